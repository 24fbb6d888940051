"""Exact long-sequence multi-head attention on MI355X (gfx950).

Python binding of liblsh.so (include/lsh.h). It only marshals arguments:
every step runs in the library's HIP kernels. PyTorch provides device
memory and streams. Tensors use the [B, S, H, D] layout with D contiguous
(any (b, s, h) strides whose byte sizes are multiples of 16); O is
float32 [B, Sq, H, D] and LSE float32 [B, H, Sq].

Functions:
  attn_fwd            dense attention forward
  attn_fwd_chunked    head-chunked two-stream forward (head-major copies
                      of each chunk on a second stream, overlapped with
                      the previous chunk's attention)
  attn_partial        attention against one KV block (a Ring round)
  attn_partial_accumulate  one KV block folded into a running (O, LSE)
  lse_merge           merge of per-block partial results
  head_permute        [B, S, H, D] -> [B, hc, S, D] copy of heads [h0, h0+hc)
  attn_fwd_blocksparse  attention restricted to a 128x128 block mask
  attn_fwd_blocksparse_noalloc  the same without a workspace (its schedule
                      goes to the library's static device array)
  attn_bwd            gradients dQ, dK, dV of the dense forward (bf16)

Submodule balance: host-side load-balance diagnostics of the block-sparse
work (imbalance ratios of head and row splits, and of the launch schedule
the library leaves in its workspace).
"""
from __future__ import annotations

import ctypes
import math

from . import _lib
from ._lib import LshError, load  # noqa: F401

__all__ = ["attn_fwd", "attn_fwd_chunked", "attn_partial", "attn_partial_accumulate",
           "lse_merge", "head_permute",
           "attn_fwd_blocksparse", "attn_fwd_blocksparse_noalloc", "attn_bwd", "bwd_workspace_bytes",
           "chunked_workspace_bytes", "blocksparse_workspace_bytes",
           "LshError", "load", "MASK_BLOCK"]

MASK_BLOCK = 128


def _torch():
    import torch
    return torch


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return _lib.LSH_BF16
    if t.dtype == torch.float32:
        return _lib.LSH_F32
    raise TypeError(f"unsupported dtype {t.dtype}; expected bfloat16 or float32")


def _check4(name, t):
    if t.dim() != 4:
        raise ValueError(f"{name} must be 4-D [B, S, H, D], got shape {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.stride(-1) != 1:
        raise ValueError(f"{name}: head_dim must be contiguous")


def _stream_ptr(stream):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _outputs(q, o, lse, Skv_ok=True):
    torch = _torch()
    B, Sq, H, D = q.shape
    if o is None:
        o = torch.empty((B, Sq, H, D), dtype=torch.float32, device=q.device)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=q.device)
    if o.dtype != torch.float32 or tuple(o.shape) != (B, Sq, H, D) or o.stride(-1) != 1:
        raise ValueError("o must be float32 [B, Sq, H, D] with contiguous head_dim")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, Sq) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, H, Sq]")
    return o, lse


def _args(q, k, v, o, lse, scale):
    _check4("q", q)
    B, Sq, H, D = q.shape
    a = _lib.AttnArgs()
    a.q = q.data_ptr()
    a.o = o.data_ptr()
    a.lse = lse.data_ptr()
    a.dtype = _dtype_code(q)
    a.reserved = 0
    a.B, a.Sq, a.H, a.D = B, Sq, H, D
    if k is not None:
        _check4("k", k)
        _check4("v", v)
        if k.dtype != q.dtype or v.dtype != q.dtype:
            raise TypeError("q, k, v must share a dtype")
        if k.shape != v.shape or k.shape[0] != B or k.shape[2] != H or k.shape[3] != D:
            raise ValueError(f"k/v shape {tuple(k.shape)}/{tuple(v.shape)} does not match q {tuple(q.shape)}")
        a.k = k.data_ptr()
        a.v = v.data_ptr()
        a.Skv = k.shape[1]
        a.k_stride[:] = [k.stride(0), k.stride(1), k.stride(2)]
        a.v_stride[:] = [v.stride(0), v.stride(1), v.stride(2)]
    else:
        a.k = a.v = None
        a.Skv = 0
    a.q_stride[:] = [q.stride(0), q.stride(1), q.stride(2)]
    a.o_stride[:] = [o.stride(0), o.stride(1), o.stride(2)]
    a.scale = float(1.0 / math.sqrt(D) if scale is None else scale)
    return a


def attn_fwd(q, k, v, scale=None, o=None, lse=None, stream=None):
    """Dense attention forward. Returns (O float32 [B,Sq,H,D], LSE float32 [B,H,Sq])."""
    lib = load()
    o, lse = _outputs(q, o, lse)
    a = _args(q, k, v, o, lse, scale)
    _lib.check("lsh_attn_fwd", lib.lsh_attn_fwd(ctypes.byref(a), _stream_ptr(stream)))
    return o, lse


def attn_partial(q, k, v, scale=None, o=None, lse=None, stream=None):
    """Attention against one KV block; k and v may hold zero keys (O = 0,
    LSE = -inf). O is normalised over the block's keys."""
    lib = load()
    o, lse = _outputs(q, o, lse)
    empty = k is None or k.shape[1] == 0
    a = _args(q, None if empty else k, None if empty else v, o, lse, scale)
    _lib.check("lsh_attn_partial", lib.lsh_attn_partial(ctypes.byref(a), _stream_ptr(stream)))
    return o, lse


def attn_partial_accumulate(q, k, v, o, lse, scale=None, stream=None):
    """Fold attention against one KV block into a running result, in
    place: o, lse hold attention over the blocks folded so far (O = 0,
    LSE = -inf before the first) and afterwards over those and this one.
    k and v may hold zero keys (nothing changes). Returns (o, lse)."""
    lib = load()
    o, lse = _outputs(q, o, lse)
    empty = k is None or k.shape[1] == 0
    a = _args(q, None if empty else k, None if empty else v, o, lse, scale)
    _lib.check("lsh_attn_partial_accumulate",
               lib.lsh_attn_partial_accumulate(ctypes.byref(a), _stream_ptr(stream)))
    return o, lse


def chunked_workspace_bytes(q, k, v):
    lib = load()
    torch = _torch()
    B, Sq, H, D = q.shape
    o = torch.empty(0, dtype=torch.float32, device=q.device)
    a = _args(q, k, v, o.new_empty((B, Sq, H, D)), o.new_empty((B, H, Sq)), None)
    return int(lib.lsh_attn_fwd_chunked_workspace(ctypes.byref(a)))


_perm_streams = {}


def _permute_stream(device):
    torch = _torch()
    key = device.index if device.index is not None else torch.cuda.current_device()
    s = _perm_streams.get(key)
    if s is None:
        s = torch.cuda.Stream(device=device)   # default priority
        _perm_streams[key] = s
    return s


def attn_fwd_chunked(q, k, v, head_chunks, scale=None, o=None, lse=None, workspace=None,
                     compute_stream=None, permute_stream=None):
    """Head-chunked forward: heads split into `head_chunks` (ascending
    contiguous ranges, sizes may differ); each chunk's Q/K/V are copied
    head-major on `permute_stream` while the previous chunk's attention runs
    on `compute_stream`. Bit-identical to attn_fwd."""
    lib = load()
    torch = _torch()
    o, lse = _outputs(q, o, lse)
    a = _args(q, k, v, o, lse, scale)
    need = int(lib.lsh_attn_fwd_chunked_workspace(ctypes.byref(a)))
    if workspace is None:
        workspace = torch.empty(need + 256, dtype=torch.uint8, device=q.device)
    base = workspace.data_ptr()
    aligned = (base + 255) // 256 * 256
    avail = workspace.numel() - (aligned - base)
    sc = torch.cuda.current_stream() if compute_stream is None else compute_stream
    sp = _permute_stream(q.device) if permute_stream is None else permute_stream
    chunks = (ctypes.c_int32 * len(head_chunks))(*[int(c) for c in head_chunks])
    st = lib.lsh_attn_fwd_chunked(ctypes.byref(a), chunks, len(head_chunks), ctypes.c_void_p(aligned),
                                  avail, ctypes.c_void_p(sc.cuda_stream), ctypes.c_void_p(sp.cuda_stream))
    _lib.check("lsh_attn_fwd_chunked", st)
    # The caching allocator must not hand these out again while another
    # stream than the current one still uses them.
    cur = torch.cuda.current_stream(q.device)
    for s_ in {sp, sc}:
        if s_ != cur:
            for t in (workspace, q, k, v, o, lse):
                t.record_stream(s_)
    return o, lse


def lse_merge(o_parts, lse_parts, o=None, lse=None, stream=None):
    """Merge n partial results: o_parts float32 [n,B,Sq,H,D], lse_parts
    float32 [n,B,H,Sq] (both contiguous). Returns (O, LSE)."""
    lib = load()
    torch = _torch()
    if o_parts.dim() != 5 or lse_parts.dim() != 4:
        raise ValueError("o_parts must be [n,B,Sq,H,D] and lse_parts [n,B,H,Sq]")
    if not (o_parts.is_contiguous() and lse_parts.is_contiguous()):
        raise ValueError("o_parts and lse_parts must be contiguous")
    if o_parts.dtype != torch.float32 or lse_parts.dtype != torch.float32:
        raise TypeError("o_parts and lse_parts must be float32")
    n, B, Sq, H, D = o_parts.shape
    if tuple(lse_parts.shape) != (n, B, H, Sq):
        raise ValueError("lse_parts shape does not match o_parts")
    if o is None:
        o = torch.empty((B, Sq, H, D), dtype=torch.float32, device=o_parts.device)
    if lse is None:
        lse = torch.empty((B, H, Sq), dtype=torch.float32, device=o_parts.device)
    if not (o.is_contiguous() and lse.is_contiguous()):
        raise ValueError("o and lse must be contiguous")
    st = lib.lsh_lse_merge(ctypes.c_void_p(o_parts.data_ptr()), ctypes.c_void_p(lse_parts.data_ptr()),
                           n, B, Sq, H, D, ctypes.c_void_p(o.data_ptr()), ctypes.c_void_p(lse.data_ptr()),
                           _stream_ptr(stream))
    _lib.check("lsh_lse_merge", st)
    return o, lse


def head_permute(x, h0, hc, out=None, stream=None):
    """[B, S, H, D] (contiguous) -> [B, hc, S, D] copy of heads [h0, h0+hc)."""
    lib = load()
    torch = _torch()
    if x.dim() != 4 or not x.is_contiguous():
        raise ValueError("x must be contiguous [B, S, H, D]")
    B, S, H, D = x.shape
    if out is None:
        out = torch.empty((B, hc, S, D), dtype=x.dtype, device=x.device)
    if tuple(out.shape) != (B, hc, S, D) or not out.is_contiguous() or out.dtype != x.dtype:
        raise ValueError("out must be contiguous [B, hc, S, D] of x's dtype")
    st = lib.lsh_head_permute(ctypes.c_void_p(x.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                              _dtype_code(x), B, S, H, D, int(h0), int(hc), _stream_ptr(stream))
    _lib.check("lsh_head_permute", st)
    return out


def blocksparse_workspace_bytes(q, k, v):
    lib = load()
    torch = _torch()
    B, Sq, H, D = q.shape
    o = torch.empty(0, dtype=torch.float32, device=q.device)
    a = _args(q, k, v, o.new_empty((B, Sq, H, D)), o.new_empty((B, H, Sq)), None)
    return int(lib.lsh_attn_fwd_blocksparse_workspace(ctypes.byref(a)))


def attn_fwd_blocksparse(q, k, v, block_mask, scale=None, o=None, lse=None, workspace=None,
                         stream=None):
    """Attention restricted to a block mask: block_mask uint8 GPU tensor
    [B, H, ceil(Sq/128), ceil(Skv/128)]; query i attends key j iff
    block_mask[b, h, i//128, j//128] != 0."""
    lib = load()
    torch = _torch()
    o, lse = _outputs(q, o, lse)
    a = _args(q, k, v, o, lse, scale)
    B, Sq, H, _ = q.shape
    Skv = k.shape[1]
    want = (B, H, -(-Sq // MASK_BLOCK), -(-Skv // MASK_BLOCK))
    if block_mask.dtype != torch.uint8 or tuple(block_mask.shape) != want or not block_mask.is_contiguous():
        raise ValueError(f"block_mask must be contiguous uint8 {want}")
    if not block_mask.is_cuda:
        raise ValueError("block_mask must be a GPU tensor")
    need = int(lib.lsh_attn_fwd_blocksparse_workspace(ctypes.byref(a)))
    if workspace is None:
        workspace = torch.empty(need + 256, dtype=torch.uint8, device=q.device)
    base = workspace.data_ptr()
    aligned = (base + 255) // 256 * 256
    st = lib.lsh_attn_fwd_blocksparse(ctypes.byref(a), ctypes.c_void_p(block_mask.data_ptr()),
                                      ctypes.c_void_p(aligned), workspace.numel() - (aligned - base),
                                      _stream_ptr(stream))
    _lib.check("lsh_attn_fwd_blocksparse", st)
    return o, lse


def attn_fwd_blocksparse_noalloc(q, k, v, block_mask, scale=None, o=None, lse=None,
                                 stream=None):
    """attn_fwd_blocksparse without a workspace: the launch schedule goes to
    the library's static device array (no allocation in the library; pass o
    and lse to allocate nothing here either). Calls overlapping on one GPU
    race on that array."""
    lib = load()
    torch = _torch()
    o, lse = _outputs(q, o, lse)
    a = _args(q, k, v, o, lse, scale)
    B, Sq, H, _ = q.shape
    Skv = k.shape[1]
    want = (B, H, -(-Sq // MASK_BLOCK), -(-Skv // MASK_BLOCK))
    if block_mask.dtype != torch.uint8 or tuple(block_mask.shape) != want or not block_mask.is_contiguous():
        raise ValueError(f"block_mask must be contiguous uint8 {want}")
    if not block_mask.is_cuda:
        raise ValueError("block_mask must be a GPU tensor")
    st = lib.lsh_attn_fwd_blocksparse_noalloc(ctypes.byref(a), ctypes.c_void_p(block_mask.data_ptr()),
                                              _stream_ptr(stream))
    _lib.check("lsh_attn_fwd_blocksparse_noalloc", st)
    return o, lse


def _bwd_args(q, k, v, dout, o, lse, dq, dk, dv, scale):
    torch = _torch()
    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _check4(name, t)
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16 (the backward supports bf16 only)")
    B, Sq, H, D = q.shape
    Skv = k.shape[1]
    if k.shape != v.shape or k.shape[0] != B or k.shape[2] != H or k.shape[3] != D:
        raise ValueError(f"k/v shape {tuple(k.shape)}/{tuple(v.shape)} does not match q {tuple(q.shape)}")
    if dout.shape != q.shape:
        raise ValueError("dout must have the shape of q")
    for name, t, shape in (("o", o, q.shape), ("dq", dq, q.shape), ("dk", dk, k.shape),
                           ("dv", dv, k.shape)):
        if t.dtype != torch.float32 or tuple(t.shape) != tuple(shape) or t.stride(-1) != 1:
            raise ValueError(f"{name} must be float32 {tuple(shape)} with contiguous head_dim")
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, Sq) or not lse.is_contiguous():
        raise ValueError("lse must be contiguous float32 [B, H, Sq]")
    a = _lib.AttnBwdArgs()
    a.q, a.k, a.v, a.dout = q.data_ptr(), k.data_ptr(), v.data_ptr(), dout.data_ptr()
    a.o, a.lse = o.data_ptr(), lse.data_ptr()
    a.dq, a.dk, a.dv = dq.data_ptr(), dk.data_ptr(), dv.data_ptr()
    a.dtype, a.reserved = _lib.LSH_BF16, 0
    a.B, a.Sq, a.Skv, a.H, a.D = B, Sq, Skv, H, D
    for field, t in (("q_stride", q), ("k_stride", k), ("v_stride", v), ("do_stride", dout),
                     ("o_stride", o), ("dq_stride", dq), ("dk_stride", dk), ("dv_stride", dv)):
        getattr(a, field)[:] = [t.stride(0), t.stride(1), t.stride(2)]
    a.scale = float(1.0 / math.sqrt(D) if scale is None else scale)
    return a


def bwd_workspace_bytes(q, k, v):
    """Workspace bytes lsh_attn_bwd needs for these shapes: the header's
    B * H * ceil(Sq / 64) * 512 (lsh_attn_bwd_workspace)."""
    B, Sq, H, _ = q.shape
    return B * H * (-(-Sq // 64)) * 512


def attn_bwd(q, k, v, dout, o, lse, scale=None, dq=None, dk=None, dv=None, workspace=None,
             stream=None):
    """Gradients of the dense forward: q, k, v, dout bfloat16 [B, S, H, D];
    o and lse the forward's float32 outputs. Returns (dQ, dK, dV) float32."""
    lib = load()
    torch = _torch()
    if dq is None:
        dq = torch.empty(q.shape, dtype=torch.float32, device=q.device)
    if dk is None:
        dk = torch.empty(k.shape, dtype=torch.float32, device=q.device)
    if dv is None:
        dv = torch.empty(v.shape, dtype=torch.float32, device=q.device)
    a = _bwd_args(q, k, v, dout, o, lse, dq, dk, dv, scale)
    need = int(lib.lsh_attn_bwd_workspace(ctypes.byref(a)))
    if need == 0:
        _lib.check("lsh_attn_bwd_workspace", _lib.LSH_ERR_INVALID)
    if workspace is None:
        workspace = torch.empty(need + 256, dtype=torch.uint8, device=q.device)
    base = workspace.data_ptr()
    aligned = (base + 255) // 256 * 256
    st = lib.lsh_attn_bwd(ctypes.byref(a), ctypes.c_void_p(aligned),
                          workspace.numel() - (aligned - base), _stream_ptr(stream))
    _lib.check("lsh_attn_bwd", st)
    return dq, dk, dv
