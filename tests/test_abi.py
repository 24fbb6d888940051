"""liblsh.so loads, exports every function include/lsh.h declares, and
rejects bad arguments before touching a device. CPU only: no kernel is
launched (pointers below are never dereferenced; validation fails first,
or no device is found)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lsh.h")

L = pytest.importorskip("long_sequence_head_amd")
from long_sequence_head_amd import _lib  # noqa: E402


def _lib_or_skip():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("liblsh.so not built")
    return _lib.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b(lsh_[a-z0-9_]+)\s*\(", text)
    return sorted(set(names))


def test_header_declares_the_boundary():
    names = declared_functions()
    for want in ["lsh_attn_fwd_chunked", "lsh_attn_partial", "lsh_lse_merge", "lsh_head_permute",
                 "lsh_attn_fwd_blocksparse", "lsh_attn_fwd"]:
        assert want in names
    assert set(names) == set(_lib.SIGNATURES), "binding and header disagree"


def test_library_exports_every_declared_symbol():
    lib = _lib_or_skip()
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s+(lsh_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_abi_version_and_status_strings():
    lib = _lib_or_skip()
    assert lib.lsh_abi_version() == 1
    for s in range(6):
        assert lib.lsh_status_str(s)
    assert lib.lsh_status_str(99) == b"unknown status"


def _valid_args(dtype=_lib.LSH_BF16, B=1, Sq=300, Skv=257, H=4, D=128):
    a = _lib.AttnArgs()
    fake = 1 << 20  # 16-byte aligned, never dereferenced
    a.q, a.k, a.v, a.o, a.lse = fake, fake * 2, fake * 3, fake * 4, fake * 5
    a.dtype, a.reserved = dtype, 0
    a.B, a.Sq, a.Skv, a.H, a.D = B, Sq, Skv, H, D
    a.q_stride[:] = [Sq * H * D, H * D, D]
    a.k_stride[:] = [Skv * H * D, H * D, D]
    a.v_stride[:] = [Skv * H * D, H * D, D]
    a.o_stride[:] = [Sq * H * D, H * D, D]
    a.scale = 0.088
    return a


def _call_fwd(lib, a):
    return lib.lsh_attn_fwd(ctypes.byref(a), None)


BAD_CASES = [
    ("null q", lambda a: setattr(a, "q", None), _lib.LSH_ERR_INVALID),
    ("null o", lambda a: setattr(a, "o", None), _lib.LSH_ERR_INVALID),
    ("null lse", lambda a: setattr(a, "lse", None), _lib.LSH_ERR_INVALID),
    ("null k", lambda a: setattr(a, "k", None), _lib.LSH_ERR_INVALID),
    ("bad dtype", lambda a: setattr(a, "dtype", 7), _lib.LSH_ERR_INVALID),
    ("reserved", lambda a: setattr(a, "reserved", 1), _lib.LSH_ERR_INVALID),
    ("B=0", lambda a: setattr(a, "B", 0), _lib.LSH_ERR_INVALID),
    ("Sq=0", lambda a: setattr(a, "Sq", 0), _lib.LSH_ERR_INVALID),
    ("Skv=0 dense", lambda a: setattr(a, "Skv", 0), _lib.LSH_ERR_INVALID),
    ("H=0", lambda a: setattr(a, "H", 0), _lib.LSH_ERR_INVALID),
    ("D=64", lambda a: setattr(a, "D", 64), _lib.LSH_ERR_UNSUPPORTED),
    ("misaligned q", lambda a: setattr(a, "q", (1 << 20) + 8), _lib.LSH_ERR_INVALID),
    ("odd stride", lambda a: a.q_stride.__setitem__(1, 4 * 128 + 3), _lib.LSH_ERR_INVALID),
    ("negative stride", lambda a: a.k_stride.__setitem__(2, -128), _lib.LSH_ERR_INVALID),
    ("nan scale", lambda a: setattr(a, "scale", float("nan")), _lib.LSH_ERR_INVALID),
    ("huge S", lambda a: setattr(a, "Sq", 1 << 31), _lib.LSH_ERR_UNSUPPORTED),
    # 2^20 keys x a 2048-element key stride x 2 bytes = 4 GiB of one head's rows
    ("K span over 2 GiB", lambda a: (setattr(a, "Skv", 1 << 20), a.k_stride.__setitem__(1, 2048)),
     _lib.LSH_ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("name,mutate,want", BAD_CASES, ids=[c[0] for c in BAD_CASES])
def test_attn_fwd_rejects(name, mutate, want):
    lib = _lib_or_skip()
    a = _valid_args()
    mutate(a)
    assert _call_fwd(lib, a) == want
    assert lib.lsh_last_error()


def test_null_args_pointer():
    lib = _lib_or_skip()
    assert lib.lsh_attn_fwd(None, None) == _lib.LSH_ERR_INVALID
    assert lib.lsh_attn_partial(None, None) == _lib.LSH_ERR_INVALID
    assert lib.lsh_attn_partial_accumulate(None, None) == _lib.LSH_ERR_INVALID
    assert lib.lsh_attn_fwd_chunked_workspace(None) == 0
    assert lib.lsh_attn_fwd_blocksparse_workspace(None) == 0


def _torch_cuda():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_torch_cuda(), reason="checks the no-device path")
def test_valid_args_without_device_report_no_device():
    lib = _lib_or_skip()
    a = _valid_args()
    assert _call_fwd(lib, a) == _lib.LSH_ERR_NO_DEVICE
    assert lib.lsh_attn_partial(ctypes.byref(a), None) == _lib.LSH_ERR_NO_DEVICE
    assert lib.lsh_attn_partial_accumulate(ctypes.byref(a), None) == _lib.LSH_ERR_NO_DEVICE
    assert lib.lsh_device_check() == _lib.LSH_ERR_NO_DEVICE


def test_partial_allows_empty_block():
    lib = _lib_or_skip()
    a = _valid_args(Skv=0)
    a.k = a.v = None
    st = lib.lsh_attn_partial(ctypes.byref(a), None)
    assert st in (_lib.LSH_OK, _lib.LSH_ERR_NO_DEVICE)   # valid arguments
    st = lib.lsh_attn_partial_accumulate(ctypes.byref(a), None)
    assert st in (_lib.LSH_OK, _lib.LSH_ERR_NO_DEVICE)
    assert lib.lsh_attn_fwd(ctypes.byref(a), None) == _lib.LSH_ERR_INVALID


def test_chunked_validation():
    lib = _lib_or_skip()
    a = _valid_args(Sq=300, Skv=300, H=40)
    need = lib.lsh_attn_fwd_chunked_workspace(ctypes.byref(a))
    assert need == 3 * ((1 * 40 * 300 * 128 * 2 + 255) // 256 * 256)
    ws = 1 << 24

    def call(chunks, ws_ptr=ws, ws_bytes=need, args=a):
        arr = (ctypes.c_int32 * max(1, len(chunks)))(*chunks)
        return lib.lsh_attn_fwd_chunked(ctypes.byref(args), arr, len(chunks), ws_ptr, ws_bytes, None, None)

    assert call([16, 12, 11]) == _lib.LSH_ERR_INVALID      # sums to 39
    assert call([16, 0, 24]) == _lib.LSH_ERR_INVALID       # empty chunk
    assert call([]) == _lib.LSH_ERR_INVALID
    assert call([16, 12, 12], ws_bytes=need - 1) == _lib.LSH_ERR_WORKSPACE
    assert call([16, 12, 12], ws_ptr=None) == _lib.LSH_ERR_WORKSPACE
    assert call([16, 12, 12], ws_ptr=ws + 16) == _lib.LSH_ERR_WORKSPACE   # alignment
    b = _valid_args(Sq=300, Skv=301, H=40)
    assert call([40], args=b) == _lib.LSH_ERR_INVALID                      # Sq != Skv
    c = _valid_args(Sq=300, Skv=300, H=40)
    c.q_stride[1] = 2 * 40 * 128
    assert call([40], args=c) == _lib.LSH_ERR_INVALID                      # non-contiguous input
    if not _torch_cuda():
        assert call([16, 12, 12]) == _lib.LSH_ERR_NO_DEVICE


def test_merge_and_permute_validation():
    lib = _lib_or_skip()
    p = 1 << 20
    assert lib.lsh_lse_merge(None, p, 2, 1, 8, 2, 128, p, p, None) == _lib.LSH_ERR_INVALID
    assert lib.lsh_lse_merge(p, p, 0, 1, 8, 2, 128, p, p, None) == _lib.LSH_ERR_INVALID
    assert lib.lsh_lse_merge(p, p, 2, 1, 8, 2, 64, p, p, None) == _lib.LSH_ERR_UNSUPPORTED
    assert lib.lsh_lse_merge(p + 4, p, 2, 1, 8, 2, 128, p, p, None) == _lib.LSH_ERR_INVALID
    assert lib.lsh_head_permute(p, p, 1, 1, 8, 4, 128, 3, 2, None) == _lib.LSH_ERR_INVALID  # 3+2 > 4
    assert lib.lsh_head_permute(p, p, 1, 1, 8, 4, 128, -1, 2, None) == _lib.LSH_ERR_INVALID
    assert lib.lsh_head_permute(p, p, 1, 1, 8, 4, 4, 0, 2, None) == _lib.LSH_ERR_INVALID    # 8-byte rows
    assert lib.lsh_head_permute(p, None, 1, 1, 8, 4, 128, 0, 2, None) == _lib.LSH_ERR_INVALID
    if not _torch_cuda():
        assert lib.lsh_lse_merge(p, p, 2, 1, 8, 2, 128, p, p, None) == _lib.LSH_ERR_NO_DEVICE
        assert lib.lsh_head_permute(p, p, 1, 1, 8, 4, 128, 0, 2, None) == _lib.LSH_ERR_NO_DEVICE


def test_blocksparse_validation():
    lib = _lib_or_skip()
    a = _valid_args(Sq=300, Skv=257, H=4)
    need = lib.lsh_attn_fwd_blocksparse_workspace(ctypes.byref(a))
    # counts and order (int32 per item), totals (int64 per head), kept lists
    # (uint16 per item and key block), XCD placement (int32 per head + 8),
    # each rounded up to 256 bytes
    assert need == 2 * ((4 * 3 * 4 + 255) // 256 * 256) + (4 * 8 + 255) // 256 * 256 + \
        (4 * 3 * 3 * 2 + 255) // 256 * 256 + ((4 + 8) * 4 + 255) // 256 * 256
    m = 1 << 22
    assert lib.lsh_attn_fwd_blocksparse(ctypes.byref(a), None, m, need, None) == _lib.LSH_ERR_INVALID
    assert lib.lsh_attn_fwd_blocksparse(ctypes.byref(a), m, m, need - 1, None) == _lib.LSH_ERR_WORKSPACE
    if not _torch_cuda():
        assert lib.lsh_attn_fwd_blocksparse(ctypes.byref(a), m, m, need, None) == _lib.LSH_ERR_NO_DEVICE


def test_blocksparse_noalloc_validation():
    """The allocation-free entry point checks its arguments like the
    workspace one and refuses, before any HIP call, a schedule larger than
    its static array (16 MiB: 8 bytes per query block, 2 per query and key
    block, 8 per head)."""
    lib = _lib_or_skip()
    a = _valid_args(Sq=300, Skv=257, H=4)
    m = 1 << 22
    fn = lib.lsh_attn_fwd_blocksparse_noalloc
    assert fn(ctypes.byref(a), None, None) == _lib.LSH_ERR_INVALID
    assert fn(None, m, None) == _lib.LSH_ERR_INVALID
    big = _valid_args(Sq=128 * 300, Skv=128, H=8192)
    for f in ("q_stride", "k_stride", "v_stride", "o_stride"):
        getattr(big, f)[:] = [0, 0, 0]
    need = lib.lsh_attn_fwd_blocksparse_workspace(ctypes.byref(big))
    assert need > (16 << 20)
    assert fn(ctypes.byref(big), m, None) == _lib.LSH_ERR_WORKSPACE
    assert b"static scratch" in lib.lsh_last_error()
    if not _torch_cuda():
        assert fn(ctypes.byref(a), m, None) == _lib.LSH_ERR_NO_DEVICE


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    with pytest.raises(RuntimeError, match="build the HIP library"):
        _lib.load(str(tmp_path / "missing.so"))


def _valid_bwd_args(B=1, Sq=300, Skv=257, H=4, D=128):
    a = _lib.AttnBwdArgs()
    fake = 1 << 20  # 16-byte aligned, never dereferenced
    (a.q, a.k, a.v, a.dout, a.o, a.lse, a.dq, a.dk, a.dv) = [fake * i for i in range(1, 10)]
    a.dtype, a.reserved = _lib.LSH_BF16, 0
    a.B, a.Sq, a.Skv, a.H, a.D = B, Sq, Skv, H, D
    for f in ("q_stride", "do_stride", "o_stride", "dq_stride"):
        getattr(a, f)[:] = [Sq * H * D, H * D, D]
    for f in ("k_stride", "v_stride", "dk_stride", "dv_stride"):
        getattr(a, f)[:] = [Skv * H * D, H * D, D]
    a.scale = 0.088
    return a


BWD_BAD_CASES = [
    ("null dout", lambda a: setattr(a, "dout", None), _lib.LSH_ERR_INVALID),
    ("null dq", lambda a: setattr(a, "dq", None), _lib.LSH_ERR_INVALID),
    ("null lse", lambda a: setattr(a, "lse", None), _lib.LSH_ERR_INVALID),
    ("f32 inputs", lambda a: setattr(a, "dtype", _lib.LSH_F32), _lib.LSH_ERR_UNSUPPORTED),
    ("bad dtype", lambda a: setattr(a, "dtype", 5), _lib.LSH_ERR_INVALID),
    ("reserved", lambda a: setattr(a, "reserved", 2), _lib.LSH_ERR_INVALID),
    ("Skv=0", lambda a: setattr(a, "Skv", 0), _lib.LSH_ERR_INVALID),
    ("D=64", lambda a: setattr(a, "D", 64), _lib.LSH_ERR_UNSUPPORTED),
    ("misaligned dk", lambda a: setattr(a, "dk", (1 << 20) + 4), _lib.LSH_ERR_INVALID),
    ("odd dO stride", lambda a: a.do_stride.__setitem__(1, 4 * 128 + 4), _lib.LSH_ERR_INVALID),
    ("odd dv stride", lambda a: a.dv_stride.__setitem__(1, 4 * 128 + 2), _lib.LSH_ERR_INVALID),
    ("inf scale", lambda a: setattr(a, "scale", float("inf")), _lib.LSH_ERR_INVALID),
    ("huge Skv", lambda a: setattr(a, "Skv", 1 << 30), _lib.LSH_ERR_UNSUPPORTED),
    # 2^20 query rows x a 2048-element stride x 2 bytes = 4 GiB of one head's rows
    ("Q span over 2 GiB", lambda a: (setattr(a, "Sq", 1 << 20), a.q_stride.__setitem__(1, 2048)),
     _lib.LSH_ERR_UNSUPPORTED),
    ("dO span over 2 GiB", lambda a: (setattr(a, "Sq", 1 << 20), a.do_stride.__setitem__(1, 2048)),
     _lib.LSH_ERR_UNSUPPORTED),
]


@pytest.mark.parametrize("name,mutate,want", BWD_BAD_CASES, ids=[c[0] for c in BWD_BAD_CASES])
def test_attn_bwd_rejects(name, mutate, want):
    lib = _lib_or_skip()
    a = _valid_bwd_args()
    need = lib.lsh_attn_bwd_workspace(ctypes.byref(a))
    mutate(a)
    assert lib.lsh_attn_bwd(ctypes.byref(a), 1 << 24, need, None) == want
    assert lib.lsh_last_error()
    assert lib.lsh_attn_bwd_workspace(ctypes.byref(a)) == 0


def test_attn_bwd_workspace():
    lib = _lib_or_skip()
    a = _valid_bwd_args(B=2, Sq=300, Skv=257, H=4)
    need = lib.lsh_attn_bwd_workspace(ctypes.byref(a))
    assert need == 2 * 4 * 5 * 512
    import torch
    q = torch.empty(2, 300, 4, 128)
    assert L.bwd_workspace_bytes(q, None, None) == need
    assert lib.lsh_attn_bwd(None, 1 << 24, need, None) == _lib.LSH_ERR_INVALID
    assert lib.lsh_attn_bwd(ctypes.byref(a), 1 << 24, need - 1, None) == _lib.LSH_ERR_WORKSPACE
    assert lib.lsh_attn_bwd(ctypes.byref(a), None, need, None) == _lib.LSH_ERR_WORKSPACE
    assert lib.lsh_attn_bwd(ctypes.byref(a), (1 << 24) + 16, need, None) == _lib.LSH_ERR_WORKSPACE
    if not _torch_cuda():
        assert lib.lsh_attn_bwd(ctypes.byref(a), 1 << 24, need, None) == _lib.LSH_ERR_NO_DEVICE


def test_row_span_limit_is_exact():
    """One head's rows may span up to 2^31 - 1 bytes: with 64 interleaved
    heads (16 KiB per row) 131072 rows are accepted and 131073 are not, for
    K/V in the forward and Q/dO in the backward."""
    lib = _lib_or_skip()
    ok = _lib.LSH_ERR_NO_DEVICE if not _torch_cuda() else _lib.LSH_OK
    a = _valid_args(Sq=130, Skv=131072, H=64)
    assert lib.lsh_attn_fwd(ctypes.byref(a), None) in (ok, _lib.LSH_ERR_NO_DEVICE)
    a = _valid_args(Sq=130, Skv=131073, H=64)
    assert lib.lsh_attn_fwd(ctypes.byref(a), None) == _lib.LSH_ERR_UNSUPPORTED
    b = _valid_bwd_args(Sq=131072, Skv=200, H=64)
    need = lib.lsh_attn_bwd_workspace(ctypes.byref(b))
    assert need > 0
    if not _torch_cuda():
        assert lib.lsh_attn_bwd(ctypes.byref(b), 1 << 24, need, None) == _lib.LSH_ERR_NO_DEVICE
    b = _valid_bwd_args(Sq=131073, Skv=200, H=64)
    assert lib.lsh_attn_bwd(ctypes.byref(b), 1 << 24, 1 << 40, None) == _lib.LSH_ERR_UNSUPPORTED
