"""fp64 oracle: softmax attention, log-sum-exp merge, head re-layout.

Test infrastructure: only tests, the smoke check and the benchmark's
CPU-baseline leg use this module. Nothing here is shared with the HIP
library.

Pages followed (cited by title and section):
  * "LLM Lab Notes 05: Attention Tensor Parallelism - Splitting QKV by
    Head, Megatron Style", section 2 (code walkthrough, annotations ③④)
    and section 3: per head, scores are q.k / sqrt(head_dim), a softmax
    over the keys turns them into weights, and the output is the
    weighted sum of the value rows; heads never interact.
  * "HCMS: Head-Chunked Multi-Stream Pipeline ...", Abstract: attention
    heads are computationally independent, so any (possibly uneven)
    partition of the heads yields the same result.
  * "CHARM+: How Cross-Hardware Attention Breaks Through Distributed
    Communication Bottlenecks", section "Where Does the Communication
    Bottleneck of Distributed Attention Come From?": Ring Attention keeps
    Q local, visits the KV blocks one by one and accumulates the partial
    results until every block has been seen. CHARM+'s "Re-Merge" (title
    of the CHARM+ arXiv listing) is read as the same accumulation.
  * "db-SP: Accelerating Sparse Attention for Visual Generative Models
    with Dual-Balanced Sequence Parallelism", Abstract: block-wise sparse
    attention computes only the dense blocks of a sparse block mask.

Readings where the pages are silent:
  * log-sum-exp (LSE) is the natural log of the sum of exp(scaled score)
    over the keys a row attends to; it is the per-row statistic that lets
    partial results be merged exactly.
  * A partial result over a KV block is normalised over that block's keys
    and carries the block's LSE.
  * A row with no key to attend to (empty block, fully masked row) has
    O = 0 and LSE = -inf; merging only such partials gives the same.
  * A masked (query block, key block) pair is excluded from the softmax
    (its scores are -inf), not given a zero score.
"""
from __future__ import annotations

import numpy as np

# Query rows processed at once. Rows are independent, so blocking rows
# changes no arithmetic on any row.
_ROW_BLOCK = 256


def attention_flops(B, H, Sq, Skv, D) -> int:
    """Algorithmic flop count of one attention forward: two products of
    2*Sq*Skv*D flops each, per batch entry and head."""
    return 4 * B * H * Sq * Skv * D


def attention_ref(q, k, v, scale, block_mask=None, mask_block=128, rows=None,
                  heads=None):
    """Exact softmax attention of every head, in float64.

    q: [B, Sq, H, D]; k, v: [B, Skv, H, D]; any real dtype (upcast to fp64).
    scale: multiplier of the scores (1/sqrt(D) for the workloads).
    block_mask: optional [B, H, ceil(Sq/mask_block), ceil(Skv/mask_block)];
        query i may attend key j only if
        block_mask[b, h, i // mask_block, j // mask_block] is non-zero.
    rows: optional 1-D array of query indices; only those rows are computed
        (output row r corresponds to query rows[r]).
    heads: optional iterable of head indices to compute; other heads are
        left as NaN in the output.

    Returns O [B, R, H, D] and LSE [B, H, R] (float64), R = len(rows) or Sq.
    For each row: s_j = scale * <q, k_j> over its admissible keys j,
    LSE = log(sum_j exp(s_j)), O = sum_j exp(s_j - LSE) * v_j.
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    B, Sq, H, D = q.shape
    Bk, Skv, Hk, Dk = k.shape
    if (Bk, Hk, Dk) != (B, H, D) or v.shape != k.shape:
        raise ValueError("q, k, v shapes disagree")
    rows = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = range(H) if heads is None else list(heads)
    R = rows.size
    out = np.full((B, R, H, D), np.nan, dtype=np.float64)
    lse = np.full((B, H, R), np.nan, dtype=np.float64)
    if block_mask is not None:
        block_mask = np.asarray(block_mask)
        nqb = -(-Sq // mask_block)
        nkb = -(-Skv // mask_block)
        if block_mask.shape != (B, H, nqb, nkb):
            raise ValueError(f"block_mask shape {block_mask.shape} != {(B, H, nqb, nkb)}")
        kblock_of = np.arange(Skv) // mask_block
    for b in range(B):
        for h in heads:
            kh = k[b, :, h, :].astype(np.float64)      # [Skv, D]
            vh = v[b, :, h, :].astype(np.float64)      # [Skv, D]
            for r0 in range(0, R, _ROW_BLOCK):
                idx = rows[r0:r0 + _ROW_BLOCK]
                qh = q[b, idx, h, :].astype(np.float64)  # [r, D]
                s = (qh @ kh.T) * float(scale)           # [r, Skv]
                if block_mask is not None:
                    allowed = block_mask[b, h][idx // mask_block][:, kblock_of] != 0
                    s = np.where(allowed, s, -np.inf)
                o_blk, l_blk = _softmax_weighted_sum(s, vh)
                out[b, r0:r0 + idx.size, h, :] = o_blk
                lse[b, h, r0:r0 + idx.size] = l_blk
    return out, lse


def _softmax_weighted_sum(s, vh):
    """Rows of s are scores over the keys (-inf = excluded). Returns the
    softmax-weighted sum of the value rows and the natural-log LSE.
    Subtracting the row maximum is an exact identity that only keeps exp
    in range. Rows with no admissible key give O = 0, LSE = -inf."""
    r, n = s.shape
    o = np.zeros((r, vh.shape[1]), dtype=np.float64)
    lse = np.full(r, -np.inf, dtype=np.float64)
    if n == 0:
        return o, lse
    m = s.max(axis=1)
    live = np.isfinite(m)
    if live.any():
        e = np.exp(s[live] - m[live, None])
        l = e.sum(axis=1)
        o[live] = (e @ vh) / l[:, None]
        lse[live] = m[live] + np.log(l)
    return o, lse


def merge_ref(o_parts, lse_parts):
    """Merge n partial results over disjoint key sets into the result over
    their union (float64).

    o_parts: [n, B, Sq, H, D], each normalised over its own keys;
    lse_parts: [n, B, H, Sq]. With M = max_k LSE_k, w_k = exp(LSE_k - M),
    Z = sum_k w_k: LSE = M + log Z and O = sum_k (w_k / Z) * O_k. Rows
    where every LSE_k is -inf give O = 0, LSE = -inf.
    """
    o_parts = np.asarray(o_parts, dtype=np.float64)
    lse_parts = np.asarray(lse_parts, dtype=np.float64)
    n, B, Sq, H, D = o_parts.shape
    if lse_parts.shape != (n, B, H, Sq):
        raise ValueError("lse_parts shape disagrees with o_parts")
    M = lse_parts.max(axis=0)                       # [B, H, Sq]
    live = np.isfinite(M)
    Msafe = np.where(live, M, 0.0)
    w = np.where(live[None], np.exp(lse_parts - Msafe[None]), 0.0)   # [n,B,H,Sq]
    Z = w.sum(axis=0)
    lse = np.where(live, Msafe + np.log(np.where(live, Z, 1.0)), -np.inf)
    coef = np.where(live[None], w / np.where(live, Z, 1.0)[None], 0.0)  # [n,B,H,Sq]
    coef = coef.transpose(0, 1, 3, 2)[..., None]    # [n, B, Sq, H, 1]
    o = (coef * o_parts).sum(axis=0)
    return o, lse


def permute_ref(x, h0, hc):
    """Head-major copy of heads [h0, h0+hc): x [B, S, H, D] -> [B, hc, S, D].

    This is the local re-layout an all-to-all performs when sequence
    sharding becomes head sharding (HCMS page, Abstract; db-SP page,
    Abstract: Ulysses splits along the head dimension)."""
    x = np.asarray(x)
    return np.ascontiguousarray(x[:, :, h0:h0 + hc, :].transpose(0, 2, 1, 3))


def inverse_permute_ref(y):
    """[B, hc, S, D] -> [B, S, hc, D]."""
    return np.ascontiguousarray(np.asarray(y).transpose(0, 2, 1, 3))


def attention_bwd_ref(q, k, v, dout, scale, rows=None, keys=None, heads=None):
    """Gradients of dense softmax attention, in float64.

    The forward is attention_ref without a mask: O = P V with
    P = softmax_j(scale * <q_i, k_j>). For a loss L with dL/dO = dout
    (called dO below), the chain rule gives, per batch entry and head:

        dV = P^T dO
        dP = dO V^T
        dS = P * (dP - rowsum(P * dP))      (softmax Jacobian, row by row)
        dQ = scale * dS K
        dK = scale * dS^T Q

    The CHARM+ pages ("CHARM+: How Cross-Hardware Attention Breaks Through
    Distributed Communication Bottlenecks", section "Measured Speedups")
    report the backward pass beside the forward; the pages give no
    formulas, so this is the plain derivative of the forward they define.

    q, dout: [B, Sq, H, D]; k, v: [B, Skv, H, D]; any real dtype.
    rows: optional query indices for dQ; keys: optional key indices for dK
    and dV (the other outputs are computed over all rows / keys as the
    definition requires). heads: optional head indices; others stay NaN.
    Returns dQ [B, R, H, D], dK [B, K, H, D], dV [B, K, H, D] (float64).
    """
    q = np.asarray(q)
    k = np.asarray(k)
    v = np.asarray(v)
    dout = np.asarray(dout)
    B, Sq, H, D = q.shape
    Skv = k.shape[1]
    if k.shape != (B, Skv, H, D) or v.shape != k.shape or dout.shape != q.shape:
        raise ValueError("q, k, v, dout shapes disagree")
    rows = np.arange(Sq) if rows is None else np.asarray(rows, dtype=np.int64)
    keys = np.arange(Skv) if keys is None else np.asarray(keys, dtype=np.int64)
    heads = range(H) if heads is None else list(heads)
    dq = np.full((B, rows.size, H, D), np.nan)
    dk = np.full((B, keys.size, H, D), np.nan)
    dv = np.full((B, keys.size, H, D), np.nan)
    row_pos = {int(r): i for i, r in enumerate(rows)}
    for b in range(B):
        for h in heads:
            kh = k[b, :, h, :].astype(np.float64)
            vh = v[b, :, h, :].astype(np.float64)
            kk = kh[keys]
            dk_acc = np.zeros((keys.size, D))
            dv_acc = np.zeros((keys.size, D))
            for r0 in range(0, Sq, _ROW_BLOCK):
                idx = np.arange(r0, min(Sq, r0 + _ROW_BLOCK))
                qh = q[b, idx, h, :].astype(np.float64)
                doh = dout[b, idx, h, :].astype(np.float64)
                s = (qh @ kh.T) * float(scale)                 # [r, Skv]
                m = s.max(axis=1, keepdims=True)
                e = np.exp(s - m)
                p = e / e.sum(axis=1, keepdims=True)             # softmax over keys
                dp = doh @ vh.T                                  # [r, Skv]
                ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
                dv_acc += p[:, keys].T @ doh
                dk_acc += float(scale) * ds[:, keys].T @ qh
                sel = [i for i, r in enumerate(idx) if int(r) in row_pos]
                if sel:
                    dq_blk = float(scale) * ds[sel] @ kh
                    for j, i in enumerate(sel):
                        dq[b, row_pos[int(idx[i])], h, :] = dq_blk[j]
            dk[b, :, h, :] = dk_acc
            dv[b, :, h, :] = dv_acc
    return dq, dk, dv
