"""Pins that tie the fp64 oracle to something other than itself.

Each pin takes the attention function (signature of
``oracle.attention_ref``) and/or the merge function (signature of
``oracle.merge_ref``) and raises AssertionError when the function
disagrees with a fact fixed by the mathematics or by the pages:
closed forms, a hand-derived worked example, brute force in arbitrary
precision, a library softmax, and invariants (KV split + merge, head
partition, key permutation, key shift, block-mask special cases).

The mutation tests run the same pins against deliberately broken copies
of the oracle and require at least one pin to fail for each.
"""
from __future__ import annotations

import math
import os

import mpmath
import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")

TOL = 1e-12


def _rng(seed):
    return np.random.default_rng(seed)


def _close(a, b, tol=TOL, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    both_inf = np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b))
    diff = np.where(both_inf, 0.0, np.abs(a - b))
    scale = np.maximum(1.0, np.where(both_inf, 1.0, np.abs(b)))
    bad = ~(diff <= tol * scale)
    assert not bad.any(), f"{what}: max err {np.nanmax(np.where(both_inf, 0, diff))}"


def _qkv(seed, B, Sq, Skv, H, D):
    r = _rng(seed)
    return (r.standard_normal((B, Sq, H, D)), r.standard_normal((B, Skv, H, D)),
            r.standard_normal((B, Skv, H, D)))


# ---------------------------------------------------------------- closed forms

def pin_constant_v(attn, merge=None):
    """v_j = c for every key  =>  O_i = c (weights sum to one)."""
    q, k, _ = _qkv(1, 2, 5, 7, 3, 4)
    c = np.array([1.5, -2.0, 0.25, 3.0])
    v = np.broadcast_to(c, k.shape).copy()
    o, _ = attn(q, k, v, 0.5)
    _close(o, np.broadcast_to(c, o.shape), what="constant V")


def pin_identical_keys(attn, merge=None):
    """k_j = kappa for every key  =>  O_i = mean_j v_j and
    LSE_i = scale*<q_i, kappa> + ln Skv."""
    B, Sq, Skv, H, D = 1, 4, 6, 2, 3
    q, _, v = _qkv(2, B, Sq, Skv, H, D)
    kappa = np.array([[0.3, -1.2, 2.0], [1.0, 0.5, -0.7]])     # per head
    k = np.broadcast_to(kappa[None, None], (B, Skv, H, D)).copy()
    scale = 0.7
    o, lse = attn(q, k, v, scale)
    for h in range(H):
        mean_v = [math.fsum(v[0, j, h, d] for j in range(Skv)) / Skv for d in range(D)]
        for i in range(Sq):
            _close(o[0, i, h], mean_v, what="identical keys O")
            dot = math.fsum(q[0, i, h, d] * kappa[h, d] for d in range(D))
            _close(lse[0, h, i], scale * dot + math.log(Skv), what="identical keys LSE")


def pin_single_key(attn, merge=None):
    """One key  =>  O = v_0 and LSE = scale*<q, k_0>."""
    q, k, v = _qkv(3, 2, 3, 1, 2, 5)
    scale = 1.3
    o, lse = attn(q, k, v, scale)
    _close(o, np.broadcast_to(v[:, :1], o.shape), what="single key O")
    want = scale * np.einsum("bshd,bhd->bhs", q, k[:, 0])
    _close(lse, want, what="single key LSE")


def pin_zero_query(attn, merge=None):
    """q = 0  =>  uniform weights: O = mean V, LSE = ln Skv."""
    _, k, v = _qkv(4, 1, 3, 9, 2, 4)
    q = np.zeros((1, 3, 2, 4))
    o, lse = attn(q, k, v, 0.9)
    _close(o, np.broadcast_to(v.mean(axis=1, keepdims=True), o.shape), what="zero q O")
    _close(lse, np.full(lse.shape, math.log(9)), what="zero q LSE")


def _golden_two_keys():
    rows = []
    with open(os.path.join(GOLDEN, "two_keys.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            t = line.split()
            rows.append(t)
    vals = {"0": 0.0, "ln3": math.log(3), "-ln3": -math.log(3), "5": 5.0}
    lse_vals = {"ln4": math.log(4), "ln2": math.log(2), "ln4-ln3": math.log(4) - math.log(3)}
    qs, os_, ls = [], [], []
    for t in rows:
        assert t[0] == "query" and t[3] == "O" and t[6] == "LSE"
        qs.append([vals[t[1]], vals[t[2]]])
        os_.append([float(t[4]), float(t[5])])
        ls.append(lse_vals[t[7]])
    return np.array(qs), np.array(os_), np.array(ls)


def pin_two_keys_golden(attn, merge=None):
    """Hand-derived worked example (tests/golden/two_keys.txt)."""
    qs, want_o, want_lse = _golden_two_keys()
    n = qs.shape[0]
    q = qs.reshape(1, n, 1, 2)
    k = np.array([[0.0, 0.0], [1.0, 0.0]]).reshape(1, 2, 1, 2)
    v = np.array([[4.0, 0.0], [0.0, 8.0]]).reshape(1, 2, 1, 2)
    o, lse = attn(q, k, v, 1.0)
    _close(o[0, :, 0, :], want_o, what="two-keys O")
    _close(lse[0, 0, :], want_lse, what="two-keys LSE")


# ------------------------------------------------------ brute force, mpmath/fsum

def brute_attention_mp(q, k, v, scale, dps=40):
    """Scalar loops in arbitrary precision: exp/log from mpmath."""
    mpmath.mp.dps = dps
    B, Sq, H, D = q.shape
    Skv = k.shape[1]
    o = np.zeros((B, Sq, H, D))
    lse = np.zeros((B, H, Sq))
    for b in range(B):
        for h in range(H):
            for i in range(Sq):
                s = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(q[b, i, h, d]) * mpmath.mpf(k[b, j, h, d])
                                                     for d in range(D)) for j in range(Skv)]
                e = [mpmath.exp(x) for x in s]
                z = mpmath.fsum(e)
                lse[b, h, i] = float(mpmath.log(z))
                for d in range(D):
                    o[b, i, h, d] = float(mpmath.fsum(e[j] * mpmath.mpf(v[b, j, h, d])
                                                      for j in range(Skv)) / z)
    return o, lse


def brute_attention_fsum(q, k, v, scale):
    """Scalar loops in Python floats with exactly rounded sums (math.fsum)."""
    B, Sq, H, D = q.shape
    Skv = k.shape[1]
    o = np.zeros((B, Sq, H, D))
    lse = np.zeros((B, H, Sq))
    ql, kl, vl = q.tolist(), k.tolist(), v.tolist()
    for b in range(B):
        for h in range(H):
            keys = [kl[b][j][h] for j in range(Skv)]
            vals = [vl[b][j][h] for j in range(Skv)]
            for i in range(Sq):
                qi = ql[b][i][h]
                s = [scale * math.fsum(a * c for a, c in zip(qi, kj)) for kj in keys]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                z = math.fsum(e)
                lse[b, h, i] = m + math.log(z)
                for d in range(D):
                    o[b, i, h, d] = math.fsum(e[j] * vals[j][d] for j in range(Skv)) / z
    return o, lse


def pin_brute_force(attn, merge=None):
    """Tiny shapes (Sq != Skv, H > 1, B > 1) against scalar brute force."""
    for seed, shp in enumerate([(1, 1, 1, 1, 1), (1, 3, 5, 2, 4), (2, 7, 3, 3, 8)]):
        B, Sq, Skv, H, D = shp
        q, k, v = _qkv(100 + seed, *shp)
        scale = 1.0 / math.sqrt(D)
        o, lse = attn(q, k, v, scale)
        ob, lb = brute_attention_mp(q, k, v, scale)
        _close(o, ob, what=f"brute O {shp}")
        _close(lse, lb, what=f"brute LSE {shp}")
    shp = (1, 130, 200, 2, 16)
    q, k, v = _qkv(110, *shp)
    o, lse = attn(q, k, v, 0.25)
    ob, lb = brute_attention_fsum(q, k, v, 0.25)
    _close(o, ob, tol=1e-11, what="brute O large")
    _close(lse, lb, tol=1e-11, what="brute LSE large")


def pin_scipy_softmax(attn, merge=None):
    """Dense case reduces to a library softmax followed by a product."""
    from scipy.special import softmax, logsumexp
    q, k, v = _qkv(5, 2, 33, 47, 3, 16)
    scale = 0.25
    o, lse = attn(q, k, v, scale)
    for b in range(2):
        for h in range(3):
            s = (q[b, :, h, :] @ k[b, :, h, :].T) * scale
            _close(o[b, :, h, :], softmax(s, axis=1) @ v[b, :, h, :], what="scipy O")
            _close(lse[b, h], logsumexp(s, axis=1), what="scipy LSE")


# ---------------------------------------------------------------- invariants

def pin_merge_split(attn, merge):
    """Any split of the keys (uneven, size-1, empty parts), each part
    attended separately, merged = attention over all keys."""
    B, Sq, Skv, H, D = 2, 9, 23, 3, 8
    q, k, v = _qkv(6, B, Sq, Skv, H, D)
    scale = 0.35
    o_full, lse_full = attn(q, k, v, scale)
    for cuts in ([0, 23], [0, 1, 23], [0, 5, 5, 17, 23], [0, 11, 12, 23, 23], [0, 0, 23]):
        ops, lps = [], []
        for a, b in zip(cuts[:-1], cuts[1:]):
            o_k, l_k = attn(q, k[:, a:b], v[:, a:b], scale)
            ops.append(o_k)
            lps.append(l_k)
        o, lse = merge(np.stack(ops), np.stack(lps))
        _close(o, o_full, tol=1e-11, what=f"merge split {cuts}")
        _close(lse, lse_full, tol=1e-11, what=f"merge split LSE {cuts}")


def pin_merge_closed_forms(attn, merge):
    """Merge algebra: equal LSEs average the outputs and add ln n; an
    all -inf part is ignored; all -inf parts give O = 0, LSE = -inf."""
    r = _rng(7)
    o1 = r.standard_normal((1, 4, 2, 3))
    o2 = r.standard_normal((1, 4, 2, 3))
    l = r.standard_normal((1, 2, 4))
    o, lse = merge(np.stack([o1, o2]), np.stack([l, l]))
    _close(o, (o1 + o2) / 2, what="merge equal O")
    _close(lse, l + math.log(2), what="merge equal LSE")
    ninf = np.full_like(l, -np.inf)
    o, lse = merge(np.stack([o1, np.zeros_like(o2)]), np.stack([l, ninf]))
    _close(o, o1, what="merge -inf part O")
    _close(lse, l, what="merge -inf part LSE")
    o, lse = merge(np.stack([np.zeros_like(o1)] * 3), np.stack([ninf] * 3))
    assert np.all(o == 0) and np.all(np.isneginf(lse)), "merge all -inf"
    # weights e^{l1}, e^{l2}: explicit two-part formula
    l2 = l + 1.0
    o, lse = merge(np.stack([o1, o2]), np.stack([l, l2]))
    w1 = 1.0 / (1.0 + math.e)
    _close(o, w1 * o1 + (1 - w1) * o2, what="merge two-part O")
    _close(lse, l + math.log(1 + math.e), what="merge two-part LSE")


def pin_head_partition_tp_demo(attn, merge=None):
    """The TP demo's check (golden/tp_demo_shape.txt): 32 heads computed as
    4 shards of 8 heads, gathered in ascending head order, equal the
    full computation, and the gathered output has the printed shape."""
    cfg = {}
    with open(os.path.join(GOLDEN, "tp_demo_shape.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            t = line.split()
            cfg[t[0]] = [int(x) for x in t[1:]]
    B, S, H, D, world = (cfg["batch"][0], cfg["seq"][0], cfg["heads"][0],
                         cfg["head_dim"][0], cfg["world"][0])
    # The page's sizes, with the sequence cut to 16 to keep the pin quick;
    # head count, head_dim and sharding are the page's.
    Ssmall = 16
    r = _rng(8)
    q = r.standard_normal((B, Ssmall, H, D))
    k = r.standard_normal((B, Ssmall, H, D))
    v = r.standard_normal((B, Ssmall, H, D))
    scale = 1.0 / math.sqrt(D)
    o_full, lse_full = attn(q, k, v, scale)
    lh = H // world
    parts = []
    for g in range(world):
        sl = slice(g * lh, (g + 1) * lh)
        o_g, l_g = attn(q[:, :, sl], k[:, :, sl], v[:, :, sl], scale)
        _close(l_g, lse_full[:, sl], what="TP shard LSE")
        parts.append(o_g.reshape(B, Ssmall, lh * D))
    gathered = np.concatenate(parts, axis=-1)
    _close(gathered, o_full.reshape(B, Ssmall, H * D), what="TP gathered O")
    assert [B, S, H * D] == cfg["output_shape"], "TP demo printed shape"
    # uneven chunking (HCMS: uneven head partitions keep results unchanged)
    ofs = 0
    for hc in (13, 1, 11, 7):
        sl = slice(ofs, ofs + hc)
        o_c, l_c = attn(q[:, :, sl], k[:, :, sl], v[:, :, sl], scale)
        _close(o_c, o_full[:, :, sl], what="uneven chunk O")
        _close(l_c, lse_full[:, sl], what="uneven chunk LSE")
        ofs += hc
    assert ofs == H


def pin_key_permutation(attn, merge=None):
    """Permuting the (key, value) rows jointly changes nothing."""
    q, k, v = _qkv(9, 1, 6, 13, 2, 5)
    perm = _rng(10).permutation(13)
    o1, l1 = attn(q, k, v, 0.6)
    o2, l2 = attn(q, k[:, perm], v[:, perm], 0.6)
    _close(o2, o1, what="key permutation O")
    _close(l2, l1, what="key permutation LSE")


def pin_key_shift(attn, merge=None):
    """k_j -> k_j + u for all j: O unchanged, LSE += scale*<q, u>."""
    q, k, v = _qkv(11, 1, 5, 8, 2, 4)
    u = np.array([[0.5, -1.0, 2.0, 0.1], [1.5, 0.0, -0.3, 0.7]])
    scale = 0.8
    o1, l1 = attn(q, k, v, scale)
    o2, l2 = attn(q, k + u[None, None], v, scale)
    _close(o2, o1, tol=1e-11, what="key shift O")
    _close(l2, l1 + scale * np.einsum("bshd,hd->bhs", q, u), tol=1e-11, what="key shift LSE")


# ------------------------------------------------------------ block mask cases

def pin_mask_all_ones(attn, merge=None):
    """All-ones mask = dense (S not a multiple of the block edge)."""
    q, k, v = _qkv(12, 1, 20, 27, 2, 4)
    blk = 8
    mask = np.ones((1, 2, 3, 4), dtype=np.uint8)
    o1, l1 = attn(q, k, v, 0.5)
    o2, l2 = attn(q, k, v, 0.5, block_mask=mask, mask_block=blk)
    _close(o2, o1, what="all-ones mask O")
    _close(l2, l1, what="all-ones mask LSE")


def pin_mask_diagonal(attn, merge=None):
    """Diagonal-only mask = independent dense problems per block."""
    blk, nb = 4, 5
    q, k, v = _qkv(13, 1, blk * nb, blk * nb, 2, 3)
    mask = np.zeros((1, 2, nb, nb), dtype=np.uint8)
    for i in range(nb):
        mask[0, :, i, i] = 1
    o, l = attn(q, k, v, 0.5, block_mask=mask, mask_block=blk)
    for i in range(nb):
        sl = slice(i * blk, (i + 1) * blk)
        ob, lb = attn(q[:, sl], k[:, sl], v[:, sl], 0.5)
        _close(o[:, sl], ob, what="diagonal mask O")
        _close(l[:, :, sl], lb, what="diagonal mask LSE")


def pin_mask_gather(attn, merge=None):
    """A query block's result equals dense attention over the keys of its
    kept key blocks; a row block with nothing kept gives O = 0, LSE = -inf."""
    blk, nqb, nkb = 4, 3, 5
    B, H = 1, 2
    q, k, v = _qkv(14, B, blk * nqb, blk * nkb - 2, H, 3)
    r = _rng(15)
    mask = (r.random((B, H, nqb, nkb)) < 0.5).astype(np.uint8)
    mask[0, 0, 1, :] = 0          # an empty row block
    mask[0, 1, 2, :] = 0
    mask[0, 1, 2, 4] = 1          # only the partial last key block
    mask[0, 0, 0, :] = 0
    mask[0, 0, 0, 3] = 1
    mask[0, 0, 0, 1] = 1
    o, l = attn(q, k, v, 0.5, block_mask=mask, mask_block=blk)
    Skv = k.shape[1]
    for h in range(H):
        for i in range(nqb):
            rows = slice(i * blk, (i + 1) * blk)
            keys = [j for j in range(Skv) if mask[0, h, i, j // blk]]
            if not keys:
                assert np.all(o[0, rows, h] == 0), "empty row block O"
                assert np.all(np.isneginf(l[0, h, rows])), "empty row block LSE"
                continue
            ob, lb = attn(q[:, rows, h:h + 1], k[:, keys, h:h + 1], v[:, keys, h:h + 1], 0.5)
            _close(o[:, rows, h:h + 1], ob, what="mask gather O")
            _close(l[:, h:h + 1, rows], lb, what="mask gather LSE")


def pin_row_subset(attn, merge=None):
    """Computing a subset of query rows equals the same rows of the full run."""
    q, k, v = _qkv(16, 2, 300, 40, 2, 4)
    rows = np.array([0, 3, 255, 256, 299])
    o1, l1 = attn(q, k, v, 0.5)
    o2, l2 = attn(q, k, v, 0.5, rows=rows)
    _close(o2, o1[:, rows], what="row subset O")
    _close(l2, l1[:, :, rows], what="row subset LSE")


ATTN_PINS = [pin_constant_v, pin_identical_keys, pin_single_key, pin_zero_query,
             pin_two_keys_golden, pin_brute_force, pin_scipy_softmax,
             pin_head_partition_tp_demo, pin_key_permutation, pin_key_shift,
             pin_mask_all_ones, pin_mask_diagonal, pin_mask_gather, pin_row_subset]
MERGE_PINS = [pin_merge_split, pin_merge_closed_forms]


# ------------------------------------------------------------------ backward
#
# Pins of the gradient oracle (signature of ``oracle.attention_bwd_ref``).
# The first differentiates the forward oracle numerically, so it pins the
# gradient to the forward definition without using the gradient formulas;
# the others are exact consequences of the softmax Jacobian.

def _bwd_case(seed, B=2, Sq=3, Skv=4, H=2, D=5):
    r = _rng(seed)
    return (r.standard_normal((B, Sq, H, D)), r.standard_normal((B, Skv, H, D)),
            r.standard_normal((B, Skv, H, D)), r.standard_normal((B, Sq, H, D)))


def pin_bwd_finite_differences(bwd, attn):
    """Central differences of L = sum(dO * O(q, k, v)) in float64 match
    every entry of dQ, dK and dV (step 1e-6: truncation ~1e-12, rounding
    ~1e-10)."""
    scale = 0.7
    q, k, v, do = _bwd_case(201)
    dq, dk, dv = bwd(q, k, v, do, scale)

    def loss(q_, k_, v_):
        o, _ = attn(q_, k_, v_, scale)
        return float((do * o).sum())

    eps = 1e-6
    for name, x, g in (("dQ", q, dq), ("dK", k, dk), ("dV", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = x.copy(); xp[idx] += eps
            xm = x.copy(); xm[idx] -= eps
            args_p = {"dQ": (xp, k, v), "dK": (q, xp, v), "dV": (q, k, xp)}[name]
            args_m = {"dQ": (xm, k, v), "dK": (q, xm, v), "dV": (q, k, xm)}[name]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        _close(g, num, tol=1e-7, what=f"finite differences {name}")


def pin_bwd_column_sums(bwd, attn=None):
    """Each row of dS sums to zero, so sum_j dK_j = 0; each row of P sums
    to one, so sum_j dV_j = sum_i dO_i (per batch entry and head)."""
    q, k, v, do = _bwd_case(202, B=2, Sq=9, Skv=13, H=3, D=6)
    dq, dk, dv = bwd(q, k, v, do, 0.45)
    _close(dk.sum(axis=1), np.zeros_like(dk.sum(axis=1)), tol=1e-12, what="sum dK")
    _close(dv.sum(axis=1), do.sum(axis=1), tol=1e-12, what="sum dV")


def pin_bwd_identical_keys(bwd, attn=None):
    """All keys equal: scores are constant along each row, P is uniform and
    dQ = scale * dS K = scale * (sum_j dS_ij) kappa = 0."""
    q, k, v, do = _bwd_case(203, B=1, Sq=6, Skv=7, H=2, D=4)
    k[:] = _rng(9).standard_normal(4)
    dq, dk, dv = bwd(q, k, v, do, 0.9)
    _close(dq, np.zeros_like(dq), tol=1e-12, what="dQ with identical keys")
    _close(dv, np.broadcast_to(do.sum(axis=1, keepdims=True) / 7, dv.shape), tol=1e-12,
           what="dV with identical keys")


def pin_bwd_single_key(bwd, attn=None):
    """One key: P = 1, dS = 0, so dQ = dK = 0 and dV_0 = sum_i dO_i."""
    q, k, v, do = _bwd_case(204, B=2, Sq=5, Skv=1, H=2, D=3)
    dq, dk, dv = bwd(q, k, v, do, 1.3)
    _close(dq, np.zeros_like(dq), what="dQ one key")
    _close(dk, np.zeros_like(dk), what="dK one key")
    _close(dv, do.sum(axis=1, keepdims=True), what="dV one key")


def pin_bwd_zero_scale(bwd, attn=None):
    """scale = 0: P uniform (1/Skv), dQ = dK = 0 (both carry the factor
    scale) and every dV_j = (1/Skv) sum_i dO_i."""
    q, k, v, do = _bwd_case(205, B=1, Sq=4, Skv=6, H=2, D=5)
    dq, dk, dv = bwd(q, k, v, do, 0.0)
    _close(dq, np.zeros_like(dq), what="dQ scale 0")
    _close(dk, np.zeros_like(dk), what="dK scale 0")
    _close(dv, np.broadcast_to(do.sum(axis=1, keepdims=True) / 6, dv.shape), what="dV scale 0")


def pin_bwd_subsets(bwd, attn=None):
    """Computing selected query rows (dQ) and keys (dK, dV) equals the same
    entries of the full run."""
    q, k, v, do = _bwd_case(206, B=1, Sq=300, Skv=37, H=2, D=4)
    dq, dk, dv = bwd(q, k, v, do, 0.5)
    rows = np.array([0, 7, 256, 299])
    keys = np.array([3, 36])
    dq2, dk2, dv2 = bwd(q, k, v, do, 0.5, rows=rows, keys=keys)
    _close(dq2, dq[:, rows], what="dQ rows")
    _close(dk2, dk[:, keys], what="dK keys")
    _close(dv2, dv[:, keys], what="dV keys")


BWD_PINS = [pin_bwd_finite_differences, pin_bwd_column_sums, pin_bwd_identical_keys,
            pin_bwd_single_key, pin_bwd_zero_scale, pin_bwd_subsets]
