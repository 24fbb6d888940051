"""Attention backward (dQ, dK, dV) on the GPU against the fp64 oracle:
small and ragged shapes that span several 64-row tiles and 128-row
blocks, strided views, peaked scores, closed forms and run-to-run
identity. The forward is the library's own (lsh_attn_fwd), as a caller
would run it; the oracle differentiates the exact forward."""
import math

import numpy as np
import pytest

import lsh_inputs as I
import oracle
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def L():
    import long_sequence_head_amd as lsh
    lsh.load()
    return lsh


def _grads(L, qg, kg, vg, dog, scale=None):
    t = G.torch()
    o, lse = L.attn_fwd(qg, kg, vg, scale=scale)
    dq = t.full(qg.shape, float("nan"), dtype=t.float32, device="cuda")
    dk = t.full(kg.shape, float("nan"), dtype=t.float32, device="cuda")
    dv = t.full(vg.shape, float("nan"), dtype=t.float32, device="cuda")
    L.attn_bwd(qg, kg, vg, dog, o, lse, scale=scale, dq=dq, dk=dk, dv=dv)
    return dq, dk, dv


def _np(ts):
    return [x.cpu().numpy() for x in ts]


BWD_SHAPES = [  # (B, Sq, Skv, H)
    (1, 1, 1, 1), (1, 2, 3, 2), (1, 63, 64, 1), (1, 64, 65, 2), (2, 127, 128, 2),
    (1, 128, 129, 3), (1, 129, 127, 1), (1, 200, 255, 2), (1, 257, 256, 2), (2, 300, 1000, 3),
    (1, 513, 77, 2), (1, 1000, 1000, 4), (1, 77, 513, 2),
]


@pytest.mark.parametrize("shape", BWD_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bwd_vs_oracle(L, shape):
    B, Sq, Skv, H = shape
    G.announce(f"bwd B={B} Sq={Sq} Skv={Skv} H={H}")
    q, k, v = I.make_custom((B, Sq, H, 128), (B, Skv, H, 128), "bf16", seed=Sq * 5 + Skv)
    do = I.make_custom_dout((B, Sq, H, 128), "bf16", seed=Sq * 5 + Skv)
    got = _grads(L, G.to_gpu(q, "bf16"), G.to_gpu(k, "bf16"), G.to_gpu(v, "bf16"),
                 G.to_gpu(do, "bf16"))
    ref = oracle.attention_bwd_ref(q.values, k.values, v.values, do.values, 1 / math.sqrt(128))
    G.check_grads(f"bwd {shape}", _np(got), ref)


def test_bwd_moderate_size(L):
    """4096 x 4096 keys, two heads: 64 query tiles and 32 key blocks."""
    B, S, H = 1, 4096, 2
    G.announce(f"bwd moderate S={S} H={H}")
    q, k, v = I.make_custom((B, S, H, 128), (B, S, H, 128), "bf16", seed=4096)
    do = I.make_custom_dout((B, S, H, 128), "bf16", seed=4096)
    got = _grads(L, G.to_gpu(q, "bf16"), G.to_gpu(k, "bf16"), G.to_gpu(v, "bf16"),
                 G.to_gpu(do, "bf16"))
    ref = oracle.attention_bwd_ref(q.values, k.values, v.values, do.values, 1 / math.sqrt(128))
    G.check_grads("bwd moderate", _np(got), ref)


def test_bwd_peaked_and_scaled(L):
    """Q scaled by 8 (softmax dominated by few keys) and a non-default
    scale."""
    B, Sq, Skv, H = 1, 260, 700, 2
    G.announce("bwd peaked")
    q, k, v = I.make_custom((B, Sq, H, 128), (B, Skv, H, 128), "bf16", seed=31)
    do = I.make_custom_dout((B, Sq, H, 128), "bf16", seed=31)
    qv = q.values * 8.0   # exact in bf16 (power of two)
    for scale in (1 / math.sqrt(128), 0.05):
        got = _grads(L, G.values_to_gpu(qv, "bf16"), G.to_gpu(k, "bf16"), G.to_gpu(v, "bf16"),
                     G.to_gpu(do, "bf16"), scale=scale)
        ref = oracle.attention_bwd_ref(qv, k.values, v.values, do.values, scale)
        G.check_grads(f"bwd peaked scale={scale:.4f}", _np(got), ref)


def test_bwd_strided_views(L):
    """Q, K, V as views into one packed [B, S, 3, H, D] buffer, dO a view of
    a wider buffer, gradients written into views of wider buffers."""
    t = G.torch()
    B, S, H, D = 2, 333, 3, 128
    G.announce("bwd strided")
    q, k, v = I.make_custom((B, S, H, D), (B, S, H, D), "bf16", seed=12)
    do = I.make_custom_dout((B, S, H, D), "bf16", seed=12)
    packed = t.stack([G.to_gpu(q, "bf16"), G.to_gpu(k, "bf16"), G.to_gpu(v, "bf16")], dim=2)
    qv, kv, vv = packed[:, :, 0], packed[:, :, 1], packed[:, :, 2]
    dwide = t.zeros((B, S, H + 1, D), dtype=t.bfloat16, device="cuda")
    dwide[:, :, 1:] = G.to_gpu(do, "bf16")
    dov = dwide[:, :, 1:]
    o, lse = L.attn_fwd(qv, kv, vv)
    outs = [t.full((B, S, H + 2, D), float("nan"), dtype=t.float32, device="cuda") for _ in range(3)]
    dq, dk, dv = (x[:, :, 1:H + 1] for x in outs)
    L.attn_bwd(qv, kv, vv, dov, o, lse, dq=dq, dk=dk, dv=dv)
    ref = oracle.attention_bwd_ref(q.values, k.values, v.values, do.values, 1 / math.sqrt(D))
    G.check_grads("bwd strided", _np((dq, dk, dv)), ref)
    for x in outs:
        assert t.isnan(x[:, :, 0]).all() and t.isnan(x[:, :, H + 1]).all(), "wrote outside"


def test_bwd_closed_forms(L):
    """dO = 0 gives zero gradients exactly. One key: P = 1, so dV = sum_i dO_i
    and dS = 0 (dQ = dK = 0 up to the rounding of dP - Delta). Constant V:
    dP_ij = <dO_i, c> = Delta_i, so dS = 0 again and dV_j = sum_i P_ij dO_i."""
    t = G.torch()
    B, Sq, Skv, H, D = 1, 190, 300, 2, 128
    G.announce("bwd closed forms")
    q, k, v = I.make_custom((B, Sq, H, D), (B, Skv, H, D), "bf16", seed=41)
    do = I.make_custom_dout((B, Sq, H, D), "bf16", seed=41)
    qg, kg, vg, dog = (G.to_gpu(x, "bf16") for x in (q, k, v, do))
    # dO = 0
    dq, dk, dv = _grads(L, qg, kg, vg, t.zeros_like(dog))
    for x in (dq, dk, dv):
        assert bool((x == 0).all()), "dO = 0 must give exact zeros"
    # one key
    dq, dk, dv = _grads(L, qg, kg[:, :1], vg[:, :1], dog)
    want_dv = do.values.astype(np.float64).sum(axis=1, keepdims=True)
    e = G.max_err(dv.cpu().numpy(), want_dv)
    assert e <= 1e-4 * max(1.0, np.abs(want_dv).max()), e
    top = float(np.abs(do.values).max())
    assert G.max_err(dq.cpu().numpy(), 0.0 * q.values) <= 1e-4 * top
    assert G.max_err(dk.cpu().numpy(), 0.0 * k.values[:, :1]) <= 1e-4 * top
    # constant V (multiples of 1/8: exact in bf16)
    c = (np.arange(D) % 17 - 8) / 8.0
    vc = np.broadcast_to(c, (B, Skv, H, D)).astype(np.float32)
    dq, dk, dv = _grads(L, qg, kg, G.values_to_gpu(vc, "bf16"), dog)
    _, _, dv_ref = oracle.attention_bwd_ref(q.values, k.values, vc, do.values, 1 / math.sqrt(D))
    e = G.max_err(dv.cpu().numpy(), dv_ref)
    assert e <= G.TOL_GRAD * np.abs(dv_ref).max(), e
    gq = float(np.abs(dq.cpu().numpy()).max())
    gk = float(np.abs(dk.cpu().numpy()).max())
    assert gq <= 2e-2 and gk <= 2e-2, (gq, gk)   # dS = 0 up to rounding


def test_bwd_run_to_run_bit_identical(L):
    t = G.torch()
    B, Sq, Skv, H = 1, 700, 900, 3
    G.announce("bwd determinism")
    q, k, v = I.make_custom((B, Sq, H, 128), (B, Skv, H, 128), "bf16", seed=51)
    do = I.make_custom_dout((B, Sq, H, 128), "bf16", seed=51)
    args = [G.to_gpu(x, "bf16") for x in (q, k, v, do)]
    a = _grads(L, *args)
    b = _grads(L, *args)
    for x, y in zip(a, b):
        assert t.equal(x, y)


def test_bwd_head_independence(L):
    """A head's gradients do not depend on the other heads: heads 1..2 of
    an H=4 run equal an H=2 run on those heads' slices, bit for bit."""
    t = G.torch()
    B, Sq, Skv = 1, 300, 260
    G.announce("bwd head independence")
    q, k, v = I.make_custom((B, Sq, 4, 128), (B, Skv, 4, 128), "bf16", seed=61)
    do = I.make_custom_dout((B, Sq, 4, 128), "bf16", seed=61)
    full = [G.to_gpu(x, "bf16") for x in (q, k, v, do)]
    part = [x[:, :, 1:3].contiguous() for x in full]
    a = _grads(L, *full)
    b = _grads(L, *part)
    for x, y in zip(a, b):
        assert t.equal(x[:, :, 1:3], y)


@pytest.mark.parametrize("B,Skv", [(1, 1), (1, 65), (1, 129), (1, 517), (2, 300)])
def test_bwd_large_grid_dq(L, B, Skv):
    """H=32, Sq=4133 (last 256-query block holds 37 rows): 544 workgroups
    of 256 queries per batch entry, so dQ runs on the two-wavefronts-per-
    SIMD kernel, over 1, 2, 3, 5 and 9 key tiles (each load-ahead case,
    ragged last tiles), and with B=2. Heads 0 and 31 against the oracle;
    every head bit-identical to calls on 4 / B heads at a time (68
    workgroups: the pipelined dQ kernel)."""
    t = G.torch()
    Sq, H = 4133, 32
    G.announce(f"bwd large-grid dQ B={B} Skv={Skv}")
    q, k, v = I.make_custom((B, Sq, H, 128), (B, Skv, H, 128), "bf16", seed=71 + Skv + B)
    do = I.make_custom_dout((B, Sq, H, 128), "bf16", seed=71 + Skv + B)
    full = [G.to_gpu(x, "bf16") for x in (q, k, v, do)]
    got = _grads(L, *full)
    heads = [0, 31]
    ref = oracle.attention_bwd_ref(q.values, k.values, v.values, do.values, 1 / math.sqrt(128),
                                   heads=heads)
    G.check_grads("bwd large grid", [x[:, :, heads] for x in _np(got)],
                  [r[:, :, heads] for r in ref])
    w = 4 // B   # heads per call: few enough workgroups for the pipelined kernel
    for h0 in range(0, H, w):
        part = [x[:, :, h0:h0 + w].contiguous() for x in full]
        sub = _grads(L, *part)
        for x, y in zip(got, sub):
            assert t.equal(x[:, :, h0:h0 + w], y), f"heads {h0}..{h0 + w - 1}"
