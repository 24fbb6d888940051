"""HIP path vs the fp64 oracle on small and odd shapes, closed forms on the
GPU, strided inputs, peaked and monotone score patterns (lazy-rescale
paths), and determinism. Sizes keep the oracle to seconds while spanning
several 64-key tiles, several query blocks and ragged tails."""
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


SHAPES = [  # (B, Sq, Skv, H)
    (1, 1, 1, 1), (1, 2, 3, 2), (1, 63, 64, 1), (1, 64, 65, 2), (2, 127, 128, 2),
    (1, 128, 129, 3), (1, 200, 255, 2), (1, 257, 256, 2), (2, 300, 1000, 3),
    (1, 1000, 1000, 4), (1, 513, 77, 2),
    # short query ranges against long key ranges, odd and even tile counts,
    # last tiles of one key
    (1, 1, 1024, 1), (1, 129, 1025, 2), (2, 300, 1100, 3), (1, 1000, 1500, 2), (1, 64, 4097, 2),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_dense_vs_oracle(L, dtype, shape):
    B, Sq, Skv, H = shape
    G.announce(f"dense {dtype} B={B} Sq={Sq} Skv={Skv} H={H}")
    q, k, v = I.make_custom((B, Sq, H, 128), (B, Skv, H, 128), dtype, seed=Sq * 7 + Skv)
    o, lse = G.poisoned_outputs(B, Sq, H)
    L.attn_fwd(G.to_gpu(q, dtype), G.to_gpu(k, dtype), G.to_gpu(v, dtype), o=o, lse=lse)
    o_ref, lse_ref = oracle.attention_ref(q.values, k.values, v.values, 1 / math.sqrt(128))
    sig = (G.bf16_weight_sigma(oracle, q.values, k.values, v.values, 1 / math.sqrt(128), lse_ref)
           if dtype == "bf16" else None)
    G.check(f"dense {dtype} {shape}", dtype, o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref,
            sigma=sig)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_closed_forms_on_gpu(L, dtype):
    """constant V -> O = c; identical keys -> O = mean V and
    LSE = scale <q, kappa> + ln Skv; one key -> O = v_0."""
    G.announce(f"closed forms {dtype}")
    t = G.torch()
    B, Sq, Skv, H, D = 1, 130, 333, 2, 128
    q, k, v = I.make_custom((B, Sq, H, D), (B, Skv, H, D), dtype, seed=5)
    scale = 1 / math.sqrt(D)
    # constant V (values exactly representable: multiples of 1/8)
    c = (np.arange(D) % 17 - 8) / 8.0
    vc = np.broadcast_to(c, (B, Skv, H, D)).astype(np.float32)
    o, lse = G.poisoned_outputs(B, Sq, H)
    L.attn_fwd(G.to_gpu(q, dtype), G.to_gpu(k, dtype), G.values_to_gpu(vc, dtype), o=o, lse=lse)
    err = G.max_err(o.cpu().numpy(), np.broadcast_to(c, (B, Sq, H, D)))
    # fp32: weights summing to one up to fp32 rounding; bf16: P is rounded
    # to bf16 in the numerator (relative 2^-9) but not in the row sum
    assert err <= (1e-5 if dtype == "f32" else 2e-3), err
    # identical keys
    kappa = np.round(np.linspace(-1, 1, D) * 8) / 8
    kc = np.broadcast_to(kappa, (B, Skv, H, D)).astype(np.float32)
    o, lse = G.poisoned_outputs(B, Sq, H)
    L.attn_fwd(G.to_gpu(q, dtype), G.values_to_gpu(kc, dtype), G.to_gpu(v, dtype), o=o, lse=lse)
    mean_v = v.values.astype(np.float64).mean(axis=1, keepdims=True)
    eo = G.max_err(o.cpu().numpy(), np.broadcast_to(mean_v, (B, Sq, H, D)))
    want_lse = scale * np.einsum("bshd,d->bhs", q.values.astype(np.float64), kappa) + math.log(Skv)
    el = G.max_err(lse.cpu().numpy(), want_lse)
    assert eo <= G.TOL_O[dtype] and el <= G.TOL_LSE, (eo, el)
    # single key
    o, lse = G.poisoned_outputs(B, Sq, H)
    kt, vt = G.to_gpu(k, dtype)[:, :1], G.to_gpu(v, dtype)[:, :1]
    L.attn_fwd(G.to_gpu(q, dtype), kt, vt, o=o, lse=lse)
    eo = G.max_err(o.cpu().numpy(), np.broadcast_to(v.values[:, :1], (B, Sq, H, D)))
    # exp2(fma(s, c, -m c)) of the single key is 1 up to the rounding of m c
    assert eo <= 1e-6, eo


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_strided_packed_qkv(L, dtype):
    """Q, K, V as views into one packed [B, S, 3, H, D] buffer; O written
    into a view of a wider buffer."""
    G.announce(f"strided {dtype}")
    t = G.torch()
    B, S, H, D = 2, 333, 3, 128
    q, k, v = I.make_custom((B, S, H, D), (B, S, H, D), dtype, seed=11)
    packed = t.stack([G.to_gpu(q, dtype), G.to_gpu(k, dtype), G.to_gpu(v, dtype)], dim=2)
    qv, kv, vv = packed[:, :, 0], packed[:, :, 1], packed[:, :, 2]
    wide = t.full((B, S, H + 2, D), float("nan"), dtype=t.float32, device="cuda")
    o = wide[:, :, 1:H + 1]
    lse = t.full((B, H, S), float("nan"), dtype=t.float32, device="cuda")
    L.attn_fwd(qv, kv, vv, o=o, lse=lse)
    o_ref, lse_ref = oracle.attention_ref(q.values, k.values, v.values, 1 / math.sqrt(D))
    sig = (G.bf16_weight_sigma(oracle, q.values, k.values, v.values, 1 / math.sqrt(D), lse_ref)
           if dtype == "bf16" else None)
    G.check(f"strided {dtype}", dtype, o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, sigma=sig)
    assert t.isnan(wide[:, :, 0]).all() and t.isnan(wide[:, :, H + 1]).all(), "wrote outside O"


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_peaked_scores(L, dtype):
    """Q scaled by 8: softmax dominated by few keys."""
    G.announce(f"peaked {dtype}")
    B, Sq, Skv, H, D = 1, 260, 700, 2, 128
    q, k, v = I.make_custom((B, Sq, H, D), (B, Skv, H, D), dtype, seed=21)
    qv = q.values * 8.0   # exact in bf16 (power of two)
    o, lse = G.poisoned_outputs(B, Sq, H)
    L.attn_fwd(G.values_to_gpu(qv, dtype), G.to_gpu(k, dtype), G.to_gpu(v, dtype), o=o, lse=lse)
    o_ref, lse_ref = oracle.attention_ref(qv, k.values, v.values, 1 / math.sqrt(D))
    sig = (G.bf16_weight_sigma(oracle, qv, k.values, v.values, 1 / math.sqrt(D), lse_ref)
           if dtype == "bf16" else None)
    G.check(f"peaked {dtype}", dtype, o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, sigma=sig)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("direction", [1, -1])
def test_monotone_scores(L, dtype, direction):
    """Scores that rise (or fall) along the keys by ~64 raw units per 64-key
    tile: with direction=1 the running max moves on every tile."""
    G.announce(f"monotone {dtype} {direction}")
    B, Sq, Skv, H, D = 1, 70, 900, 2, 128
    q = np.zeros((B, Sq, H, D), np.float32)
    q[..., 0] = 8.0
    q[..., 1] = np.linspace(-1, 1, Sq, dtype=np.float32)[None, :, None]
    k = np.zeros((B, Skv, H, D), np.float32)
    k[..., 0] = direction * np.arange(Skv, dtype=np.float32)[None, :, None] / 8.0
    k[..., 1] = 1.0
    k = k.astype(np.float32)
    if dtype == "bf16":
        import lsh_inputs as II
        k = II.bf16_bits_to_f32(II.bf16_bits(k))
        q = II.bf16_bits_to_f32(II.bf16_bits(q))
    _, _, v = I.make_custom((B, Sq, H, D), (B, Skv, H, D), dtype, seed=31)
    o, lse = G.poisoned_outputs(B, Sq, H)
    L.attn_fwd(G.values_to_gpu(q, dtype), G.values_to_gpu(k, dtype), G.to_gpu(v, dtype), o=o, lse=lse)
    o_ref, lse_ref = oracle.attention_ref(q, k, v.values, 1 / math.sqrt(D))
    sig = (G.bf16_weight_sigma(oracle, q, k, v.values, 1 / math.sqrt(D), lse_ref)
           if dtype == "bf16" else None)
    G.check(f"monotone {dtype} {direction}", dtype, o.cpu().numpy(), lse.cpu().numpy(), o_ref,
            lse_ref, sigma=sig)


def test_rescale_paths_large_grid(L):
    """Scores that rise along the keys at four rates, one per group of 16
    heads (raw slope 1, 0.75 and 0.25 per key, and falling), plus a per-row
    offset: the running max moves on every tile, every other tile, every
    few tiles (with tile sums past the bound that skips the row max), or
    never after the first. H=64 and Sq=2048 give 512 workgroups of 256
    rows, so the 256-row kernel runs (two 16-query groups per wavefront);
    an all-ones block mask runs the block-sparse kernel. Both must equal,
    bit for bit, calls on 4 heads at a time (64 workgroups: the 128-row
    kernel, one 16-query group per wavefront); heads 0, 20, 40 and 60 are
    checked against the oracle."""
    G.announce("rescale paths, large grid")
    t = G.torch()
    B, Sq, Skv, H, D = 1, 2048, 1500, 64, 128
    import lsh_inputs as II
    rates = np.repeat(np.array([1.0, 0.75, 0.25, -1.0], np.float32), 16)
    q = np.zeros((B, Sq, H, D), np.float32)
    q[..., 0] = 8.0
    q[..., 1] = np.linspace(-4, 4, Sq, dtype=np.float32)[None, :, None]
    k = np.zeros((B, Skv, H, D), np.float32)
    k[..., 0] = np.arange(Skv, dtype=np.float32)[None, :, None] / 8.0 * rates[None, None, :]
    k[..., 1] = 1.0
    q = II.bf16_bits_to_f32(II.bf16_bits(q))
    k = II.bf16_bits_to_f32(II.bf16_bits(k))
    _, _, v = I.make_custom((B, Sq, H, D), (B, Skv, H, D), "bf16", seed=37)
    qg, kg, vg = G.values_to_gpu(q, "bf16"), G.values_to_gpu(k, "bf16"), G.to_gpu(v, "bf16")
    o, lse = L.attn_fwd(qg, kg, vg)
    nb = -(-Sq // 128), -(-Skv // 128)
    o_s, lse_s = L.attn_fwd_blocksparse(qg, kg, vg, t.ones((B, H) + nb, dtype=t.uint8, device="cuda"))
    assert t.equal(o, o_s) and t.equal(lse, lse_s), "block-sparse kernel differs"
    for h0 in range(0, H, 4):
        sl = slice(h0, h0 + 4)
        o4, l4 = L.attn_fwd(qg[:, :, sl].contiguous(), kg[:, :, sl].contiguous(),
                            vg[:, :, sl].contiguous())
        assert t.equal(o[:, :, sl], o4) and t.equal(lse[:, sl], l4), f"heads {h0}..{h0 + 3}"
    heads = [0, 20, 40, 60]
    o_ref, lse_ref = oracle.attention_ref(q, k, v.values, 1 / math.sqrt(D), heads=heads)
    sig = G.bf16_weight_sigma(oracle, q, k, v.values, 1 / math.sqrt(D), lse_ref, heads=heads)
    og, lg = o.cpu().numpy(), lse.cpu().numpy()
    G.check("rescale paths", "bf16", og[:, :, heads], lg[:, heads], o_ref[:, :, heads],
            lse_ref[:, heads], sigma=sig[:, :, heads])


def test_odd_tile_count_bitwise(L):
    """Sq = Skv = 1025 (17 key tiles, the last holding one key; the last
    query block one row). Against the oracle on every row; an all-ones block
    mask, a {1, 2} head chunking and each batch entry on its own give the
    same bits."""
    G.announce("odd tile count")
    t = G.torch()
    B, Sq, Skv, H = 2, 1025, 1025, 3
    q, k, v = I.make_custom((B, Sq, H, 128), (B, Skv, H, 128), "bf16", seed=97)
    qg, kg, vg = G.to_gpu(q, "bf16"), G.to_gpu(k, "bf16"), G.to_gpu(v, "bf16")
    o, lse = G.poisoned_outputs(B, Sq, H)
    L.attn_fwd(qg, kg, vg, o=o, lse=lse)
    o_ref, lse_ref = oracle.attention_ref(q.values, k.values, v.values, 1 / math.sqrt(128))
    sig = G.bf16_weight_sigma(oracle, q.values, k.values, v.values, 1 / math.sqrt(128), lse_ref)
    G.check("odd tile count", "bf16", o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref, sigma=sig)
    ones = t.ones((B, H, -(-Sq // 128), -(-Skv // 128)), dtype=t.uint8, device="cuda")
    o2, l2 = L.attn_fwd_blocksparse(qg, kg, vg, ones)
    assert t.equal(o, o2) and t.equal(lse, l2), "block-sparse all-ones differs"
    o3, l3 = L.attn_fwd_chunked(qg, kg, vg, [1, 2])
    t.cuda.synchronize()
    assert t.equal(o, o3) and t.equal(lse, l3), "chunked differs"
    for b in range(B):
        o4, l4 = L.attn_fwd(qg[b:b + 1], kg[b:b + 1], vg[b:b + 1])
        assert t.equal(o[b:b + 1], o4) and t.equal(lse[b:b + 1], l4), f"batch entry {b}"


def test_run_to_run_bit_identical(L):
    G.announce("run-to-run")
    t = G.torch()
    q, k, v = I.make_custom((1, 1500, 4, 128), (1, 1500, 4, 128), "bf16", seed=41)
    qg, kg, vg = G.to_gpu(q, "bf16"), G.to_gpu(k, "bf16"), G.to_gpu(v, "bf16")
    o1, l1 = L.attn_fwd(qg, kg, vg)
    for _ in range(3):
        o2, l2 = L.attn_fwd(qg, kg, vg)
        assert t.equal(o1, o2) and t.equal(l1, l2)


def test_workgroup_size_does_not_change_bits(L):
    """All 8 heads (512 workgroups of 256 rows: the 256-row kernel) vs head
    0 alone (128 workgroups of 128 rows: the 128-row kernel) and a {1, 7}
    chunking (its 1-head chunk on the 128-row kernel, its 7-head chunk on
    the 256-row one): neither the kernel, the grid size nor the chunking may
    change a bit."""
    G.announce("workgroup-size invariance")
    t = G.torch()
    S, H = 16384, 8
    q, k, v = I.make_custom((1, S, H, 128), (1, S, H, 128), "bf16", seed=43)
    qg, kg, vg = G.to_gpu(q, "bf16"), G.to_gpu(k, "bf16"), G.to_gpu(v, "bf16")
    o1, l1 = L.attn_fwd(qg, kg, vg)
    o2, l2 = L.attn_fwd_chunked(qg, kg, vg, [1, 7])
    t.cuda.synchronize()
    assert t.equal(o1, o2) and t.equal(l1, l2)
    o3, l3 = L.attn_fwd(qg[:, :, :1].contiguous(), kg[:, :, :1].contiguous(), vg[:, :, :1].contiguous())
    assert t.equal(o1[:, :, :1], o3) and t.equal(l1[:, :1], l3)


def test_large_grid_strided(L):
    """B=2, Sq=777 (last 256-row block holds 9 rows), Skv=333, H=64: 512
    workgroups, so the 256-row kernel runs, here on Q, K, V as views of one
    packed [B, S, 3, H, D] buffer with O written into a wider one. Four
    heads against the oracle on every row; every head bit-identical to
    calls on 4 heads at a time (56-workgroup grids: the 128-row kernel)."""
    G.announce("large grid, strided")
    t = G.torch()
    B, Sq, Skv, H, D = 2, 777, 333, 64, 128
    q, k, v = I.make_custom((B, Sq, H, D), (B, Skv, H, D), "bf16", seed=77)
    qg = G.to_gpu(q, "bf16")
    packed = t.zeros((B, Sq, 3, H, D), dtype=t.bfloat16, device="cuda")
    packed[:, :, 0] = qg
    packed[:, :Skv, 1] = G.to_gpu(k, "bf16")
    packed[:, :Skv, 2] = G.to_gpu(v, "bf16")
    qv, kv, vv = packed[:, :, 0], packed[:, :Skv, 1], packed[:, :Skv, 2]
    wide = t.full((B, Sq, H + 2, D), float("nan"), dtype=t.float32, device="cuda")
    o = wide[:, :, 1:H + 1]
    lse = t.full((B, H, Sq), float("nan"), dtype=t.float32, device="cuda")
    L.attn_fwd(qv, kv, vv, o=o, lse=lse)
    heads = [0, 1, 37, 63]
    o_ref, lse_ref = oracle.attention_ref(q.values, k.values, v.values, 1 / math.sqrt(D),
                                          heads=heads)
    sig = G.bf16_weight_sigma(oracle, q.values, k.values, v.values, 1 / math.sqrt(D), lse_ref,
                              heads=heads)
    og, lg = o.cpu().numpy(), lse.cpu().numpy()
    G.check("large grid strided", "bf16", og[:, :, heads], lg[:, heads], o_ref[:, :, heads],
            lse_ref[:, heads], sigma=sig[:, :, heads])
    assert t.isnan(wide[:, :, 0]).all() and t.isnan(wide[:, :, H + 1]).all(), "wrote outside O"
    assert not t.isnan(o).any() and not t.isnan(lse).any(), "unwritten output"
    for h0 in range(0, H, 4):
        sl = slice(h0, h0 + 4)
        o4, l4 = L.attn_fwd(qv[:, :, sl], kv[:, :, sl], vv[:, :, sl])
        assert t.equal(o[:, :, sl], o4) and t.equal(lse[:, sl], l4), f"heads {h0}..{h0 + 3}"


@pytest.mark.parametrize("B,H,packed", [(1, 32, False), (2, 16, True)], ids=["B1H32", "B2H16-packed"])
def test_tail_halves_bitwise(L, B, H, packed):
    """S=4133 with B*H = 32: 544 items of 256 rows, 68 per XCD (the 4
    (b, h) pairs 4x .. 4x + 3 of XCD x; with B=2 the upper XCDs hold batch
    entry 1); 64 run whole and the last 4 (query blocks 13..16 of pair
    4x + 3, the last holding 37 rows, so its second half none) as 128-row
    halves in the same launch (the empty half returns at once). The B=2
    case reads Q, K, V as views of one packed [B, S, 3, H, D] buffer and
    writes O into a wider one. Every head bit-identical to calls on 4 heads
    at a time (no split: the 128-row kernel for B=1, the plain 256-row one
    for B=2); split and whole rows of the first and last batch entry
    against the oracle."""
    G.announce(f"256-row grid with split tail B={B} H={H} packed={packed}")
    t = G.torch()
    S, D = 4133, 128
    plan = G.dense_bf16_launch(B, S, H)
    assert plan == ("256-row, split tail", 576, 4), plan
    assert G.dense_bf16_launch(B, S, 4)[0] in ("128-row", "256-row")   # no split tail
    q, k, v = I.make_custom((B, S, H, D), (B, S, H, D), "bf16", seed=96 + B)
    qg, kg, vg = G.to_gpu(q, "bf16"), G.to_gpu(k, "bf16"), G.to_gpu(v, "bf16")
    if packed:
        buf = t.zeros((B, S, 3, H, D), dtype=t.bfloat16, device="cuda")
        buf[:, :, 0], buf[:, :, 1], buf[:, :, 2] = qg, kg, vg
        qg, kg, vg = buf[:, :, 0], buf[:, :, 1], buf[:, :, 2]
        wide = t.full((B, S, H + 2, D), float("nan"), dtype=t.float32, device="cuda")
        o = wide[:, :, 1:H + 1]
        lse = t.full((B, H, S), float("nan"), dtype=t.float32, device="cuda")
    else:
        o, lse = G.poisoned_outputs(B, S, H)
    L.attn_fwd(qg, kg, vg, o=o, lse=lse)
    t.cuda.synchronize()
    assert not t.isnan(o).any() and not t.isnan(lse).any(), "unwritten output"
    if packed:
        assert t.isnan(wide[:, :, 0]).all() and t.isnan(wide[:, :, H + 1]).all(), "wrote outside O"
    for h0 in range(0, H, 4):
        sl = slice(h0, h0 + 4)
        o4, l4 = L.attn_fwd(qg[:, :, sl].contiguous(), kg[:, :, sl].contiguous(),
                            vg[:, :, sl].contiguous())
        assert t.equal(o[:, :, sl], o4) and t.equal(lse[:, sl], l4), f"heads {h0}..{h0 + 3}"
    rows = np.unique(np.concatenate([np.arange(0, 64), np.arange(3328, 3328 + 64),
                                     np.arange(3520, 3600), np.arange(4090, S)]))
    heads = [0, 3, H - 1]
    o_ref, lse_ref = oracle.attention_ref(q.values, k.values, v.values, 1 / math.sqrt(D),
                                          heads=heads, rows=rows)
    ridx = t.from_numpy(rows).cuda()
    og = o.index_select(1, ridx).cpu().numpy()[:, :, heads]
    lg = lse.index_select(2, ridx).cpu().numpy()[:, heads]
    G.check("split tail", "bf16", og, lg, o_ref[:, :, heads], lse_ref[:, heads])


def test_permute_bit_exact(L):
    G.announce("permute")
    t = G.torch()
    for dtype, shape in [("bf16", (2, 333, 5, 128)), ("f32", (1, 200, 7, 128)), ("bf16", (1, 70, 3, 64))]:
        x = I.make_tensor(shape, dtype, 77, 0, seed=1)
        xg = G.to_gpu(x, dtype)
        H = shape[2]
        for h0, hc in [(0, H), (1, H - 1), (H - 1, 1)]:
            y = L.head_permute(xg, h0, hc)
            want = oracle.permute_ref(x.device_array, h0, hc)
            got = y.cpu()
            got = got.view(t.int16).numpy().view(np.uint16) if dtype == "bf16" else got.numpy()
            assert np.array_equal(got, want), (dtype, shape, h0, hc)


def test_chunked_small_bit_identical(L):
    G.announce("chunked small")
    t = G.torch()
    B, S, H = 2, 777, 7
    q, k, v = I.make_custom((B, S, H, 128), (B, S, H, 128), "bf16", seed=51)
    qg, kg, vg = G.to_gpu(q, "bf16"), G.to_gpu(k, "bf16"), G.to_gpu(v, "bf16")
    o1, l1 = L.attn_fwd(qg, kg, vg)
    for chunks in ([7], [3, 4], [1, 1, 5], [2, 2, 2, 1]):
        o2, l2 = G.poisoned_outputs(B, S, H)
        L.attn_fwd_chunked(qg, kg, vg, chunks, o=o2, lse=l2)
        t.cuda.synchronize()
        assert t.equal(o1, o2) and t.equal(l1, l2), chunks
    # same stream for both roles
    o3, l3 = G.poisoned_outputs(B, S, H)
    s = t.cuda.current_stream()
    L.attn_fwd_chunked(qg, kg, vg, [3, 4], o=o3, lse=l3, compute_stream=s, permute_stream=s)
    assert t.equal(o1, o3) and t.equal(l1, l3)
    o_ref, lse_ref = oracle.attention_ref(q.values, k.values, v.values, 1 / math.sqrt(128))
    G.check("chunked small", "bf16", o1.cpu().numpy(), l1.cpu().numpy(), o_ref, lse_ref)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_partial_and_merge_small(L, dtype):
    """Uneven KV split incl. an empty block; GPU partials + GPU merge vs the
    oracle's full attention, and the GPU merge vs the oracle merge of the
    same partials."""
    G.announce(f"partial+merge {dtype}")
    t = G.torch()
    B, Sq, Skv, H = 1, 300, 1000, 3
    q, k, v = I.make_custom((B, Sq, H, 128), (B, Skv, H, 128), dtype, seed=61)
    qg, kg, vg = G.to_gpu(q, dtype), G.to_gpu(k, dtype), G.to_gpu(v, dtype)
    cuts = [0, 1, 64, 64, 500, 1000]
    n = len(cuts) - 1
    o_parts = t.full((n, B, Sq, H, 128), float("nan"), dtype=t.float32, device="cuda")
    l_parts = t.full((n, B, H, Sq), float("nan"), dtype=t.float32, device="cuda")
    for i, (a, b) in enumerate(zip(cuts[:-1], cuts[1:])):
        L.attn_partial(qg, kg[:, a:b], vg[:, a:b], o=o_parts[i], lse=l_parts[i])
    assert t.isneginf(l_parts[2]).all() and (o_parts[2] == 0).all(), "empty block"
    o, lse = L.lse_merge(o_parts, l_parts)
    o_ref, lse_ref = oracle.attention_ref(q.values, k.values, v.values, 1 / math.sqrt(128))
    G.check(f"merge-vs-full {dtype}", dtype, o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref)
    om, lm = oracle.merge_ref(o_parts.cpu().numpy(), l_parts.cpu().numpy())
    G.check(f"merge-vs-oracle-merge {dtype}", dtype, o.cpu().numpy(), lse.cpu().numpy(), om, lm,
            tol_o=1e-5, tol_lse=1e-5)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_partial_accumulate_small(L, dtype):
    """The same uneven KV split (incl. an empty block) folded block by block
    into a running (O, LSE) that starts at O = 0, LSE = -inf: against the
    oracle's full attention, against the oracle merge of the same blocks'
    partials, and the first fold bit-identical to lsh_attn_partial. Folding
    an empty block leaves even a NaN-filled (O, LSE) untouched."""
    G.announce(f"partial accumulate {dtype}")
    t = G.torch()
    B, Sq, Skv, H = 1, 300, 1000, 3
    q, k, v = I.make_custom((B, Sq, H, 128), (B, Skv, H, 128), dtype, seed=61)
    qg, kg, vg = G.to_gpu(q, dtype), G.to_gpu(k, dtype), G.to_gpu(v, dtype)
    cuts = [0, 1, 64, 64, 500, 1000]
    o = t.zeros((B, Sq, H, 128), dtype=t.float32, device="cuda")
    lse = t.full((B, H, Sq), float("-inf"), dtype=t.float32, device="cuda")
    parts = []
    for i, (a, b) in enumerate(zip(cuts[:-1], cuts[1:])):
        parts.append(L.attn_partial(qg, kg[:, a:b], vg[:, a:b]))
        L.attn_partial_accumulate(qg, kg[:, a:b], vg[:, a:b], o, lse)
        if i == 0:
            assert t.equal(o, parts[0][0]) and t.equal(lse, parts[0][1]), "first fold"
    o_ref, lse_ref = oracle.attention_ref(q.values, k.values, v.values, 1 / math.sqrt(128))
    G.check(f"accumulate-vs-full {dtype}", dtype, o.cpu().numpy(), lse.cpu().numpy(), o_ref,
            lse_ref)
    om, lm = oracle.merge_ref(np.stack([p[0].cpu().numpy() for p in parts]),
                              np.stack([p[1].cpu().numpy() for p in parts]))
    G.check(f"accumulate-vs-oracle-merge {dtype}", dtype, o.cpu().numpy(), lse.cpu().numpy(), om,
            lm, tol_o=1e-5, tol_lse=1e-5)
    on, ln = G.poisoned_outputs(B, Sq, H)
    L.attn_partial_accumulate(qg, kg[:, :0], vg[:, :0], on, ln)
    t.cuda.synchronize()
    assert t.isnan(on).all() and t.isnan(ln).all(), "an empty block changed the result"


def test_partial_accumulate_large_grid(L):
    """H=32, Sq=4133: each fold is a launch of 544 items of 256 rows (the
    last 4 of each XCD's 68 as 128-row halves). Three blocks (1500, 1500,
    37 keys) against the
    oracle on heads 0 and 31; the first fold bit-identical to
    lsh_attn_partial."""
    G.announce("partial accumulate, large grid")
    t = G.torch()
    B, Sq, Skv, H = 1, 4133, 3037, 32
    q, k, v = I.make_custom((B, Sq, H, 128), (B, Skv, H, 128), "bf16", seed=67)
    qg, kg, vg = G.to_gpu(q, "bf16"), G.to_gpu(k, "bf16"), G.to_gpu(v, "bf16")
    o = t.zeros((B, Sq, H, 128), dtype=t.float32, device="cuda")
    lse = t.full((B, H, Sq), float("-inf"), dtype=t.float32, device="cuda")
    cuts = [0, 1500, 3000, 3037]
    for i, (a, b) in enumerate(zip(cuts[:-1], cuts[1:])):
        L.attn_partial_accumulate(qg, kg[:, a:b], vg[:, a:b], o, lse)
        if i == 0:
            o1, l1 = L.attn_partial(qg, kg[:, a:b], vg[:, a:b])
            assert t.equal(o, o1) and t.equal(lse, l1), "first fold"
    heads = [0, 31]
    o_ref, lse_ref = oracle.attention_ref(q.values, k.values, v.values, 1 / math.sqrt(128),
                                          heads=heads)
    og, lg = o.cpu().numpy(), lse.cpu().numpy()
    G.check("accumulate large grid", "bf16", og[:, :, heads], lg[:, heads], o_ref[:, :, heads],
            lse_ref[:, heads])


@pytest.mark.parametrize("n", [1, 8, 9, 17])
def test_merge_counts_vs_oracle(L, n):
    """n partials (one, exactly one group of 8, and counts that leave a
    partial group) with random outputs and LSEs, some -inf: GPU merge vs the
    oracle merge of the same values."""
    G.announce(f"merge n={n}")
    t = G.torch()
    B, Sq, H, D = 2, 37, 3, 128
    rng = np.random.default_rng(500 + n)
    o_parts = rng.standard_normal((n, B, Sq, H, D)).astype(np.float32)
    l_parts = (rng.standard_normal((n, B, H, Sq)) * 4).astype(np.float32)
    l_parts[rng.random(l_parts.shape) < 0.2] = -np.inf
    o_parts[np.broadcast_to(np.isneginf(l_parts).transpose(0, 1, 3, 2)[..., None], o_parts.shape)] = 0
    o, lse = L.lse_merge(t.from_numpy(o_parts).cuda(), t.from_numpy(l_parts).cuda())
    om, lm = oracle.merge_ref(o_parts, l_parts)
    G.check(f"merge n={n}", "f32", o.cpu().numpy(), lse.cpu().numpy(), om, lm,
            tol_o=1e-5, tol_lse=1e-5)


def test_merge_all_empty(L):
    G.announce("merge all empty")
    t = G.torch()
    o_parts = t.zeros((3, 1, 5, 2, 128), dtype=t.float32, device="cuda")
    l_parts = t.full((3, 1, 2, 5), float("-inf"), dtype=t.float32, device="cuda")
    o, lse = L.lse_merge(o_parts, l_parts)
    assert (o == 0).all() and t.isneginf(lse).all()


SPARSE_CASES = [  # (Sq, Skv, H, B)
    (128, 128, 1, 1), (300, 257, 2, 1), (640, 1000, 2, 1), (1024, 1024, 3, 1),
    # last key block holding exactly 64 keys (its second half is empty) and 65
    (256, 320, 2, 1), (256, 321, 2, 1),
    # two batch entries with different masks
    (700, 900, 3, 2),
    # last key block of 65 keys (its second half holds one), and of exactly
    # 64 (second half empty), over many blocks
    (700, 1089, 2, 2), (1000, 1344, 1, 1),
]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", SPARSE_CASES, ids=lambda s: "x".join(map(str, s)))
def test_blocksparse_vs_oracle(L, dtype, case):
    Sq, Skv, H, B = case
    G.announce(f"sparse {dtype} {case}")
    t = G.torch()
    q, k, v = I.make_custom((B, Sq, H, 128), (B, Skv, H, 128), dtype, seed=Sq + Skv)
    nqb, nkb = -(-Sq // 128), -(-Skv // 128)
    rng = np.random.default_rng(Sq * 31 + Skv)
    mask = (rng.random((B, H, nqb, nkb)) < 0.4).astype(np.uint8)
    mask[0, 0, 0, :] = 0          # a query block with no kept key block
    if nkb > 1:
        mask[-1, -1, -1, :] = 0
        mask[-1, -1, -1, nkb - 1] = 1   # only the partial last key block
    o, lse = G.poisoned_outputs(B, Sq, H)
    L.attn_fwd_blocksparse(G.to_gpu(q, dtype), G.to_gpu(k, dtype), G.to_gpu(v, dtype),
                           t.from_numpy(mask).cuda(), o=o, lse=lse)
    o_ref, lse_ref = oracle.attention_ref(q.values, k.values, v.values, 1 / math.sqrt(128),
                                          block_mask=mask)
    sig = (G.bf16_weight_sigma(oracle, q.values, k.values, v.values, 1 / math.sqrt(128), lse_ref,
                               block_mask=mask) if dtype == "bf16" else None)
    G.check(f"sparse {dtype} {case}", dtype, o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref,
            sigma=sig)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_blocksparse_all_ones_equals_dense_bitwise(L, dtype):
    """Both dtypes: the block-sparse kernel over an all-ones mask keeps the
    dense kernel's keys per wavefront in the same order (the fp32 kernel
    also splits them between the same two wavefronts)."""
    G.announce(f"sparse all-ones {dtype}")
    t = G.torch()
    Sq, Skv, H = 700, 650, 3
    q, k, v = I.make_custom((1, Sq, H, 128), (1, Skv, H, 128), dtype, seed=91)
    qg, kg, vg = G.to_gpu(q, dtype), G.to_gpu(k, dtype), G.to_gpu(v, dtype)
    mask = t.ones((1, H, 6, 6), dtype=t.uint8, device="cuda")
    o1, l1 = L.attn_fwd_blocksparse(qg, kg, vg, mask)
    o2, l2 = L.attn_fwd(qg, kg, vg)
    assert t.equal(o1, o2) and t.equal(l1, l2)


def test_blocksparse_all_ones_large_grid_equals_dense_bitwise(L):
    """H=32, S=4133: 1056 sparse workgroups, two to a CU, against the dense
    call (544 items of 256 rows, 68 per XCD: 64 run whole and the last 4
    as 128-row halves); the last key block holds 37 keys."""
    G.announce("sparse all-ones, large grid")
    t = G.torch()
    S, H = 4133, 32
    q, k, v = I.make_custom((1, S, H, 128), (1, S, H, 128), "bf16", seed=95)
    qg, kg, vg = G.to_gpu(q, "bf16"), G.to_gpu(k, "bf16"), G.to_gpu(v, "bf16")
    nb = -(-S // 128)
    mask = t.ones((1, H, nb, nb), dtype=t.uint8, device="cuda")
    o1, l1 = L.attn_fwd_blocksparse(qg, kg, vg, mask)
    o2, l2 = L.attn_fwd(qg, kg, vg)
    assert t.equal(o1, o2) and t.equal(l1, l2)


def test_blocksparse_diagonal_is_blockwise_dense(L):
    G.announce("sparse diagonal")
    t = G.torch()
    S, H = 640, 2
    q, k, v = I.make_custom((1, S, H, 128), (1, S, H, 128), "bf16", seed=93)
    qg, kg, vg = G.to_gpu(q, "bf16"), G.to_gpu(k, "bf16"), G.to_gpu(v, "bf16")
    mask = t.eye(5, dtype=t.uint8, device="cuda").expand(1, H, 5, 5).contiguous()
    o1, l1 = L.attn_fwd_blocksparse(qg, kg, vg, mask)
    for i in range(5):
        sl = slice(128 * i, 128 * (i + 1))
        o2, l2 = L.attn_fwd(qg[:, sl], kg[:, sl], vg[:, sl])
        assert t.equal(o1[:, sl], o2) and t.equal(l1[:, :, sl], l2), i


def _expected_schedule(mask):
    """The launch schedule lsh.h documents, computed from the mask: heads
    dealt whole to the 8 XCDs by kept-block total, each XCD's list (its
    heads in the order dealt, each head's rows heaviest first) interleaved
    slot by slot."""
    B, H, nq, _ = mask.shape
    G = B * H
    counts = (mask != 0).sum(axis=-1).reshape(-1).astype(np.int64)
    totals = counts.reshape(G, nq).sum(axis=1)
    heads = sorted(range(G), key=lambda g: (-totals[g], g))
    cap = -(-G // 8)
    load, xcd_heads = [0] * 8, [[] for _ in range(8)]
    for g in heads:
        x = min((x for x in range(8) if len(xcd_heads[x]) < cap), key=lambda x: (load[x], x))
        xcd_heads[x].append(g)
        load[x] += int(totals[g])
    lists = [[g * nq + r for g in hs for r in sorted(range(nq), key=lambda r: (-counts[g * nq + r], r))]
             for hs in xcd_heads]
    order = []
    for j in range(max(len(lst) for lst in lists)):
        order += [lst[j] for lst in lists if j < len(lst)]
    return counts, totals, np.array(order, dtype=np.int64)




@pytest.mark.parametrize("case", [(2, 700, 900, 3, 0), (1, 4097 * 128, 128, 1, 1)],
                         ids=["B2_H3", "4097_query_blocks"])
def test_blocksparse_schedule(L, case):
    """The schedule left in the workspace equals its definition (exact
    integer comparison). Equal masks across batch entries tie the head
    totals; the second case has more query blocks per head than one LDS
    chunk of the ranking kernel, with counts of 0 or 1 only."""
    B, Sq, Skv, H, seed = case
    G.announce(f"sparse schedule B={B} Sq={Sq} Skv={Skv} H={H}")
    t = G.torch()
    nq, nk = -(-Sq // 128), -(-Skv // 128)
    mask, _ = I.make_block_mask(B, H, nq, nk, seed=seed, lo=0.2, hi=0.8)
    if nk == 1:   # one key block: drop the diagonal rule so that rows differ
        mask = I.rng_for(5, 3, seed + 100).integers(0, 2, size=mask.shape).astype(np.uint8)
    q, k, v = I.make_custom((B, Sq, H, 128), (B, Skv, H, 128), "bf16", seed=17)
    qg, kg, vg = G.to_gpu(q, "bf16"), G.to_gpu(k, "bf16"), G.to_gpu(v, "bf16")
    need = L.blocksparse_workspace_bytes(qg, kg, vg)
    ws = t.zeros(need, dtype=t.uint8, device="cuda")
    assert ws.data_ptr() % 256 == 0
    L.attn_fwd_blocksparse(qg, kg, vg, t.from_numpy(mask).cuda(), workspace=ws)
    t.cuda.synchronize()
    want = _expected_schedule(mask)
    from long_sequence_head_amd import balance as BL
    counts, order, totals = BL.schedule_from_workspace(ws.cpu().numpy(), B * H * nq, B * H)
    got = (counts, totals, order)
    for name, g, w in zip(("counts", "totals", "order"), got, want):
        assert np.array_equal(g.astype(np.int64), w), name


@pytest.mark.parametrize("Skv", [1, 63, 64, 65, 128, 129, 191, 333, 1000, 4097])
def test_large_grid_ragged_keys(L, Skv):
    """Sq=16400, H=8: 520 items of 256 rows, 65 per XCD (two rounds of 32,
    the last item of each XCD as 128-row halves): sampled query rows (incl.
    the ragged last query tile) against the oracle over key counts that end
    mid-tile, at one tile, and below the prefetch depth."""
    G.announce(f"large grid ragged Skv={Skv}")
    t = G.torch()
    B, Sq, H = 1, 16400, 8
    q, k, v = I.make_custom((B, Sq, H, 128), (B, Skv, H, 128), "bf16", seed=700 + Skv)
    o, lse = G.poisoned_outputs(B, Sq, H)
    L.attn_fwd(G.to_gpu(q, "bf16"), G.to_gpu(k, "bf16"), G.to_gpu(v, "bf16"), o=o, lse=lse)
    t.cuda.synchronize()
    assert not t.isnan(o).any() and not t.isnan(lse).any(), "unwritten output"
    rows = I.sample_rows(Sq, 200, seed=Skv)
    o_ref, lse_ref = oracle.attention_ref(q.values, k.values, v.values, 1 / math.sqrt(128), rows=rows)
    sig = G.bf16_weight_sigma(oracle, q.values, k.values, v.values, 1 / math.sqrt(128), lse_ref,
                              rows=rows)
    ridx = t.from_numpy(rows).cuda()
    G.check(f"large grid Skv={Skv}", "bf16", o.index_select(1, ridx).cpu().numpy(),
            lse.index_select(2, ridx).cpu().numpy(), o_ref, lse_ref, sigma=sig)
