"""The five workloads at full size, in the launch configuration bench.py
times, against the fp64 oracle on sampled rows (every row of the last,
ragged query tile is always included), plus the bit-identity checks of the
chunked pipeline. Inputs are the seeded synthetic tensors of lsh_inputs."""
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


def _upload(w, seed=0):
    q, k, v = I.make_qkv(w, seed=seed)
    return (q, k, v), (G.to_gpu(q, w.dtype), G.to_gpu(k, w.dtype), G.to_gpu(v, w.dtype))


def _check_rows(name, w, o, lse, q, k, v, rows, heads, mask=None):
    o_ref, lse_ref = oracle.attention_ref(q.values, k.values, v.values, w.scale, rows=rows,
                                          heads=heads, block_mask=mask)
    t = G.torch()
    ridx = t.from_numpy(rows).cuda()
    og = o.index_select(1, ridx).cpu().numpy()
    lg = lse.index_select(2, ridx).cpu().numpy()
    hs = list(heads)
    sig = None
    if w.dtype == "bf16":
        sig = G.bf16_weight_sigma(oracle, q.values, k.values, v.values, w.scale, lse_ref, rows=rows,
                                  heads=heads, block_mask=mask)[:, :, hs]
    return G.check(name, w.dtype, og[:, :, hs], lg[:, hs], o_ref[:, :, hs], lse_ref[:, hs],
                   sigma=sig)


def test_workload1_dense_f32_full(L):
    w = I.WORKLOADS[1]
    G.announce(w.name)
    (q, k, v), (qg, kg, vg) = _upload(w)
    o, lse = G.poisoned_outputs(w.B, w.Sq, w.H)
    L.attn_fwd(qg, kg, vg, o=o, lse=lse)
    o_ref, lse_ref = oracle.attention_ref(q.values, k.values, v.values, w.scale)
    G.check(w.name, w.dtype, o.cpu().numpy(), lse.cpu().numpy(), o_ref, lse_ref)
    # the TP page's gathered output shape
    assert tuple(o.reshape(w.B, w.Sq, w.H * w.D).shape) == (4, 128, 4096)


def test_workload2_ring_partials_merge(L):
    w = I.WORKLOADS[2]
    G.announce(w.name)
    t = G.torch()
    (q, k, v), (qg, kg, vg) = _upload(w)
    n = w.kv_blocks
    blk = w.Skv // n
    o_parts = t.full((n, w.B, w.Sq, w.H, w.D), float("nan"), dtype=t.float32, device="cuda")
    l_parts = t.full((n, w.B, w.H, w.Sq), float("nan"), dtype=t.float32, device="cuda")
    for i in range(n):
        L.attn_partial(qg, kg[:, i * blk:(i + 1) * blk], vg[:, i * blk:(i + 1) * blk],
                       o=o_parts[i], lse=l_parts[i])
    o, lse = L.lse_merge(o_parts, l_parts)
    rows = I.sample_rows(w.Sq, 96, seed=2)
    _check_rows(w.name + " merged", w, o, lse, q, k, v, rows, range(w.H))
    # one partial against the oracle over its own block
    i = 5
    ob, lb = oracle.attention_ref(q.values, k.values[:, i * blk:(i + 1) * blk],
                                  v.values[:, i * blk:(i + 1) * blk], w.scale, rows=rows)
    ridx = t.from_numpy(rows).cuda()
    G.check(w.name + " partial 5", w.dtype, o_parts[i].index_select(1, ridx).cpu().numpy(),
            l_parts[i].index_select(2, ridx).cpu().numpy(), ob, lb)
    # GPU merge vs the oracle merge of the same GPU partials, all rows
    om, lm = oracle.merge_ref(o_parts.cpu().numpy(), l_parts.cpu().numpy())
    G.check(w.name + " merge-vs-oracle-merge", w.dtype, o.cpu().numpy(), lse.cpu().numpy(), om, lm,
            tol_o=1e-5, tol_lse=1e-5)


def test_workload3_chunked_two_streams(L):
    w = I.WORKLOADS[3]
    G.announce(w.name)
    t = G.torch()
    (q, k, v), (qg, kg, vg) = _upload(w)
    o1, l1 = G.poisoned_outputs(w.B, w.Sq, w.H)
    L.attn_fwd_chunked(qg, kg, vg, list(w.head_chunks), o=o1, lse=l1)
    o2, l2 = G.poisoned_outputs(w.B, w.Sq, w.H)
    L.attn_fwd(qg, kg, vg, o=o2, lse=l2)
    t.cuda.synchronize()
    assert t.equal(o1, o2) and t.equal(l1, l2), "chunked and unchunked differ"
    o3, l3 = G.poisoned_outputs(w.B, w.Sq, w.H)
    L.attn_fwd_chunked(qg, kg, vg, [w.H], o=o3, lse=l3)
    t.cuda.synchronize()
    assert t.equal(o1, o3) and t.equal(l1, l3), "chunking {16,12,12} vs {40} differ"
    rows = I.sample_rows(w.Sq, 48, seed=3)
    _check_rows(w.name, w, o1, l1, q, k, v, rows, [0, 15, 16, 27, 28, 39])
    # permute of each chunk, bit-exact
    h0 = 0
    for hc in w.head_chunks:
        y = L.head_permute(kg, h0, hc)
        got = y.cpu().view(t.int16).numpy().view(np.uint16)
        assert np.array_equal(got, oracle.permute_ref(k.bits, h0, hc)), (h0, hc)
        del y
        h0 += hc


def test_workload4_dense_bf16_56k(L):
    w = I.WORKLOADS[4]
    G.announce(w.name)
    t = G.torch()
    (q, k, v), (qg, kg, vg) = _upload(w)
    o, lse = G.poisoned_outputs(w.B, w.Sq, w.H)
    L.attn_fwd(qg, kg, vg, o=o, lse=lse)
    t.cuda.synchronize()
    assert not t.isnan(o).any() and not t.isnan(lse).any(), "unwritten output"
    rows = I.sample_rows(w.Sq, 48, seed=4)
    _check_rows(w.name, w, o, lse, q, k, v, rows, [0, 13, 26, 39])
    o2, l2 = L.attn_fwd(qg, kg, vg)
    assert t.equal(o, o2) and t.equal(lse, l2), "run-to-run"


def test_workload5_blocksparse(L):
    w = I.WORKLOADS[5]
    G.announce(w.name)
    t = G.torch()
    (q, k, v), (qg, kg, vg) = _upload(w)
    nb = w.Sq // I.MASK_BLOCK
    mask, dens = I.make_block_mask(w.B, w.H, nb, nb, seed=0)
    o, lse = G.poisoned_outputs(w.B, w.Sq, w.H)
    L.attn_fwd_blocksparse(qg, kg, vg, t.from_numpy(mask).cuda(), o=o, lse=lse)
    t.cuda.synchronize()
    assert not t.isnan(o).any() and not t.isnan(lse).any(), "unwritten output"
    heads = sorted({int(np.argmin(dens)), int(np.argmax(dens)), 0, 19, 39})
    rows = I.sample_rows(w.Sq, 48, seed=5)
    _check_rows(w.name, w, o, lse, q, k, v, rows, heads, mask=mask)


def test_workload6_backward_sampled(L):
    """Backward at S=32760, H=40 as bench.py runs it (library forward, then
    lsh_attn_bwd): dQ on sampled query rows and dK, dV on sampled keys of
    head 37 against the oracle (which still sums over every row and key);
    the last ragged 128-row block and key block are always included."""
    w = I.WORKLOADS[6]
    G.announce(w.name)
    t = G.torch()
    (q, k, v), (qg, kg, vg) = _upload(w)
    do = I.make_dout(w)
    dog = G.to_gpu(do, w.dtype)
    o, lse = L.attn_fwd(qg, kg, vg)
    ws = t.empty(L.bwd_workspace_bytes(qg, kg, vg) + 256, dtype=t.uint8, device="cuda")
    dq, dk, dv = L.attn_bwd(qg, kg, vg, dog, o, lse, workspace=ws)
    del o, lse, qg, kg, vg, dog
    h = 37
    rows = I.sample_rows(w.Sq, 64, seed=6)
    keys = I.sample_rows(w.Skv, 64, seed=7)
    ref = oracle.attention_bwd_ref(q.values, k.values, v.values, do.values, w.scale, rows=rows,
                                   keys=keys, heads=[h])
    ridx, kidx = t.from_numpy(rows).cuda(), t.from_numpy(keys).cuda()
    got = (dq.index_select(1, ridx)[:, :, h].cpu().numpy(),
           dk.index_select(1, kidx)[:, :, h].cpu().numpy(),
           dv.index_select(1, kidx)[:, :, h].cpu().numpy())
    G.check_grads(w.name + " head 37", got, [r[:, :, h] for r in ref])
    assert t.isfinite(dq).all() and t.isfinite(dk).all() and t.isfinite(dv).all()
