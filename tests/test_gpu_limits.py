"""Edge sizes on the GPU against the fp64 oracle: one query against a very
long key sequence and the reverse, and heads whose rows span just under the
2 GiB that the kernels' 32-bit buffer offsets allow (the validation limit
of lsh.h), for the forward (K and V rows) and the backward (Q and dO
rows)."""
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


@pytest.mark.parametrize("Sq,Skv", [(1, 100003), (100003, 1)], ids=["one_query", "one_key"])
def test_long_and_degenerate_sequences(L, Sq, Skv):
    B, H = 1, 2
    G.announce(f"edge Sq={Sq} Skv={Skv}")
    q, k, v = I.make_custom((B, Sq, H, 128), (B, Skv, H, 128), "bf16", seed=Sq + 2 * Skv)
    o, lse = G.poisoned_outputs(B, Sq, H)
    L.attn_fwd(G.to_gpu(q, "bf16"), G.to_gpu(k, "bf16"), G.to_gpu(v, "bf16"), o=o, lse=lse)
    rows = I.sample_rows(Sq, 300, seed=3)
    o_ref, lse_ref = oracle.attention_ref(q.values, k.values, v.values, 1 / math.sqrt(128),
                                          rows=rows)
    sig = G.bf16_weight_sigma(oracle, q.values, k.values, v.values, 1 / math.sqrt(128), lse_ref,
                              rows=rows)
    t = G.torch()
    ridx = t.from_numpy(rows).cuda()
    G.check(f"edge Sq={Sq} Skv={Skv}", "bf16", o.index_select(1, ridx).cpu().numpy(),
            lse.index_select(2, ridx).cpu().numpy(), o_ref, lse_ref, sigma=sig)
    assert not t.isnan(o).any() and not t.isnan(lse).any(), "unwritten output"


def _span_bytes(S, H):
    return (S - 1) * H * 128 * 2 + 128 * 2


def test_forward_head_rows_at_2gib(L):
    """H=64 interleaved heads and Skv=131072, the largest key count the
    validation accepts for that layout: one head's K (and V) rows span
    2^31 - 16128 bytes. Heads 0 and 63 (the last, whose rows end nearest
    the limit) are checked on every query row."""
    B, Sq, Skv, H = 1, 130, 131072, 64
    assert 0 < 2 ** 31 - _span_bytes(Skv, H) <= 2 * 128 * H
    G.announce(f"forward span {_span_bytes(Skv, H) / 2 ** 30:.3f} GiB")
    q, k, v = I.make_custom((B, Sq, H, 128), (B, Skv, H, 128), "bf16", seed=64)
    o, lse = G.poisoned_outputs(B, Sq, H)
    L.attn_fwd(G.to_gpu(q, "bf16"), G.to_gpu(k, "bf16"), G.to_gpu(v, "bf16"), o=o, lse=lse)
    heads = [0, 63]
    o_ref, lse_ref = oracle.attention_ref(q.values, k.values, v.values, 1 / math.sqrt(128),
                                          heads=heads)
    sig = G.bf16_weight_sigma(oracle, q.values, k.values, v.values, 1 / math.sqrt(128), lse_ref,
                              heads=heads)
    og, lg = o.cpu().numpy(), lse.cpu().numpy()
    G.check("forward at the 2 GiB span", "bf16", og[:, :, heads], lg[:, heads], o_ref[:, :, heads],
            lse_ref[:, heads], sigma=sig[:, :, heads])


def test_backward_head_rows_at_2gib(L):
    """H=64 interleaved heads with Sq=131072: one head's Q (and dO) rows
    span 2^31 - 16128 bytes, the largest the validation accepts. dK and dV
    of head 63 are checked on every key (each is a sum over all 131072
    queries), dQ on sampled rows."""
    B, Sq, Skv, H = 1, 131072, 200, 64
    assert 0 < 2 ** 31 - _span_bytes(Sq, H) <= 2 * 128 * H
    G.announce(f"backward span {_span_bytes(Sq, H) / 2 ** 30:.3f} GiB")
    t = G.torch()
    q, k, v = I.make_custom((B, Sq, H, 128), (B, Skv, H, 128), "bf16", seed=65)
    do = I.make_custom_dout((B, Sq, H, 128), "bf16", seed=65)
    qg, kg, vg, dog = (G.to_gpu(x, "bf16") for x in (q, k, v, do))
    o, lse = L.attn_fwd(qg, kg, vg)
    dq, dk, dv = L.attn_bwd(qg, kg, vg, dog, o, lse)
    t.cuda.synchronize()
    del o, lse, qg, kg, vg, dog
    h = 63
    rows = I.sample_rows(Sq, 128, seed=5)
    ref = oracle.attention_bwd_ref(q.values, k.values, v.values, do.values, 1 / math.sqrt(128),
                                   rows=rows, heads=[h])
    ridx = t.from_numpy(rows).cuda()
    got = (dq.index_select(1, ridx)[:, :, h].cpu().numpy(), dk[:, :, h].cpu().numpy(),
           dv[:, :, h].cpu().numpy())
    G.check_grads("backward at the 2 GiB span, head 63", got, [r[:, :, h] for r in ref])
    assert t.isfinite(dk).all() and t.isfinite(dv).all()
