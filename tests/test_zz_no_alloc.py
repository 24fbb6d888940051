"""The allocation-free block-sparse entry point (static device scratch)
against the workspace entry point and the fp64 oracle: two calls in a row,
the second with a smaller input, each bitwise equal to
lsh_attn_fwd_blocksparse on the same inputs (same kernels, same schedule)
and within the bf16 bars of the oracle."""
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


def _case(L, B, Sq, Skv, H, seed):
    t = G.torch()
    G.announce(f"noalloc sparse B={B} Sq={Sq} Skv={Skv} H={H}")
    nq, nk = -(-Sq // 128), -(-Skv // 128)
    q, k, v = I.make_custom((B, Sq, H, 128), (B, Skv, H, 128), "bf16", seed=seed)
    mask, _ = I.make_block_mask(B, H, nq, nk, seed=seed, lo=0.2, hi=0.7)
    mask[0, 0, 0, :] = 0   # a query block with no kept key block: O = 0, LSE = -inf
    qg, kg, vg = G.to_gpu(q, "bf16"), G.to_gpu(k, "bf16"), G.to_gpu(v, "bf16")
    mg = t.from_numpy(mask).cuda()
    o1, l1 = G.poisoned_outputs(B, Sq, H)
    L.attn_fwd_blocksparse_noalloc(qg, kg, vg, mg, o=o1, lse=l1)
    o2, l2 = G.poisoned_outputs(B, Sq, H)
    L.attn_fwd_blocksparse(qg, kg, vg, mg, o=o2, lse=l2)
    t.cuda.synchronize()
    assert t.equal(o1, o2), "O differs from the workspace entry point"
    assert t.equal(l1, l2), "LSE differs from the workspace entry point"
    o_ref, lse_ref = oracle.attention_ref(q.values, k.values, v.values, 1 / math.sqrt(128),
                                          block_mask=mask)
    sig = G.bf16_weight_sigma(oracle, q.values, k.values, v.values, 1 / math.sqrt(128), lse_ref,
                              block_mask=mask)
    G.check(f"noalloc sparse B={B} Sq={Sq} H={H}", "bf16", o1.cpu().numpy(), l1.cpu().numpy(),
            o_ref, lse_ref, sigma=sig)


def test_noalloc_two_calls_second_smaller(L):
    _case(L, 2, 1100, 900, 3, seed=41)
    _case(L, 1, 300, 260, 2, seed=42)
