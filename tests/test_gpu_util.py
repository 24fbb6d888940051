"""CPU checks of the parity-test helpers in tests/gpu_util.py."""
import math

import numpy as np

import oracle
from tests import gpu_util as G


def test_bf16_weight_sigma_equals_direct_sum():
    """sigma = 2^-8 / sqrt(3) * sqrt(sum_j w_j^2 v_j^2), with the weights
    w = softmax(scale q k^T) formed directly here, on a tiny case with a
    block mask that empties one query block."""
    rng = np.random.default_rng(0)
    q = rng.standard_normal((2, 5, 2, 8))
    k = rng.standard_normal((2, 7, 2, 8))
    v = rng.standard_normal((2, 7, 2, 8)).astype(np.float32)
    sc = 0.3
    o, lse = oracle.attention_ref(q, k, v, sc)
    sig = G.bf16_weight_sigma(oracle, q, k, v, sc, lse)
    s = np.einsum("bihd,bjhd->bhij", q, k) * sc
    w = np.exp(s - s.max(-1, keepdims=True))
    w /= w.sum(-1, keepdims=True)
    direct = G.U_BF16 / math.sqrt(3) * np.sqrt(
        np.einsum("bhij,bjhd->bihd", w ** 2, v.astype(np.float64) ** 2))
    assert np.allclose(sig, direct, rtol=1e-6, atol=1e-12)


def test_bf16_weight_sigma_empty_rows_are_zero():
    rng = np.random.default_rng(1)
    q = rng.standard_normal((1, 200, 1, 4))
    k = rng.standard_normal((1, 300, 1, 4))
    v = rng.standard_normal((1, 300, 1, 4)).astype(np.float32)
    mask = np.ones((1, 1, 2, 3), dtype=np.uint8)
    mask[0, 0, 1] = 0                       # query rows 128..199 attend to nothing
    o, lse = oracle.attention_ref(q, k, v, 0.5, block_mask=mask)
    sig = G.bf16_weight_sigma(oracle, q, k, v, 0.5, lse, block_mask=mask)
    assert np.all(sig[:, 128:] == 0) and np.all(sig[:, :128] > 0)


def test_dense_bf16_launch_cases():
    """The launch rule on the workloads' shapes and on the shapes the GPU
    tests use to reach each path (256 CUs)."""
    # 56160 queries x 40 heads: 8800 items, 1100 per XCD = 34 rounds + 12
    assert G.dense_bf16_launch(1, 56160, 40) == ("256-row, split tail", 8800 + 8 * 12, 12)
    # head chunks of S = 32760: 128 blocks per head, rounds of 32 per XCD
    assert G.dense_bf16_launch(1, 32760, 16) == ("256-row", 2048)
    assert G.dense_bf16_launch(1, 32760, 12) == ("256-row", 1536)
    assert G.dense_bf16_launch(1, 32760, 40) == ("256-row", 5120)
    # a ring round: 128 items of 256 rows would leave half the CUs idle
    assert G.dense_bf16_launch(1, 4096, 8) == ("128-row", 256)
    # 544 items, 68 per XCD: the last 4 of each as halves
    assert G.dense_bf16_launch(1, 4133, 32) == ("256-row, split tail", 576, 4)
    # remainders above half an XCD, or one round only, stay whole
    assert G.dense_bf16_launch(1, 256 * 52, 8) == ("256-row", 416)
    assert G.dense_bf16_launch(1, 16384, 8) == ("256-row", 512)
    assert G.dense_bf16_launch(1, 16400, 8) == ("256-row, split tail", 528, 1)
