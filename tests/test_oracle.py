"""The fp64 oracle against its pins (closed forms, worked example, brute
force, library softmax, invariants). CPU only."""
import numpy as np
import pytest

import oracle
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ATTN_PINS, ids=lambda f: f.__name__)
def test_attention_pin(pin):
    pin(oracle.attention_ref, oracle.merge_ref)


@pytest.mark.parametrize("pin", P.MERGE_PINS, ids=lambda f: f.__name__)
def test_merge_pin(pin):
    pin(oracle.attention_ref, oracle.merge_ref)


@pytest.mark.parametrize("pin", P.BWD_PINS, ids=lambda f: f.__name__)
def test_backward_pin(pin):
    pin(oracle.attention_bwd_ref, oracle.attention_ref)


def test_permute_indexwise():
    """dst[b, h-h0, s, :] == src[b, s, h, :], checked element by element."""
    r = np.random.default_rng(0)
    x = r.integers(0, 1 << 16, size=(2, 5, 7, 3), dtype=np.uint16)
    for h0, hc in [(0, 7), (2, 3), (6, 1)]:
        y = oracle.permute_ref(x, h0, hc)
        assert y.shape == (2, hc, 5, 3)
        for b in range(2):
            for hh in range(hc):
                for s in range(5):
                    for d in range(3):
                        assert y[b, hh, s, d] == x[b, s, h0 + hh, d]
        assert np.array_equal(oracle.inverse_permute_ref(y), x[:, :, h0:h0 + hc])


def test_permute_chunks_cover_heads():
    """Chunks {16,12,12} of 40 heads, concatenated, are the full head-major copy."""
    r = np.random.default_rng(1)
    x = r.integers(0, 1 << 16, size=(1, 9, 40, 4), dtype=np.uint16)
    parts, h0 = [], 0
    for hc in (16, 12, 12):
        parts.append(oracle.permute_ref(x, h0, hc))
        h0 += hc
    assert np.array_equal(np.concatenate(parts, axis=1), oracle.permute_ref(x, 0, 40))


def test_flops():
    assert oracle.attention_flops(1, 40, 56160, 56160, 128) == 4 * 40 * 56160 ** 2 * 128
    assert oracle.attention_flops(4, 32, 128, 128, 128) == 1073741824
