"""Plant mistakes in copies of the oracle (on the CPU) and check that the
pins catch each one: a dropped term, a wrong sign, a wrong index, a
transposed operand."""
import numpy as np
import pytest

import oracle
from oracle import attention as A
from tests import oracle_pins as P


def _fails_some_pin(attn, merge, pins):
    for pin in pins:
        try:
            pin(attn, merge)
        except AssertionError:
            return True
    return False


def _with_patched_core(core):
    def attn(q, k, v, scale, **kw):
        saved = A._softmax_weighted_sum
        A._softmax_weighted_sum = core
        try:
            return A.attention_ref(q, k, v, scale, **kw)
        finally:
            A._softmax_weighted_sum = saved
    return attn


def _core_no_normalise(s, vh):
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    return e @ vh, m + np.log(e.sum(axis=1))


def _core_lse_without_max(s, vh):
    m = s.max(axis=1)
    e = np.exp(s - m[:, None])
    l = e.sum(axis=1)
    return (e @ vh) / l[:, None], np.log(l)


def _core_wrong_sign(s, vh):
    m = s.min(axis=1)
    e = np.exp(-(s - m[:, None]))
    l = e.sum(axis=1)
    return (e @ vh) / l[:, None], -m + np.log(l)


def _core_softmax_over_queries(s, vh):
    m = s.max(axis=0)
    e = np.exp(s - m[None, :])
    l = e.sum(axis=0)
    p = e / l[None, :]
    return p @ vh, np.log(e.sum(axis=1)) + s.max(axis=1)


MUTANTS = {
    "no_normalisation": (_with_patched_core(_core_no_normalise), oracle.merge_ref),
    "lse_without_max": (_with_patched_core(_core_lse_without_max), oracle.merge_ref),
    "wrong_sign": (_with_patched_core(_core_wrong_sign), oracle.merge_ref),
    "softmax_over_queries": (_with_patched_core(_core_softmax_over_queries), oracle.merge_ref),
    "scale_squared": (lambda q, k, v, s, **kw: oracle.attention_ref(q, k, v, s * s, **kw), oracle.merge_ref),
    "k_v_swapped": (lambda q, k, v, s, **kw: oracle.attention_ref(q, v, k, s, **kw), oracle.merge_ref),
    "last_key_dropped": (lambda q, k, v, s, **kw: oracle.attention_ref(q, k[:, :-1] if k.shape[1] > 1 else k,
                                                                        v[:, :-1] if v.shape[1] > 1 else v, s, **kw),
                         oracle.merge_ref),
    "heads_shifted": (lambda q, k, v, s, **kw: oracle.attention_ref(q, np.roll(k, 1, axis=2), v, s, **kw),
                      oracle.merge_ref),
    "mask_transposed": (lambda q, k, v, s, block_mask=None, **kw: oracle.attention_ref(
        q, k, v, s, block_mask=None if block_mask is None else _transpose_mask(block_mask), **kw),
        oracle.merge_ref),
}


def _transpose_mask(m):
    t = np.swapaxes(m, 2, 3)
    if t.shape == m.shape:
        return np.ascontiguousarray(t)
    # non-square masks: reflect the kept blocks inside the original shape
    out = np.zeros_like(m)
    n = min(m.shape[2], m.shape[3])
    out[..., :n, :n] = t[..., :n, :n]
    return out


def _merge_unnormalised(o_parts, lse_parts):
    o, lse = oracle.merge_ref(o_parts, lse_parts)
    M = np.max(lse_parts, axis=0)
    w = np.exp(lse_parts - M[None]).transpose(0, 1, 3, 2)[..., None]
    return (w * o_parts).sum(axis=0), lse


def _merge_lse_without_max(o_parts, lse_parts):
    o, _ = oracle.merge_ref(o_parts, lse_parts)
    M = np.max(lse_parts, axis=0)
    return o, np.log(np.exp(lse_parts - M[None]).sum(axis=0))


MERGE_MUTANTS = {"merge_unnormalised": _merge_unnormalised,
                 "merge_lse_without_max": _merge_lse_without_max}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_attention_mutant_is_caught(name):
    attn, merge = MUTANTS[name]
    assert _fails_some_pin(attn, merge, P.ATTN_PINS + P.MERGE_PINS), name


@pytest.mark.parametrize("name", sorted(MERGE_MUTANTS))
def test_merge_mutant_is_caught(name):
    assert _fails_some_pin(oracle.attention_ref, MERGE_MUTANTS[name], P.MERGE_PINS), name
