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


# ------------------------------------------------------------------ backward

def _bwd_mutant(kind):
    """A gradient implementation with one planted mistake."""
    def bwd(q, k, v, do, scale, rows=None, keys=None, heads=None):
        q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
        B, Sq, H, D = q.shape
        dq = np.zeros_like(q)
        dk = np.zeros_like(k)
        dv = np.zeros_like(v)
        for b in range(B):
            for h in range(H):
                qh, kh, vh, doh = q[b, :, h], k[b, :, h], v[b, :, h], do[b, :, h]
                s = scale * qh @ kh.T
                e = np.exp(s - s.max(axis=1, keepdims=True))
                p = e if kind == "p_unnormalised" else e / e.sum(axis=1, keepdims=True)
                dp = doh @ vh.T
                delta = (p * dp).sum(axis=1, keepdims=True)
                if kind == "no_delta":
                    ds = p * dp
                elif kind == "delta_sign":
                    ds = p * (dp + delta)
                else:
                    ds = p * (dp - delta)
                dq[b, :, h] = (1.0 if kind == "dq_no_scale" else scale) * ds @ (
                    vh if kind == "dq_uses_v" else kh)
                dk[b, :, h] = scale * ds.T @ (doh if kind == "dk_uses_do" else qh)
                dv[b, :, h] = (ds if kind == "dv_uses_ds" else p).T @ doh
        if rows is not None:
            dq = dq[:, np.asarray(rows)]
        if keys is not None:
            dk, dv = dk[:, np.asarray(keys)], dv[:, np.asarray(keys)]
        return dq, dk, dv
    return bwd


BWD_MUTANTS = ["no_delta", "delta_sign", "dq_no_scale", "dq_uses_v", "dk_uses_do",
               "dv_uses_ds", "p_unnormalised"]


def test_backward_mutant_helper_is_faithful():
    """Without a planted mistake the helper passes every pin, so a failing
    mutant fails because of its mistake."""
    for pin in P.BWD_PINS:
        pin(_bwd_mutant("none"), oracle.attention_ref)


@pytest.mark.parametrize("kind", BWD_MUTANTS)
def test_backward_mutant_is_caught(kind):
    bwd = _bwd_mutant(kind)
    caught = False
    for pin in P.BWD_PINS:
        try:
            pin(bwd, oracle.attention_ref)
        except AssertionError:
            caught = True
            break
    assert caught, f"no pin catches backward mutant {kind}"
