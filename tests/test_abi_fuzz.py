"""Property-based fuzz of the C ABI's argument checks (CPU only: no kernel
is launched; every call either fails validation or, with no device present,
stops at the device check).

The expected status comes from the rules include/lsh.h states, restated
here in exact integer arithmetic and in the order lsh.h gives them; the
library must return that status for any argument block, including sizes
and strides whose products leave the 64-bit range."""
import ctypes
import math
import os

import pytest

hyp = pytest.importorskip("hypothesis")
from hypothesis import given, settings, strategies as st  # noqa: E402

from long_sequence_head_amd import _lib  # noqa: E402

OK, INVALID, UNSUPPORTED, NO_DEVICE = (_lib.LSH_OK, _lib.LSH_ERR_INVALID,
                                       _lib.LSH_ERR_UNSUPPORTED, _lib.LSH_ERR_NO_DEVICE)
D = 128
LIM = 1 << 30
BIG = 1 << 31


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("liblsh.so not built")
    lib = _lib.load()
    if lib.lsh_device_check() == OK:
        pytest.skip("a device is present: valid arguments would launch kernels")
    return lib


sizes = st.one_of(st.integers(-2, 5), st.integers(1, 5000),
                  st.sampled_from([LIM - 1, LIM, 1 << 29, (1 << 29) + 7, 1 << 40]))
strides = st.one_of(st.sampled_from([0, 8, 64, 128, 136, 1 << 20]), st.integers(-256, 1 << 24),
                    st.sampled_from([1 << 33, 1 << 40, (1 << 61) + 8, (1 << 62), -(1 << 62)]))
pointers = st.sampled_from([0, 1 << 20, (1 << 20) + 8, 1 << 44])


def expected_fwd(a, allow_empty_kv):
    """The checks of an attention argument block, first failing one wins."""
    if a["dtype"] not in (_lib.LSH_F32, _lib.LSH_BF16):
        return INVALID
    if a["reserved"] != 0:
        return INVALID
    B, Sq, Skv, H, Dd = a["B"], a["Sq"], a["Skv"], a["H"], a["D"]
    if B < 1 or Sq < 1 or H < 1 or Dd < 1:
        return INVALID
    if Skv < (0 if allow_empty_kv else 1):
        return INVALID
    if Dd != D:
        return UNSUPPORTED
    if B >= LIM or Sq >= LIM or Skv >= LIM or H >= LIM:
        return UNSUPPORTED
    if B * H * -(-Sq // 128) >= BIG or B * Sq * H >= BIG:
        return UNSUPPORTED
    if not a["q"] or not a["o"] or not a["lse"]:
        return INVALID
    need_kv = Skv > 0
    if need_kv and (not a["k"] or not a["v"]):
        return INVALID
    if not math.isfinite(a["scale"]):
        return INVALID
    for p in (a["q"], a["k"], a["v"], a["o"], a["lse"]):
        if p and p % 16:
            return INVALID
    eb = 4 if a["dtype"] == _lib.LSH_F32 else 2
    if a["dtype"] == _lib.LSH_BF16 and need_kv:
        for s in (a["k_stride"], a["v_stride"]):
            if (Skv - 1) * s[1] * eb + D * eb >= BIG:
                return UNSUPPORTED
    for t, (s, e) in enumerate(((a["q_stride"], eb), (a["k_stride"], eb), (a["v_stride"], eb),
                                (a["o_stride"], 4))):
        if t in (1, 2) and not need_kv:
            continue
        for x in s:
            if x < 0 or (x * e) % 16:
                return INVALID
    return NO_DEVICE


def to_struct(a):
    s = _lib.AttnArgs()
    for f in ("q", "k", "v", "o", "lse"):
        setattr(s, f, a[f] or None)
    for f in ("dtype", "reserved", "B", "Sq", "Skv", "H", "D"):
        setattr(s, f, a[f])
    for f in ("q_stride", "k_stride", "v_stride", "o_stride"):
        getattr(s, f)[:] = a[f]
    s.scale = a["scale"]
    return s


attn_args = st.fixed_dictionaries({
    "q": pointers, "k": pointers, "v": pointers, "o": pointers, "lse": pointers,
    "dtype": st.sampled_from([_lib.LSH_F32, _lib.LSH_BF16, 7]),
    "reserved": st.sampled_from([0, 0, 0, 1]),
    "B": sizes, "Sq": sizes, "Skv": st.one_of(st.just(0), sizes), "H": sizes,
    "D": st.sampled_from([128, 128, 128, 64]),
    "q_stride": st.tuples(strides, strides, strides),
    "k_stride": st.tuples(strides, strides, strides),
    "v_stride": st.tuples(strides, strides, strides),
    "o_stride": st.tuples(strides, strides, strides),
    "scale": st.sampled_from([0.088, 1.0, float("inf"), float("nan"), -0.5]),
})


@settings(max_examples=2000, deadline=None, derandomize=True)
@given(a=attn_args)
def test_fwd_and_partial_validation_matches_the_rules(lib, a):
    s = to_struct(a)
    if s.scale != a["scale"] and math.isfinite(a["scale"]):
        a = dict(a, scale=s.scale)   # the float the library sees
    assert lib.lsh_attn_fwd(ctypes.byref(s), None) == expected_fwd(a, False), a
    assert lib.lsh_attn_partial(ctypes.byref(s), None) == expected_fwd(a, True), a


def expected_bwd(a):
    if a["dtype"] not in (_lib.LSH_F32, _lib.LSH_BF16):
        return INVALID
    if a["reserved"] != 0:
        return INVALID
    B, Sq, Skv, H, Dd = a["B"], a["Sq"], a["Skv"], a["H"], a["D"]
    if B < 1 or Sq < 1 or Skv < 1 or H < 1 or Dd < 1:
        return INVALID
    if Dd != D:
        return UNSUPPORTED
    if a["dtype"] != _lib.LSH_BF16:
        return UNSUPPORTED
    if B >= LIM or Sq >= LIM or Skv >= LIM or H >= LIM:
        return UNSUPPORTED
    bh = B * H
    if (bh * -(-Sq // 128) >= BIG or bh * -(-Skv // 128) >= BIG or bh * -(-Sq // 64) * 4 >= BIG
            or B * Sq * H >= BIG or B * Skv * H >= BIG):
        return UNSUPPORTED
    for p in (a["q"], a["k"], a["v"], a["dout"], a["o"], a["lse"], a["dq"], a["dk"], a["dv"]):
        if not p or p % 16:
            return INVALID
    if not math.isfinite(a["scale"]):
        return INVALID
    names = ("q_stride", "k_stride", "v_stride", "do_stride", "o_stride", "dq_stride",
             "dk_stride", "dv_stride")
    ebs = (2, 2, 2, 2, 4, 4, 4, 4)
    for n, e in zip(names, ebs):
        for x in a[n]:
            if x < 0 or (x * e) % 16:
                return INVALID
    for rows, n in ((Sq, "q_stride"), (Skv, "k_stride"), (Skv, "v_stride"), (Sq, "do_stride")):
        if (rows - 1) * a[n][1] * 2 + D * 2 >= BIG:
            return UNSUPPORTED
    return NO_DEVICE


bwd_args = st.fixed_dictionaries({
    **{p: pointers for p in ("q", "k", "v", "dout", "o", "lse", "dq", "dk", "dv")},
    "dtype": st.sampled_from([_lib.LSH_BF16, _lib.LSH_BF16, _lib.LSH_F32, 7]),
    "reserved": st.sampled_from([0, 0, 0, 1]),
    "B": sizes, "Sq": sizes, "Skv": sizes, "H": sizes,
    "D": st.sampled_from([128, 128, 128, 64]),
    **{n: st.tuples(strides, strides, strides) for n in (
        "q_stride", "k_stride", "v_stride", "do_stride", "o_stride", "dq_stride", "dk_stride",
        "dv_stride")},
    "scale": st.sampled_from([0.088, float("inf"), float("nan")]),
})


@settings(max_examples=2000, deadline=None, derandomize=True)
@given(a=bwd_args)
def test_bwd_validation_matches_the_rules(lib, a):
    s = _lib.AttnBwdArgs()
    for f in ("q", "k", "v", "dout", "o", "lse", "dq", "dk", "dv"):
        setattr(s, f, a[f] or None)
    for f in ("dtype", "reserved", "B", "Sq", "Skv", "H", "D"):
        setattr(s, f, a[f])
    for f in ("q_stride", "k_stride", "v_stride", "do_stride", "o_stride", "dq_stride",
              "dk_stride", "dv_stride"):
        getattr(s, f)[:] = a[f]
    s.scale = a["scale"]
    ws = ctypes.c_void_p(1 << 20)
    got = lib.lsh_attn_bwd(ctypes.byref(s), ws, 1 << 40, None)
    assert got == expected_bwd(a), a


big_ints = st.one_of(st.integers(-2, 300), st.sampled_from([1 << 22, 1 << 31, 1 << 40, 1 << 62]))


@settings(max_examples=1500, deadline=None, derandomize=True)
@given(n=st.sampled_from([0, 1, 8, 4096, 4097]), B=big_ints, Sq=big_ints, H=big_ints,
       Dd=st.sampled_from([128, 64, 1 << 40]), p=pointers)
def test_merge_validation_matches_the_rules(lib, n, B, Sq, H, Dd, p):
    if not p:
        want = INVALID
    elif n < 1 or n > 4096 or B < 1 or Sq < 1 or H < 1 or Dd < 1:
        want = INVALID
    elif Dd != D:
        want = UNSUPPORTED
    elif B * Sq * H >= BIG:
        want = UNSUPPORTED
    elif p % 16:
        want = INVALID
    else:
        want = NO_DEVICE
    ptr = ctypes.c_void_p(p or None)
    got = lib.lsh_lse_merge(ptr, ptr, n, B, Sq, H, Dd, ptr, ptr, None)
    assert got == want, (n, B, Sq, H, Dd, p)


@settings(max_examples=1500, deadline=None, derandomize=True)
@given(dtype=st.sampled_from([_lib.LSH_F32, _lib.LSH_BF16, 5]), B=big_ints, S=big_ints,
       H=big_ints, Dd=st.sampled_from([128, 64, 4, 12, (1 << 62) + 8]),
       h0=st.integers(-1, 40), hc=st.integers(0, 40), p=pointers)
def test_permute_validation_matches_the_rules(lib, dtype, B, S, H, Dd, h0, hc, p):
    eb = 4 if dtype == _lib.LSH_F32 else 2
    if not p:
        want = INVALID
    elif dtype not in (_lib.LSH_F32, _lib.LSH_BF16):
        want = INVALID
    elif B < 1 or S < 1 or H < 1 or Dd < 1:
        want = INVALID
    elif h0 < 0 or hc < 1 or h0 + hc > H:
        want = INVALID
    elif (Dd * eb) % 16:
        want = INVALID
    elif S * (Dd * eb // 16) >= BIG or B * hc > 65535:
        want = UNSUPPORTED
    elif p % 16:
        want = INVALID
    else:
        want = NO_DEVICE
    ptr = ctypes.c_void_p(p or None)
    got = lib.lsh_head_permute(ptr, ptr, dtype, B, S, H, Dd, h0, hc, None)
    assert got == want, (dtype, B, S, H, Dd, h0, hc, p)
