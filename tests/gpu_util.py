"""Helpers of the GPU parity tests: upload seeded inputs, NaN-poisoned
outputs, error measures. Tolerances of the HIP path against the fp64
oracle (max |difference| over all elements; any NaN or Inf fails):
  O: <= 1e-4 for float32 inputs, <= 2e-2 for bfloat16 inputs (N(0,1) data)
  LSE: <= 1e-3
For bfloat16 inputs the 2e-2 bar is the worst case of rounding every
attention weight to bfloat16, so it alone would miss, e.g., a dropped key
tile at long S. Checks that pass `sigma` (bf16_weight_sigma: the per-element
standard deviation of that rounding error, from the oracle) also fail when
an O error exceeds SIGMA_ALARM = 8 sigma (+1e-6); the largest seen over
every bf16 case is 3.5 sigma.
Gradients of the backward (bfloat16 inputs; dQ, dK, dV in float32), per
tensor: max |got - ref| <= 2e-2 * max |ref|. The inputs and dO are exact in
both; the GPU rounds P and dS to bfloat16 before the products dV = P^T dO,
dK = scale dS^T Q and dQ = scale dS K (relative error <= 2^-8 per term,
random in sign, so a sum is off by about 2^-8 / sqrt(3) of its typical
size), and takes Delta = rowsum(dO * O) from the forward's O, itself within
the bfloat16 bar above. Measured over the backward cases: median 2.0e-3,
largest 4.5e-3 of max |ref| (peaked scores).
"""
from __future__ import annotations

import sys

import numpy as np

TOL_O = {"f32": 1e-4, "bf16": 2e-2}
TOL_LSE = 1e-3
TOL_GRAD = 2e-2
U_BF16 = 2.0 ** -8   # unit roundoff of bfloat16 (round to nearest even)
SIGMA_ALARM = 8.0    # bf16 O errors beyond this many sigma of weight rounding fail


def dense_bf16_launch(B: int, Sq: int, H: int, n_cu: int = 256):
    """Which dense bf16 forward kernel a call of this shape launches, as
    ("256-row", blocks), ("256-row, split tail", blocks, halves per XCD) or
    ("128-row", blocks): the launcher's rule, restated so that tests can
    check that their shapes reach the path they are meant for.
    256-row items win unless their rounds over the CUs are more than 3/5 of
    the 128-row kernel's; then, when the items and CUs split evenly over the
    8 XCDs and each XCD's last round holds at most half its CUs' worth of
    items (with more than one round), those items run as 128-row halves."""
    big = B * H * -(-Sq // 256)
    small = B * H * -(-Sq // 128)
    if not 5 * -(-big // n_cu) <= 3 * -(-small // n_cu):
        return ("128-row", small)
    if n_cu % 8 == 0 and big % 8 == 0:
        per, cu_x = big // 8, n_cu // 8
        r = per % cu_x
        if 0 < r and 2 * r <= cu_x and per > cu_x:
            return ("256-row, split tail", big + 8 * r, r)
    return ("256-row", big)


def torch():
    import torch as t
    return t


def to_gpu(tensor, dtype: str):
    """lsh_inputs.Tensor -> GPU tensor with exactly the values the oracle sees."""
    t = torch()
    if dtype == "bf16":
        return t.from_numpy(np.ascontiguousarray(tensor.bits).view(np.int16)).view(t.bfloat16).cuda()
    return t.from_numpy(np.ascontiguousarray(tensor.values)).cuda()


def values_to_gpu(values: np.ndarray, dtype: str):
    """float array whose values are already representable in `dtype`."""
    t = torch()
    x = t.from_numpy(np.ascontiguousarray(values, dtype=np.float32))
    if dtype == "bf16":
        y = x.to(t.bfloat16)
        assert t.equal(y.float(), x), "values not exactly representable in bf16"
        return y.cuda()
    return x.cuda()


def poisoned_outputs(B, Sq, H, D=128):
    t = torch()
    o = t.full((B, Sq, H, D), float("nan"), dtype=t.float32, device="cuda")
    lse = t.full((B, H, Sq), float("nan"), dtype=t.float32, device="cuda")
    return o, lse


def max_err(got, want) -> float:
    """max |got - want| in float64; inf if any NaN, or if infinities disagree."""
    g = np.asarray(got, dtype=np.float64)
    w = np.asarray(want, dtype=np.float64)
    assert g.shape == w.shape, (g.shape, w.shape)
    if np.isnan(g).any() or np.isnan(w).any():
        return float("inf")
    same_inf = np.isinf(g) & np.isinf(w) & (np.sign(g) == np.sign(w))
    if (np.isinf(g) ^ np.isinf(w)).any():
        return float("inf")
    with np.errstate(invalid="ignore"):
        d = np.where(same_inf, 0.0, np.abs(g - w))
    return float(d.max()) if d.size else 0.0


def bf16_weight_sigma(oracle, q, k, v, scale, lse_ref, **kw):
    """Per-element standard deviation of the O error that rounding each
    attention weight to bfloat16 causes, from the oracle alone.

    With weights w_j = softmax_j(s) and relative rounding errors d_j of
    zero mean and variance <= U_BF16^2 / 3 (round to nearest even), the error
    sum_j w_j d_j v_j has variance <= U_BF16^2 / 3 * sum_j w_j^2 v_j^2, and
      sum_j w_j^2 v_j^2 = exp(LSE(2 s) - 2 LSE(s)) * sum_j softmax_j(2 s) v_j^2,
    i.e. one more oracle call with scale doubled and V squared. Rows with no
    key (LSE = -inf) get 0. kw is passed through (rows, heads, block_mask)."""
    v2 = np.square(np.asarray(v, dtype=np.float32))   # exact: bf16 values square into 16 bits
    o2, lse2 = oracle.attention_ref(q, k, v2, 2.0 * scale, **kw)
    with np.errstate(invalid="ignore", over="ignore"):
        ratio = np.where(np.isfinite(lse_ref), np.exp(lse2 - 2.0 * lse_ref), 0.0)
    ratio = np.nan_to_num(ratio)                              # [B, H, rows]
    var = np.transpose(ratio, (0, 2, 1))[..., None] * np.nan_to_num(o2)
    return U_BF16 / np.sqrt(3.0) * np.sqrt(np.maximum(var, 0.0))


def check(name, dtype, o_got, lse_got, o_ref, lse_ref, tol_o=None, tol_lse=TOL_LSE, sigma=None):
    eo = max_err(o_got, o_ref)
    el = max_err(lse_got, lse_ref)
    ratio, rmax = "", None
    if sigma is not None:
        with np.errstate(invalid="ignore"):
            r = np.abs(np.asarray(o_got, np.float64) - np.asarray(o_ref, np.float64)) / (sigma + 1e-6)
        rmax = float(np.nanmax(r)) if np.isfinite(eo) else float("inf")
        ratio = f" max|dO|/(sigma+1e-6)={rmax:.2f}"
    print(f"[parity] {name}: max|dO|={eo:.3e} max|dLSE|={el:.3e}{ratio}", file=sys.stderr, flush=True)
    tol_o = TOL_O[dtype] if tol_o is None else tol_o
    assert eo <= tol_o, f"{name}: O error {eo} > {tol_o}"
    assert el <= tol_lse, f"{name}: LSE error {el} > {tol_lse}"
    if rmax is not None:
        assert rmax <= SIGMA_ALARM, (f"{name}: O error {rmax:.2f} sigma of bf16 weight rounding "
                                     f"(alarm at {SIGMA_ALARM})")
    return eo, el


def announce(msg):
    print(f"[case] {msg}", file=sys.stderr, flush=True)


def check_grads(name, got, ref, tol=TOL_GRAD):
    """got, ref: (dQ, dK, dV) arrays of equal shapes. Each gradient's max
    abs error must be <= tol * its max |ref|. Returns the relative errors."""
    errs = []
    for label, g, r in zip(("dQ", "dK", "dV"), got, ref):
        r = np.asarray(r, dtype=np.float64)
        top = float(np.abs(r).max()) if r.size else 0.0
        e = max_err(g, r)
        rel = e / top if top > 0 else e
        errs.append(rel)
        print(f"[parity] {name} {label}: max|err|={e:.3e} max|ref|={top:.3e} rel={rel:.3e}",
              file=sys.stderr, flush=True)
        assert rel <= tol, f"{name}: {label} error {e} > {tol} * {top}"
    return errs
