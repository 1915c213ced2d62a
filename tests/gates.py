"""Acceptance gates used by the GPU parity tests (test infrastructure).

* fp32 workloads: normwise relative error max|g - r| / max|r| <= 1e-5.
* bf16-KV workloads (fp32 accumulate): max absolute error <= 1e-2, and the
  stronger internal gate normwise relative error <= 1e-3 (both sides read
  the same bf16 cache values and accumulate in at least fp32, so the
  expected error is ~1e-5; the absolute gate alone would accept an all-zero
  output at these value scales).
* INT8-KV workloads: the bf16 gates.  Both sides read the same codes and
  scales, so the only difference is arithmetic (products of exact codes
  with q to ~2^-22 and p to ~2^-21, fp32 accumulation); quantisation error
  is not part of the comparison.
* Causal prefill (gqa_prefill_attn, dtype "prefill"): q * scale and the
  probabilities enter the matrix cores rounded once to bf16, as in
  FlashAttention-2 in bf16.  Rounding each weight to bf16 perturbs it by up
  to 2^-9 relative (1.1e-3 rms); the output is normalised by the sum of the
  unrounded weights, so its error is that perturbation averaged over V:
  about 1e-3 relative per element.  lse comes from the same sum, so only
  the rounding of q moves it.  An fp64 emulation of exactly these roundings
  (rows of 2 to 2000 tokens, q gain 1 to 32) gave normwise output errors of
  1.5e-3 to 3.0e-3 and lse errors up to 1.5e-3 * max(1, |lse|) (2 tokens at
  q gain 32; 3e-4 otherwise); normalising by the sum of the rounded weights
  instead gives the same errors to within the spread of the trials.  Gates: max abs
  <= 1e-2 (the bf16 gate), normwise <= 1e-2, lse <= 5e-3 * max(1, |r|).
* lse (natural log): |g - r| <= tol_lse * max(1, |r|).
* Cache append and block-table indexing: bit-exact.
"""
import numpy as np

FP32_NORM_TOL = 1e-5
BF16_ABS_TOL = 1e-2
BF16_NORM_TOL = 1e-3
LSE_TOL = {"f32": 1e-5, "bf16": 1e-4, "i8": 1e-4, "prefill": 5e-3}
PREFILL_NORM_TOL = 1e-2


def normwise_rel_err(got, ref) -> float:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.abs(ref).max()
    if den == 0:
        return float(np.abs(got).max())
    return float(np.abs(got - ref).max() / den)


def out_errors(got, ref):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    return {"max_abs": float(np.abs(got - ref).max()) if got.size else 0.0,
            "normwise": normwise_rel_err(got, ref) if got.size else 0.0,
            "finite": bool(np.isfinite(got).all())}


def out_ok(got, ref, dtype) -> bool:
    e = out_errors(got, ref)
    if not e["finite"]:
        return False
    if dtype == "f32":
        return e["normwise"] <= FP32_NORM_TOL
    if dtype == "prefill":
        return e["max_abs"] <= BF16_ABS_TOL and e["normwise"] <= PREFILL_NORM_TOL
    return e["max_abs"] <= BF16_ABS_TOL and e["normwise"] <= BF16_NORM_TOL


def lse_ok(got, ref, dtype) -> bool:
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    both_inf = np.isneginf(got) & np.isneginf(ref)
    diff = np.where(both_inf, 0.0, np.abs(got - ref))
    return bool((diff <= LSE_TOL[dtype] * np.maximum(1.0, np.abs(ref))).all())


def assert_out(got, ref, dtype, what=""):
    e = out_errors(got, ref)
    assert out_ok(got, ref, dtype), f"{what}: {e}"
    return e


def assert_lse(got, ref, dtype, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert lse_ok(got, ref, dtype), f"{what}: max |dlse| = {np.nanmax(np.abs(got - ref))}"
