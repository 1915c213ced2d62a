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
* lse (natural log): |g - r| <= tol_lse * max(1, |r|).
* Cache append and block-table indexing: bit-exact.
"""
import numpy as np

FP32_NORM_TOL = 1e-5
BF16_ABS_TOL = 1e-2
BF16_NORM_TOL = 1e-3
LSE_TOL = {"f32": 1e-5, "bf16": 1e-4, "i8": 1e-4}


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
