"""Comparison of GEMM outputs against the fp64 oracle.

TEST INFRASTRUCTURE ONLY (tests, smoke check and bench's CPU leg).

Criterion R1.  The target tolerance is a maximum relative error of 2e-3 for
GEMM outputs accumulated in fp32.  The outputs are bf16, whose unit roundoff
(2^-8) already exceeds 2e-3, and relative error is unbounded for outputs near
zero.  R1 therefore charges the unavoidable half-ulp of the final bf16 rounding
to the epilogue and applies 2e-3 to the rest, floored at sigma/16:

    |g - r| <= 0.5 * ulp_bf16(max(|g|, |r|)) + 2e-3 * max(|r|, sigma / 16)
               + U_MFMA * sum_k |x_k * y_k|

with g the result, r the fp64 oracle value and sigma the RMS of r over the
output.  The last term is the classical dot-product error bound (unit
roundoff times the sum of the absolute products).  The block-scaled MFMA of
the target GPU does not sum its products exactly in fp32: measured against
exact sums, a single instruction deviates by up to 2^-13.2 of its largest
product, and whole GEMMs by up to 2.1e-4 (K=384) and 3.3e-5 (K=5120) of
sum_k |x_k y_k|.  U_MFMA = 2^-11 keeps a margin of more than 2x over the
worst case seen.  Pass abs_terms=None to apply R1 without that term.
"""

from __future__ import annotations

import numpy as np

REL_TOL = 2e-3
U_MFMA = 2.0 ** -11


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32)
    with np.errstate(invalid="ignore"):
        return (b << np.uint32(16)).view(np.float32).astype(np.float64)


def ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |x| (8 significant bits; subnormal floor 2^-133)."""
    a = np.abs(np.asarray(x, dtype=np.float64))
    _, p = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(p - 1, -126)
    return np.exp2(e - 7.0)


def rne_bf16(r: np.ndarray) -> np.ndarray:
    """Round fp64 values to the nearest bf16 (ties to even), returned as fp64."""
    r = np.asarray(r, dtype=np.float64)
    a = np.abs(r)
    _, p = np.frexp(np.where(a > 0, a, 1.0))
    e = np.maximum(p - 1, -126)
    q = np.exp2(e - 7.0)
    return np.sign(r) * np.rint(a / q) * q


def r1_check(g_bits: np.ndarray, r: np.ndarray, sigma: float | None = None,
             abs_terms: np.ndarray | None = None, f32: bool = False) -> dict:
    """Return a report dict; ``ok`` is True iff every element satisfies R1.

    g_bits: bf16 bit patterns (or fp32 values with f32=True, no half-ulp term);
    abs_terms: sum_k |x_k y_k| per element (same shape as r), or None.
    """
    g = np.asarray(g_bits, dtype=np.float64) if f32 else bf16_bits_to_f64(g_bits)
    r = np.asarray(r, dtype=np.float64)
    assert g.shape == r.shape, (g.shape, r.shape)
    if sigma is None:
        sigma = float(np.sqrt(np.mean(r * r))) if r.size else 0.0
    err = np.abs(g - r)
    tol = REL_TOL * np.maximum(np.abs(r), sigma / 16.0)
    if not f32:
        tol = tol + 0.5 * ulp_bf16(np.maximum(np.abs(g), np.abs(r)))
    plain_bad = ~(err <= tol)
    if abs_terms is not None:
        tol = tol + U_MFMA * np.asarray(abs_terms, dtype=np.float64)
    bad = ~(err <= tol)
    nrm = float(np.linalg.norm(r))
    rep = {
        "ok": not bool(bad.any()),
        "n": int(r.size),
        "n_bad": int(bad.sum()),
        "max_err_over_tol": float(np.max(err / np.maximum(tol, 1e-300))) if r.size else 0.0,
        "normwise_rel": float(np.linalg.norm(g - r) / nrm) if nrm > 0 else float(np.linalg.norm(g)),
        "exact_rne_rate": float(np.mean(g == rne_bf16(r))) if r.size else 1.0,
        "plain_r1_violations": int(plain_bad.sum()),
        "max_err_over_abs_terms": float(np.max(err / np.maximum(abs_terms, 1e-300))) if abs_terms is not None and r.size else None,
        "sigma": sigma,
    }
    if bad.any():
        idx = np.argwhere(bad)[:5]
        rep["first_bad"] = [(tuple(int(v) for v in i), float(g[tuple(i)]), float(r[tuple(i)])) for i in idx]
    return rep
