"""Comparison helpers for HIP-versus-oracle parity.

Tolerances (stated for the path: fp16 storage, fp32 arithmetic):
  * fp16 outputs (Y, H, dX): |gpu - ref16| <= 2 ulp16(ref16), where ref16 is
    the oracle's float64 value rounded once to fp16 (nearest, ties to even)
    and ulp16(v) = 2^(max(floor(log2|v|), -14) - 10) (2^-24 at zero); +0 and
    -0 are equal, NaN matches NaN, an infinity matches the same infinity.
    The named workloads are held to this bound on every checked element.
    Other cases may admit an element whose exact value is a cancellation of
    much larger fp32 terms (dX = rstd*(g - xhat*c1 [- c2]) [+ dH], LayerNorm
    y = xhat*gamma + beta) when |gpu - ref| <= 64 * 2^-24 * scale, scale being
    the magnitude of those terms; no fp32 evaluation of the formula can do
    better there, while a wrong term or index misses by O(scale).
  * fp32 statistics (mean, rstd): |gpu - ref| <= 1e-5 |ref| (+ an absolute
    term for means of rows centred at zero, stated where used).
  * fp32 parameter gradients (dgamma, dbeta): |gpu - ref| <= 1e-3 + 5e-4 |ref|.
"""
from __future__ import annotations

import numpy as np

import oracle


def ulp16(ref16: np.ndarray) -> np.ndarray:
    a = np.abs(ref16.astype(np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, -14.0)
    u = np.exp2(e - 10.0)
    return np.where(a > 0, u, 2.0 ** -24)


# fp32 evaluation allowance for elements whose value is a cancellation of
# larger fp32 terms: |gpu - ref| <= FP32_K * 2^-24 * scale, where `scale` is
# the magnitude of the terms the kernel adds in fp32 (tests/gpu_cases.py, cancel_scales).
FP32_K = 64.0


def check_f16(gpu16: np.ndarray, ref64: np.ndarray, what: str, max_ulp: float = 2.0,
              scale: np.ndarray = None):
    """Element-wise fp16 check. Returns (worst error in ulp over the elements
    that meet the ulp bound, number of elements admitted only by the fp32
    cancellation allowance). Without ``scale`` every element must meet the
    ulp bound."""
    assert gpu16.shape == ref64.shape, f"{what}: shape {gpu16.shape} vs {ref64.shape}"
    ref16 = oracle.f64_to_f16(ref64)
    g = gpu16.astype(np.float64)
    r = ref16.astype(np.float64)
    nan_g, nan_r = np.isnan(g), np.isnan(r)
    assert (nan_g == nan_r).all(), f"{what}: NaN pattern differs ({int((nan_g != nan_r).sum())})"
    fin = ~nan_r
    inf_r = np.isinf(r) & fin
    assert (g[inf_r] == r[inf_r]).all(), f"{what}: infinities differ"
    ok = fin & ~inf_r
    err = np.abs(g[ok] - r[ok]) / ulp16(ref16[ok])
    over = err > max_ulp
    admitted = 0
    if over.any() and scale is not None:
        gi, ri, si = g[ok][over], ref64[ok][over], scale[ok][over]
        fine = np.abs(gi - ri) <= FP32_K * 2.0 ** -24 * si
        admitted = int(fine.sum())
        over_idx = np.flatnonzero(over)
        over[over_idx[fine]] = False
    if over.any():
        e = np.where(over, err, -1.0)
        idx = np.argwhere(ok)[np.argmax(e)]
        raise AssertionError(
            f"{what}: {int(over.sum())} of {err.size} elements beyond {max_ulp} ulp"
            f"{'' if scale is None else ' and beyond the fp32 cancellation allowance'}; "
            f"worst {float(e.max()):.2f} ulp at {tuple(idx)}: gpu {g[tuple(idx)]!r} "
            f"ref {ref64[tuple(idx)]!r}")
    worst = float(err[err <= max_ulp].max()) if (err <= max_ulp).any() else 0.0
    return worst, admitted


def check_stat(gpu32: np.ndarray, ref64: np.ndarray, what: str, rtol: float = 1e-5,
               atol=0.0):
    g = gpu32.astype(np.float64)
    err = np.abs(g - ref64)
    lim = rtol * np.abs(ref64) + atol
    bad = ~(err <= lim)
    if bad.any():
        i = int(np.argmax(np.where(bad, err, -1)))
        raise AssertionError(f"{what}: {int(bad.sum())} of {g.size} beyond tolerance; worst at {i}: "
                             f"gpu {g.flat[i]!r} ref {ref64.flat[i]!r}")
    return float(np.max(err / np.maximum(np.abs(ref64), 1e-300))) if g.size else 0.0


def check_grad(gpu32: np.ndarray, ref64: np.ndarray, what: str, atol: float = 1e-3,
               rtol: float = 5e-4):
    g = gpu32.astype(np.float64)
    err = np.abs(g - ref64)
    lim = atol + rtol * np.abs(ref64)
    bad = ~(err <= lim)
    if bad.any():
        i = int(np.argmax(np.where(bad, err, -1)))
        raise AssertionError(f"{what}: {int(bad.sum())} of {g.size} beyond tolerance; worst at {i}: "
                             f"gpu {g.flat[i]!r} ref {ref64.flat[i]!r}")
    return float((err / lim).max()) if g.size else 0.0
