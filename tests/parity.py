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
    the magnitude of those terms (for LayerNorm xhat counts as
    rstd*(|x| + |mean|), since it is formed from x and the rounded mean); no
    fp32 evaluation of the formula can do better there, while a wrong term
    or index misses by O(scale).
  * bfloat16 outputs: the same rule with ulp_bf16(v) = 2^(max(floor(log2|v|),
    -126) - 7) (2^-133 at zero).
  * float32 outputs: |gpu - ref| <= 64 * 2^-24 * scale on every element, scale
    being the magnitude of the fp32 terms (|ref| itself where the value is a
    plain product, such as RMSNorm y); a float32 H must equal fl32(x + r).
  * fp32 statistics (mean, rstd): |gpu - ref| <= 1e-5 |ref|; outside the named
    workloads a mean may also take 64 * 2^-24 * mean(|x|) of absolute error
    (a row centred near zero makes its mean a cancellation).
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


def allowance_bound(D: int, storage: str) -> float:
    """Largest fraction of a case's 16-bit output elements (Y and dX) that
    the fp32 cancellation allowance may admit.

    * D <= 2: the row sums are no longer means of many independent terms.
      RMSNorm at D = 1 gives dX = rstd * g * eps / (x^2 + eps), a cancellation
      of two terms of size |g| / |x| in 1 - xhat^2; LayerNorm at D = 2 has
      xhat = +-1 / sqrt(1 + eps / var) likewise. A few per cent of the
      elements need the allowance (measured: up to 4.5 %); bound 10 %.
    * fp16 from 16 columns on: none. c1 and c2 are then means of many
      independent products, so a dX near zero needs a small g = dY * gamma
      and every fp32 term is as small as the result. Below 16 columns an
      occasional element (measured: 1 of 16,368 at LayerNorm D = 8); bound
      1e-3.
    * bfloat16 keeps its relative precision down to 2^-126, so deep
      cancellations (dX near zero, LayerNorm y where gamma * xhat ~ -beta)
      stay visible at any width (measured: at most 2e-6 of the elements from
      16 columns on); bound 1e-5, and 1e-3 below 16 columns.
    """
    if D <= 2:
        return 0.1
    if storage == "f16":
        return 0.0 if D >= 16 else 1e-3
    return 1e-5 if D >= 16 else 1e-3


# storage name -> (mantissa bits, minimum normal exponent)
_FORMAT = {"f16": (10, -14), "bf16": (7, -126)}


def storage_of(a: np.ndarray) -> str:
    return {np.dtype(np.float16): "f16", np.dtype(np.uint16): "bf16",
            np.dtype(np.float32): "f32"}[a.dtype]


def ulp_of(ref_rounded: np.ndarray, storage: str) -> np.ndarray:
    m, emin = _FORMAT[storage]
    a = np.abs(ref_rounded.astype(np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(e, float(emin))
    return np.where(a > 0, np.exp2(e - m), 2.0 ** (emin - m))


def as_f64(a: np.ndarray) -> np.ndarray:
    """Values of a storage array (bfloat16 given as uint16 bits)."""
    return oracle.bf16_to_f64(a) if a.dtype == np.uint16 else a.astype(np.float64)


def check_out(gpu: np.ndarray, ref64: np.ndarray, what: str, max_ulp: float = 2.0,
              scale: np.ndarray = None):
    """Element-wise check of a stored output against the float64 oracle, in
    the output's own storage type (see the module docstring). Returns (worst
    error, number of elements admitted only by the fp32 allowance); the worst
    error is in ulps for 16-bit types and in units of 2^-24 * scale for
    float32."""
    st = storage_of(gpu)
    if st == "f16":
        return check_f16(gpu, ref64, what, max_ulp, scale)
    assert gpu.shape == ref64.shape, f"{what}: shape {gpu.shape} vs {ref64.shape}"
    g = as_f64(gpu)
    nan_g, nan_r = np.isnan(g), np.isnan(ref64)
    assert (nan_g == nan_r).all(), f"{what}: NaN pattern differs ({int((nan_g != nan_r).sum())})"
    ok = ~nan_r
    ref_r = ref64 if st == "f32" else as_f64(oracle.round_to(ref64, np.uint16))
    inf_r = np.isinf(ref_r) & ok
    assert (g[inf_r] == ref_r[inf_r]).all(), f"{what}: infinities differ"
    ok &= ~inf_r
    if st == "f32":
        sc = np.abs(ref64) if scale is None else np.maximum(scale, np.abs(ref64))
        err = np.abs(g[ok] - ref64[ok]) / (2.0 ** -24 * np.maximum(sc[ok], 1e-300))
        bad = err > FP32_K
        if bad.any():
            i = np.argwhere(ok)[np.argmax(np.where(bad, err, -1.0))]
            raise AssertionError(
                f"{what}: {int(bad.sum())} of {err.size} elements beyond {FP32_K} * 2^-24 * scale; "
                f"worst {float(err.max()):.1f} at {tuple(i)}: gpu {g[tuple(i)]!r} "
                f"ref {ref64[tuple(i)]!r}")
        return (float(err.max()) if err.size else 0.0), 0
    err = np.abs(g[ok] - ref_r[ok]) / ulp_of(ref_r[ok], st)
    over = err > max_ulp
    admitted = 0
    if over.any() and scale is not None:
        fine = np.abs(g[ok][over] - ref64[ok][over]) <= FP32_K * 2.0 ** -24 * scale[ok][over]
        admitted = int(fine.sum())
        idx = np.flatnonzero(over)
        over[idx[fine]] = False
    if over.any():
        e = np.where(over, err, -1.0)
        i = np.argwhere(ok)[np.argmax(e)]
        raise AssertionError(
            f"{what}: {int(over.sum())} of {err.size} elements beyond {max_ulp} ulp; worst "
            f"{float(e.max()):.2f} ulp at {tuple(i)}: gpu {g[tuple(i)]!r} ref {ref64[tuple(i)]!r}")
    within = err[err <= max_ulp]
    return (float(within.max()) if within.size else 0.0), admitted


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
