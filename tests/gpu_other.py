"""Run a Dynamic Tanh, PolyNorm or Modulated RMSNorm case through the HIP
library and through the oracle, and compare them element by element.

Outputs in 16-bit storage are held to 2 ulp of their type; an element that
misses it is admitted only when its exact value is a cancellation of much
larger fp32 terms and it is within 64 * 2^-24 * scale of the oracle (the
allowance of parity.check_out). float32 outputs are held to that bound on
every element. Parameter gradients use parity.check_grad (the scalar ones
scaled by the number of summed terms, see ``grad_scalar``); saved statistics
parity.check_stat.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

import every_row
import oracle
import parity
import workloads
import row_wise_normalization_amd as mn
from gpu_cases import dev, empty, host

# The scalar parameters as the GPU receives them (float32); the oracle is fed
# the same float32 values.
ALPHA = float(np.float32(workloads.DYT_ALPHA[0]))
POLY = np.array(workloads.POLY_PARAMS, dtype=np.float32).astype(np.float64)


def _f64(a):
    return parity.as_f64(a)


def run(kind: str, d: Dict[str, np.ndarray], eps: float, offset: int = 0,
        dx_dtype: Optional[torch.dtype] = None, alpha: float = ALPHA,
        params=POLY) -> Dict[str, np.ndarray]:
    """Forward, then backward fed with the forward's own saved statistics."""
    N, D = d["X"].shape
    X = dev(d["X"], offset)
    dY = dev(d["dY"], offset)
    act = X.dtype
    dxt = act if dx_dtype is None else dx_dtype
    Y = empty((N, D), act, offset)
    dX = empty((N, D), dxt, offset)
    out: Dict[str, np.ndarray] = {}
    if kind == "dyt":
        g = dev(d["gamma"], offset)
        b = dev(d["beta"], offset)
        a = torch.tensor([alpha], dtype=torch.float32, device="cuda")
        mn.mn_dyt_forward_ex(X, a, g, b, Y)
        da = torch.empty(1, dtype=torch.float32, device="cuda")
        dg = torch.empty(D, dtype=torch.float32, device="cuda")
        db = torch.empty(D, dtype=torch.float32, device="cuda")
        ws = mn.new_workspace(mn.MN_DYT, N, D)
        mn.mn_dyt_backward_ex(X, a, g, dY, dX, da, dg, db, ws)
        out.update(dalpha=host(da), dgamma=host(dg), dbeta=host(db))
    elif kind == "poly":
        p = torch.tensor(np.asarray(params, dtype=np.float32), device="cuda")
        rstd = torch.empty(N, 3, dtype=torch.float32, device="cuda")
        mn.mn_polynorm_forward_ex(X, p, Y, rstd, eps)
        dp = torch.empty(4, dtype=torch.float32, device="cuda")
        ws = mn.new_workspace(mn.MN_POLYNORM, N, D)
        mn.mn_polynorm_backward_ex(X, p, rstd, dY, dX, dp, ws)
        out.update(rstd=host(rstd), dparams=host(dp))
    elif kind == "mod":
        g = dev(d["gamma"], offset)
        sc = dev(d["scale"], offset)
        sh = dev(d["shift"], offset)
        B = sc.shape[0]
        rstd = torch.empty(N, dtype=torch.float32, device="cuda")
        mn.mn_mod_rmsnorm_forward_ex(X, g, sc, sh, Y, rstd, eps)
        dg = torch.empty(D, dtype=torch.float32, device="cuda")
        dsc = torch.empty(B, D, dtype=torch.float32, device="cuda")
        dsh = torch.empty(B, D, dtype=torch.float32, device="cuda")
        ws = mn.new_workspace(mn.MN_MOD_RMSNORM, N, D, B=B)
        mn.mn_mod_rmsnorm_backward_ex(X, g, sc, rstd, dY, dX, dg, dsc, dsh, ws)
        out.update(rstd=host(rstd), dgamma=host(dg), dscale=host(dsc), dshift=host(dsh))
    else:
        raise ValueError(kind)
    torch.cuda.synchronize()
    out.update(Y=host(Y), dX=host(dX))
    return out


def reference(kind: str, d: Dict[str, np.ndarray], eps: float, rows=None, alpha: float = ALPHA,
              params=POLY, per_row: bool = True, grads: bool = True) -> Dict[str, np.ndarray]:
    """Oracle results: per-row outputs for ``rows`` (all when None; an index
    array, or a slice that for "mod" lies inside one sample) and parameter
    gradients over all rows. Either half can be left out."""
    sub = (lambda a: a) if rows is None else (lambda a: np.ascontiguousarray(a[rows]))
    X, dY = d["X"], d["dY"]
    o: Dict[str, np.ndarray] = {}
    if kind == "dyt":
        if per_row:
            o["Y"] = oracle.dyt_forward(sub(X), alpha, d["gamma"], d["beta"])
            o["dX"] = oracle.dyt_backward(sub(X), alpha, d["gamma"], sub(dY))[0]
        if grads:
            _, da, o["dgamma"], o["dbeta"] = oracle.dyt_backward(X, alpha, d["gamma"], dY,
                                                                 want_dx=False)
            o["dalpha"] = np.array([da])
    elif kind == "poly":
        w, b = np.asarray(params[:3], np.float64), float(params[3])
        if per_row:
            o["Y"], o["rstd"] = oracle.polynorm_forward(sub(X), w, b, eps)
            o["dX"] = oracle.polynorm_backward(sub(X), w, sub(dY), eps)[0]
        if grads:
            _, dw, db = oracle.polynorm_backward(X, w, dY, eps, want_dx=False)
            o["dparams"] = np.concatenate([dw, [db]])
    elif kind == "mod":
        S = X.shape[0] // d["scale"].shape[0]
        if per_row and rows is None:
            o["Y"], o["rstd"] = oracle.modrms_forward(X, d["gamma"], d["scale"], d["shift"], eps)
            o["dX"] = oracle.modrms_backward(X, d["gamma"], d["scale"], dY, eps)[0]
        elif per_row and isinstance(rows, slice):
            # a block of rows of one sample: that sample's scale and shift
            b = rows.start // S
            assert (rows.stop - 1) // S == b, "a row block must lie inside one sample"
            sci, shi = d["scale"][b:b + 1], d["shift"][b:b + 1]
            o["Y"], o["rstd"] = oracle.modrms_forward(sub(X), d["gamma"], sci, shi, eps)
            o["dX"] = oracle.modrms_backward(sub(X), d["gamma"], sci, sub(dY), eps)[0]
        elif per_row:
            # per-row outputs of sampled rows: one row at a time with its sample's
            # scale and shift
            Ys, rs, dXs = [], [], []
            for i in rows:
                b = i // S
                xi, dyi = X[i:i + 1], dY[i:i + 1]
                sci, shi = d["scale"][b:b + 1], d["shift"][b:b + 1]
                y, r = oracle.modrms_forward(xi, d["gamma"], sci, shi, eps)
                Ys.append(y[0]); rs.append(r[0])
                dXs.append(oracle.modrms_backward(xi, d["gamma"], sci, dyi, eps)[0][0])
            o["Y"], o["rstd"], o["dX"] = np.array(Ys), np.array(rs), np.array(dXs)
        if grads:
            _, o["dgamma"], o["dscale"], o["dshift"] = oracle.modrms_backward(
                X, d["gamma"], d["scale"], dY, eps, want_dx=False)
    return o


def scales(kind: str, d, ref, rows=None, alpha: float = ALPHA, params=POLY):
    """Magnitude of the fp32 terms behind each Y and dX element."""
    sub = (lambda a: a) if rows is None else (lambda a: a[rows])
    x = _f64(sub(d["X"]))
    dy = _f64(sub(d["dY"]))
    if kind == "dyt":
        g = _f64(d["gamma"])[None, :]
        b = _f64(d["beta"])[None, :]
        t = np.tanh(alpha * x)
        return np.abs(g * t) + np.abs(b), np.abs(dy * g * alpha)
    if kind == "poly":
        rs = ref["rstd"]
        w = np.asarray(params, np.float64)
        n = [x ** p * rs[:, p - 1:p] for p in (1, 2, 3)]
        sy = sum(np.abs(w[p] * n[p]) for p in range(3)) + abs(w[3])
        sdx = 0.0
        for p in range(3):
            c = np.abs(dy * n[p]).mean(axis=1, keepdims=True)
            sdx = sdx + np.abs((p + 1) * x ** p * w[p] * rs[:, p:p + 1]) * (np.abs(dy) +
                                                                          np.abs(n[p]) * c)
        return sy, sdx
    # mod
    S = d["X"].shape[0] // d["scale"].shape[0]
    if rows is None:
        idx = np.arange(d["X"].shape[0])
    elif isinstance(rows, slice):
        idx = np.arange(rows.start, rows.stop)
    else:
        idx = np.asarray(rows)
    smp = idx // S
    sc = _f64(d["scale"])[smp]
    sh = _f64(d["shift"])[smp]
    g = _f64(d["gamma"])[None, :]
    rs = ref["rstd"][:, None]
    xh = x * rs
    m = g * (1 + sc)
    gg = dy * m
    A = np.abs(gg * xh).mean(axis=1, keepdims=True)
    return np.abs(xh * g) * (1 + np.abs(sc)) + np.abs(sh), rs * (np.abs(gg) + np.abs(xh) * A)


def grad_scalar(gpu, ref, what, terms: int, mag: float):
    """A scalar sum of `terms` fp32 products of size ~mag: the fp32
    accumulation error grows like sqrt(terms) * 2^-24 * mag per level; the
    bound is the dgamma bound plus 2^-16 * mag * sqrt(terms)."""
    atol = 1e-3 + 2.0 ** -16 * mag * np.sqrt(terms)
    return parity.check_grad(gpu, ref, what, atol=atol)


def compare(kind: str, gpu, ref, d, what: str, rows=None, strict: bool = False,
            alpha: float = ALPHA, params=POLY, per_row: bool = True,
            grads: bool = True) -> Dict[str, float]:
    sel = (lambda a: a) if rows is None else (lambda a: a[rows])
    w: Dict[str, float] = {}
    n = d["X"].size
    if grads:
        if kind == "dyt":
            w["dgamma"] = parity.check_grad(gpu["dgamma"], ref["dgamma"], f"{what} dgamma")
            w["dbeta"] = parity.check_grad(gpu["dbeta"], ref["dbeta"], f"{what} dbeta")
            mag = float(np.abs(_f64(d["dY"]) * _f64(d["X"])).mean() *
                        np.abs(_f64(d["gamma"])).max())
            w["dalpha"] = grad_scalar(gpu["dalpha"], ref["dalpha"], f"{what} dalpha", n, mag)
        elif kind == "poly":
            mag = float(np.abs(_f64(d["dY"])).mean())
            w["dparams"] = grad_scalar(gpu["dparams"], ref["dparams"], f"{what} dparams", n,
                                       mag)
        else:
            w["dgamma"] = parity.check_grad(gpu["dgamma"], ref["dgamma"], f"{what} dgamma")
            w["dscale"] = parity.check_grad(gpu["dscale"], ref["dscale"], f"{what} dscale")
            w["dshift"] = parity.check_grad(gpu["dshift"], ref["dshift"], f"{what} dshift")
    if not per_row:
        return w
    sy, sdx = scales(kind, d, ref, rows, alpha, params)
    if strict and gpu["Y"].dtype != np.float32:
        sy = sdx = None
    w["Y"], w["Y_admitted"] = parity.check_out(sel(gpu["Y"]), ref["Y"], f"{what} Y", scale=sy)
    w["dX"], w["dX_admitted"] = parity.check_out(sel(gpu["dX"]), ref["dX"], f"{what} dX",
                                                 scale=sdx)
    if kind != "dyt":
        w["rstd"] = parity.check_stat(sel(gpu["rstd"]), ref["rstd"], f"{what} rstd")
    return w


def compare_every_row(kind: str, gpu, d, eps: float, what: str, strict: bool = False,
                      alpha: float = ALPHA, params=POLY) -> Dict[str, float]:
    """compare() over every row of a full-size call, the oracle on blocks of
    rows (for "mod" blocks never straddle two samples); parameter gradients
    once over all rows."""
    N, D = d["X"].shape
    w = compare(kind, gpu, reference(kind, d, eps, alpha=alpha, params=params, per_row=False),
                d, what, per_row=False, alpha=alpha, params=params)
    align = 1
    if kind == "mod":
        S = N // d["scale"].shape[0]
        # blocks of whole samples, or of a divisor of the sample's rows
        rows = max(1, every_row.BLOCK_ELEMS // D)
        align = S if rows >= S else max(r for r in range(1, rows + 1) if S % r == 0)

    def block(rows):
        ref = reference(kind, d, eps, rows=rows, alpha=alpha, params=params, grads=False)
        return compare(kind, gpu, ref, d, what, rows=rows, strict=strict, alpha=alpha,
                       params=params, grads=False)

    w.update(every_row.run_blocks(N, D, block, align=align))
    return w
