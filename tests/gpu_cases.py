"""Run one case through the HIP library (via the binding) and through the
oracle, and compare them with the parity helpers."""
from __future__ import annotations

import sys
from typing import Dict, Optional

import numpy as np
import torch

import oracle
import parity
import row_wise_normalization_amd as mn


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray, offset: int = 0) -> torch.Tensor:
    """Upload ``a`` as a contiguous GPU tensor whose first element sits
    ``offset`` elements past a 256-byte aligned allocation."""
    t = torch.from_numpy(np.ascontiguousarray(a))
    if offset == 0:
        return t.to("cuda")
    buf = torch.empty(t.numel() + offset + 64, dtype=t.dtype, device="cuda")
    v = buf[offset:offset + t.numel()].view(t.shape)
    v.copy_(t)
    return v


def empty(shape, dtype, offset: int = 0) -> torch.Tensor:
    n = int(np.prod(shape))
    if offset == 0:
        return torch.empty(shape, dtype=dtype, device="cuda")
    buf = torch.empty(n + offset + 64, dtype=dtype, device="cuda")
    return buf[offset:offset + n].view(shape)


def host(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    return None if t is None else t.detach().cpu().numpy()


def run_gpu(kind: str, d: Dict[str, np.ndarray], eps: float, offset: int = 0,
            use_dh: bool = True) -> Dict[str, np.ndarray]:
    """Forward, then backward fed with the forward's own saved statistics."""
    N, D = d["X"].shape
    X = dev(d["X"], offset)
    g = dev(d["gamma"], offset)
    dY = dev(d["dY"], offset)
    out: Dict[str, np.ndarray] = {}
    Y = empty((N, D), torch.float16, offset)
    rstd = torch.empty(N, dtype=torch.float32, device="cuda")
    dX = empty((N, D), torch.float16, offset)
    dgamma = torch.empty(D, dtype=torch.float32, device="cuda")
    if kind == "rms":
        mn.mn_rmsnorm_forward(X, g, Y, rstd, eps)
        ws = mn.new_workspace(mn.MN_RMSNORM, N, D)
        mn.mn_rmsnorm_backward(X, g, rstd, dY, dX, dgamma, ws)
    elif kind == "ln":
        b = dev(d["beta"], offset)
        mean = torch.empty(N, dtype=torch.float32, device="cuda")
        dbeta = torch.empty(D, dtype=torch.float32, device="cuda")
        mn.mn_layernorm_forward(X, g, b, Y, mean, rstd, eps)
        ws = mn.new_workspace(mn.MN_LAYERNORM, N, D)
        mn.mn_layernorm_backward(X, g, mean, rstd, dY, dX, dgamma, dbeta, ws)
        out["mean"] = host(mean)
        out["dbeta"] = host(dbeta)
    elif kind == "add":
        R = dev(d["R"], offset)
        dH = dev(d["dH"], offset) if use_dh else None
        Hs = empty((N, D), torch.float16, offset)
        mn.mn_add_rmsnorm_forward(X, R, g, Hs, Y, rstd, eps)
        ws = mn.new_workspace(mn.MN_ADD_RMSNORM, N, D)
        mn.mn_add_rmsnorm_backward(X, R, g, rstd, dY, dH, dX, dgamma, ws)
        out["H"] = host(Hs)
    else:
        raise ValueError(kind)
    torch.cuda.synchronize()
    out.update(Y=host(Y), rstd=host(rstd), dX=host(dX), dgamma=host(dgamma))
    return out


def reference(kind: str, d: Dict[str, np.ndarray], eps: float, rows: Optional[np.ndarray] = None,
              use_dh: bool = True) -> Dict[str, np.ndarray]:
    """Oracle results: per-row outputs for ``rows`` (all rows when None) and
    parameter gradients over all rows."""
    sub = (lambda a: a) if rows is None else (lambda a: np.ascontiguousarray(a[rows]))
    X, dY = d["X"], d["dY"]
    o: Dict[str, np.ndarray] = {}
    if kind == "rms":
        o["Y"], o["rstd"] = oracle.rmsnorm_forward(sub(X), d["gamma"], eps)
        o["dX"], _ = oracle.rmsnorm_backward(sub(X), d["gamma"], sub(dY), eps)
        _, o["dgamma"] = oracle.rmsnorm_backward(X, d["gamma"], dY, eps, want_dx=False)
    elif kind == "ln":
        o["Y"], o["mean"], o["rstd"] = oracle.layernorm_forward(sub(X), d["gamma"], d["beta"], eps)
        o["dX"], _, _ = oracle.layernorm_backward(sub(X), d["gamma"], sub(dY), eps)
        _, o["dgamma"], o["dbeta"] = oracle.layernorm_backward(X, d["gamma"], dY, eps,
                                                               want_dx=False)
    elif kind == "add":
        R = d["R"]
        dH = d["dH"] if use_dh else None
        _, o["H16"], o["Y"], o["rstd"] = oracle.add_rmsnorm_forward(sub(X), sub(R), d["gamma"], eps)
        o["dX"], _ = oracle.add_rmsnorm_backward(sub(X), sub(R), d["gamma"], sub(dY),
                                                 None if dH is None else sub(dH), eps)
        _, o["dgamma"] = oracle.add_rmsnorm_backward(X, R, d["gamma"], dY, dH, eps, want_dx=False)
    return o


def _f64(a):
    return a.astype(np.float64)


def cancel_scales(kind: str, d: Dict[str, np.ndarray], ref: Dict[str, np.ndarray],
                  rows: Optional[np.ndarray], use_dh: bool = True):
    """Magnitude of the fp32 terms whose sum gives each dX element (and each
    LayerNorm y element), from the inputs and the oracle statistics."""
    sub = (lambda a: a) if rows is None else (lambda a: a[rows])
    x = _f64(sub(d["X"]))
    if kind == "add":
        x = x + _f64(sub(d["R"]))
    rs = ref["rstd"][:, None]
    mu = ref["mean"][:, None] if kind == "ln" else 0.0
    xh = (x - mu) * rs
    g = _f64(sub(d["dY"])) * _f64(d["gamma"])[None, :]
    A = np.abs(g * xh).mean(axis=1, keepdims=True)
    sdx = rs * (np.abs(g) + np.abs(xh) * A)
    if kind == "ln":
        sdx = sdx + rs * np.abs(g).mean(axis=1, keepdims=True)
    if kind == "add" and use_dh:
        sdx = sdx + np.abs(_f64(sub(d["dH"])))
    sy = None
    if kind == "ln":
        sy = np.abs(xh * _f64(d["gamma"])[None, :]) + np.abs(_f64(d["beta"]))[None, :]
    return sdx, sy


def compare(kind: str, gpu: Dict[str, np.ndarray], ref: Dict[str, np.ndarray], what: str,
            rows: Optional[np.ndarray] = None, mean_atol: float = 0.0,
            inputs: Optional[Dict[str, np.ndarray]] = None, use_dh: bool = True
            ) -> Dict[str, float]:
    """Check every element of the GPU outputs (restricted to ``rows``)
    against the oracle; returns the worst error per output. With ``inputs``
    the fp32 cancellation allowance of parity.check_f16 applies; without it
    every element must be within 2 ulp."""
    sel = (lambda a: a) if rows is None else (lambda a: a[rows])
    sdx = sy = None
    if inputs is not None:
        sdx, sy = cancel_scales(kind, inputs, ref, rows, use_dh)
    w: Dict[str, float] = {}
    w["Y_ulp"], w["Y_fp32_admitted"] = parity.check_f16(sel(gpu["Y"]), ref["Y"], f"{what} Y",
                                                        scale=sy)
    w["dX_ulp"], w["dX_fp32_admitted"] = parity.check_f16(sel(gpu["dX"]), ref["dX"],
                                                          f"{what} dX", scale=sdx)
    w["rstd_rel"] = parity.check_stat(sel(gpu["rstd"]), ref["rstd"], f"{what} rstd")
    w["dgamma"] = parity.check_grad(gpu["dgamma"], ref["dgamma"], f"{what} dgamma")
    if kind == "ln":
        w["mean_rel"] = parity.check_stat(sel(gpu["mean"]), ref["mean"], f"{what} mean",
                                          atol=mean_atol)
        w["dbeta"] = parity.check_grad(gpu["dbeta"], ref["dbeta"], f"{what} dbeta")
    if kind == "add":
        h = sel(gpu["H"]).view(np.uint16)
        r = ref["H16"].view(np.uint16)
        # +0 and -0 are the same sum; otherwise H must be the exact rounded sum
        same = (h == r) | (((h | r) & 0x7FFF) == 0)
        assert same.all(), f"{what} H: {int((~same).sum())} elements differ from fp16(x + r)"
    return w
