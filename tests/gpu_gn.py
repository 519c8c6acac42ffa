"""Run a GroupNorm case through the HIP library and through the oracle, and
compare them element by element.

A GroupNorm slice (one sample, one group of C / G channels) is a LayerNorm
row of (C / G) * L values whose gamma and beta vary by channel, so the bar
is the LayerNorm one: Y and dX within 2 ulp of their storage type (binary32:
64 * 2^-24 of the size of the fp32 terms on every element), an element that
misses 2 ulp admitted only when its exact value is a cancellation of much
larger fp32 terms and it is within 64 * 2^-24 of their size; mean and rstd
to 1e-5 relative; dgamma and dbeta to 1e-3 + 5e-4 |ref|.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch

import oracle
import parity
import workloads
import row_wise_normalization_amd as mn
from gpu_cases import dev, empty, host


def case(N: int, C: int, L: int, G: int, seed: int, act: str = "f16",
         param: Optional[str] = None, x_loc: float = 0.5) -> Dict[str, np.ndarray]:
    d = workloads.random_case("gn", N, C * L, seed, x_loc=x_loc, act=act, param=param,
                              channels=C, groups=G)
    d["X"] = d["X"].reshape(N, C, L)
    d["dY"] = d["dY"].reshape(N, C, L)
    return d


def run(d, G: int, eps: float, offset: int = 0, dx_dtype: Optional[torch.dtype] = None):
    """Forward, then backward fed with the forward's own statistics."""
    N, C, L = d["X"].shape
    X = dev(d["X"], offset)
    dY = dev(d["dY"], offset)
    g = dev(d["gamma"], offset)
    b = dev(d["beta"], offset)
    Y = empty((N, C, L), X.dtype, offset)
    dX = empty((N, C, L), X.dtype if dx_dtype is None else dx_dtype, offset)
    mean = torch.empty(N, G, dtype=torch.float32, device="cuda")
    rstd = torch.empty(N, G, dtype=torch.float32, device="cuda")
    mn.mn_groupnorm_forward_ex(X, g, b, Y, mean, rstd, G, eps)
    dg = torch.empty(C, dtype=torch.float32, device="cuda")
    db = torch.empty(C, dtype=torch.float32, device="cuda")
    ws = torch.empty(max(16, mn.groupnorm_workspace_bytes(N, C, L, G)) // 4, dtype=torch.float32,
                     device="cuda")
    mn.mn_groupnorm_backward_ex(X, g, mean, rstd, dY, dX, dg, db, G, ws)
    torch.cuda.synchronize()
    return {"Y": host(Y), "dX": host(dX), "mean": host(mean), "rstd": host(rstd),
            "dgamma": host(dg), "dbeta": host(db)}


def reference(d, G: int, eps: float):
    Y, mean, rstd = oracle.groupnorm_forward(d["X"], d["gamma"], d["beta"], G, eps)
    dX, dg, db = oracle.groupnorm_backward(d["X"], d["gamma"], d["dY"], G, eps)
    return {"Y": Y, "dX": dX, "mean": mean, "rstd": rstd, "dgamma": dg, "dbeta": db}


def _per_element(v: np.ndarray, N: int, L: int) -> np.ndarray:
    """[C] per-channel values as [N, C, L]."""
    return np.broadcast_to(parity.as_f64(v)[None, :, None], (N, v.shape[0], L))


def scales(d, ref, G: int):
    """Size of the fp32 terms behind each Y and dX element (the LayerNorm
    terms of the slice, gamma and beta per channel)."""
    N, C, L = d["X"].shape
    x = parity.as_f64(d["X"]).reshape(N, G, -1)
    rs = ref["rstd"][:, :, None]
    mu = ref["mean"][:, :, None]
    xs = (np.abs(x) + np.abs(mu)) * rs
    ge = _per_element(d["gamma"], N, L).reshape(N, G, -1)
    be = _per_element(d["beta"], N, L).reshape(N, G, -1)
    g = parity.as_f64(d["dY"]).reshape(N, G, -1) * ge
    A = (np.abs(g) * xs).mean(axis=2, keepdims=True)
    sdx = rs * (np.abs(g) + xs * A) + rs * np.abs(g).mean(axis=2, keepdims=True)
    sy = xs * np.abs(ge) + np.abs(be)
    return sy.reshape(N, C, L), sdx.reshape(N, C, L)


def compare(gpu, ref, d, G: int, what: str) -> Dict[str, float]:
    sy, sdx = scales(d, ref, G)
    w: Dict[str, float] = {}
    w["Y"], w["Y_admitted"] = parity.check_out(gpu["Y"], ref["Y"], f"{what} Y", scale=sy)
    w["dX"], w["dX_admitted"] = parity.check_out(gpu["dX"], ref["dX"], f"{what} dX", scale=sdx)
    N = d["X"].shape[0]
    xa = np.abs(parity.as_f64(d["X"])).reshape(N, G, -1).mean(axis=2)
    w["mean"] = parity.check_stat(gpu["mean"], ref["mean"], f"{what} mean",
                                  atol=parity.FP32_K * 2.0 ** -24 * xa)
    w["rstd"] = parity.check_stat(gpu["rstd"], ref["rstd"], f"{what} rstd")
    w["dgamma"] = parity.check_grad(gpu["dgamma"], ref["dgamma"], f"{what} dgamma")
    w["dbeta"] = parity.check_grad(gpu["dbeta"], ref["dbeta"], f"{what} dbeta")
    return w
