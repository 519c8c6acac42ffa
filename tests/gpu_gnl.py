"""Channels-last GroupNorm through the HIP library, compared with the
channels-first oracle: the same seeded case as tests/gpu_gn.py, its X and dY
transposed to [N, L, C] for the GPU, and the GPU's Y and dX transposed back
([N, C, L]) for the element-by-element comparison (gpu_gn.compare, the same
tolerances). Transposing moves values only; the oracle's arithmetic is the
channels-first one, which the pins cover.
"""
from __future__ import annotations

from typing import Optional

import numpy as np
import torch

import row_wise_normalization_amd as mn
from gpu_cases import dev, empty, host


def to_nlc(a: np.ndarray) -> np.ndarray:
    return np.ascontiguousarray(np.swapaxes(a, 1, 2))


def run(d, G: int, eps: float, offset: int = 0, dx_dtype: Optional[torch.dtype] = None,
        ws_fill: Optional[int] = None):
    """Forward, then backward fed with the forward's own statistics, on the
    channels-last layout; returns the outputs in the channels-first layout."""
    N, C, L = d["X"].shape
    X = dev(to_nlc(d["X"]), offset)
    dY = dev(to_nlc(d["dY"]), offset)
    g = dev(d["gamma"], offset)
    b = dev(d["beta"], offset)
    Y = empty((N, L, C), X.dtype, offset)
    dX = empty((N, L, C), X.dtype if dx_dtype is None else dx_dtype, offset)
    mean = torch.empty(N, G, dtype=torch.float32, device="cuda")
    rstd = torch.empty(N, G, dtype=torch.float32, device="cuda")
    nb = mn.groupnorm_nlc_workspace_bytes(N, L, C, G)
    assert nb > 0
    ws = torch.empty(nb // 4, dtype=torch.float32, device="cuda")
    if ws_fill is not None:
        ws.view(torch.int32).fill_(ws_fill)
    mn.mn_groupnorm_nlc_forward_ex(X, g, b, Y, mean, rstd, G, eps, ws)
    dg = torch.empty(C, dtype=torch.float32, device="cuda")
    db = torch.empty(C, dtype=torch.float32, device="cuda")
    mn.mn_groupnorm_nlc_backward_ex(X, g, mean, rstd, dY, dX, dg, db, G, ws)
    torch.cuda.synchronize()
    back = lambda t: np.ascontiguousarray(np.swapaxes(host(t), 1, 2))
    return {"Y": back(Y), "dX": back(dX), "mean": host(mean), "rstd": host(rstd),
            "dgamma": host(dg), "dbeta": host(db)}
