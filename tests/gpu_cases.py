"""Run one case through the HIP library (via the binding) and through the
oracle, and compare them with the parity helpers."""
from __future__ import annotations

import sys
from typing import Dict, Optional

import numpy as np
import torch

import every_row
import oracle
import parity
import row_wise_normalization_amd as mn


def say(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


_TORCH = {np.dtype(np.float16): torch.float16, np.dtype(np.uint16): torch.bfloat16,
          np.dtype(np.float32): torch.float32}


def dev(a: np.ndarray, offset: int = 0) -> torch.Tensor:
    """Upload ``a`` as a contiguous GPU tensor whose first element sits
    ``offset`` elements past a 256-byte aligned allocation (uint16 arrays
    are bfloat16 bit patterns)."""
    a = np.ascontiguousarray(a)
    bf16 = a.dtype == np.uint16
    t = torch.from_numpy(a.view(np.int16) if bf16 else a)
    if bf16:
        t = t.view(torch.bfloat16)
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
    """Download a GPU tensor (bfloat16 comes back as uint16 bit patterns)."""
    if t is None:
        return None
    t = t.detach()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def run_gpu(kind: str, d: Dict[str, np.ndarray], eps: float, offset: int = 0,
            use_dh: bool = True, typed: Optional[bool] = None,
            dx_dtype: Optional[torch.dtype] = None) -> Dict[str, np.ndarray]:
    """Forward, then backward fed with the forward's own saved statistics.
    All-fp16 cases go through the fp16 entry points, any other storage (or
    ``typed=True``) through the ``_ex`` entry points; dX is stored in
    ``dx_dtype`` (default: the activation type)."""
    N, D = d["X"].shape
    act = _TORCH[d["X"].dtype]
    dxt = act if dx_dtype is None else dx_dtype
    if typed is None:
        typed = not (d["X"].dtype == np.float16 and d["gamma"].dtype == np.float16 and
                     d["dY"].dtype == np.float16 and dxt == torch.float16)
    X = dev(d["X"], offset)
    g = dev(d["gamma"], offset)
    dY = dev(d["dY"], offset)
    out: Dict[str, np.ndarray] = {}
    Y = empty((N, D), act, offset)
    rstd = torch.empty(N, dtype=torch.float32, device="cuda")
    dX = empty((N, D), dxt, offset)
    dgamma = torch.empty(D, dtype=torch.float32, device="cuda")
    x = "_ex" if typed else ""
    if kind == "rms":
        getattr(mn, "mn_rmsnorm_forward" + x)(X, g, Y, rstd, eps)
        ws = mn.new_workspace(mn.MN_RMSNORM, N, D)
        getattr(mn, "mn_rmsnorm_backward" + x)(X, g, rstd, dY, dX, dgamma, ws)
    elif kind == "ln":
        b = dev(d["beta"], offset)
        mean = torch.empty(N, dtype=torch.float32, device="cuda")
        dbeta = torch.empty(D, dtype=torch.float32, device="cuda")
        getattr(mn, "mn_layernorm_forward" + x)(X, g, b, Y, mean, rstd, eps)
        ws = mn.new_workspace(mn.MN_LAYERNORM, N, D)
        getattr(mn, "mn_layernorm_backward" + x)(X, g, mean, rstd, dY, dX, dgamma, dbeta, ws)
        out["mean"] = host(mean)
        out["dbeta"] = host(dbeta)
    elif kind == "add":
        R = dev(d["R"], offset)
        dH = dev(d["dH"], offset) if use_dh else None
        Hs = empty((N, D), act, offset)
        getattr(mn, "mn_add_rmsnorm_forward" + x)(X, R, g, Hs, Y, rstd, eps)
        ws = mn.new_workspace(mn.MN_ADD_RMSNORM, N, D)
        getattr(mn, "mn_add_rmsnorm_backward" + x)(X, R, g, rstd, dY, dH, dX, dgamma, ws)
        out["H"] = host(Hs)
    else:
        raise ValueError(kind)
    torch.cuda.synchronize()
    out.update(Y=host(Y), rstd=host(rstd), dX=host(dX), dgamma=host(dgamma))
    return out


def reference(kind: str, d: Dict[str, np.ndarray], eps: float, rows=None,
              use_dh: bool = True, per_row: bool = True, grads: bool = True
              ) -> Dict[str, np.ndarray]:
    """Oracle results: per-row outputs for ``rows`` (all rows when None; an
    index array or a slice) and parameter gradients over all rows. Either
    half can be left out (``per_row``, ``grads``)."""
    sub = (lambda a: a) if rows is None else (lambda a: np.ascontiguousarray(a[rows]))
    X, dY = d["X"], d["dY"]
    o: Dict[str, np.ndarray] = {}
    if kind == "rms":
        if per_row:
            o["Y"], o["rstd"] = oracle.rmsnorm_forward(sub(X), d["gamma"], eps)
            o["dX"], _ = oracle.rmsnorm_backward(sub(X), d["gamma"], sub(dY), eps)
        if grads:
            _, o["dgamma"] = oracle.rmsnorm_backward(X, d["gamma"], dY, eps, want_dx=False)
    elif kind == "ln":
        if per_row:
            o["Y"], o["mean"], o["rstd"] = oracle.layernorm_forward(sub(X), d["gamma"],
                                                                   d["beta"], eps)
            o["dX"], _, _ = oracle.layernorm_backward(sub(X), d["gamma"], sub(dY), eps)
        if grads:
            _, o["dgamma"], o["dbeta"] = oracle.layernorm_backward(X, d["gamma"], dY, eps,
                                                                   want_dx=False)
    elif kind == "add":
        R = d["R"]
        dH = d["dH"] if use_dh else None
        if per_row:
            _, o["H16"], o["Y"], o["rstd"] = oracle.add_rmsnorm_forward(sub(X), sub(R),
                                                                        d["gamma"], eps)
            o["dX"], _ = oracle.add_rmsnorm_backward(sub(X), sub(R), d["gamma"], sub(dY),
                                                     None if dH is None else sub(dH), eps)
        if grads:
            _, o["dgamma"] = oracle.add_rmsnorm_backward(X, R, d["gamma"], dY, dH, eps,
                                                         want_dx=False)
    return o


def _f64(a):
    return parity.as_f64(a)


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
    # xhat = (x - mean) * rstd is formed from x and the fp32 mean, so its
    # rounding error scales with |x| + |mean|, not with |x - mean|
    xs = (np.abs(x) + np.abs(mu)) * rs
    g = _f64(sub(d["dY"])) * _f64(d["gamma"])[None, :]
    A = (np.abs(g) * xs).mean(axis=1, keepdims=True)
    sdx = rs * (np.abs(g) + xs * A)
    if kind == "ln":
        sdx = sdx + rs * np.abs(g).mean(axis=1, keepdims=True)
    if kind == "add" and use_dh:
        sdx = sdx + np.abs(_f64(sub(d["dH"])))
    sy = None
    if kind == "ln":
        sy = xs * np.abs(_f64(d["gamma"]))[None, :] + np.abs(_f64(d["beta"]))[None, :]
    return sdx, sy


def compare(kind: str, gpu: Dict[str, np.ndarray], ref: Dict[str, np.ndarray], what: str,
            rows=None, mean_atol: float = 0.0,
            inputs: Optional[Dict[str, np.ndarray]] = None, use_dh: bool = True,
            per_row: bool = True, grads: bool = True) -> Dict[str, float]:
    """Check every element of the GPU outputs (restricted to ``rows``, an
    index array or a slice) against the oracle; returns the worst error per
    output and, for 16-bit outputs, how many elements only the fp32
    cancellation allowance admitted. With ``inputs`` that allowance of
    parity.check_out applies; without it every element must be within
    2 ulp. float32 outputs need ``inputs`` (their bound is relative to the
    fp32 terms). ``per_row`` and ``grads`` select the halves to check."""
    sel = (lambda a: a) if rows is None else (lambda a: a[rows])
    w: Dict[str, float] = {}
    if grads:
        w["dgamma"] = parity.check_grad(gpu["dgamma"], ref["dgamma"], f"{what} dgamma")
        if kind == "ln":
            w["dbeta"] = parity.check_grad(gpu["dbeta"], ref["dbeta"], f"{what} dbeta")
    if not per_row:
        return w
    sdx = sy = None
    if inputs is not None:
        sdx, sy = cancel_scales(kind, inputs, ref, rows, use_dh)
    if inputs is None and np.float32 in (gpu["Y"].dtype, gpu["dX"].dtype):
        raise ValueError("float32 outputs are checked against the scale of their fp32 terms; "
                         "pass the inputs")
    w["Y_ulp"], w["Y_fp32_admitted"] = parity.check_out(sel(gpu["Y"]), ref["Y"], f"{what} Y",
                                                        scale=sy)
    w["dX_ulp"], w["dX_fp32_admitted"] = parity.check_out(sel(gpu["dX"]), ref["dX"],
                                                          f"{what} dX", scale=sdx)
    w["rstd_rel"] = parity.check_stat(sel(gpu["rstd"]), ref["rstd"], f"{what} rstd")
    if kind == "ln":
        if inputs is not None:
            # a mean near zero is a cancellation of fp32 terms of size mean|x|
            sub = (lambda a: a) if rows is None else (lambda a: a[rows])
            xa = np.abs(_f64(sub(inputs["X"]))).mean(axis=1)
            mean_atol = np.maximum(mean_atol, parity.FP32_K * 2.0 ** -24 * xa)
        w["mean_rel"] = parity.check_stat(sel(gpu["mean"]), ref["mean"], f"{what} mean",
                                          atol=mean_atol)
    if kind == "add":
        hg, hr = sel(gpu["H"]), ref["H16"]
        assert hg.dtype == hr.dtype, f"{what} H: {hg.dtype} vs {hr.dtype}"
        bits = np.uint32 if hg.dtype == np.float32 else np.uint16
        sign = bits(0x80000000 if bits is np.uint32 else 0x8000)
        h, r = hg.view(bits), hr.view(bits)
        # +0 and -0 are the same sum; otherwise H must be the exact rounded sum
        same = (h == r) | (((h | r) & ~sign) == 0)
        assert same.all(), f"{what} H: {int((~same).sum())} elements differ from round(x + r)"
    return w


def compare_every_row(kind: str, gpu: Dict[str, np.ndarray], d: Dict[str, np.ndarray],
                      eps: float, what: str, inputs: Optional[Dict[str, np.ndarray]] = None,
                      use_dh: bool = True) -> Dict[str, float]:
    """compare() over every row of a full-size call: the oracle runs on
    blocks of rows (bounded host memory, several blocks at a time), the
    parameter gradients once over all rows. Returns the worst error per
    output, the admitted counts summed over the blocks and ``rows_checked``."""
    N, D = d["X"].shape
    ref_g = reference(kind, d, eps, use_dh=use_dh, per_row=False)
    w = compare(kind, gpu, ref_g, what, per_row=False)

    def block(rows):
        ref = reference(kind, d, eps, rows=rows, use_dh=use_dh, grads=False)
        return compare(kind, gpu, ref, what, rows=rows, inputs=inputs, use_dh=use_dh,
                       grads=False)

    w.update(every_row.run_blocks(N, D, block))
    return w
