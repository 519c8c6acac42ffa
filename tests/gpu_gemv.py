"""Run a fused RMSNorm / LayerNorm + GEMV case through the HIP library and
through the oracle, and compare them element by element.

Each output is held to 2 ulp of its storage type. An element that misses it
is admitted only within the fp32 summation bound of the kernel: the longest
chain of fp32 roundings behind an output (at most 64 products per lane, the
lane and wave additions, one addition per K slice, at most ceil(K / 64)
slices, and a few for the statistics and the final combination), each worth
2^-24 of the size of the summed terms. The kernel sums the shifted rows
(x - c) * gamma against W (c = 0 for RMSNorm, the row's first element for
LayerNorm) and applies rstd, and for LayerNorm (mean - c) times the column
sums of gamma * W and the column sums of beta * W, afterwards; the size of
the terms is rstd * (sum_k |(x - c) g W| + |mean - c| sum_k |g W|)
+ sum_k |b W|. The pages' own acceptance measure, the RMS error over the RMS
of the reference (at most 5e-3), is checked and reported beside it.
"""
import numpy as np
import torch

import oracle
import parity
import workloads
import row_wise_normalization_amd as mn
from gpu_cases import dev, empty, host, say


def run(d, eps, ln, offset=0):
    X = dev(d["X"], offset)
    g = dev(d["gamma"], offset)
    W = dev(d["W"], offset)
    b = dev(d["beta"], offset) if ln else None
    M, K = X.shape
    N = W.shape[1]
    Y = empty((M, N), X.dtype, offset)
    mn.mn_fused_norm_gemv_ex(X, g, W, Y, eps, workspace(M, N, K), beta=b)
    torch.cuda.synchronize()
    return host(Y)


_WS = [None]


def workspace(M, N, K):
    """One zero-filled workspace kept across calls (any shape, RMSNorm or
    LayerNorm), as the entry point allows: every call must leave its arrival
    counters at zero for the next."""
    nb = max(16, mn.norm_gemv_workspace_bytes(M, N, K))
    if _WS[0] is None or _WS[0].numel() * 4 < nb:
        _WS[0] = torch.zeros(max(nb // 4, 1 << 20), dtype=torch.float32, device="cuda")
    return _WS[0]


def reference(d, eps, ln):
    return oracle.norm_gemv(d["X"], d["gamma"], d["W"], eps, beta=d["beta"] if ln else None)


def _terms(d, eps, ln):
    """Size of the fp32 terms behind each output (see the module docstring)."""
    x = parity.as_f64(d["X"])
    g = parity.as_f64(d["gamma"])
    aw = np.abs(parity.as_f64(d["W"]))
    c = x[:, :1] if ln else 0.0
    mu = x.mean(axis=1, keepdims=True) if ln else 0.0
    var = ((x - mu) ** 2).mean(axis=1, keepdims=True)
    rs = 1.0 / np.sqrt(var + eps)
    t = rs * (np.abs((x - c) * g) @ aw)
    if ln:
        t += rs * np.abs(mu - c) * (np.abs(g) @ aw)[None, :]
        t += (np.abs(parity.as_f64(d["beta"])) @ aw)[None, :]
    return t


def compare(gpu, ref, d, eps, ln, what):
    K = d["X"].shape[1]
    chain = 64 + 8 + -(-K // 64) + 8
    terms = _terms(d, eps, ln)
    worst, admitted = parity.check_out(gpu, ref, f"{what} Y",
                                       scale=terms * (chain / parity.FP32_K))
    g = parity.as_f64(gpu)
    rms = float(np.sqrt(np.mean((g - ref) ** 2)) / max(np.sqrt(np.mean(ref ** 2)), 1e-300))
    assert rms <= 5e-3, f"{what}: rms_scaled {rms}"
    return {"ulp": worst, "admitted": admitted, "rms_scaled": rms}


def case(M, K, N, seed, ln, act="f16", param=None, x_loc=None):
    kind = "ln_gemv" if ln else "rms_gemv"
    loc = (0.5 if ln else 0.0) if x_loc is None else x_loc
    return workloads.random_case(kind, M, K, seed, x_loc=loc, act=act, param=param, Nout=N)
