"""The no-allocation RMSNorm backward against the workspace entry point.

mn_rmsnorm_backward_noalloc runs the same two kernels as
mn_rmsnorm_backward with the library's fixed device scratch array in place
of the caller's workspace, so dX and dgamma must be bitwise those of the
workspace call. Calls follow one another through the one array: the second
is smaller than the first (the array still holds the first call's partial
rows), the third is on the element-wise path, the fourth on a stream of its
own. Every call is also held to the oracle's bar on dgamma.
"""
import numpy as np
import pytest
import torch

import parity
import row_wise_normalization_amd as mn
import workloads
from gpu_cases import dev, reference, say

pytestmark = pytest.mark.gpu


def _bits(a):
    return a.view(np.uint32 if a.dtype == np.float32 else np.uint16)


def _one(N, D, seed, stream=None):
    d = workloads.random_case("rms", N, D, seed)
    X, g, dY = dev(d["X"]), dev(d["gamma"]), dev(d["dY"])
    Y = torch.empty_like(X)
    rstd = torch.empty(N, dtype=torch.float32, device="cuda")
    mn.mn_rmsnorm_forward(X, g, Y, rstd, 1e-5)
    # the workspace entry point
    dX_a = torch.empty_like(X)
    dg_a = torch.empty(D, dtype=torch.float32, device="cuda")
    mn.mn_rmsnorm_backward(X, g, rstd, dY, dX_a, dg_a, mn.new_workspace(mn.MN_RMSNORM, N, D))
    torch.cuda.synchronize()
    # the no-allocation one (outputs pre-filled so a skipped write shows)
    dX_b = torch.full_like(X, 7.0)
    dg_b = torch.full((D,), 7.0, dtype=torch.float32, device="cuda")
    if stream is None:
        mn.mn_rmsnorm_backward_noalloc(X, g, rstd, dY, dX_b, dg_b)
    else:
        with torch.cuda.stream(stream):
            mn.mn_rmsnorm_backward_noalloc(X, g, rstd, dY, dX_b, dg_b, stream=stream)
        stream.synchronize()
    torch.cuda.synchronize()
    a_dx, b_dx = dX_a.cpu().numpy(), dX_b.cpu().numpy()
    a_dg, b_dg = dg_a.cpu().numpy(), dg_b.cpu().numpy()
    assert (_bits(a_dx) == _bits(b_dx)).all(), f"{N}x{D}: dX differs"
    assert (_bits(a_dg) == _bits(b_dg)).all(), f"{N}x{D}: dgamma differs"
    ref = reference("rms", d, 1e-5, per_row=False)
    parity.check_grad(b_dg, ref["dgamma"], f"noalloc {N}x{D} dgamma")
    say(f"[noalloc] {N}x{D}: bitwise equal to the workspace call")


def test_noalloc_matches_workspace_entry_point_in_sequence():
    _one(2048, 8192, 1)                     # fills the whole 8 MiB array
    _one(16384, 4096, 5)                    # the headline shape
    _one(1000, 1024, 2)                     # smaller: stale partials must not leak
    _one(129, 257, 3)                       # element-wise path
    _one(3, 8192, 4, stream=torch.cuda.Stream())   # fewer rows than workgroups, own stream


def test_noalloc_rejects_bad_arguments():
    X = torch.zeros(4, 64, dtype=torch.float16, device="cuda")
    g = torch.ones(64, dtype=torch.float16, device="cuda")
    r = torch.ones(4, dtype=torch.float32, device="cuda")
    dX = torch.empty_like(X)
    dg = torch.empty(64, dtype=torch.float32, device="cuda")
    with pytest.raises(mn.MnError, match="MN_ERR_ALIAS"):
        mn.mn_rmsnorm_backward_noalloc(X, g, r, X, X, dg)
    L = mn.lib()
    assert L.mn_rmsnorm_backward_noalloc(X.data_ptr(), g.data_ptr(), r.data_ptr(), X.data_ptr(),
                                         dX.data_ptr(), dg.data_ptr(), 0, 64, None) == 2
