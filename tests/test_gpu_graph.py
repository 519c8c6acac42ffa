"""The library's calls can be captured in a HIP graph (they allocate nothing
and enqueue only kernels): capture forward + backward once, then replay it
several times with fresh inputs copied in between, with eager work and
synchronizations between replays; every replay must match the eager calls
bit for bit."""
import numpy as np
import pytest
import torch

import row_wise_normalization_amd as mn
import workloads
from gpu_cases import say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("kind,N,D", [("rms", 4096, 4096), ("ln", 1024, 1024), ("add", 512, 8192),
                                      ("rms", 8192, 128)])
def test_graph_replay_matches_eager(kind, N, D):
    say(f"[graph] {kind} {N}x{D}")
    dev = torch.device("cuda", 0)
    cases = [workloads.random_case(kind, N, D, seed=50 + i) for i in range(3)]
    t = {k: torch.from_numpy(v).to(dev) for k, v in cases[0].items()}
    out = {"Y": torch.empty(N, D, dtype=torch.float16, device=dev),
           "dX": torch.empty(N, D, dtype=torch.float16, device=dev),
           "rstd": torch.empty(N, dtype=torch.float32, device=dev),
           "mean": torch.empty(N, dtype=torch.float32, device=dev),
           "H": torch.empty(N, D, dtype=torch.float16, device=dev),
           "dgamma": torch.empty(D, dtype=torch.float32, device=dev),
           "dbeta": torch.empty(D, dtype=torch.float32, device=dev)}
    code = {"rms": mn.MN_RMSNORM, "ln": mn.MN_LAYERNORM, "add": mn.MN_ADD_RMSNORM}[kind]
    ws = mn.new_workspace(code, N, D, dev)

    def run(t, o, stream=None):
        if kind == "rms":
            mn.mn_rmsnorm_forward(t["X"], t["gamma"], o["Y"], o["rstd"], 1e-5, stream)
            mn.mn_rmsnorm_backward(t["X"], t["gamma"], o["rstd"], t["dY"], o["dX"], o["dgamma"],
                                   ws, stream)
        elif kind == "ln":
            mn.mn_layernorm_forward(t["X"], t["gamma"], t["beta"], o["Y"], o["mean"], o["rstd"],
                                    1e-5, stream)
            mn.mn_layernorm_backward(t["X"], t["gamma"], o["mean"], o["rstd"], t["dY"], o["dX"],
                                     o["dgamma"], o["dbeta"], ws, stream)
        else:
            mn.mn_add_rmsnorm_forward(t["X"], t["R"], t["gamma"], o["H"], o["Y"], o["rstd"], 1e-5,
                                      stream)
            mn.mn_add_rmsnorm_backward(t["X"], t["R"], t["gamma"], o["rstd"], t["dY"], t["dH"],
                                       o["dX"], o["dgamma"], ws, stream)

    # warm up on a side stream, as graph capture requires
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run(t, out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(t, out)
    torch.cuda.synchronize()

    keys = ["Y", "dX", "rstd", "dgamma"] + (["mean", "dbeta"] if kind == "ln" else []) + \
           (["H"] if kind == "add" else [])
    for i, case in enumerate(cases + cases[:1]):
        for k, v in case.items():
            t[k].copy_(torch.from_numpy(v))
        # unrelated eager work between replays
        junk = torch.randn(1 << 20, device=dev).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {k: out[k].clone() for k in keys}
        ref = {k: torch.empty_like(out[k]) for k in out}
        run(t, ref)          # eager, same inputs, separate outputs
        torch.cuda.synchronize()
        for k in keys:
            a = got[k].cpu().numpy()
            b = ref[k].cpu().numpy()
            view = np.uint32 if a.dtype == np.float32 else np.uint16
            assert (a.view(view) == b.view(view)).all(), f"replay {i}: {k} differs from eager"
        del junk


@pytest.mark.parametrize("layout,N,C,L,G", [("ncl", 4, 320, 1024, 32), ("ncl", 2, 64, 20001, 4),
                                            ("nlc", 4, 320, 1024, 32), ("nlc", 2, 300, 77, 10)])
def test_graph_replay_groupnorm(layout, N, C, L, G):
    """GroupNorm forward + backward in a captured graph: the register path,
    the split path (slices beyond one workgroup) and the channels-last
    passes, replayed with new inputs, bitwise the eager result."""
    say(f"[graph] groupnorm {layout} {N}x{C}x{L} G={G}")
    dev = torch.device("cuda", 0)
    shape = (N, C, L) if layout == "ncl" else (N, L, C)

    def case(seed):
        d = workloads.random_case("gn", N, C * L, seed, x_loc=0.5, channels=C, groups=G)
        for k in ("X", "dY"):
            a = d[k].reshape(N, C, L)
            d[k] = np.ascontiguousarray(a if layout == "ncl" else a.swapaxes(1, 2))
        return d

    cases = [case(60 + i) for i in range(3)]
    t = {k: torch.from_numpy(v).to(dev) for k, v in cases[0].items()}

    def outputs():
        return {"Y": torch.empty(shape, dtype=torch.float16, device=dev),
                "dX": torch.empty(shape, dtype=torch.float16, device=dev),
                "mean": torch.empty(N, G, dtype=torch.float32, device=dev),
                "rstd": torch.empty(N, G, dtype=torch.float32, device=dev),
                "dgamma": torch.empty(C, dtype=torch.float32, device=dev),
                "dbeta": torch.empty(C, dtype=torch.float32, device=dev)}

    out = outputs()
    nb = (mn.groupnorm_workspace_bytes(N, C, L, G) if layout == "ncl"
          else mn.groupnorm_nlc_workspace_bytes(N, L, C, G))
    ws = torch.empty(max(16, nb) // 4, dtype=torch.float32, device=dev)

    def run(t, o, stream=None):
        if layout == "ncl":
            mn.mn_groupnorm_forward_ex(t["X"], t["gamma"], t["beta"], o["Y"], o["mean"], o["rstd"],
                                       G, 1e-5, stream)
            mn.mn_groupnorm_backward_ex(t["X"], t["gamma"], o["mean"], o["rstd"], t["dY"], o["dX"],
                                        o["dgamma"], o["dbeta"], G, ws, stream)
        else:
            mn.mn_groupnorm_nlc_forward_ex(t["X"], t["gamma"], t["beta"], o["Y"], o["mean"],
                                           o["rstd"], G, 1e-5, ws, stream)
            mn.mn_groupnorm_nlc_backward_ex(t["X"], t["gamma"], o["mean"], o["rstd"], t["dY"],
                                            o["dX"], o["dgamma"], o["dbeta"], G, ws, stream)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        run(t, out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run(t, out)
    torch.cuda.synchronize()
    for i, c in enumerate(cases + cases[:1]):
        for k, v in c.items():
            t[k].copy_(torch.from_numpy(v))
        junk = torch.randn(1 << 20, device=dev).sum()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = {k: v.clone() for k, v in out.items()}
        ref = outputs()
        run(t, ref)
        torch.cuda.synchronize()
        for k in got:
            a = got[k].cpu().numpy()
            b = ref[k].cpu().numpy()
            view = np.uint32 if a.dtype == np.float32 else np.uint16
            assert (a.view(view) == b.view(view)).all(), f"replay {i}: {k} differs from eager"
        del junk
