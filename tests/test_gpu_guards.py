"""No writes outside the caller's buffers, on every kernel path.

Every output, statistic, parameter gradient and workspace of a call sits in
a device allocation with canary bytes before and after it; after the call
the canaries must be intact, and the inputs bit for bit unchanged (no
in-place mutation: the [meTile] contract, section "Exact native
normalization contract"). The shapes cover each path's tail handling: the
16-byte vector path, the element-wise path (widths that are not a multiple
of 8, and tensors starting 2 bytes past a 16-byte boundary), the narrow-row
layout with a ragged last tile, the widest rows, and a row count below the
backward's workgroup count. Parity tests compare only inside the outputs, so
they cannot see such writes.
"""
from __future__ import annotations

from typing import Dict, List, Tuple

import numpy as np
import pytest
import torch

import row_wise_normalization_amd as mn
import workloads
from gpu_cases import say

pytestmark = pytest.mark.gpu

GUARD = 4096           # canary bytes on each side
CANARY = 0xA5

T = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


class Guarded:
    """A tensor of `shape` and `dtype` whose first element sits `offset`
    elements past a 4096-byte canary region, followed by another one."""

    def __init__(self, shape, dtype, offset: int = 0, fill: int = CANARY):
        esz = torch.empty((), dtype=dtype).element_size()
        n = int(np.prod(shape))
        self.start = GUARD + offset * esz
        self.nbytes = n * esz
        self.raw = torch.full((self.start + self.nbytes + GUARD,), CANARY, dtype=torch.uint8,
                              device="cuda")
        if fill != CANARY:
            self.raw[self.start:self.start + self.nbytes].fill_(fill)
        self.t = self.raw[self.start:self.start + self.nbytes].view(dtype).view(shape)

    def intact(self) -> bool:
        h = self.raw.cpu()
        return bool((h[:self.start] == CANARY).all() and
                    (h[self.start + self.nbytes:] == CANARY).all())


def upload(a: np.ndarray, offset: int = 0) -> Guarded:
    """An input copied into a guarded allocation (bfloat16 as uint16 bits)."""
    bf16 = a.dtype == np.uint16
    src = torch.from_numpy(np.ascontiguousarray(a).view(np.int16) if bf16 else
                           np.ascontiguousarray(a))
    if bf16:
        src = src.view(torch.bfloat16)
    g = Guarded(a.shape, src.dtype, offset)
    g.t.copy_(src)
    return g


def workspace(nbytes: int, fill: int = CANARY) -> Guarded:
    return Guarded((max(4, (nbytes + 3) // 4),), torch.float32, 0, fill)


def snapshot(inputs: Dict[str, Guarded]):
    """The inputs' bytes (guards included) before the call."""
    torch.cuda.synchronize()
    return {k: v.raw.cpu().clone() for k, v in inputs.items()}


def verify(outputs: Dict[str, Guarded], inputs: Dict[str, Guarded], before, what: str):
    torch.cuda.synchronize()
    for k, g in outputs.items():
        assert g.intact(), f"{what}: write outside {k}"
    for k, g in inputs.items():
        assert torch.equal(g.raw.cpu(), before[k]), f"{what}: input {k} was modified"
    say(f"[guards] {what}: {len(outputs)} outputs intact, {len(inputs)} inputs unchanged")


# (N, D, element offset): vector path, element-wise unaligned, element-wise
# ragged width, narrow rows with a ragged tile, widest rows, fewer rows than
# the backward's workgroups
PAIR_SHAPES = [(300, 4096, 0), (301, 4096, 1), (129, 257, 0), (1001, 128, 0), (333, 8192, 0),
               (5, 1000, 0), (77, 64, 1)]


@pytest.mark.parametrize("N,D,off", PAIR_SHAPES)
@pytest.mark.parametrize("kind", ["rms", "ln", "add"])
def test_training_pair_guards(kind, N, D, off):
    _pair(kind, N, D, off, "f16", "f16", "f16", "f16")


@pytest.mark.parametrize("act,param,cot,dxt", [("bf16", "f32", "bf16", "bf16"),
                                               ("f16", "f16", "f32", "f32"),
                                               ("f32", "f32", "f32", "f32")])
@pytest.mark.parametrize("N,D,off", [(300, 4096, 0), (129, 257, 1), (1001, 128, 0)])
@pytest.mark.parametrize("kind", ["rms", "ln", "add"])
def test_training_pair_guards_storage(kind, N, D, off, act, param, cot, dxt):
    _pair(kind, N, D, off, act, param, cot, dxt)


def _pair(kind, N, D, off, act, param, cot, dxt):
    what = f"{kind} {N}x{D}+{off} {act}/{param}/{cot}/{dxt}"
    d = workloads.random_case(kind, N, D, 40 + D, x_loc=0.5 if kind == "ln" else 0.0,
                              act=act, param=param, cot=cot)
    ins = {k: upload(v, off) for k, v in d.items()}
    a = T[act]
    outs = {"Y": Guarded((N, D), a, off), "rstd": Guarded((N,), torch.float32),
            "dX": Guarded((N, D), T[dxt], off), "dgamma": Guarded((D,), torch.float32)}
    kcode = {"rms": mn.MN_RMSNORM, "ln": mn.MN_LAYERNORM, "add": mn.MN_ADD_RMSNORM}[kind]
    outs["ws"] = workspace(mn.workspace_bytes(kcode, N, D))
    if kind == "ln":
        outs["mean"] = Guarded((N,), torch.float32)
        outs["dbeta"] = Guarded((D,), torch.float32)
    if kind == "add":
        outs["H"] = Guarded((N, D), a, off)
    before = snapshot(ins)
    o = {k: v.t for k, v in outs.items()}
    i = {k: v.t for k, v in ins.items()}
    if kind == "rms":
        mn.mn_rmsnorm_forward_ex(i["X"], i["gamma"], o["Y"], o["rstd"], 1e-5)
        mn.mn_rmsnorm_backward_ex(i["X"], i["gamma"], o["rstd"], i["dY"], o["dX"], o["dgamma"],
                                  o["ws"])
    elif kind == "ln":
        mn.mn_layernorm_forward_ex(i["X"], i["gamma"], i["beta"], o["Y"], o["mean"], o["rstd"],
                                   1e-5)
        mn.mn_layernorm_backward_ex(i["X"], i["gamma"], o["mean"], o["rstd"], i["dY"], o["dX"],
                                    o["dgamma"], o["dbeta"], o["ws"])
    else:
        mn.mn_add_rmsnorm_forward_ex(i["X"], i["R"], i["gamma"], o["H"], o["Y"], o["rstd"], 1e-5)
        mn.mn_add_rmsnorm_backward_ex(i["X"], i["R"], i["gamma"], o["rstd"], i["dY"], i["dH"],
                                      o["dX"], o["dgamma"], o["ws"])
    verify(outs, ins, before, what)


@pytest.mark.parametrize("N,D,off", [(300, 4096, 0), (301, 4096, 1), (129, 257, 0),
                                     (1000, 128, 0), (90, 8192, 0), (6, 1000, 0)])
@pytest.mark.parametrize("kind", ["dyt", "poly", "mod"])
def test_other_norm_guards(kind, N, D, off):
    what = f"{kind} {N}x{D}+{off}"
    B = 3 if N % 3 == 0 else 1
    d = workloads.random_case(kind, N, D, 60 + D, B=B) if kind == "mod" else \
        workloads.random_case(kind, N, D, 60 + D)
    ins = {k: upload(v, off) for k, v in d.items()}
    outs = {"Y": Guarded((N, D), torch.float16, off), "dX": Guarded((N, D), torch.float16, off)}
    if kind == "dyt":
        ins["alpha"] = upload(np.array([0.5], np.float32))
        outs.update(dalpha=Guarded((1,), torch.float32), dgamma=Guarded((D,), torch.float32),
                    dbeta=Guarded((D,), torch.float32),
                    ws=workspace(mn.workspace_bytes(mn.MN_DYT, N, D)))
    elif kind == "poly":
        ins["params"] = upload(np.array(workloads.POLY_PARAMS, np.float32))
        outs.update(rstd=Guarded((N, 3), torch.float32), dparams=Guarded((4,), torch.float32),
                    ws=workspace(mn.workspace_bytes(mn.MN_POLYNORM, N, D)))
    else:
        outs.update(rstd=Guarded((N,), torch.float32), dgamma=Guarded((D,), torch.float32),
                    dscale=Guarded((B, D), torch.float32), dshift=Guarded((B, D), torch.float32),
                    ws=workspace(mn.mod_rmsnorm_workspace_bytes(B, N, D)))
    before = snapshot(ins)
    o = {k: v.t for k, v in outs.items()}
    i = {k: v.t for k, v in ins.items()}
    if kind == "dyt":
        mn.mn_dyt_forward_ex(i["X"], i["alpha"], i["gamma"], i["beta"], o["Y"])
        mn.mn_dyt_backward_ex(i["X"], i["alpha"], i["gamma"], i["dY"], o["dX"], o["dalpha"],
                              o["dgamma"], o["dbeta"], o["ws"])
    elif kind == "poly":
        mn.mn_polynorm_forward_ex(i["X"], i["params"], o["Y"], o["rstd"], 1e-5)
        mn.mn_polynorm_backward_ex(i["X"], i["params"], o["rstd"], i["dY"], o["dX"],
                                   o["dparams"], o["ws"])
    else:
        mn.mn_mod_rmsnorm_forward_ex(i["X"], i["gamma"], i["scale"], i["shift"], o["Y"],
                                     o["rstd"], 1e-5)
        mn.mn_mod_rmsnorm_backward_ex(i["X"], i["gamma"], i["scale"], o["rstd"], i["dY"],
                                      o["dX"], o["dgamma"], o["dscale"], o["dshift"], o["ws"])
    verify(outs, ins, before, what)


# (N, C, L, G, offset): the vector path at several lane shapes, the
# element-wise path (L not a multiple of 8), unaligned tensors, G = C
# the last three take the split path (slices beyond one workgroup), on
# 16-byte chunks, element-wise with several units per channel row, and with
# many short channel rows
GN_SHAPES = [(2, 64, 256, 8, 0), (2, 12, 100, 3, 0), (3, 32, 4096, 32, 0), (2, 40, 64, 4, 1),
             (1, 16, 8, 16, 0), (4, 320, 1024, 32, 0), (2, 32, 16384, 2, 0),
             (1, 8, 20001, 1, 1), (2, 3000, 9, 1, 0)]


@pytest.mark.parametrize("N,C,L,G,off", GN_SHAPES)
def test_groupnorm_guards(N, C, L, G, off):
    what = f"groupnorm {N}x{C}x{L} G={G}+{off}"
    d = workloads.random_case("gn", N, C * L, 80 + L, x_loc=0.5, channels=C, groups=G)
    d["X"] = d["X"].reshape(N, C, L)
    d["dY"] = d["dY"].reshape(N, C, L)
    ins = {k: upload(v, off) for k, v in d.items()}
    outs = {"Y": Guarded((N, C, L), torch.float16, off),
            "dX": Guarded((N, C, L), torch.float16, off),
            "mean": Guarded((N, G), torch.float32), "rstd": Guarded((N, G), torch.float32),
            "dgamma": Guarded((C,), torch.float32), "dbeta": Guarded((C,), torch.float32),
            "ws": workspace(mn.groupnorm_workspace_bytes(N, C, L, G))}
    before = snapshot(ins)
    o = {k: v.t for k, v in outs.items()}
    i = {k: v.t for k, v in ins.items()}
    mn.mn_groupnorm_forward_ex(i["X"], i["gamma"], i["beta"], o["Y"], o["mean"], o["rstd"], G,
                               1e-5)
    mn.mn_groupnorm_backward_ex(i["X"], i["gamma"], o["mean"], o["rstd"], i["dY"], o["dX"],
                                o["dgamma"], o["dbeta"], G, o["ws"])
    verify(outs, ins, before, what)


# Channels-last GroupNorm (X [N, L, C]): 16-byte chunks with several rows
# per pass and with two channel blocks, the element-wise path (C not a
# multiple of 8, and unaligned tensors), G = C, one position
GNL_SHAPES = [(2, 320, 1000, 32, 0), (1, 2560, 40, 32, 0), (2, 300, 50, 10, 0),
              (2, 64, 256, 8, 1), (2, 16, 128, 16, 0), (3, 8, 1, 1, 0)]


@pytest.mark.parametrize("N,C,L,G,off", GNL_SHAPES)
def test_groupnorm_nlc_guards(N, C, L, G, off):
    what = f"groupnorm nlc {N}x{L}x{C} G={G}+{off}"
    d = workloads.random_case("gn", N, C * L, 90 + L, x_loc=0.5, channels=C, groups=G)
    d["X"] = np.ascontiguousarray(d["X"].reshape(N, C, L).swapaxes(1, 2))
    d["dY"] = np.ascontiguousarray(d["dY"].reshape(N, C, L).swapaxes(1, 2))
    ins = {k: upload(v, off) for k, v in d.items()}
    outs = {"Y": Guarded((N, L, C), torch.float16, off),
            "dX": Guarded((N, L, C), torch.float16, off),
            "mean": Guarded((N, G), torch.float32), "rstd": Guarded((N, G), torch.float32),
            "dgamma": Guarded((C,), torch.float32), "dbeta": Guarded((C,), torch.float32),
            "ws": workspace(mn.groupnorm_nlc_workspace_bytes(N, L, C, G))}
    before = snapshot(ins)
    o = {k: v.t for k, v in outs.items()}
    i = {k: v.t for k, v in ins.items()}
    mn.mn_groupnorm_nlc_forward_ex(i["X"], i["gamma"], i["beta"], o["Y"], o["mean"], o["rstd"],
                                   G, 1e-5, o["ws"])
    mn.mn_groupnorm_nlc_backward_ex(i["X"], i["gamma"], o["mean"], o["rstd"], i["dY"], o["dX"],
                                    o["dgamma"], o["dbeta"], G, o["ws"])
    verify(outs, ins, before, what)


@pytest.mark.parametrize("M,K,N,off", [(4, 4096, 12288, 0), (3, 1000, 1032, 0), (1, 4096, 14336, 0),
                                       (8, 512, 100, 1), (2, 64, 4099, 0)])
@pytest.mark.parametrize("ln", [False, True])
def test_gemv_guards(M, K, N, off, ln):
    """The GEMV's Y and its workspace; the workspace must also come back with
    its counters at zero, i.e. exactly as zero-filled as it was given."""
    what = f"{'ln' if ln else 'rms'}_gemv {M}x{K}x{N}+{off}"
    d = workloads.random_case("ln_gemv" if ln else "rms_gemv", M, K, 90 + K, Nout=N,
                              x_loc=0.5 if ln else 0.0)
    ins = {k: upload(v, off) for k, v in d.items() if k in ("X", "gamma", "W") or
           (ln and k == "beta")}
    outs = {"Y": Guarded((M, N), torch.float16, off),
            "ws": workspace(mn.norm_gemv_workspace_bytes(M, N, K), fill=0)}
    before = snapshot(ins)
    o = {k: v.t for k, v in outs.items()}
    i = {k: v.t for k, v in ins.items()}
    mn.mn_fused_norm_gemv_ex(i["X"], i["gamma"], i["W"], o["Y"], 1e-5, o["ws"],
                             beta=i.get("beta"))
    verify(outs, ins, before, what)
    # the arrival counters (16,384 words after 64 words of row statistics)
    counters = o["ws"][64:64 + 16384].view(torch.int32).cpu()
    assert (counters == 0).all(), f"{what}: counters not back at zero"
