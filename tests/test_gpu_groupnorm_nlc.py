"""Channels-last GroupNorm (X [N, L, C]) forward and backward: the HIP path
against the fp64 oracle on every element (transposed to the oracle's
channels-first layout; tolerances in tests/gpu_gn.py)."""
import numpy as np
import pytest
import torch

import workloads
from gpu_cases import say
from gpu_gn import case, compare, reference
from gpu_gnl import run

pytestmark = pytest.mark.gpu

# (N, C, L, G): 16-byte chunks with one to several rows per pass (C = 8 to
# 2048 channels), more than 256 chunks per position (two channel blocks),
# the element-wise path (C not a multiple of 8, one and two channel blocks),
# G = 1 and G = C (chunks spanning several groups), one position, one
# channel, positions not a multiple of the rows per pass, and enough
# samples that each takes one position chunk
SHAPES = [
    (2, 64, 256, 8), (3, 320, 1000, 32), (2, 8, 64, 1), (2, 2048, 33, 32), (1, 2560, 40, 32),
    (2, 12, 100, 3), (2, 300, 50, 10), (1, 520, 70, 4), (2, 16, 128, 16), (3, 1, 17, 1),
    (2, 7, 1, 7), (1, 32, 16384, 4), (4, 96, 999, 6), (3000, 16, 9, 4), (1, 8, 1, 1),
]


@pytest.mark.parametrize("N,C,L,G", SHAPES)
def test_every_element(N, C, L, G):
    say(f"[gn nlc] N={N} C={C} L={L} G={G}")
    d = case(N, C, L, G, 80 + C + L)
    w = compare(run(d, G, 1e-5), reference(d, G, 1e-5), d, G, f"nlc {N}x{C}x{L} G={G}")
    say(f"[gn nlc] {N}x{C}x{L} G={G}: {w}")


TORCH = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


@pytest.mark.parametrize("act,param,dxt", [("bf16", "bf16", "bf16"), ("bf16", "f32", "f32"),
                                           ("f32", "f32", "f32"), ("f16", "f32", "f32"),
                                           ("f32", "f16", "f32")])
@pytest.mark.parametrize("N,C,L,G", [(2, 64, 1024, 32), (2, 30, 100, 5), (1, 320, 256, 32)])
def test_storage_types(N, C, L, G, act, param, dxt):
    d = case(N, C, L, G, 83, act=act, param=param)
    compare(run(d, G, 1e-5, dx_dtype=TORCH[dxt]), reference(d, G, 1e-5), d, G,
            f"nlc {act}/{param}/{dxt} {N}x{C}x{L}")


@pytest.mark.parametrize("N,C,L,G", [(2, 64, 256, 8), (1, 320, 300, 32)])
def test_unaligned(N, C, L, G):
    d = case(N, C, L, G, 84)
    compare(run(d, G, 1e-5, offset=1), reference(d, G, 1e-5), d, G, "nlc unaligned")


@pytest.mark.parametrize("N,C,L,G", [(2, 64, 1024, 8), (1, 320, 4096, 32)])
def test_large_mean(N, C, L, G):
    d = case(N, C, L, G, 85, x_loc=20.0)
    compare(run(d, G, 1e-5), reference(d, G, 1e-5), d, G, "nlc mean 20")


@pytest.mark.parametrize("N,C,L,G", [(4, 320, 1024, 32), (2, 300, 77, 10)])
def test_deterministic_any_workspace(N, C, L, G):
    """Bitwise the same on a rerun, whatever the workspace held before."""
    d = case(N, C, L, G, 86)
    a = run(d, G, 1e-5, ws_fill=0)
    b = run(d, G, 1e-5, ws_fill=-1)
    for k in a:
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k


def test_full_size():
    """The GroupNorm benchmark shape (32 images, 320 channels, 64 x 64
    positions, 32 groups) in the channels-last layout, every element."""
    w = workloads.WORKLOADS["gn_32x320x4096_g32"]
    N, C = w.N, w.channels
    L = w.D // C
    say(f"[gn nlc] full {w.name}: generating")
    d = workloads.generate(w)
    d["X"] = d["X"].reshape(N, C, L)
    d["dY"] = d["dY"].reshape(N, C, L)
    say(f"[gn nlc] full {w.name}: gpu")
    gpu = run(d, w.groups, w.eps)
    say(f"[gn nlc] full {w.name}: oracle")
    r = compare(gpu, reference(d, w.groups, w.eps), d, w.groups, f"nlc {w.name}")
    say(f"[gn nlc] full {w.name}: {r}")
