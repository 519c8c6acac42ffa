"""GroupNorm forward and backward: the HIP path against the fp64 oracle on
every element (tolerances in tests/gpu_gn.py)."""
import numpy as np
import pytest
import torch

import workloads
from gpu_cases import say
from gpu_gn import case, compare, reference, run

pytestmark = pytest.mark.gpu

# (N, C, L, G): the vector path at every lane shape (L = 8 .. 16384), the
# element-wise path (L not a multiple of 8), one to 64 channels per group,
# G = 1 (one slice per sample) and G = C (one channel per slice), and slices
# up to the 65,536-value limit
SHAPES = [
    (2, 4, 8, 2), (3, 6, 64, 3), (4, 64, 256, 32), (2, 320, 1024, 32), (1, 128, 4096, 32),
    (2, 64, 8192, 16), (1, 8, 16384, 4), (2, 1280, 64, 32), (1, 128, 1024, 2),
    (3, 40, 1000, 4), (2, 32, 49, 8), (2, 12, 100, 3), (1, 7, 13, 7), (2, 8, 512, 1),
    (2, 16, 2048, 16), (5, 96, 120, 6), (1, 64, 2048, 2),
    (3, 1, 1, 1), (2, 3, 1, 3), (4, 2, 8, 1),   # one-value slices, L = 1, the smallest vector row
]


@pytest.mark.parametrize("N,C,L,G", SHAPES)
def test_every_element(N, C, L, G):
    say(f"[gn] N={N} C={C} L={L} G={G}")
    d = case(N, C, L, G, 10 + C + L)
    w = compare(run(d, G, 1e-5), reference(d, G, 1e-5), d, G, f"{N}x{C}x{L} G={G}")
    say(f"[gn] {N}x{C}x{L} G={G}: {w}")


TORCH = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


@pytest.mark.parametrize("act,param,dxt", [("bf16", "bf16", "bf16"), ("bf16", "f32", "f32"),
                                           ("f32", "f32", "f32"), ("f16", "f32", "f32"),
                                           ("f32", "f16", "f32")])
@pytest.mark.parametrize("N,C,L,G", [(2, 64, 1024, 32), (2, 30, 100, 5), (1, 32, 4096, 4)])
def test_storage_types(N, C, L, G, act, param, dxt):
    d = case(N, C, L, G, 33, act=act, param=param)
    compare(run(d, G, 1e-5, dx_dtype=TORCH[dxt]), reference(d, G, 1e-5), d, G,
            f"{act}/{param}/{dxt} {N}x{C}x{L}")


@pytest.mark.parametrize("N,C,L,G", [(2, 64, 256, 8), (1, 32, 1024, 4)])
def test_unaligned(N, C, L, G):
    d = case(N, C, L, G, 44)
    compare(run(d, G, 1e-5, offset=1), reference(d, G, 1e-5), d, G, "unaligned")


def test_large_mean():
    d = case(2, 64, 1024, 8, 55, x_loc=20.0)
    compare(run(d, 8, 1e-5), reference(d, 8, 1e-5), d, 8, "mean 20")


def test_deterministic():
    d = case(4, 320, 1024, 32, 66)
    a = run(d, 32, 1e-5)
    b = run(d, 32, 1e-5)
    for k in a:
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k


def test_full_size():
    w = workloads.WORKLOADS["gn_32x320x4096_g32"]
    N, C = w.N, w.channels
    L = w.D // C
    say(f"[gn] full {w.name}: generating")
    d = workloads.generate(w)
    d["X"] = d["X"].reshape(N, C, L)
    d["dY"] = d["dY"].reshape(N, C, L)
    say(f"[gn] full {w.name}: gpu")
    gpu = run(d, w.groups, w.eps)
    say(f"[gn] full {w.name}: oracle")
    r = compare(gpu, reference(d, w.groups, w.eps), d, w.groups, w.name)
    say(f"[gn] full {w.name}: {r}")
