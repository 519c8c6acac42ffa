"""GroupNorm forward and backward: the HIP path against the fp64 oracle on
every element (tolerances in tests/gpu_gn.py)."""
import numpy as np
import pytest
import torch

import workloads
from gpu_cases import say
from gpu_gn import case, compare, reference, run

pytestmark = pytest.mark.gpu

# (N, C, L, G): the register path at every lane shape (L = 8 .. 16384), the
# element-wise path (L not a multiple of 8), one to 64 channels per group,
# G = 1 (one slice per sample) and G = C (one channel per slice), slices up
# to 65,536 values, and more slices than workgroups (each persistent
# workgroup takes several in turn, the last round ragged)
SHAPES = [
    (2, 4, 8, 2), (3, 6, 64, 3), (4, 64, 256, 32), (2, 320, 1024, 32), (1, 128, 4096, 32),
    (2, 64, 8192, 16), (1, 8, 16384, 4), (2, 1280, 64, 32), (1, 128, 1024, 2),
    (3, 40, 1000, 4), (2, 32, 49, 8), (2, 12, 100, 3), (1, 7, 13, 7), (2, 8, 512, 1),
    (2, 16, 2048, 16), (5, 96, 120, 6), (1, 64, 2048, 2),
    (3, 1, 1, 1), (2, 3, 1, 3), (4, 2, 8, 1),   # one-value slices, L = 1, the smallest vector row
    (300, 64, 1024, 32), (40, 320, 4096, 32), (5000, 8, 100, 2),
]

# Slices larger than one workgroup holds (the split path): 16-byte chunks
# with one and with several units per channel row, the element-wise path
# with several units per row and with many short rows, G = 1, and a
# 32 x 320 x 128 x 128 (G = 32) shape beside the benchmark one
SPLIT_SHAPES = [
    (2, 320, 16384, 32), (1, 128, 65536, 32), (2, 16, 20001, 2), (1, 2048, 9, 1),
    (3, 64, 3000, 1), (2, 40, 16384, 4), (1, 20000, 5, 2),
]


@pytest.mark.parametrize("N,C,L,G", SHAPES)
def test_every_element(N, C, L, G):
    say(f"[gn] N={N} C={C} L={L} G={G}")
    d = case(N, C, L, G, 10 + C + L)
    w = compare(run(d, G, 1e-5), reference(d, G, 1e-5), d, G, f"{N}x{C}x{L} G={G}")
    say(f"[gn] {N}x{C}x{L} G={G}: {w}")


@pytest.mark.parametrize("N,C,L,G", SPLIT_SHAPES)
def test_split_every_element(N, C, L, G):
    say(f"[gn] split N={N} C={C} L={L} G={G}")
    d = case(N, C, L, G, 20 + C + L)
    w = compare(run(d, G, 1e-5), reference(d, G, 1e-5), d, G, f"split {N}x{C}x{L} G={G}")
    say(f"[gn] split {N}x{C}x{L} G={G}: {w}")


TORCH = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


@pytest.mark.parametrize("act,param,dxt", [("bf16", "bf16", "bf16"), ("bf16", "f32", "f32"),
                                           ("f32", "f32", "f32"), ("f16", "f32", "f32"),
                                           ("f32", "f16", "f32")])
@pytest.mark.parametrize("N,C,L,G", [(2, 64, 1024, 32), (2, 30, 100, 5), (1, 32, 4096, 4),
                                     (1, 32, 16384, 4), (2, 8, 20001, 2)])
def test_storage_types(N, C, L, G, act, param, dxt):
    d = case(N, C, L, G, 33, act=act, param=param)
    compare(run(d, G, 1e-5, dx_dtype=TORCH[dxt]), reference(d, G, 1e-5), d, G,
            f"{act}/{param}/{dxt} {N}x{C}x{L}")


@pytest.mark.parametrize("N,C,L,G", [(2, 64, 256, 8), (1, 32, 1024, 4), (2, 32, 16384, 2)])
def test_unaligned(N, C, L, G):
    d = case(N, C, L, G, 44)
    compare(run(d, G, 1e-5, offset=1), reference(d, G, 1e-5), d, G, "unaligned")


@pytest.mark.parametrize("N,C,L,G", [(2, 64, 1024, 8), (1, 64, 16384, 4)])
def test_large_mean(N, C, L, G):
    d = case(N, C, L, G, 55, x_loc=20.0)
    compare(run(d, G, 1e-5), reference(d, G, 1e-5), d, G, "mean 20")


@pytest.mark.parametrize("N,C,L,G", [(4, 320, 1024, 32), (2, 320, 16384, 32)])
def test_deterministic(N, C, L, G):
    d = case(N, C, L, G, 66)
    a = run(d, G, 1e-5)
    b = run(d, G, 1e-5)
    for k in a:
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k


@pytest.mark.slow
def test_split_full_size():
    """32 images of 320 channels at 128 x 128 positions in 32 groups: slices
    of 163,840 values, every element."""
    N, C, L, G = 32, 320, 16384, 32
    say(f"[gn] split full {N}x{C}x{L} G={G}: generating")
    d = case(N, C, L, G, 77)
    say("[gn] split full: gpu")
    gpu = run(d, G, 1e-5)
    say("[gn] split full: oracle")
    r = compare(gpu, reference(d, G, 1e-5), d, G, "split full")
    say(f"[gn] split full {N}x{C}x{L} G={G}: {r}")


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
