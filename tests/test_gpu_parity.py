"""HIP path versus the fp64 oracle, element by element.

Small workloads and a width/row sweep are compared on every element; the
full-size workloads on a sample of rows (always including the first and last
row) for Y, H, dX and the statistics, and on every column for dgamma/dbeta
(the oracle sums all rows in fp64). The backward is fed the statistics saved
by the GPU forward, as in training.
"""
import numpy as np
import pytest

import workloads
from gpu_cases import compare, reference, run_gpu, say

pytestmark = pytest.mark.gpu

KINDS = ["rms", "ln", "add"]


def _case(kind, N, D, seed):
    return workloads.random_case(kind, N, D, seed, x_loc=0.5 if kind == "ln" else 0.0)


@pytest.mark.parametrize("name", ["rms_17x257", "ln_128x1024"])
def test_small_workload_every_element(name):
    w = workloads.WORKLOADS[name]
    say(f"[parity] {name} N={w.N} D={w.D}")
    d = workloads.generate(w)
    worst = compare(w.kind, run_gpu(w.kind, d, w.eps), reference(w.kind, d, w.eps), name)
    say(f"[parity] {name} worst {worst}")


D_SWEEP = [1, 2, 7, 8, 16, 63, 64, 127, 128, 200, 256, 257, 512, 1000, 1024, 2048, 2056, 3000,
           3072, 4095, 4096, 5000, 5120, 6000, 6144, 8191, 8192]


@pytest.mark.parametrize("D", D_SWEEP)
@pytest.mark.parametrize("kind", KINDS)
def test_width_sweep(kind, D):
    # several tiles and workgroup ranges plus a ragged tail of rows
    N = 1023 if D <= 1024 else 333
    say(f"[parity] sweep {kind} N={N} D={D}")
    d = _case(kind, N, D, seed=1000 + D)
    w = compare(kind, run_gpu(kind, d, 1e-5), reference(kind, d, 1e-5), f"{kind} {N}x{D}",
                inputs=d)
    say(f"[parity] sweep {kind} N={N} D={D}: {w}")


@pytest.mark.parametrize("N", [1, 2, 3, 5, 31, 513, 1025, 4097])
@pytest.mark.parametrize("kind", KINDS)
def test_row_sweep(kind, N):
    D = 1024 if N > 1000 else 4096
    say(f"[parity] rows {kind} N={N} D={D}")
    d = _case(kind, N, D, seed=2000 + N)
    compare(kind, run_gpu(kind, d, 1e-5), reference(kind, d, 1e-5), f"{kind} {N}x{D}", inputs=d)


@pytest.mark.parametrize("D", [8, 128, 1024, 4096, 8192, 257])
@pytest.mark.parametrize("kind", KINDS)
def test_unaligned_pointers(kind, D):
    # every tensor starts 2 bytes past a 16-byte boundary: element-wise kernels
    N = 129
    say(f"[parity] unaligned {kind} N={N} D={D}")
    d = _case(kind, N, D, seed=3000 + D)
    compare(kind, run_gpu(kind, d, 1e-5, offset=1), reference(kind, d, 1e-5),
            f"{kind} {N}x{D} unaligned", inputs=d)


def test_add_without_residual_cotangent():
    d = _case("add", 300, 1024, seed=4)
    compare("add", run_gpu("add", d, 1e-5, use_dh=False),
            reference("add", d, 1e-5, use_dh=False), "add dH=NULL", inputs=d, use_dh=False)


@pytest.mark.parametrize("eps", [1e-6, 1e-3, 1.0])
def test_epsilon_values(eps):
    for kind in KINDS:
        d = _case(kind, 64, 512, seed=5)
        compare(kind, run_gpu(kind, d, eps), reference(kind, d, eps), f"{kind} eps={eps}",
                inputs=d)


FULL = ["rms_16384x4096", "add_rms_32768x8192", "rms_1048576x128", "ln_16384x4096"]


@pytest.mark.slow
@pytest.mark.parametrize("name", FULL)
def test_full_size_workload(name):
    w = workloads.WORKLOADS[name]
    say(f"[parity] full {name}: generating")
    d = workloads.generate(w)
    say(f"[parity] full {name}: gpu")
    gpu = run_gpu(w.kind, d, w.eps)
    rows = workloads.sample_rows(w.N, 2048)
    say(f"[parity] full {name}: oracle on {len(rows)} rows + all-row parameter gradients")
    ref = reference(w.kind, d, w.eps, rows=rows)
    worst = compare(w.kind, gpu, ref, name, rows=rows)
    say(f"[parity] full {name}: worst {worst}")
