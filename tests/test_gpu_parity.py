"""HIP path versus the fp64 oracle, element by element.

Every output element of every case is compared, the full-size workloads
included (the oracle runs there on blocks of rows, see every_row.py); the
parameter gradients on every column, the oracle summing all rows in fp64.
The backward is fed the statistics saved by the GPU forward, as in training.

The named workloads are held to 2 ulp on every element with no allowance.
The sweeps may admit an element whose exact value is a cancellation of much
larger fp32 terms (parity.check_out); how many were admitted is printed for
every case and bounded by parity.allowance_bound: from 16 columns on none
may be, since the row sums c1, c2 are then means of many independent terms,
so a dX near zero needs a small g = dY*gamma and the fp32 terms are as small
as the result.
"""
import numpy as np
import pytest

import workloads
import every_row
import parity
import record
from gpu_cases import compare, compare_every_row, reference, run_gpu, say

pytestmark = pytest.mark.gpu

KINDS = ["rms", "ln", "add"]


def _case(kind, N, D, seed):
    return workloads.random_case(kind, N, D, seed, x_loc=0.5 if kind == "ln" else 0.0)


def admitted(w):
    return int(w.get("Y_fp32_admitted", 0)) + int(w.get("dX_fp32_admitted", 0))


def check_admitted(w, N, D, what, storage="f16"):
    """Record and print the admitted count and hold it to
    parity.allowance_bound (zero for fp16 from 16 columns on)."""
    n = admitted(w)
    say(f"[parity] {what}: admitted {n} (Y {w.get('Y_fp32_admitted', 0)}, "
        f"dX {w.get('dX_fp32_admitted', 0)})")
    record.admitted(what, n, 2 * N * D)
    bound = parity.allowance_bound(D, storage) * 2 * N * D
    assert n <= bound, f"{what}: {n} elements needed the fp32 cancellation allowance"


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
    check_admitted(w, N, D, f"sweep {kind} {N}x{D}")


@pytest.mark.parametrize("N", [1, 2, 3, 5, 31, 513, 1025, 4097])
@pytest.mark.parametrize("kind", KINDS)
def test_row_sweep(kind, N):
    D = 1024 if N > 1000 else 4096
    say(f"[parity] rows {kind} N={N} D={D}")
    d = _case(kind, N, D, seed=2000 + N)
    w = compare(kind, run_gpu(kind, d, 1e-5), reference(kind, d, 1e-5), f"{kind} {N}x{D}",
                inputs=d)
    check_admitted(w, N, D, f"rows {kind} {N}x{D}")


@pytest.mark.parametrize("D", [8, 128, 1024, 4096, 8192, 257])
@pytest.mark.parametrize("kind", KINDS)
def test_unaligned_pointers(kind, D):
    # every tensor starts 2 bytes past a 16-byte boundary: element-wise kernels
    N = 129
    say(f"[parity] unaligned {kind} N={N} D={D}")
    d = _case(kind, N, D, seed=3000 + D)
    w = compare(kind, run_gpu(kind, d, 1e-5, offset=1), reference(kind, d, 1e-5),
                f"{kind} {N}x{D} unaligned", inputs=d)
    check_admitted(w, N, D, f"unaligned {kind} {N}x{D}")


def test_add_without_residual_cotangent():
    d = _case("add", 300, 1024, seed=4)
    w = compare("add", run_gpu("add", d, 1e-5, use_dh=False),
                reference("add", d, 1e-5, use_dh=False), "add dH=NULL", inputs=d, use_dh=False)
    check_admitted(w, 300, 1024, "add dH=NULL 300x1024")


@pytest.mark.parametrize("eps", [1e-6, 1e-3, 1.0])
def test_epsilon_values(eps):
    for kind in KINDS:
        d = _case(kind, 64, 512, seed=5)
        w = compare(kind, run_gpu(kind, d, eps), reference(kind, d, eps), f"{kind} eps={eps}",
                    inputs=d)
        check_admitted(w, 64, 512, f"{kind} 64x512 eps={eps}")


FULL = ["rms_16384x4096", "add_rms_32768x8192", "rms_1048576x128", "ln_16384x4096"]


@pytest.mark.slow
@pytest.mark.parametrize("name", FULL)
def test_full_size_workload(name):
    """Every row of the full-size workload, in the launch configuration the
    benchmark times, at the strict 2-ulp bar."""
    w = workloads.WORKLOADS[name]
    say(f"[parity] full {name}: generating")
    d = workloads.generate(w)
    say(f"[parity] full {name}: gpu")
    gpu = run_gpu(w.kind, d, w.eps)
    say(f"[parity] full {name}: oracle on every row, {every_row.THREADS} threads")
    r = compare_every_row(w.kind, gpu, d, w.eps, name)
    msg = (f"full {name}: rows checked = {r['rows_checked']} of {w.N}, "
           f"admitted = {admitted(r)}, worst Y {r['Y_ulp']:.0f} ulp, dX {r['dX_ulp']:.0f} ulp")
    say(f"[parity] {msg}; {r}")
    record.line(msg)
    assert r["rows_checked"] == w.N
    assert admitted(r) == 0
