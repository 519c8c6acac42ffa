"""Dynamic Tanh, PolyNorm and Modulated RMSNorm: HIP path versus the fp64
oracle, element by element (tolerances in tests/gpu_other.py)."""
import numpy as np
import pytest
import torch

import parity
import record
import workloads
from gpu_cases import say
from gpu_other import compare, compare_every_row, reference, run

pytestmark = pytest.mark.gpu

KINDS = ["dyt", "poly", "mod"]
TORCH = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def _case(kind, N, D, seed, act="f16", param=None, B=None):
    if kind == "mod":
        B = B or (4 if N % 4 == 0 else 1)
        return workloads.random_case("mod", N, D, seed, act=act, param=param, B=B)
    return workloads.random_case(kind, N, D, seed, act=act, param=param)


@pytest.mark.parametrize("N,D", [(17, 257), (128, 1024), (64, 4096)])
@pytest.mark.parametrize("kind", KINDS)
def test_small_every_element(kind, N, D):
    say(f"[other] {kind} N={N} D={D}")
    d = _case(kind, N, D, 100 + D)
    w = compare(kind, run(kind, d, 1e-5), reference(kind, d, 1e-5), d, f"{kind} {N}x{D}")
    say(f"[other] {kind} {N}x{D}: {w}")


D_SWEEP = [1, 2, 7, 8, 64, 127, 128, 256, 1000, 1024, 2048, 2056, 3072, 4095, 4096, 5120, 6000,
           6144, 8191, 8192]


@pytest.mark.parametrize("D", D_SWEEP)
@pytest.mark.parametrize("kind", KINDS)
def test_width_sweep(kind, D):
    N = 1020 if D <= 1024 else 332      # several tiles and a ragged tail
    say(f"[other] sweep {kind} N={N} D={D}")
    d = _case(kind, N, D, 200 + D)
    w = compare(kind, run(kind, d, 1e-5), reference(kind, d, 1e-5), d, f"{kind} {N}x{D}")
    n = w["Y_admitted"] + w["dX_admitted"]
    record.admitted(f"other sweep {kind} {N}x{D}", n, 2 * N * D)
    assert n <= parity.allowance_bound(D, "f16") * 2 * N * D, f"{kind} {N}x{D}: {n} admitted"


@pytest.mark.parametrize("act,dxt", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32"),
                                     ("f16", "f32")])
@pytest.mark.parametrize("D", [1024, 4096, 257])
@pytest.mark.parametrize("kind", KINDS)
def test_storage_types(kind, D, act, dxt):
    N = 300
    say(f"[other] {kind} {act}/{dxt} N={N} D={D}")
    d = _case(kind, N, D, 300 + D, act=act, param="f32")
    compare(kind, run(kind, d, 1e-5, dx_dtype=TORCH[dxt]), reference(kind, d, 1e-5), d,
            f"{kind} {act}/{dxt} {N}x{D}")


@pytest.mark.parametrize("D", [8, 1024, 4096, 257])
@pytest.mark.parametrize("kind", KINDS)
def test_unaligned(kind, D):
    N = 132
    d = _case(kind, N, D, 400 + D)
    compare(kind, run(kind, d, 1e-5, offset=1), reference(kind, d, 1e-5), d,
            f"{kind} {N}x{D} unaligned")


@pytest.mark.parametrize("B,N", [(1, 300), (3, 300), (300, 300), (7, 7 * 129), (64, 64 * 16)])
def test_mod_samples(B, N):
    """One sample, a few, one row per sample, and more samples than tiles."""
    D = 1024
    say(f"[other] mod B={B} N={N}")
    d = workloads.random_case("mod", N, D, 500 + B, B=B)
    compare("mod", run("mod", d, 1e-5), reference("mod", d, 1e-5), d, f"mod B={B} N={N}")


def test_mod_ragged_samples_at_benchmark_width():
    """Samples of 101 rows at 3072 columns: tiles are laid out per sample, so
    every sample ends in a part-filled tile."""
    d = workloads.random_case("mod", 6 * 101, 3072, 510, B=6)
    compare("mod", run("mod", d, 1e-5), reference("mod", d, 1e-5), d, "mod B=6 N=606 D=3072")


@pytest.mark.parametrize("x_scale", [1e-3, 0.02])
def test_dyt_small_arguments(x_scale):
    """alpha * x around and below the 1/128 switch of the kernel's tanh, with
    beta = 0 so that every output is as small as tanh itself: relative
    accuracy on both sides of the switch."""
    d = workloads.random_case("dyt", 256, 1024, 520, x_scale=x_scale)
    d["beta"][:] = 0
    compare("dyt", run("dyt", d, 1e-5), reference("dyt", d, 1e-5), d, f"dyt x~{x_scale}")


def test_mod_without_modulation_is_rmsnorm():
    """scale = shift = 0 gives the RMSNorm outputs of the training-pair path."""
    from gpu_cases import run_gpu
    d = workloads.random_case("mod", 256, 4096, 7, B=4)
    d["scale"][:] = 0
    d["shift"][:] = 0
    a = run("mod", d, 1e-5)
    b = run_gpu("rms", {"X": d["X"], "gamma": d["gamma"], "dY": d["dY"]}, 1e-5)
    assert np.array_equal(a["rstd"], b["rstd"])
    assert (np.abs(a["Y"].astype(np.float64) - b["Y"].astype(np.float64)) <=
            np.abs(b["Y"].astype(np.float64)) * 2 ** -10 + 2 ** -24).all()


@pytest.mark.parametrize("kind", KINDS)
def test_deterministic(kind):
    d = _case(kind, 1000, 4096, 9)
    a = run(kind, d, 1e-5)
    b = run(kind, d, 1e-5)
    for k in a:
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k


FULL = ["dyt_16384x4096", "poly_16384x4096", "mod_rms_16384x3072"]


@pytest.mark.slow
@pytest.mark.parametrize("name", FULL)
def test_full_size(name):
    """Every row of the full-size workload."""
    w = workloads.WORKLOADS[name]
    say(f"[other] full {name}: generating")
    d = workloads.generate(w)
    say(f"[other] full {name}: gpu")
    gpu = run(w.kind, d, w.eps)
    say(f"[other] full {name}: oracle on every row")
    r = compare_every_row(w.kind, gpu, d, w.eps, name)
    n = r.get('Y_admitted', 0) + r.get('dX_admitted', 0)
    msg = f"full {name}: rows checked = {r['rows_checked']} of {w.N}, admitted = {n}"
    say(f"[other] {msg}; worst {r}")
    record.line(msg)
    assert r["rows_checked"] == w.N
    assert n == 0
