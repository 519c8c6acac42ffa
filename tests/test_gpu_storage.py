"""bfloat16 and float32 storage through the typed (``_ex``) entry points,
versus the fp64 oracle fed the same stored values.

The activations X, R and forward outputs Y, H take one storage type, gamma
and beta another (every pairing of fp16, bf16 and float32 is run), the
cotangents dY, dH a third and dX a fourth (every backward combination the
library provides is run). The arithmetic is fp32 in every case, so only the
rounding of the stored outputs differs: bf16 outputs are held to 2 bf16 ulp,
float32 outputs to the fp32 evaluation bound (parity.check_out), and a
stored H must equal round(x + r) in its own type.
"""
import itertools

import numpy as np
import pytest
import torch

import parity
import record
import workloads
from gpu_cases import compare_every_row, compare, reference, run_gpu, say

pytestmark = pytest.mark.gpu

KINDS = ["rms", "ln", "add"]
STORAGE = ["f16", "bf16", "f32"]
PAIRS = list(itertools.product(STORAGE, STORAGE))


def _case(kind, N, D, seed, act, param, cot=None):
    return workloads.random_case(kind, N, D, seed, x_loc=0.5 if kind == "ln" else 0.0,
                                 act=act, param=param, cot=cot)


TORCH = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}


def _admitted(w, N, D, act, what):
    """Record the elements the fp32 cancellation allowance admitted and hold
    them to parity.allowance_bound (binary32 outputs take no allowance)."""
    n = w["Y_fp32_admitted"] + w["dX_fp32_admitted"]
    record.admitted(what, n, 2 * N * D)
    if act != "f32":
        assert n <= parity.allowance_bound(D, act) * 2 * N * D, f"{what}: {n} admitted"

# backward storage combinations (act, cot, dX) the library provides
BWD_TYPES = ([(a, c, o) for a in ("f16", "bf16") for c in (a, "f32") for o in (a, "f32")] +
             [("f32", c, "f32") for c in ("f16", "bf16", "f32")])


@pytest.mark.parametrize("D", [257, 1024, 4096, 8192])
@pytest.mark.parametrize("act,param", PAIRS)
@pytest.mark.parametrize("kind", KINDS)
def test_storage_pairs(kind, act, param, D):
    N = 300
    say(f"[storage] {kind} act={act} param={param} N={N} D={D}")
    d = _case(kind, N, D, 7000 + D, act, param)
    w = compare(kind, run_gpu(kind, d, 1e-5), reference(kind, d, 1e-5),
                f"{kind} {act}/{param} {N}x{D}", inputs=d)
    say(f"[storage] {kind} act={act} param={param} D={D}: {w}")


D_SWEEP = [1, 2, 3, 4, 7, 8, 63, 64, 127, 128, 200, 256, 260, 1000, 2048, 2056, 3000, 3072,
           4095, 5120, 6000, 6144, 8191]


@pytest.mark.parametrize("D", D_SWEEP)
@pytest.mark.parametrize("act", ["bf16", "f32"])
@pytest.mark.parametrize("kind", KINDS)
def test_storage_width_sweep(kind, act, D):
    # several tiles and workgroup ranges plus a ragged tail of rows
    N = 1023 if D <= 1024 else 333
    say(f"[storage] sweep {kind} {act} N={N} D={D}")
    d = _case(kind, N, D, 8000 + D, act, act)
    w = compare(kind, run_gpu(kind, d, 1e-5), reference(kind, d, 1e-5),
                f"{kind} {act} {N}x{D}", inputs=d)
    _admitted(w, N, D, act, f"storage sweep {kind} {act} {N}x{D}")


@pytest.mark.parametrize("D", [8, 128, 1024, 4096, 257])
@pytest.mark.parametrize("act", ["bf16", "f32"])
@pytest.mark.parametrize("kind", KINDS)
def test_storage_unaligned(kind, act, D):
    # every tensor starts one element past a 16-byte boundary: element-wise kernels
    N = 129
    say(f"[storage] unaligned {kind} {act} N={N} D={D}")
    d = _case(kind, N, D, 9000 + D, act, act)
    w = compare(kind, run_gpu(kind, d, 1e-5, offset=1), reference(kind, d, 1e-5),
                f"{kind} {act} {N}x{D} unaligned", inputs=d)
    _admitted(w, N, D, act, f"storage unaligned {kind} {act} {N}x{D}")


@pytest.mark.parametrize("D", [1024, 257])
@pytest.mark.parametrize("act,cot,dxt", BWD_TYPES)
@pytest.mark.parametrize("kind", KINDS)
def test_cotangent_and_dx_types(kind, act, cot, dxt, D):
    N = 300
    say(f"[storage] {kind} act={act} cot={cot} dX={dxt} N={N} D={D}")
    d = _case(kind, N, D, 10000 + D, act, "f32", cot)
    gpu = run_gpu(kind, d, 1e-5, dx_dtype=TORCH[dxt])
    assert gpu["dX"].dtype == workloads.STORAGE[dxt]
    w = compare(kind, gpu, reference(kind, d, 1e-5), f"{kind} {act}/{cot}/{dxt} {N}x{D}",
                inputs=d)
    say(f"[storage] {kind} act={act} cot={cot} dX={dxt} D={D}: {w}")


@pytest.mark.parametrize("kind", KINDS)
def test_float32_dx_is_the_unrounded_16bit_dx(kind):
    """A float32 dX rounded to fp16 (nearest, ties to even) equals the fp16
    dX of the same call: both are the same fp32 value, stored once as is and
    once rounded."""
    d = _case(kind, 200, 4096, 13, "f16", "f16")
    a = run_gpu(kind, d, 1e-5)
    b = run_gpu(kind, d, 1e-5, dx_dtype=torch.float32)
    assert np.array_equal(b["dX"].astype(np.float16), a["dX"])
    for k in ("Y", "rstd", "dgamma"):
        assert np.array_equal(a[k], b[k]), k


@pytest.mark.parametrize("kind", KINDS)
def test_typed_entry_points_match_fp16_ones(kind):
    """With fp16 for both types the ``_ex`` entry points run the fp16 path."""
    d = _case(kind, 500, 4096, 11, "f16", "f16")
    a = run_gpu(kind, d, 1e-5, typed=False)
    b = run_gpu(kind, d, 1e-5, typed=True)
    for k in a:
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k


@pytest.mark.parametrize("act", ["bf16", "f32"])
def test_add_without_residual_cotangent_storage(act):
    d = _case("add", 300, 1024, 12, act, "f32")
    compare("add", run_gpu("add", d, 1e-5, use_dh=False),
            reference("add", d, 1e-5, use_dh=False), f"add {act} dH=NULL", inputs=d,
            use_dh=False)


# Full-size shapes: bf16 activations with float32 parameters (the usual
# mixed-precision training layout), float32 throughout, and fp16 storage
# with float32 gradients (dX and the cotangents in float32 as well).
FULL = [("rms_16384x4096", "bf16", "f32", "bf16", "bf16"),
        ("add_rms_32768x8192", "bf16", "f32", "bf16", "bf16"),
        ("rms_1048576x128", "bf16", "bf16", "bf16", "bf16"),
        ("ln_16384x4096", "bf16", "f32", "bf16", "bf16"),
        ("rms_16384x4096", "f32", "f32", "f32", "f32"),
        ("ln_16384x4096", "f32", "f32", "f32", "f32"),
        ("rms_16384x4096", "f16", "f16", "f16", "f32"),
        ("ln_16384x4096", "f16", "f16", "f32", "f32")]


@pytest.mark.slow
@pytest.mark.parametrize("name,act,param,cot,dxt", FULL)
def test_full_size_storage(name, act, param, cot, dxt):
    w = workloads.WORKLOADS[name]
    tag = f"{name} {act}/{param}/{cot}/{dxt}"
    say(f"[storage] full {tag}: generating")
    d = workloads.generate(w, act=act, param=param, cot=cot)
    say(f"[storage] full {tag}: gpu")
    gpu = run_gpu(w.kind, d, w.eps, dx_dtype=TORCH[dxt])
    say(f"[storage] full {tag}: oracle on every row")
    # bfloat16 keeps full relative precision down to 2^-126, so an output that
    # is a deep cancellation of fp32 terms (dX near zero, LayerNorm y where
    # gamma*xhat ~ -beta) can sit a few bf16 ulp off; those elements take the
    # fp32 allowance, every other one the 2 ulp bound (binary32 outputs are
    # held to the fp32 bound on every element)
    r = compare_every_row(w.kind, gpu, d, w.eps, tag, inputs=d)
    n = r.get('Y_fp32_admitted', 0) + r.get('dX_fp32_admitted', 0)
    msg = f"full {tag}: rows checked = {r['rows_checked']} of {w.N}, admitted = {n}"
    say(f"[storage] {msg}; worst {r}")
    record.line(msg)
    assert r["rows_checked"] == w.N
    assert n <= parity.allowance_bound(w.D, act) * 2 * w.N * w.D
