"""The comparison helpers themselves, on the CPU: outputs made by rounding
the oracle's own float64 results to the storage type must pass, and a
planted error (an element a few ulp off, a wrong sign, one H bit) must fail.
"""
import numpy as np
import pytest

import oracle
import parity
import workloads
from gpu_cases import compare, reference


def _fake_gpu(kind, ref, like):
    """What an exact kernel would store: oracle results rounded once."""
    out = {"Y": oracle.round_to(ref["Y"], like), "dX": oracle.round_to(ref["dX"], like),
           "rstd": ref["rstd"].astype(np.float32), "dgamma": ref["dgamma"].astype(np.float32)}
    if kind == "ln":
        out["mean"] = ref["mean"].astype(np.float32)
        out["dbeta"] = ref["dbeta"].astype(np.float32)
    if kind == "add":
        out["H"] = ref["H16"].copy()
    return out


@pytest.mark.parametrize("act", ["f16", "bf16", "f32"])
@pytest.mark.parametrize("kind", ["rms", "ln", "add"])
def test_rounded_oracle_passes_and_planted_errors_fail(kind, act):
    d = workloads.random_case(kind, 9, 40, 3, act=act, param="f32")
    ref = reference(kind, d, 1e-5)
    like = workloads.STORAGE[act]
    gpu = _fake_gpu(kind, ref, like)
    w = compare(kind, gpu, ref, "exact", inputs=d)
    assert w["Y_fp32_admitted"] == 0 and w["dX_fp32_admitted"] == 0

    bad = {k: v.copy() for k, v in gpu.items()}
    bad["dX"] = oracle.round_to(-ref["dX"], like)            # a sign error
    with pytest.raises(AssertionError):
        compare(kind, bad, ref, "sign", inputs=d)

    bad = {k: v.copy() for k, v in gpu.items()}
    y = parity.as_f64(gpu["Y"])
    i = int(np.argmax(np.abs(y)))
    step = 8.0 * 2.0 ** -24 * 64 if act == "f32" else 3.0 * 2.0 ** -7
    y.flat[i] *= 1.0 + step                                   # beyond the bound
    bad["Y"] = oracle.round_to(y, like)
    with pytest.raises(AssertionError):
        compare(kind, bad, ref, "one element", inputs=d)

    if kind == "add":
        bad = {k: v.copy() for k, v in gpu.items()}
        bits = bad["H"].view(np.uint32 if act == "f32" else np.uint16)
        bits.flat[5] ^= 1
        with pytest.raises(AssertionError):
            compare(kind, bad, ref, "H bit", inputs=d)


def test_bf16_ulp_definition():
    one = oracle.f64_to_bf16(np.array([1.0, 3.0, 2.0 ** -126, 2.0 ** -130, 0.0]))
    u = parity.ulp_of(parity.as_f64(one), "bf16")
    assert list(u) == [2.0 ** -7, 2.0 ** -6, 2.0 ** -133, 2.0 ** -133, 2.0 ** -133]
    assert parity.ulp_of(np.array([1.0]), "f16")[0] == 2.0 ** -10
