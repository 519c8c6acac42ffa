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


def test_row_blocks_cover_every_row_once():
    import every_row
    for N, D, align in [(1, 1, 1), (17, 257, 1), (32768, 8192, 1), (1048576, 128, 1),
                        (16384, 3072, 2048), (5, 1 << 23, 1)]:
        bs = every_row.blocks(N, D, align)
        assert bs[0][0] == 0 and bs[-1][1] == N
        assert all(a[1] == b[0] for a, b in zip(bs, bs[1:]))
        assert all(hi > lo for lo, hi in bs)
        assert all((hi - lo) % align == 0 for lo, hi in bs[:-1])


@pytest.mark.parametrize("kind", ["rms", "ln", "add"])
def test_every_row_check_catches_one_bad_row(kind, monkeypatch):
    """The block-wise full-size check passes an exact result and fails when
    one element of one late row is 3 ulp off (small blocks, so the planted
    row is in neither the first nor the last block)."""
    import every_row
    from gpu_cases import compare_every_row
    monkeypatch.setattr(every_row, "BLOCK_ELEMS", 64 * 40)
    d = workloads.random_case(kind, 700, 40, 4, x_loc=0.5 if kind == "ln" else 0.0)
    ref = reference(kind, d, 1e-5)
    gpu = _fake_gpu(kind, ref, np.float16)
    w = compare_every_row(kind, gpu, d, 1e-5, "exact")
    assert w["rows_checked"] == 700
    assert w["Y_fp32_admitted"] == 0 and w["dX_fp32_admitted"] == 0
    bad = {k: v.copy() for k, v in gpu.items()}
    y = ref["dX"].copy()
    y[413, 7] *= 1.0 + 3.0 * 2.0 ** -10
    bad["dX"] = oracle.round_to(y, np.float16)
    with pytest.raises(AssertionError, match="dX"):
        compare_every_row(kind, bad, d, 1e-5, "planted")


def test_every_row_check_other_norms(monkeypatch):
    """The same for Modulated RMSNorm, whose blocks must not straddle two
    samples, and for PolyNorm."""
    import every_row
    import gpu_other
    monkeypatch.setattr(every_row, "BLOCK_ELEMS", 32 * 48)
    for kind, kw in (("mod", {"B": 6}), ("poly", {}), ("dyt", {})):
        d = workloads.random_case(kind, 6 * 50, 48, 5, **kw)
        ref = gpu_other.reference(kind, d, 1e-5)
        gpu = {"Y": oracle.round_to(ref["Y"], np.float16),
               "dX": oracle.round_to(ref["dX"], np.float16)}
        for k in ("rstd", "dgamma", "dbeta", "dscale", "dshift", "dalpha", "dparams"):
            if k in ref:
                gpu[k] = ref[k].astype(np.float32)
        w = gpu_other.compare_every_row(kind, gpu, d, 1e-5, kind)
        assert w["rows_checked"] == 300
        bad = dict(gpu)
        y = ref["Y"].copy()
        y[251, 3] += 4.0 * parity.ulp_of(oracle.round_to(y[251:252, 3:4], np.float16), "f16")[0, 0]
        bad["Y"] = oracle.round_to(y, np.float16)
        with pytest.raises(AssertionError, match="Y"):
            gpu_other.compare_every_row(kind, bad, d, 1e-5, kind)
