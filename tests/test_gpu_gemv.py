"""Fused RMSNorm / LayerNorm + GEMV ([tensorcore] "Fused Norm + GEMV"): the
HIP path against the fp64 oracle on every output element (tolerances in
tests/gpu_gemv.py)."""
import numpy as np
import pytest
import torch

import parity
import workloads
import row_wise_normalization_amd as mn
from gpu_cases import dev, say
from gpu_gemv import case as _case, compare, reference, run, workspace

pytestmark = pytest.mark.gpu


# the last two take the wide tiles of one or two X rows (a ragged last tile,
# and K not a multiple of the slice)
SHAPES = [(1, 1, 1), (1, 64, 8), (2, 257, 130), (3, 1000, 1000), (4, 4096, 4096),
          (5, 2048, 520), (8, 1024, 2056), (1, 3000, 7), (4, 300, 4104), (6, 8192, 512),
          (2, 4096, 12296), (1, 5000, 16384)]


@pytest.mark.parametrize("ln", [False, True], ids=["rms", "ln"])
@pytest.mark.parametrize("M,K,N", SHAPES)
def test_every_element(M, K, N, ln):
    say(f"[gemv] {'ln' if ln else 'rms'} M={M} K={K} N={N}")
    d = _case(M, K, N, 10 + M + K, ln)
    w = compare(run(d, 1e-5, ln), reference(d, 1e-5, ln), d, 1e-5, ln, f"{M}x{K}x{N}")
    say(f"[gemv] {M}x{K}x{N}: {w}")


@pytest.mark.parametrize("act,param", [("bf16", "bf16"), ("bf16", "f32"), ("f16", "f32"),
                                       ("f16", "bf16")])
@pytest.mark.parametrize("ln", [False, True], ids=["rms", "ln"])
def test_storage_types(act, param, ln):
    M, K, N = 4, 1024, 1032
    d = _case(M, K, N, 77, ln, act=act, param=param)
    compare(run(d, 1e-5, ln), reference(d, 1e-5, ln), d, 1e-5, ln, f"{act}/{param}")


@pytest.mark.parametrize("ln", [False, True], ids=["rms", "ln"])
def test_unaligned(ln):
    """Operands one element past an aligned address take the element-wise path."""
    M, K, N = 3, 512, 1024
    d = _case(M, K, N, 5, ln)
    compare(run(d, 1e-5, ln, offset=1), reference(d, 1e-5, ln), d, 1e-5, ln, "unaligned")


@pytest.mark.parametrize("ln", [False, True], ids=["rms", "ln"])
@pytest.mark.parametrize("M", [3, 4, 8])
@pytest.mark.parametrize("xs,gs", [(2.0 ** 12, 2.0 ** 4), (2.0 ** -12, 2.0 ** -6)],
                         ids=["large", "small"])
def test_product_row_range(M, ln, xs, gs):
    """X and gamma scaled by powers of two (exact in binary16): products of
    the shifted rows and gamma far above the binary16 range, or deep in its
    subnormals. The normalised result is the same function of the stored
    inputs; the matrix-core tiles (RMSNorm in binary16) rescale each product
    row of a tile by a power of two before splitting it into two binary16
    rows, and the vector-ALU tiles (LayerNorm) keep it in fp32."""
    d = _case(M, 1024, 1040, 31 + M, ln)
    d["X"] = (d["X"].astype(np.float64) * xs).astype(np.float16)
    d["gamma"] = (d["gamma"].astype(np.float64) * gs).astype(np.float16)
    if ln:
        d["beta"] = (d["beta"].astype(np.float64) * gs).astype(np.float16)
    assert np.isfinite(d["X"].astype(np.float64)).all()
    w = compare(run(d, 1e-5, ln), reference(d, 1e-5, ln), d, 1e-5, ln, f"range {xs} {gs}")
    say(f"[gemv] range M={M} xs={xs} gs={gs}: {w}")


def test_large_mean_layernorm():
    """Rows with a mean 20 times their spread: the shifted sums and the
    centred statistics keep the result to the bar."""
    d = _case(4, 4096, 1024, 6, True, x_loc=20.0)
    compare(run(d, 1e-5, True), reference(d, 1e-5, True), d, 1e-5, True, "mean 20")


def test_deterministic_and_row_independent():
    """Bitwise repeatable, and an output row does not depend on the other rows
    of the batch (each row's statistics and sums are its own). Another input
    runs through the shared workspace between the repeats, so a repeat that
    read a stale partial or statistic of its own earlier call could not pass
    by reading the same bits again."""
    d = _case(4, 4096, 2048, 8, False)
    other = _case(4, 4096, 2048, 9, False)
    a = run(d, 1e-5, False)
    b = run(other, 1e-5, False)
    assert not np.array_equal(a.view(np.uint16), b.view(np.uint16))
    assert np.array_equal(a.view(np.uint16), run(d, 1e-5, False).view(np.uint16))
    one = {k: (v[1:2] if k == "X" else v) for k, v in d.items()}
    run(other, 1e-5, False)
    assert np.array_equal(a[1:2].view(np.uint16), run(one, 1e-5, False).view(np.uint16))


@pytest.mark.parametrize("ln", [False, True], ids=["rms", "ln"])
def test_long_rows_few_columns(ln):
    """K = 131072 against one 64-column tile: 256 short K slices finish while
    the statistics workgroup still sums its long row, so the statistics
    workgroup is usually the one that completes the tile and adds its
    partials."""
    M, K, N = 1, 131072, 64
    d = _case(M, K, N, 12, ln)
    compare(run(d, 1e-5, ln), reference(d, 1e-5, ln), d, 1e-5, ln, f"{M}x{K}x{N}")


@pytest.mark.parametrize("M,K,N,ln", [(4, 4096, 12288, False), (4, 4096, 12288, True),
                                     (1, 4096, 14336, False), (8, 1024, 4096, True),
                                     (1, 131072, 64, False)])
def test_repeated_calls_bitwise(M, K, N, ln):
    """400 back-to-back calls through one workspace, two different inputs in
    turn (other X rows, gamma, beta and W): every call gives the bits of the
    first call on its own input. A workgroup that completed a tile from a
    partial or statistic not yet visible would read the other input's value
    left in the workspace by the call before, and differ."""
    sets = []
    for seed in (21, 22):
        d = _case(M, K, N, seed, ln)
        sets.append((dev(d["X"]), dev(d["gamma"]), dev(d["W"]),
                     dev(d["beta"]) if ln else None))
    ws = workspace(M, N, K)
    ys = [torch.empty(M, N, dtype=sets[0][0].dtype, device="cuda") for _ in range(400)]
    for i, y in enumerate(ys):
        X, g, W, b = sets[i % 2]
        mn.mn_fused_norm_gemv_ex(X, g, W, y, 1e-5, ws, beta=b)
    torch.cuda.synchronize()
    first = [ys[0].view(torch.int16), ys[1].view(torch.int16)]
    assert not torch.equal(first[0], first[1])
    bad = [i for i, y in enumerate(ys) if not torch.equal(y.view(torch.int16), first[i % 2])]
    assert not bad, f"{M}x{K}x{N}: calls {bad[:8]} differ from the first call on their input"


def test_counters_back_at_zero():
    """Each call leaves every word of the shared workspace's counter area
    (16384 words after the 64 of statistics) at zero: the block that
    finishes a column tile resets its counter."""
    for M, K, N, ln in ((4, 4096, 12288, False), (3, 1000, 1000, True), (1, 5000, 16384, False)):
        d = _case(M, K, N, 3, ln)
        run(d, 1e-5, ln)
        ws = workspace(M, N, K)[:64 + 16384].view(torch.int32).cpu()
        assert not ws[64:].any(), f"{M}x{K}x{N}: counters left {ws[64:].nonzero().flatten()[:8]}"


def test_matches_separate_norm_then_matmul():
    """The pages validate the fusion against the separate norm forward and a
    GEMM: the same rms_scaled bound against our RMSNorm forward (fp16 rows)
    followed by a float32 matmul."""
    M, K, N = 4, 4096, 4096
    d = _case(M, K, N, 9, False)
    X, g, W = dev(d["X"]), dev(d["gamma"]), dev(d["W"])
    Yn = torch.empty_like(X)
    rstd = torch.empty(M, dtype=torch.float32, device="cuda")
    mn.mn_rmsnorm_forward(X, g, Yn, rstd, 1e-5)
    sep = (Yn.float() @ W.float()).cpu().numpy().astype(np.float64)
    fused = parity.as_f64(run(d, 1e-5, False))
    rms = float(np.sqrt(np.mean((fused - sep) ** 2)) / np.sqrt(np.mean(sep ** 2)))
    say(f"[gemv] fused vs separate rms_scaled {rms:.2e}")
    assert rms <= 5e-3


FULL = ["rms_gemv_4x4096x12288", "ln_gemv_4x4096x12288", "rms_gemv_1x4096x14336"]


@pytest.mark.parametrize("name", FULL)
def test_full_size(name):
    w = workloads.WORKLOADS[name]
    ln = w.kind == "ln_gemv"
    say(f"[gemv] full {name}")
    d = workloads.generate(w)
    r = compare(run(d, w.eps, ln), reference(d, w.eps, ln), d, w.eps, ln, name)
    say(f"[gemv] full {name}: {r}")
