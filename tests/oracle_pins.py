"""Pins that tie the CPU oracle to facts outside itself.

Each ``pin_*`` function takes an ``oracle.Oracle`` instance and raises
AssertionError when the oracle disagrees with:

* a library routine that computes the same definition (numpy's float16
  conversion; torch's bfloat16 conversion and addition; torch fp64
  ``rms_norm``, ``native_layer_norm``, ``_fused_rms_norm`` and autograd),
* central finite differences of the oracle's own forward functions,
* closed forms for constant, zero and hand-derivable rows (including the
  LayerNorm example of the meTile contract page),
* invariants every row satisfies whatever its values,
* agreement of the typed entry points across storage types on values that
  every type represents exactly.

The functions are shared by ``test_oracle_pins.py`` (the real oracle must pass
all of them) and ``test_oracle_mutants.py`` (each planted mistake must fail at
least one of them).
"""
from __future__ import annotations

import json
import os

import numpy as np
import torch
import torch.nn.functional as F

import workloads

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _close(a, b, rtol, atol=0.0, what=""):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    err = np.abs(a - b)
    lim = atol + rtol * np.abs(b)
    bad = ~(err <= lim)
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {a.size} differ, max err "
                           f"{float(np.nanmax(err)):.3e}")


def _f64(a):
    return a.astype(np.float64)


# ---------------------------------------------------------------------------
# binary16 codec versus numpy
# ---------------------------------------------------------------------------

def pin_codec_decode(o):
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = o.f16_to_f64(bits.view(np.float16))
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all(), "NaN patterns decode differently"
    assert (got[~nan] == ref[~nan]).all(), "finite or infinite patterns decode differently"
    assert (np.signbit(got[~nan]) == np.signbit(ref[~nan])).all(), "sign of zero differs"


def _encode_probe_values():
    finite = np.arange(65536, dtype=np.uint16).view(np.float16)
    finite = finite[np.isfinite(finite)].astype(np.float64)
    pos = np.unique(np.abs(finite))
    mids = (pos[:-1] + pos[1:]) / 2.0               # exact ties between neighbours
    up = np.nextafter(mids, np.inf)
    down = np.nextafter(mids, -np.inf)
    rng = np.random.default_rng(123)
    rnd = np.exp2(rng.uniform(-30.0, 17.0, 200000)) * rng.choice([-1.0, 1.0], 200000)
    special = np.array([0.0, -0.0, np.inf, -np.inf, 65504.0, 65519.99, 65520.0, 65536.0,
                        1e6, -65520.0, 2.0 ** -25, 3 * 2.0 ** -26, 2.0 ** -26, 2.0 ** -14,
                        2.0 ** -14 - 2.0 ** -25, 1e-30, -1e-30])
    return np.concatenate([finite, mids, -mids, up, down, rnd, special])


def pin_codec_encode(o):
    v = _encode_probe_values()
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    got = o.f64_to_f16(v).view(np.uint16)
    bad = ref != got
    assert not bad.any(), (f"{int(bad.sum())} encodings differ from numpy, e.g. "
                           f"{v[bad][:4]} -> {got[bad][:4]} vs {ref[bad][:4]}")
    nan = o.f64_to_f16(np.array([np.nan]))
    assert np.isnan(nan[0]), "NaN does not encode to NaN"


# ---------------------------------------------------------------------------
# torch fp64 library routines and autograd
# ---------------------------------------------------------------------------

_SHAPES = [(1, 1), (3, 2), (4, 7), (5, 64), (3, 257), (2, 1024)]


def _torch_case(kind, N, D, seed):
    d = workloads.random_case(kind, N, D, seed, x_loc=0.3 if kind == "ln" else 0.0)
    t = {k: torch.tensor(_f64(v)) for k, v in d.items()}
    return d, t


def pin_torch_rmsnorm(o):
    for i, (N, D) in enumerate(_SHAPES):
        eps = [1e-5, 1e-6, 0.1][i % 3]
        d, t = _torch_case("rms", N, D, 10 + i)
        Y, rstd = o.rmsnorm_forward(d["X"], d["gamma"], eps)
        x = t["X"].clone().requires_grad_(True)
        g = t["gamma"].clone().requires_grad_(True)
        ty = F.rms_norm(x, (D,), g, eps)
        _, trstd = torch.ops.aten._fused_rms_norm(t["X"], [D], t["gamma"], eps)
        _close(Y, ty.detach().numpy(), 1e-12, 1e-15, f"rms Y {N}x{D}")
        _close(rstd, trstd.reshape(-1).numpy(), 1e-12, 0, f"rms rstd {N}x{D}")
        (ty * t["dY"]).sum().backward()
        dX, dg = o.rmsnorm_backward(d["X"], d["gamma"], d["dY"], eps)
        _close(dX, x.grad.numpy(), 1e-10, 1e-12, f"rms dX {N}x{D}")
        _close(dg, g.grad.numpy(), 1e-10, 1e-12, f"rms dgamma {N}x{D}")


def pin_torch_layernorm(o):
    for i, (N, D) in enumerate(_SHAPES):
        eps = [1e-5, 1e-6, 0.1][i % 3]
        d, t = _torch_case("ln", N, D, 20 + i)
        Y, mean, rstd = o.layernorm_forward(d["X"], d["gamma"], d["beta"], eps)
        ty, tmean, trstd = torch.native_layer_norm(t["X"], [D], t["gamma"], t["beta"], eps)
        _close(Y, ty.numpy(), 1e-12, 1e-14, f"ln Y {N}x{D}")
        _close(mean, tmean.reshape(-1).numpy(), 1e-12, 1e-15, f"ln mean {N}x{D}")
        _close(rstd, trstd.reshape(-1).numpy(), 1e-12, 0, f"ln rstd {N}x{D}")
        x = t["X"].clone().requires_grad_(True)
        g = t["gamma"].clone().requires_grad_(True)
        b = t["beta"].clone().requires_grad_(True)
        (F.layer_norm(x, (D,), g, b, eps) * t["dY"]).sum().backward()
        dX, dg, db = o.layernorm_backward(d["X"], d["gamma"], d["dY"], eps)
        _close(dX, x.grad.numpy(), 1e-9, 1e-12, f"ln dX {N}x{D}")
        _close(dg, g.grad.numpy(), 1e-10, 1e-12, f"ln dgamma {N}x{D}")
        _close(db, b.grad.numpy(), 1e-12, 1e-14, f"ln dbeta {N}x{D}")


def pin_torch_add_rmsnorm(o):
    for i, (N, D) in enumerate(_SHAPES):
        eps = [1e-5, 1e-6, 0.1][i % 3]
        d, t = _torch_case("add", N, D, 30 + i)
        S, H, Y, rstd = o.add_rmsnorm_forward(d["X"], d["R"], d["gamma"], eps)
        x = t["X"].clone().requires_grad_(True)
        r = t["R"].clone().requires_grad_(True)
        g = t["gamma"].clone().requires_grad_(True)
        s = x + r
        ty = F.rms_norm(s, (D,), g, eps)
        _close(S, s.detach().numpy(), 0, 0, f"add S {N}x{D}")
        ref_h = (_f64(d["X"]) + _f64(d["R"])).astype(np.float16)
        assert (H.view(np.uint16) == ref_h.view(np.uint16)).all(), f"add H {N}x{D}"
        _close(Y, ty.detach().numpy(), 1e-12, 1e-15, f"add Y {N}x{D}")
        _, trstd = torch.ops.aten._fused_rms_norm(s.detach(), [D], t["gamma"], eps)
        _close(rstd, trstd.reshape(-1).numpy(), 1e-12, 0, f"add rstd {N}x{D}")
        ((ty * t["dY"]).sum() + (s * t["dH"]).sum()).backward()
        dX, dg = o.add_rmsnorm_backward(d["X"], d["R"], d["gamma"], d["dY"], d["dH"], eps)
        _close(dX, x.grad.numpy(), 1e-10, 1e-12, f"add dX {N}x{D}")
        _close(dX, r.grad.numpy(), 1e-10, 1e-12, f"add dR {N}x{D}")
        _close(dg, g.grad.numpy(), 1e-10, 1e-12, f"add dgamma {N}x{D}")


# ---------------------------------------------------------------------------
# Central finite differences of the oracle's own forward (fp64 inputs)
# ---------------------------------------------------------------------------

def _fd(f, v, j):
    h = 1e-6 * max(1.0, abs(v.flat[j]))
    a = v.copy(); a.flat[j] += h
    b = v.copy(); b.flat[j] -= h
    return (f(a) - f(b)) / (2 * h)


def _fd_check(name, f, v, grad):
    for j in range(v.size):
        num = _fd(f, v, j)
        ana = grad.flat[j]
        assert abs(num - ana) <= 1e-6 * max(1.0, abs(ana)), (
            f"{name}[{j}]: finite difference {num:.9g} vs analytic {ana:.9g}")


def pin_finite_differences(o):
    rng = np.random.default_rng(5)
    for N, D in [(1, 1), (2, 2), (3, 3), (2, 5), (1, 7), (2, 9)]:
        eps = 1e-3
        x = rng.standard_normal((N, D)) + 0.2
        r = 2 * rng.standard_normal((N, D))
        g = 1 + 0.3 * rng.standard_normal(D)
        b = 0.3 * rng.standard_normal(D)
        dy = rng.standard_normal((N, D))
        dh = rng.standard_normal((N, D))

        loss = lambda xx, gg: float((o.rmsnorm_forward(xx, gg, eps, f64=True)[0] * dy).sum())
        dX, dg = o.rmsnorm_backward(x, g, dy, eps, f64=True)
        _fd_check(f"rms dX {N}x{D}", lambda v: loss(v, g), x, dX)
        _fd_check(f"rms dgamma {N}x{D}", lambda v: loss(x, v), g, dg)

        lloss = lambda xx, gg, bb: float(
            (o.layernorm_forward(xx, gg, bb, eps, f64=True)[0] * dy).sum())
        dX, dg, db = o.layernorm_backward(x, g, dy, eps, f64=True)
        _fd_check(f"ln dX {N}x{D}", lambda v: lloss(v, g, b), x, dX)
        _fd_check(f"ln dgamma {N}x{D}", lambda v: lloss(x, v, b), g, dg)
        _fd_check(f"ln dbeta {N}x{D}", lambda v: lloss(x, g, v), b, db)

        def aloss(xx, rr, gg):
            S, _, Y, _ = o.add_rmsnorm_forward(xx, rr, gg, eps, f64=True)
            return float((Y * dy).sum() + (S * dh).sum())

        dX, dg = o.add_rmsnorm_backward(x, r, g, dy, dh, eps, f64=True)
        _fd_check(f"add dX {N}x{D}", lambda v: aloss(v, r, g), x, dX)
        _fd_check(f"add dR {N}x{D}", lambda v: aloss(x, v, g), r, dX)
        _fd_check(f"add dgamma {N}x{D}", lambda v: aloss(x, r, v), g, dg)


# ---------------------------------------------------------------------------
# Closed forms
# ---------------------------------------------------------------------------

def pin_constant_rows(o):
    rng = np.random.default_rng(9)
    for D in (1, 2, 7, 128, 257, 4096, 8192):
        cs = np.array([0.0, 1.0, -1.0, 0.5, -3.25, 100.0, 2.0 ** -10], dtype=np.float16)
        X = np.repeat(cs[:, None], D, axis=1)
        gam = (1 + 0.1 * rng.standard_normal(D)).astype(np.float16)
        bet = (0.1 * rng.standard_normal(D)).astype(np.float16)
        dY = rng.standard_normal((len(cs), D)).astype(np.float16)
        eps = 1e-5
        c = _f64(cs)[:, None]
        g64, b64, dy64 = _f64(gam)[None, :], _f64(bet)[None, :], _f64(dY)
        # LayerNorm: the centred row is exactly zero, so y = beta exactly and
        # rstd = 1/sqrt(eps); dX = (g - mean(g)) / sqrt(eps) since xhat = 0.
        Y, mean, rstd = o.layernorm_forward(X, gam, bet, eps)
        assert (Y == np.broadcast_to(b64, Y.shape)).all(), f"ln constant row y != beta, D={D}"
        assert (mean == c[:, 0]).all(), f"ln constant row mean, D={D}"
        _close(rstd, np.full(len(cs), 1 / np.sqrt(eps)), 1e-15, 0, f"ln const rstd D={D}")
        dX, _, _ = o.layernorm_backward(X, gam, dY, eps)
        gg = dy64 * g64
        _close(dX, (gg - gg.mean(axis=1, keepdims=True)) / np.sqrt(eps), 1e-12, 1e-9,
               f"ln const dX D={D}")
        # RMSNorm: y = c * gamma / sqrt(c^2 + eps), which tends to sign(c) * gamma.
        Y, rstd = o.rmsnorm_forward(X, gam, eps)
        _close(Y, c * g64 / np.sqrt(c * c + eps), 1e-14, 1e-300, f"rms const Y D={D}")
        big = np.abs(cs) >= 0.5
        _close(Y[big], (np.sign(c) * g64 * np.ones_like(Y))[big], 1e-4, 0,
               f"rms const sign*gamma D={D}")
        # dX = rstd * (g - xhat^2 * mean(g)) with xhat = c * rstd for every column.
        dX, _ = o.rmsnorm_backward(X, gam, dY, eps)
        rs = 1 / np.sqrt(c * c + eps)
        xh = c * rs
        _close(dX, rs * (gg - xh * xh * gg.mean(axis=1, keepdims=True)), 1e-11, 1e-9,
               f"rms const dX D={D}")


def pin_zero_rows(o):
    D = 33
    X = np.zeros((2, D), dtype=np.float16)
    rng = np.random.default_rng(3)
    gam = (1 + 0.1 * rng.standard_normal(D)).astype(np.float16)
    dY = rng.standard_normal((2, D)).astype(np.float16)
    eps = 1e-6
    Y, rstd = o.rmsnorm_forward(X, gam, eps)
    assert (Y == 0).all()
    _close(rstd, np.full(2, 1 / np.sqrt(eps)), 1e-15, 0, "zero-row rstd")
    dX, dg = o.rmsnorm_backward(X, gam, dY, eps)
    _close(dX, _f64(dY) * _f64(gam) / np.sqrt(eps), 1e-12, 0, "zero-row rms dX = g/sqrt(eps)")
    assert (dg == 0).all(), "zero rows give zero dgamma"


def pin_worked_example(o):
    with open(os.path.join(GOLDEN, "layernorm_worked_example.json")) as f:
        ex = json.load(f)
    R, C, div, eps = ex["rows"], ex["cols"], ex["arange_divisor"], ex["epsilon"]
    vals = (np.arange(R * C, dtype=np.float32).reshape(R, C) / np.float32(div)).astype(np.float64)
    w = np.ones(C)
    b = np.zeros(C)
    dy = np.full((R, C), ex["cotangent_value"])
    Y, mean, rstd = o.layernorm_forward(vals, w, b, eps, f64=True)
    dX, dg, db = o.layernorm_backward(vals, w, dy, eps, f64=True)
    assert list(Y.shape) == ex["asserted_shapes"]["output"]
    assert list(dX.shape) == ex["asserted_shapes"]["source_gradient"]
    assert list(dg.shape) == ex["asserted_shapes"]["weight_gradient"]
    assert list(db.shape) == ex["asserted_shapes"]["bias_gradient"]
    # Closed form from the decimal values (float32 storage perturbs them by
    # about 1e-8 relative, hence the tolerances).
    _close(mean, 0.7 * np.arange(R) + 0.3, 1e-7, 0, "example mean")
    rs = 1 / np.sqrt(0.04 + eps)
    _close(rstd, np.full(R, rs), 1e-6, 0, "example rstd")
    yrow = (np.arange(C) - 3) * 0.1 * rs
    _close(Y, np.broadcast_to(yrow, (R, C)), 0, 1e-6, "example y")
    _close(dX, np.zeros((R, C)), 0, 1e-9, "example source gradient")
    _close(db, np.full(C, 3.0), 0, 0, "example bias gradient")
    _close(dg, 3 * yrow, 0, 3e-6, "example weight gradient")
    # The same example at arange(21)/8, where every input is exact in fp16:
    # mean = (7 i + 3) / 8, variance = 1/16 exactly.
    v16 = (np.arange(R * C).reshape(R, C) / 8.0).astype(np.float16)
    Y, mean, rstd = o.layernorm_forward(v16, np.ones(C, np.float16), np.zeros(C, np.float16), eps)
    rs = 1 / np.sqrt(1 / 16 + eps)
    _close(mean, (7 * np.arange(R) + 3) / 8, 0, 0, "example/8 mean")
    _close(rstd, np.full(R, rs), 1e-15, 0, "example/8 rstd")
    _close(Y, np.broadcast_to((np.arange(C) - 3) / 8 * rs, (R, C)), 1e-15, 1e-16, "example/8 y")
    dX, dg, db = o.layernorm_backward(v16, np.ones(C, np.float16),
                                      np.ones((R, C), np.float16), eps)
    _close(dX, np.zeros((R, C)), 0, 1e-12, "example/8 dX")
    _close(dg, 3 * (np.arange(C) - 3) / 8 * rs, 1e-14, 1e-15, "example/8 dgamma")


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------

def pin_invariants(o):
    for seed, (N, D) in enumerate([(6, 257), (4, 1024), (3, 4096), (8, 7)]):
        eps = 1e-2 if D == 7 else 1e-5
        d = workloads.random_case("ln", N, D, 40 + seed, x_loc=0.5)
        X, gam, bet, dY = d["X"], d["gamma"], d["beta"], d["dY"]
        ones = np.ones(D, np.float16)
        zeros = np.zeros(D, np.float16)
        # LayerNorm with unit weight and zero bias: rows of y sum to zero and
        # mean(y^2) = var / (var + eps) = 1 - eps * rstd^2.
        Y1, mean, rstd = o.layernorm_forward(X, ones, zeros, eps)
        _close(Y1.sum(axis=1), np.zeros(N), 0, 1e-11 * D, "ln sum(xhat) = 0")
        _close((Y1 * Y1).mean(axis=1), 1 - eps * rstd ** 2, 1e-12, 0, "ln mean(xhat^2)")
        # Backward: sum(dX) = 0 and <dX, x - mean> = eps * rstd^2 * <dY, y - beta>.
        Y, mean, rstd = o.layernorm_forward(X, gam, bet, eps)
        dX, dg, db = o.layernorm_backward(X, gam, dY, eps)
        scale = np.abs(dX).sum(axis=1)
        _close(dX.sum(axis=1), np.zeros(N), 0, 1e-12 * scale.max(), "ln sum(dX) = 0")
        lhs = (dX * (_f64(X) - mean[:, None])).sum(axis=1)
        rhs = eps * rstd ** 2 * (_f64(dY) * (Y - _f64(bet)[None, :])).sum(axis=1)
        _close(lhs, rhs, 1e-6, 1e-11 * scale.max(), "ln <dX, x - mean>")
        _close(db, _f64(dY).sum(axis=0), 1e-13, 1e-13, "ln dbeta = column sums of dY")
        # RMSNorm: mean(y^2) = 1 - eps * rstd^2 at unit weight, and
        # <dX, x> = eps * rstd^2 * <dY, y>.
        Y1, rstd = o.rmsnorm_forward(X, ones, eps)
        _close((Y1 * Y1).mean(axis=1), 1 - eps * rstd ** 2, 1e-12, 0, "rms mean(xhat^2)")
        Y, rstd = o.rmsnorm_forward(X, gam, eps)
        dX, dg = o.rmsnorm_backward(X, gam, dY, eps)
        scale = np.abs(dX * _f64(X)).sum(axis=1)
        lhs = (dX * _f64(X)).sum(axis=1)
        rhs = eps * rstd ** 2 * (_f64(dY) * Y).sum(axis=1)
        _close(lhs, rhs, 1e-6, 1e-12 * scale.max(), "rms <dX, x>")
        # dgamma is linear in dY (float64 inputs).
        rng = np.random.default_rng(seed)
        a = rng.standard_normal((N, D))
        b = rng.standard_normal((N, D))
        x64 = _f64(X); g64 = _f64(gam)
        for fn in (lambda dy: o.rmsnorm_backward(x64, g64, dy, eps, f64=True)[1],
                   lambda dy: o.layernorm_backward(x64, g64, dy, eps, f64=True)[1]):
            _close(fn(a + 2 * b), fn(a) + 2 * fn(b), 1e-9, 1e-11, "dgamma linear in dY")


def pin_scaling(o):
    # RMSNorm(2x; 4 eps) = RMSNorm(x; eps) exactly (power-of-two scaling is
    # exact in binary arithmetic) and rstd halves; the same for LayerNorm
    # after a shift, up to rounding.
    rng = np.random.default_rng(11)
    D = 100
    x = rng.standard_normal((4, D))
    g = 1 + 0.1 * rng.standard_normal(D)
    b = 0.1 * rng.standard_normal(D)
    eps = 1e-4
    Y1, r1 = o.rmsnorm_forward(x, g, eps, f64=True)
    Y2, r2 = o.rmsnorm_forward(2 * x, g, 4 * eps, f64=True)
    assert (Y1 == Y2).all() and (r2 == r1 / 2).all(), "rms not scale-equivariant (eps placement)"
    Y1, m1, r1 = o.layernorm_forward(x, g, b, eps, f64=True)
    Y2, m2, r2 = o.layernorm_forward(3 * x + 1.5, g, b, 9 * eps, f64=True)
    _close(Y2, Y1, 1e-12, 1e-13, "ln affine invariance (eps placement)")
    _close(m2, 3 * m1 + 1.5, 1e-14, 1e-14, "ln mean shift")
    _close(r2, r1 / 3, 1e-12, 0, "ln rstd scale")


def pin_fused_special_cases(o):
    d = workloads.random_case("add", 5, 96, 77)
    X, R, gam, dY, dH = d["X"], d["R"], d["gamma"], d["dY"], d["dH"]
    eps = 1e-5
    Z = np.zeros_like(X)
    # R = 0: H = X, and the fused forward equals the plain RMSNorm forward.
    S, H, Y, rstd = o.add_rmsnorm_forward(X, Z, gam, eps)
    Yr, rr = o.rmsnorm_forward(X, gam, eps)
    assert (H.view(np.uint16) == X.view(np.uint16)).all(), "H != X when R = 0"
    assert (Y == Yr).all() and (rstd == rr).all(), "fused(R=0) != rmsnorm"
    dXa, dga = o.add_rmsnorm_backward(X, Z, gam, dY, None, eps)
    dXr, dgr = o.rmsnorm_backward(X, gam, dY, eps)
    assert (dXa == dXr).all() and (dga == dgr).all(), "fused bwd(R=0, dH=0) != rmsnorm bwd"
    # dY = 0: the gradient is exactly dH.
    dX, dg = o.add_rmsnorm_backward(X, R, gam, Z, dH, eps)
    assert (dX == _f64(dH)).all() and (dg == 0).all(), "dY = 0 must give dX = dH"
    # A missing dH is a zero cotangent.
    a, _ = o.add_rmsnorm_backward(X, R, gam, dY, None, eps)
    b, _ = o.add_rmsnorm_backward(X, R, gam, dY, Z, eps)
    assert (a == b).all(), "dH = None differs from dH = 0"
    # The fused sum is the source: fused(X, R) == rmsnorm(fp64 sum) on f64 inputs.
    S, H, Y, rstd = o.add_rmsnorm_forward(X, R, gam, eps)
    Y2, r2 = o.rmsnorm_forward(_f64(X) + _f64(R), _f64(gam), eps, f64=True)
    assert (Y == Y2).all() and (rstd == r2).all(), "fused forward is not rmsnorm of x + r"


# ---------------------------------------------------------------------------
# bfloat16 codec versus torch, and the typed entry points
# ---------------------------------------------------------------------------

def _torch_bf16_bits(v32: np.ndarray) -> np.ndarray:
    """torch's float32 -> bfloat16 conversion (round to nearest even)."""
    t = torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def pin_bf16_codec_decode(o):
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = o.bf16_to_f64(bits)
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all(), "bf16 NaN patterns decode differently"
    assert (got[~nan] == ref[~nan]).all(), "bf16 patterns decode differently from torch"
    assert (np.signbit(got[~nan]) == np.signbit(ref[~nan])).all(), "bf16 sign of zero differs"


def pin_bf16_codec_encode(o):
    # float32-representable probes, where torch rounds once (float32 -> bf16)
    bits = np.arange(65536, dtype=np.uint16)
    vals = o.bf16_to_f64(bits)
    fin = np.unique(np.abs(vals[np.isfinite(vals)]))
    mids = (fin[:-1] + fin[1:]) / 2.0                 # ties, exact in float32
    m32 = mids.astype(np.float32)
    assert (m32.astype(np.float64) == mids).all()
    up = np.nextafter(m32, np.float32(np.inf))
    down = np.nextafter(m32, np.float32(-np.inf))
    rng = np.random.default_rng(321)
    rnd = (np.exp2(rng.uniform(-140.0, 129.0, 200000)) *
           rng.choice([-1.0, 1.0], 200000)).astype(np.float32)
    probe = np.concatenate([fin.astype(np.float32), m32, -m32, up, down, rnd,
                            np.array([0.0, -0.0, np.inf, -np.inf, 3.4e38, -3.4e38],
                                     dtype=np.float32)])
    got = o.f64_to_bf16(probe.astype(np.float64))
    ref = _torch_bf16_bits(probe)
    bad = got != ref
    assert not bad.any(), (f"{int(bad.sum())} bf16 encodings differ from torch, e.g. "
                           f"{probe[bad][:4]} -> {got[bad][:4]} vs {ref[bad][:4]}")
    # doubles off the float32 grid: the encoding is the nearer bf16 neighbour
    # (ties to even), checked by brute force on exact double distances
    v = np.exp2(rng.uniform(-120.0, 120.0, 50000)) * rng.choice([-1.0, 1.0], 50000)
    b = o.f64_to_bf16(v)
    here = o.bf16_to_f64(b)
    lo = o.bf16_to_f64((b.astype(np.int32) - 1).astype(np.uint16))
    hi = o.bf16_to_f64((b.astype(np.int32) + 1).astype(np.uint16))
    d0 = np.abs(v - here)
    assert (d0 <= np.abs(v - lo)).all() and (d0 <= np.abs(v - hi)).all(), \
        "bf16 encoding is not the nearest value"


def pin_storage_types_agree(o):
    """Values every storage type holds exactly give identical fp64 results
    through the binary16, bfloat16, binary32 and binary64 entry points."""
    rng = np.random.default_rng(17)
    N, D = 5, 96
    xs = rng.integers(-96, 97, (N, D)) / 16.0          # 7 significant bits at most
    rs = rng.integers(-64, 65, (N, D)) / 8.0
    gs = 1 + rng.integers(-16, 17, D) / 64.0
    bs = rng.integers(-16, 17, D) / 32.0
    dys = rng.integers(-128, 129, (N, D)) / 64.0
    dhs = rng.integers(-32, 33, (N, D)) / 32.0

    def as_type(a, t):
        if t == "f16":
            return a.astype(np.float16)
        if t == "bf16":
            return o.f64_to_bf16(a)
        if t == "f32":
            return a.astype(np.float32)
        return np.ascontiguousarray(a, dtype=np.float64)

    results = {}
    for t in ("f64", "f16", "bf16", "f32"):
        X, R, g, b = as_type(xs, t), as_type(rs, t), as_type(gs, t), as_type(bs, t)
        dY, dH = as_type(dys, t), as_type(dhs, t)
        r = []
        r += list(o.rmsnorm_forward(X, g, 1e-5))
        r += list(o.layernorm_forward(X, g, b, 1e-5))
        S, H, Y, rs_ = o.add_rmsnorm_forward(X, R, g, 1e-5)
        r += [S, Y, rs_]
        r += list(o.rmsnorm_backward(X, g, dY, 1e-5))
        r += list(o.layernorm_backward(X, g, dY, 1e-5))
        r += list(o.add_rmsnorm_backward(X, R, g, dY, dH, 1e-5))
        results[t] = r
    for t in ("f16", "bf16", "f32"):
        for i, (a, b_) in enumerate(zip(results["f64"], results[t])):
            assert (a == b_).all(), f"{t} entry points differ from f64 (output {i})"
    # mixed types per group: bf16 activations, f32 parameters, f16 cotangents
    dX, dg = o.rmsnorm_backward(as_type(xs, "bf16"), as_type(gs, "f32"), as_type(dys, "f16"),
                                1e-5)
    assert (dX == results["f64"][8]).all() and (dg == results["f64"][9]).all(), \
        "mixed storage types differ"


def pin_bf16_fused_sum(o):
    """The fused add's H for bfloat16 inputs is the bfloat16 rounding of the
    exact sum: torch's bf16 addition agrees wherever its float32 sum is
    exact (exponents within 16 binades)."""
    rng = np.random.default_rng(23)
    N, D = 64, 257
    x = o.f64_to_bf16(rng.standard_normal((N, D)) * np.exp2(rng.integers(-6, 7, (N, D))))
    r = o.f64_to_bf16(rng.standard_normal((N, D)) * np.exp2(rng.integers(-6, 7, (N, D))))
    g = o.f64_to_bf16(1 + 0.1 * rng.standard_normal(D))
    S, H, Y, rstd = o.add_rmsnorm_forward(x, r, g, 1e-5)
    tx = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16)
    tr = torch.from_numpy(r.view(np.int16)).view(torch.bfloat16)
    ref = (tx + tr).view(torch.int16).numpy().view(np.uint16)
    same = (H == ref) | (((H | ref) & 0x7FFF) == 0)
    assert same.all(), f"bf16 H differs from torch in {int((~same).sum())} elements"
    assert (S == o.bf16_to_f64(x) + o.bf16_to_f64(r)).all(), "S is not the exact sum"


# ---------------------------------------------------------------------------
# The other row-wise norms (Dynamic Tanh, PolyNorm, Modulated RMSNorm,
# GroupNorm)
# ---------------------------------------------------------------------------

def pin_dyt(o):
    rng = np.random.default_rng(31)
    # closed forms: tanh through the exponential, odd symmetry, alpha = 0
    N, D = 6, 77
    x = rng.standard_normal((N, D)) * 1.5
    g = 1 + 0.2 * rng.standard_normal(D)
    b = 0.2 * rng.standard_normal(D)
    for alpha in (0.5, 1.7):
        Y = o.dyt_forward(x, alpha, g, b, f64=True)
        e = np.exp(2 * alpha * x)
        _close(Y, g[None, :] * (e - 1) / (e + 1) + b[None, :], 1e-13, 1e-15, "dyt via exp")
        Ym = o.dyt_forward(-x, alpha, g, b, f64=True)
        _close(Ym - b[None, :], -(Y - b[None, :]), 1e-14, 1e-16, "dyt odd symmetry")
    Y0 = o.dyt_forward(x, 0.0, g, b, f64=True)
    assert (Y0 == np.broadcast_to(b, (N, D))).all(), "dyt alpha = 0 must give beta"
    dy = rng.standard_normal((N, D))
    dX, da, dg, db = o.dyt_backward(x, 0.0, g, dy, f64=True)
    assert (dX == 0).all() and (dg == 0).all(), "dyt alpha = 0: dX and dgamma vanish"
    _close(da, (dy * g[None, :] * x).sum(), 1e-13, 1e-13, "dyt alpha = 0: dalpha")
    _close(db, dy.sum(axis=0), 1e-14, 1e-14, "dyt dbeta = column sums")
    # saturation: tanh(+-40) = +-1 in double, so y = beta +- gamma and dX = 0
    xs = np.sign(rng.standard_normal((2, D))) * 40.0
    Ys = o.dyt_forward(xs, 1.0, g, b, f64=True)
    _close(Ys, np.sign(xs) * g[None, :] + b[None, :], 1e-15, 1e-15, "dyt saturation")
    # central finite differences
    for (n, d), alpha in (((2, 3), 0.8), ((3, 5), 1.3), ((1, 7), -0.6)):
        x = rng.standard_normal((n, d))
        g = 1 + 0.3 * rng.standard_normal(d)
        b = 0.3 * rng.standard_normal(d)
        dy = rng.standard_normal((n, d))
        loss = lambda xx, aa, gg, bb: float((o.dyt_forward(xx, aa, gg, bb, f64=True) * dy).sum())
        dX, da, dg, db = o.dyt_backward(x, alpha, g, dy, f64=True)
        _fd_check(f"dyt dX {n}x{d}", lambda v: loss(v, alpha, g, b), x, dX)
        _fd_check(f"dyt dgamma {n}x{d}", lambda v: loss(x, alpha, v, b), g, dg)
        _fd_check(f"dyt dbeta {n}x{d}", lambda v: loss(x, alpha, g, v), b, db)
        _fd_check(f"dyt dalpha {n}x{d}", lambda v: loss(x, float(v[0]), g, b),
                  np.array([alpha]), np.array([da]))


def pin_polynorm(o):
    rng = np.random.default_rng(37)
    eps = 1e-5
    # each power on its own is torch's RMSNorm (no weight) of x^p
    x = rng.standard_normal((5, 96)) + 0.1
    for p in (1, 2, 3):
        w = np.zeros(3); w[p - 1] = 1.0
        Y, rstd = o.polynorm_forward(x, w, 0.0, eps, f64=True)
        ref = F.rms_norm(torch.from_numpy(x ** p), (96,), eps=eps).numpy()
        _close(Y, ref, 1e-12, 1e-14, f"polynorm power {p} vs torch rms_norm")
        _close(rstd[:, p - 1], 1 / np.sqrt((x ** (2 * p)).mean(axis=1) + eps), 1e-13, 0,
               f"polynorm rstd {p}")
    # linear in (w, b)
    w = np.array([0.3, -0.7, 1.1])
    Y, _ = o.polynorm_forward(x, w, 0.25, eps, f64=True)
    parts = [o.polynorm_forward(x, np.eye(3)[k], 0.0, eps, f64=True)[0] for k in range(3)]
    _close(Y, sum(w[k] * parts[k] for k in range(3)) + 0.25, 1e-13, 1e-14, "polynorm linear")
    dy = rng.standard_normal(x.shape)
    dX, dw, db = o.polynorm_backward(x, w, dy, eps, f64=True)
    _close(dw, [(dy * parts[k]).sum() for k in range(3)], 1e-12, 1e-12, "polynorm dw")
    _close(db, dy.sum(), 1e-13, 1e-13, "polynorm db")
    # central finite differences
    for n, d in ((1, 1), (2, 3), (2, 6), (1, 9)):
        x = rng.standard_normal((n, d)) + 0.2
        w = rng.standard_normal(3)
        dy = rng.standard_normal((n, d))
        loss = lambda xx, ww, bb: float((o.polynorm_forward(xx, ww, bb, 1e-3, f64=True)[0]
                                         * dy).sum())
        dX, dw, db = o.polynorm_backward(x, w, dy, 1e-3, f64=True)
        _fd_check(f"polynorm dX {n}x{d}", lambda v: loss(v, w, 0.1), x, dX)
        _fd_check(f"polynorm dw {n}x{d}", lambda v: loss(x, v, 0.1), w, dw)
        _fd_check(f"polynorm db {n}x{d}", lambda v: loss(x, w, float(v[0])), np.array([0.1]),
                  np.array([db]))


def pin_modrms(o):
    rng = np.random.default_rng(41)
    eps = 1e-5
    B, S, D = 3, 4, 80
    N = B * S
    x = rng.standard_normal((N, D))
    g = 1 + 0.1 * rng.standard_normal(D)
    sc = 0.3 * rng.standard_normal((B, D))
    sh = 0.3 * rng.standard_normal((B, D))
    dy = rng.standard_normal((N, D))
    zero = np.zeros((B, D))
    # no modulation: torch's RMSNorm and its autograd
    Y, rstd = o.modrms_forward(x, g, zero, zero, eps, f64=True)
    tx = torch.from_numpy(x).requires_grad_(True)
    tg = torch.from_numpy(g).requires_grad_(True)
    ty = F.rms_norm(tx, (D,), tg, eps)
    ty.backward(torch.from_numpy(dy))
    _close(Y, ty.detach().numpy(), 1e-12, 1e-14, "modrms unmodulated Y")
    dX, dg, dsc, dsh = o.modrms_backward(x, g, zero, dy, eps, f64=True)
    _close(dX, tx.grad.numpy(), 1e-10, 1e-12, "modrms unmodulated dX")
    _close(dg, tg.grad.numpy(), 1e-10, 1e-12, "modrms unmodulated dgamma")
    # with modulation: torch RMSNorm times (1 + scale) plus shift, per sample
    tx = torch.from_numpy(x).requires_grad_(True)
    tg = torch.from_numpy(g).requires_grad_(True)
    ts = torch.from_numpy(sc).requires_grad_(True)
    th = torch.from_numpy(sh).requires_grad_(True)
    rep = torch.arange(N) // S
    ty = F.rms_norm(tx, (D,), tg, eps) * (1 + ts[rep]) + th[rep]
    ty.backward(torch.from_numpy(dy))
    Y, _ = o.modrms_forward(x, g, sc, sh, eps, f64=True)
    dX, dg, dsc, dsh = o.modrms_backward(x, g, sc, dy, eps, f64=True)
    _close(Y, ty.detach().numpy(), 1e-12, 1e-14, "modrms Y")
    _close(dX, tx.grad.numpy(), 1e-10, 1e-12, "modrms dX")
    _close(dg, tg.grad.numpy(), 1e-10, 1e-12, "modrms dgamma")
    _close(dsc, ts.grad.numpy(), 1e-10, 1e-12, "modrms dscale")
    _close(dsh, dy.reshape(B, S, D).sum(axis=1), 1e-13, 1e-13, "modrms dshift = sums per sample")
    # central finite differences
    for b_, s_, d in ((1, 1, 3), (2, 2, 3), (3, 1, 5)):
        n = b_ * s_
        x = rng.standard_normal((n, d))
        g = 1 + 0.3 * rng.standard_normal(d)
        sc = 0.4 * rng.standard_normal((b_, d))
        sh = 0.4 * rng.standard_normal((b_, d))
        dy = rng.standard_normal((n, d))
        loss = lambda xx, gg, ss, hh: float((o.modrms_forward(xx, gg, ss, hh, 1e-3, f64=True)[0]
                                             * dy).sum())
        dX, dg, dsc, dsh = o.modrms_backward(x, g, sc, dy, 1e-3, f64=True)
        _fd_check(f"modrms dX {n}x{d}", lambda v: loss(v, g, sc, sh), x, dX)
        _fd_check(f"modrms dgamma {n}x{d}", lambda v: loss(x, v, sc, sh), g, dg)
        _fd_check(f"modrms dscale {n}x{d}", lambda v: loss(x, g, v, sh), sc, dsc)
        _fd_check(f"modrms dshift {n}x{d}", lambda v: loss(x, g, sc, v), sh, dsh)


def pin_groupnorm(o):
    rng = np.random.default_rng(43)
    eps = 1e-5
    for N, C, L, G in ((2, 8, 5, 4), (3, 6, 7, 1), (2, 6, 3, 6), (1, 12, 16, 3)):
        x = rng.standard_normal((N, C, L)) + 0.3
        g = 1 + 0.2 * rng.standard_normal(C)
        b = 0.2 * rng.standard_normal(C)
        dy = rng.standard_normal((N, C, L))
        tx = torch.from_numpy(x).requires_grad_(True)
        tg = torch.from_numpy(g).requires_grad_(True)
        tb = torch.from_numpy(b).requires_grad_(True)
        ty = F.group_norm(tx, G, tg, tb, eps)
        ty.backward(torch.from_numpy(dy))
        Y, mean, rstd = o.groupnorm_forward(x, g, b, G, eps, f64=True)
        dX, dg, db = o.groupnorm_backward(x, g, dy, G, eps, f64=True)
        what = f"groupnorm {N}x{C}x{L} G={G}"
        _close(Y, ty.detach().numpy(), 1e-12, 1e-13, what + " Y")
        sl = x.reshape(N, G, -1)
        _close(mean, sl.mean(axis=2), 1e-13, 1e-15, what + " mean")
        _close(rstd, 1 / np.sqrt(sl.var(axis=2) + eps), 1e-12, 0, what + " rstd")
        _close(dX, tx.grad.numpy(), 1e-10, 1e-12, what + " dX")
        _close(dg, tg.grad.numpy(), 1e-10, 1e-12, what + " dgamma")
        _close(db, tb.grad.numpy(), 1e-12, 1e-12, what + " dbeta")
    # central finite differences
    for N, C, L, G in ((1, 2, 2, 1), (2, 4, 1, 2), (1, 3, 2, 3)):
        x = rng.standard_normal((N, C, L))
        g = 1 + 0.3 * rng.standard_normal(C)
        b = 0.3 * rng.standard_normal(C)
        dy = rng.standard_normal((N, C, L))
        loss = lambda xx, gg, bb: float((o.groupnorm_forward(xx, gg, bb, G, 1e-3, f64=True)[0]
                                         * dy).sum())
        dX, dg, db = o.groupnorm_backward(x, g, dy, G, 1e-3, f64=True)
        _fd_check(f"groupnorm dX {N}x{C}x{L}", lambda v: loss(v, g, b), x, dX)
        _fd_check(f"groupnorm dgamma {N}x{C}x{L}", lambda v: loss(x, v, b), g, dg)
        _fd_check(f"groupnorm dbeta {N}x{C}x{L}", lambda v: loss(x, g, v), b, db)


def pin_norm_gemv(o):
    rng = np.random.default_rng(47)
    eps = 1e-5
    for M, K, N in ((1, 1, 1), (3, 64, 40), (4, 257, 33), (2, 1024, 96)):
        X = rng.standard_normal((M, K)).astype(np.float16)
        g = (1 + 0.1 * rng.standard_normal(K)).astype(np.float16)
        b = (0.1 * rng.standard_normal(K)).astype(np.float16)
        W = (rng.standard_normal((K, N)) / np.sqrt(K)).astype(np.float16)
        tx, tg, tb, tw = (torch.from_numpy(a.astype(np.float64)) for a in (X, g, b, W))
        ref = F.rms_norm(tx, (K,), tg, eps) @ tw
        _close(o.norm_gemv(X, g, W, eps), ref.numpy(), 1e-12, 1e-13, f"rms gemv {M}x{K}x{N}")
        ref = F.layer_norm(tx, (K,), tg, tb, eps) @ tw
        _close(o.norm_gemv(X, g, W, eps, beta=b), ref.numpy(), 1e-12, 1e-13,
               f"ln gemv {M}x{K}x{N}")
    # an identity W returns the normalised rows; a column selector picks one
    M, K = 3, 48
    X = rng.standard_normal((M, K))
    g = 1 + 0.2 * rng.standard_normal(K)
    b = 0.2 * rng.standard_normal(K)
    tx, tg, tb = (torch.from_numpy(a) for a in (X, g, b))
    _close(o.norm_gemv(X, g, np.eye(K), eps, f64=True),
           F.rms_norm(tx, (K,), tg, eps).numpy(), 1e-13, 1e-15, "rms gemv identity")
    sel = np.zeros((K, 5)); sel[[7, 0, 47, 20, 7], range(5)] = 1.0
    _close(o.norm_gemv(X, g, sel, eps, beta=b, f64=True),
           F.layer_norm(tx, (K,), tg, tb, eps).numpy()[:, [7, 0, 47, 20, 7]], 1e-13, 1e-15,
           "ln gemv column selector")
    # linear in W
    W1 = rng.standard_normal((K, 9)); W2 = rng.standard_normal((K, 9))
    _close(o.norm_gemv(X, g, W1 + 2 * W2, eps, f64=True),
           o.norm_gemv(X, g, W1, eps, f64=True) + 2 * o.norm_gemv(X, g, W2, eps, f64=True),
           1e-12, 1e-12, "gemv linear in W")


ALL_PINS = [
    pin_codec_decode, pin_codec_encode, pin_torch_rmsnorm, pin_torch_layernorm,
    pin_torch_add_rmsnorm, pin_finite_differences, pin_constant_rows, pin_zero_rows,
    pin_worked_example, pin_invariants, pin_scaling, pin_fused_special_cases,
    pin_bf16_codec_decode, pin_bf16_codec_encode, pin_storage_types_agree, pin_bf16_fused_sum,
    pin_dyt, pin_polynorm, pin_modrms, pin_groupnorm, pin_norm_gemv,
]
