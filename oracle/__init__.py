"""CPU fp64 oracle for the row-wise normalization training pair.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use it; the product package never imports it, and it
imports nothing from the product. The arithmetic lives in ``mn_oracle.c``
(plain C, double precision, one row at a time, sums in ascending order); this
module builds it with gcc and marshals numpy arrays through ctypes.

Inputs are numpy arrays whose dtype names their storage type: float16,
uint16 (bfloat16 bit patterns), float32, or float64 (used by the
finite-difference pins). Outputs are float64 arrays; ``round_to`` rounds them
once to a storage type (nearest, ties to even, straight from double) for
comparison with GPU results.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC_PATH = os.path.join(_HERE, "mn_oracle.c")
LIB_PATH = os.path.join(_HERE, "libmn_oracle.so")

_P16 = ctypes.POINTER(ctypes.c_uint16)
_PD = ctypes.POINTER(ctypes.c_double)
_I64 = ctypes.c_int64
_DBL = ctypes.c_double


def compile_library(src: str, out: str, extra_flags=()) -> str:
    """gcc build: no fast-math and no FMA contraction, so every operation in
    the oracle is one IEEE double rounding. ``extra_flags`` adds options (the
    sanitizer builds of the tests)."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", *extra_flags, "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    if not force and os.path.exists(LIB_PATH):
        return LIB_PATH
    return compile_library(SRC_PATH, LIB_PATH)


def _nd(X: np.ndarray) -> Tuple[int, int]:
    if X.ndim != 2:
        raise ValueError("X must be [N, D]")
    return int(X.shape[0]), int(X.shape[1])


# Storage-type codes of the C oracle (MNO_F16, MNO_BF16, MNO_F32, MNO_F64).
# bfloat16 arrays are carried as numpy uint16 bit patterns.
_TYPE = {np.dtype(np.float16): 0, np.dtype(np.uint16): 1, np.dtype(np.float32): 2,
         np.dtype(np.float64): 3}
_VP = ctypes.c_void_p


class Oracle:
    """ctypes view of one build of mn_oracle.c.

    Inputs are numpy arrays whose dtype names their storage type: float16,
    uint16 (bfloat16 bit patterns), float32 or float64. X and R share a type,
    gamma and beta share one, dY and dH share one. ``f64=True`` converts
    every input to float64 first (used by the finite-difference pins)."""

    def __init__(self, lib_path: str = LIB_PATH):
        lib = ctypes.CDLL(lib_path)
        lib.mno_f16_to_f64.restype = _DBL
        lib.mno_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.mno_f64_to_f16.restype = ctypes.c_uint16
        lib.mno_f64_to_f16.argtypes = [_DBL]
        lib.mno_bf16_to_f64.restype = _DBL
        lib.mno_bf16_to_f64.argtypes = [ctypes.c_uint16]
        lib.mno_f64_to_bf16.restype = ctypes.c_uint16
        lib.mno_f64_to_bf16.argtypes = [_DBL]
        for name in ("mno_decode_f16", "mno_decode_bf16"):
            getattr(lib, name).argtypes = [_P16, _PD, _I64]
        for name in ("mno_encode_f16", "mno_encode_bf16"):
            getattr(lib, name).argtypes = [_PD, _P16, _I64]
        I = ctypes.c_int
        sig = {
            "mno_rmsnorm_forward_t": [_VP, I, _VP, I, _I64, _I64, _DBL, _PD, _PD],
            "mno_layernorm_forward_t": [_VP, I, _VP, _VP, I, _I64, _I64, _DBL, _PD, _PD, _PD],
            "mno_add_rmsnorm_forward_t": [_VP, _VP, I, _VP, I, _I64, _I64, _DBL, _PD, _PD, _PD],
            "mno_rmsnorm_backward_t": [_VP, I, _VP, I, _VP, I, _I64, _I64, _DBL, _PD, _PD],
            "mno_layernorm_backward_t": [_VP, I, _VP, I, _VP, I, _I64, _I64, _DBL, _PD, _PD,
                                         _PD],
            "mno_add_rmsnorm_backward_t": [_VP, _VP, I, _VP, I, _VP, _VP, I, _I64, _I64, _DBL,
                                           _PD, _PD],
            "mno_dyt_forward_t": [_VP, I, _DBL, _VP, _VP, I, _I64, _I64, _PD],
            "mno_dyt_backward_t": [_VP, I, _DBL, _VP, I, _VP, I, _I64, _I64, _PD, _PD, _PD, _PD],
            "mno_polynorm_forward_t": [_VP, I, _PD, _DBL, _I64, _I64, _DBL, _PD, _PD],
            "mno_polynorm_backward_t": [_VP, I, _PD, _VP, I, _I64, _I64, _DBL, _PD, _PD, _PD],
            "mno_modrms_forward_t": [_VP, I, _VP, I, _VP, _VP, I, _I64, _I64, _I64, _DBL, _PD,
                                     _PD],
            "mno_modrms_backward_t": [_VP, I, _VP, I, _VP, I, _VP, I, _I64, _I64, _I64, _DBL,
                                      _PD, _PD, _PD, _PD],
            "mno_groupnorm_forward_t": [_VP, I, _VP, _VP, I, _I64, _I64, _I64, _I64, _DBL, _PD,
                                        _PD, _PD],
            "mno_groupnorm_backward_t": [_VP, I, _VP, I, _VP, I, _I64, _I64, _I64, _I64, _DBL,
                                         _PD, _PD, _PD],
            "mno_rmsnorm_gemv_t": [_VP, I, _VP, I, _VP, I, _I64, _I64, _I64, _DBL, _PD],
            "mno_layernorm_gemv_t": [_VP, I, _VP, _VP, I, _VP, I, _I64, _I64, _I64, _DBL, _PD],
        }
        for name, argtypes in sig.items():
            fn = getattr(lib, name)
            fn.argtypes = argtypes
            fn.restype = ctypes.c_int
        self.lib = lib

    # -- marshalling -------------------------------------------------------

    @staticmethod
    def _group(arrays, f64: bool):
        """Pointers and the shared storage-type code of one operand group."""
        keep, ptrs, code = [], [], None
        for a in arrays:
            if a is None:
                ptrs.append(None)
                continue
            a = np.ascontiguousarray(a, dtype=np.float64) if f64 else a
            if not a.flags.c_contiguous or a.dtype not in _TYPE:
                raise TypeError("oracle inputs must be C-contiguous float16, uint16 (bfloat16), "
                                "float32 or float64 arrays")
            c = _TYPE[a.dtype]
            if code is not None and c != code:
                raise TypeError("operands of one group must share a storage type")
            code = c
            keep.append(a)
            ptrs.append(a.ctypes.data_as(_VP))
        return ptrs, (3 if code is None else code), keep

    @staticmethod
    def _out(a):
        return None if a is None else a.ctypes.data_as(_PD)

    def _check(self, name, rc):
        if rc != 0:
            raise RuntimeError(f"{name} returned {rc}")

    # -- storage-type codecs ----------------------------------------------

    def f16_to_f64(self, a: np.ndarray) -> np.ndarray:
        a = np.ascontiguousarray(a, dtype=np.float16)
        out = np.empty(a.shape, dtype=np.float64)
        self.lib.mno_decode_f16(a.ctypes.data_as(_P16), out.ctypes.data_as(_PD), a.size)
        return out

    def f64_to_f16(self, a: np.ndarray) -> np.ndarray:
        """Round float64 values to fp16, to nearest with ties to even."""
        a = np.ascontiguousarray(a, dtype=np.float64)
        out = np.empty(a.shape, dtype=np.uint16)
        self.lib.mno_encode_f16(a.ctypes.data_as(_PD), out.ctypes.data_as(_P16), a.size)
        return out.view(np.float16)

    def bf16_to_f64(self, bits: np.ndarray) -> np.ndarray:
        bits = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(bits.shape, dtype=np.float64)
        self.lib.mno_decode_bf16(bits.ctypes.data_as(_P16), out.ctypes.data_as(_PD), bits.size)
        return out

    def f64_to_bf16(self, a: np.ndarray) -> np.ndarray:
        """Round float64 values to bfloat16 (bit patterns), nearest, ties to even."""
        a = np.ascontiguousarray(a, dtype=np.float64)
        out = np.empty(a.shape, dtype=np.uint16)
        self.lib.mno_encode_bf16(a.ctypes.data_as(_PD), out.ctypes.data_as(_P16), a.size)
        return out

    def round_to(self, a: np.ndarray, like: np.dtype) -> np.ndarray:
        """Round float64 values once to the storage type `like` (float16,
        uint16 = bfloat16 bits, or float32)."""
        like = np.dtype(like)
        if like == np.float16:
            return self.f64_to_f16(a)
        if like == np.uint16:
            return self.f64_to_bf16(a)
        if like == np.float32:
            return np.ascontiguousarray(a, dtype=np.float64).astype(np.float32)
        raise TypeError(like)

    # -- forward -----------------------------------------------------------

    def rmsnorm_forward(self, X, gamma, eps, f64: bool = False):
        """(Y [N, D], rstd [N]), float64."""
        N, D = _nd(X)
        (x,), tx, k1 = self._group([X], f64)
        (g,), tg, k2 = self._group([gamma], f64)
        Y = np.empty((N, D)); rstd = np.empty(N)
        self._check("rmsnorm_forward", self.lib.mno_rmsnorm_forward_t(
            x, tx, g, tg, N, D, float(eps), self._out(Y), self._out(rstd)))
        return Y, rstd

    def layernorm_forward(self, X, gamma, beta, eps, f64: bool = False):
        """(Y [N, D], mean [N], rstd [N]), float64."""
        N, D = _nd(X)
        (x,), tx, k1 = self._group([X], f64)
        (g, b), tg, k2 = self._group([gamma, beta], f64)
        Y = np.empty((N, D)); mean = np.empty(N); rstd = np.empty(N)
        self._check("layernorm_forward", self.lib.mno_layernorm_forward_t(
            x, tx, g, b, tg, N, D, float(eps), self._out(Y), self._out(mean), self._out(rstd)))
        return Y, mean, rstd

    def add_rmsnorm_forward(self, X, R, gamma, eps, f64: bool = False):
        """(S = x + r unrounded, H = S rounded to X's storage type, Y, rstd);
        S, Y, rstd float64. H is float16 for float16 inputs, bfloat16 bits
        for uint16 inputs, float32 for float32 inputs, float64 for float64."""
        N, D = _nd(X)
        (x, r), tx, k1 = self._group([X, R], f64)
        (g,), tg, k2 = self._group([gamma], f64)
        S = np.empty((N, D)); Y = np.empty((N, D)); rstd = np.empty(N)
        self._check("add_rmsnorm_forward", self.lib.mno_add_rmsnorm_forward_t(
            x, r, tx, g, tg, N, D, float(eps), self._out(S), self._out(Y), self._out(rstd)))
        H = S if tx == 3 else self.round_to(S, {0: np.float16, 1: np.uint16, 2: np.float32}[tx])
        return S, H, Y, rstd

    # -- backward ----------------------------------------------------------

    def rmsnorm_backward(self, X, gamma, dY, eps, want_dx: bool = True, f64: bool = False):
        """(dX [N, D] or None, dgamma [D]), float64."""
        N, D = _nd(X)
        (x,), tx, k1 = self._group([X], f64)
        (g,), tg, k2 = self._group([gamma], f64)
        (dy,), ty, k3 = self._group([dY], f64)
        dX = np.empty((N, D)) if want_dx else None
        dg = np.empty(D)
        self._check("rmsnorm_backward", self.lib.mno_rmsnorm_backward_t(
            x, tx, g, tg, dy, ty, N, D, float(eps), self._out(dX), self._out(dg)))
        return dX, dg

    def layernorm_backward(self, X, gamma, dY, eps, want_dx: bool = True, f64: bool = False):
        """(dX or None, dgamma, dbeta), float64."""
        N, D = _nd(X)
        (x,), tx, k1 = self._group([X], f64)
        (g,), tg, k2 = self._group([gamma], f64)
        (dy,), ty, k3 = self._group([dY], f64)
        dX = np.empty((N, D)) if want_dx else None
        dg = np.empty(D); db = np.empty(D)
        self._check("layernorm_backward", self.lib.mno_layernorm_backward_t(
            x, tx, g, tg, dy, ty, N, D, float(eps), self._out(dX), self._out(dg), self._out(db)))
        return dX, dg, db

    def add_rmsnorm_backward(self, X, R, gamma, dY, dH, eps, want_dx: bool = True,
                             f64: bool = False):
        """(dX = dR or None, dgamma), float64. dH None means a zero cotangent."""
        N, D = _nd(X)
        (x, r), tx, k1 = self._group([X, R], f64)
        (g,), tg, k2 = self._group([gamma], f64)
        (dy, dh), ty, k3 = self._group([dY, dH], f64)
        dX = np.empty((N, D)) if want_dx else None
        dg = np.empty(D)
        self._check("add_rmsnorm_backward", self.lib.mno_add_rmsnorm_backward_t(
            x, r, tx, g, tg, dy, dh, ty, N, D, float(eps), self._out(dX), self._out(dg)))
        return dX, dg

    # -- the other row-wise norms -------------------------------------------

    def dyt_forward(self, X, alpha, gamma, beta, f64: bool = False):
        """Dynamic Tanh: Y [N, D] = gamma * tanh(alpha * X) + beta, float64."""
        N, D = _nd(X)
        (x,), tx, k1 = self._group([X], f64)
        (g, b), tg, k2 = self._group([gamma, beta], f64)
        Y = np.empty((N, D))
        self._check("dyt_forward", self.lib.mno_dyt_forward_t(
            x, tx, float(alpha), g, b, tg, N, D, self._out(Y)))
        return Y

    def dyt_backward(self, X, alpha, gamma, dY, want_dx: bool = True, f64: bool = False):
        """(dX or None, dalpha (float), dgamma [D], dbeta [D])."""
        N, D = _nd(X)
        (x,), tx, k1 = self._group([X], f64)
        (g,), tg, k2 = self._group([gamma], f64)
        (dy,), ty, k3 = self._group([dY], f64)
        dX = np.empty((N, D)) if want_dx else None
        da = np.empty(1); dg = np.empty(D); db = np.empty(D)
        self._check("dyt_backward", self.lib.mno_dyt_backward_t(
            x, tx, float(alpha), g, tg, dy, ty, N, D, self._out(dX), self._out(da),
            self._out(dg), self._out(db)))
        return dX, float(da[0]), dg, db

    def polynorm_forward(self, X, w, b, eps, f64: bool = False):
        """PolyNorm: (Y [N, D], rstd [N, 3]) with rstd[:, p-1] the p-th power's."""
        N, D = _nd(X)
        (x,), tx, k1 = self._group([X], f64)
        wv = np.ascontiguousarray(w, dtype=np.float64).reshape(3)
        Y = np.empty((N, D)); rstd = np.empty((N, 3))
        self._check("polynorm_forward", self.lib.mno_polynorm_forward_t(
            x, tx, self._out(wv), float(b), N, D, float(eps), self._out(Y), self._out(rstd)))
        return Y, rstd

    def polynorm_backward(self, X, w, dY, eps, want_dx: bool = True, f64: bool = False):
        """(dX or None, dw [3], db (float))."""
        N, D = _nd(X)
        (x,), tx, k1 = self._group([X], f64)
        (dy,), ty, k3 = self._group([dY], f64)
        wv = np.ascontiguousarray(w, dtype=np.float64).reshape(3)
        dX = np.empty((N, D)) if want_dx else None
        dw = np.empty(3); db = np.empty(1)
        self._check("polynorm_backward", self.lib.mno_polynorm_backward_t(
            x, tx, self._out(wv), dy, ty, N, D, float(eps), self._out(dX), self._out(dw),
            self._out(db)))
        return dX, dw, float(db[0])

    def modrms_forward(self, X, gamma, scale, shift, eps, f64: bool = False):
        """Modulated RMSNorm with B = scale.shape[0] samples of N / B rows:
        (Y [N, D], rstd [N])."""
        N, D = _nd(X)
        B = int(scale.shape[0])
        (x,), tx, k1 = self._group([X], f64)
        (g,), tg, k2 = self._group([gamma], f64)
        (sc, sh), ts, k3 = self._group([scale, shift], f64)
        Y = np.empty((N, D)); rstd = np.empty(N)
        self._check("modrms_forward", self.lib.mno_modrms_forward_t(
            x, tx, g, tg, sc, sh, ts, B, N, D, float(eps), self._out(Y), self._out(rstd)))
        return Y, rstd

    def modrms_backward(self, X, gamma, scale, dY, eps, want_dx: bool = True, f64: bool = False):
        """(dX or None, dgamma [D], dscale [B, D], dshift [B, D])."""
        N, D = _nd(X)
        B = int(scale.shape[0])
        (x,), tx, k1 = self._group([X], f64)
        (g,), tg, k2 = self._group([gamma], f64)
        (sc,), ts, k3 = self._group([scale], f64)
        (dy,), ty, k4 = self._group([dY], f64)
        dX = np.empty((N, D)) if want_dx else None
        dg = np.empty(D); dsc = np.empty((B, D)); dsh = np.empty((B, D))
        self._check("modrms_backward", self.lib.mno_modrms_backward_t(
            x, tx, g, tg, sc, ts, dy, ty, B, N, D, float(eps), self._out(dX), self._out(dg),
            self._out(dsc), self._out(dsh)))
        return dX, dg, dsc, dsh

    def groupnorm_forward(self, X, gamma, beta, groups, eps, f64: bool = False):
        """GroupNorm on X [N, C, L]: (Y [N, C, L], mean [N, G], rstd [N, G])."""
        N, C, L = (int(v) for v in X.shape)
        (x,), tx, k1 = self._group([X], f64)
        (g, b), tg, k2 = self._group([gamma, beta], f64)
        Y = np.empty((N, C, L)); mean = np.empty((N, groups)); rstd = np.empty((N, groups))
        self._check("groupnorm_forward", self.lib.mno_groupnorm_forward_t(
            x, tx, g, b, tg, N, C, L, int(groups), float(eps), self._out(Y), self._out(mean),
            self._out(rstd)))
        return Y, mean, rstd

    def groupnorm_backward(self, X, gamma, dY, groups, eps, want_dx: bool = True,
                           f64: bool = False):
        """(dX [N, C, L] or None, dgamma [C], dbeta [C])."""
        N, C, L = (int(v) for v in X.shape)
        (x,), tx, k1 = self._group([X], f64)
        (g,), tg, k2 = self._group([gamma], f64)
        (dy,), ty, k3 = self._group([dY], f64)
        dX = np.empty((N, C, L)) if want_dx else None
        dg = np.empty(C); db = np.empty(C)
        self._check("groupnorm_backward", self.lib.mno_groupnorm_backward_t(
            x, tx, g, tg, dy, ty, N, C, L, int(groups), float(eps), self._out(dX),
            self._out(dg), self._out(db)))
        return dX, dg, db

    # -- fused normalization + GEMV (inference) ---------------------------------

    def norm_gemv(self, X, gamma, W, eps, beta=None, f64: bool = False):
        """Y [M, N] = Norm(X) @ W: RMSNorm, or LayerNorm when beta is given;
        float64, the normalised rows unrounded."""
        M, K = _nd(X)
        N = int(W.shape[1])
        (x,), tx, k1 = self._group([X], f64)
        (g, b), tg, k2 = self._group([gamma, beta], f64)
        (w,), tw, k3 = self._group([W], f64)
        Y = np.empty((M, N))
        if beta is None:
            rc = self.lib.mno_rmsnorm_gemv_t(x, tx, g, tg, w, tw, M, N, K, float(eps),
                                             self._out(Y))
        else:
            rc = self.lib.mno_layernorm_gemv_t(x, tx, g, b, tg, w, tw, M, N, K, float(eps),
                                               self._out(Y))
        self._check("norm_gemv", rc)
        return Y


_default: Optional[Oracle] = None


def get() -> Oracle:
    """The oracle built from this directory's source (built on first use)."""
    global _default
    if _default is None:
        if not os.path.exists(LIB_PATH) or os.path.getmtime(LIB_PATH) < os.path.getmtime(SRC_PATH):
            build()
        _default = Oracle(LIB_PATH)
    return _default


def __getattr__(name):
    # Module-level shortcuts: oracle.rmsnorm_forward(...) etc.
    if name.startswith("_"):
        raise AttributeError(name)
    return getattr(get(), name)
