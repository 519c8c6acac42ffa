"""CPU fp64 oracle for the row-wise normalization training pair.

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the benchmark's
CPU-baseline leg use it; the product package never imports it, and it
imports nothing from the product. The arithmetic lives in ``mn_oracle.c``
(plain C, double precision, one row at a time, sums in ascending order); this
module builds it with gcc and marshals numpy arrays through ctypes.

Inputs are fp16 numpy arrays (the path's storage type) or, through the
``*_f64`` functions, float64 arrays (used by the finite-difference pins).
Outputs are float64 arrays; ``f64_to_f16`` rounds them to fp16 (nearest, ties
to even, straight from double) for comparison with fp16 results.
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


def compile_library(src: str, out: str) -> str:
    """gcc build: no fast-math and no FMA contraction, so every operation in
    the oracle is one IEEE double rounding."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
           "-fno-fast-math", "-Wall", "-Wextra", "-o", tmp, src, "-lm"]
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


class Oracle:
    """ctypes view of one build of mn_oracle.c."""

    def __init__(self, lib_path: str = LIB_PATH):
        lib = ctypes.CDLL(lib_path)
        lib.mno_f16_to_f64.restype = _DBL
        lib.mno_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.mno_f64_to_f16.restype = ctypes.c_uint16
        lib.mno_f64_to_f16.argtypes = [_DBL]
        lib.mno_decode_f16.argtypes = [_P16, _PD, _I64]
        lib.mno_encode_f16.argtypes = [_PD, _P16, _I64]
        for suffix, P in (("", _P16), ("_f64", _PD)):
            sig = {
                "mno_rmsnorm_forward": [P, P, _I64, _I64, _DBL, _PD, _PD],
                "mno_layernorm_forward": [P, P, P, _I64, _I64, _DBL, _PD, _PD, _PD],
                "mno_add_rmsnorm_forward": [P, P, P, _I64, _I64, _DBL, _PD, _PD, _PD],
                "mno_rmsnorm_backward": [P, P, P, _I64, _I64, _DBL, _PD, _PD],
                "mno_layernorm_backward": [P, P, P, _I64, _I64, _DBL, _PD, _PD, _PD],
                "mno_add_rmsnorm_backward": [P, P, P, P, P, _I64, _I64, _DBL, _PD, _PD],
            }
            for name, argtypes in sig.items():
                fn = getattr(lib, name + suffix)
                fn.argtypes = argtypes
                fn.restype = ctypes.c_int
        self.lib = lib

    # -- marshalling -------------------------------------------------------

    @staticmethod
    def _in(a: Optional[np.ndarray], f64: bool):
        if a is None:
            return None
        if f64:
            a = np.ascontiguousarray(a, dtype=np.float64)
            return a.ctypes.data_as(_PD), a
        if a.dtype != np.float16 or not a.flags.c_contiguous:
            raise TypeError("oracle fp16 inputs must be C-contiguous float16 arrays")
        return a.ctypes.data_as(_P16), a

    def _call(self, name: str, f64: bool, ins, tail):
        fn = getattr(self.lib, name + ("_f64" if f64 else ""))
        keep = []
        args = []
        for a in ins:
            m = self._in(a, f64)
            if m is None:
                args.append(None)
            else:
                args.append(m[0])
                keep.append(m[1])
        args += [None if t is None else (t.ctypes.data_as(_PD) if isinstance(t, np.ndarray) else t)
                 for t in tail]
        rc = fn(*args)
        if rc != 0:
            raise RuntimeError(f"{name} returned {rc}")

    # -- binary16 codec ----------------------------------------------------

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

    # -- forward -----------------------------------------------------------

    def rmsnorm_forward(self, X, gamma, eps, f64: bool = False):
        """(Y [N, D], rstd [N]), float64."""
        N, D = _nd(X)
        Y = np.empty((N, D)); rstd = np.empty(N)
        self._call("mno_rmsnorm_forward", f64, (X, gamma), (N, D, float(eps), Y, rstd))
        return Y, rstd

    def layernorm_forward(self, X, gamma, beta, eps, f64: bool = False):
        """(Y [N, D], mean [N], rstd [N]), float64."""
        N, D = _nd(X)
        Y = np.empty((N, D)); mean = np.empty(N); rstd = np.empty(N)
        self._call("mno_layernorm_forward", f64, (X, gamma, beta),
                   (N, D, float(eps), Y, mean, rstd))
        return Y, mean, rstd

    def add_rmsnorm_forward(self, X, R, gamma, eps, f64: bool = False):
        """(S = x + r unrounded, H = fp16(S), Y, rstd); all float64 but H."""
        N, D = _nd(X)
        S = np.empty((N, D)); Y = np.empty((N, D)); rstd = np.empty(N)
        self._call("mno_add_rmsnorm_forward", f64, (X, R, gamma),
                   (N, D, float(eps), S, Y, rstd))
        return S, self.f64_to_f16(S), Y, rstd

    # -- backward ----------------------------------------------------------

    def rmsnorm_backward(self, X, gamma, dY, eps, want_dx: bool = True, f64: bool = False):
        """(dX [N, D] or None, dgamma [D]), float64."""
        N, D = _nd(X)
        dX = np.empty((N, D)) if want_dx else None
        dg = np.empty(D)
        self._call("mno_rmsnorm_backward", f64, (X, gamma, dY), (N, D, float(eps), dX, dg))
        return dX, dg

    def layernorm_backward(self, X, gamma, dY, eps, want_dx: bool = True, f64: bool = False):
        """(dX or None, dgamma, dbeta), float64."""
        N, D = _nd(X)
        dX = np.empty((N, D)) if want_dx else None
        dg = np.empty(D); db = np.empty(D)
        self._call("mno_layernorm_backward", f64, (X, gamma, dY),
                   (N, D, float(eps), dX, dg, db))
        return dX, dg, db

    def add_rmsnorm_backward(self, X, R, gamma, dY, dH, eps, want_dx: bool = True,
                             f64: bool = False):
        """(dX = dR or None, dgamma), float64. dH None means a zero cotangent."""
        N, D = _nd(X)
        dX = np.empty((N, D)) if want_dx else None
        dg = np.empty(D)
        self._call("mno_add_rmsnorm_backward", f64, (X, R, gamma, dY, dH),
                   (N, D, float(eps), dX, dg))
        return dX, dg


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
