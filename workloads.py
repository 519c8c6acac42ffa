"""Seeded synthetic inputs for the row-wise normalization training pair.

This module is shared by the tests, the benchmark and the smoke check. It
holds the workload table (shapes, epsilon, value distributions) and the
seeded generators, and nothing of the normalization arithmetic itself: both
the CPU oracle and the HIP library receive the arrays it returns.

Recipe (fixed, so that every run sees the same bits):

* Tensors are drawn in the order the workload lists them (tensor index t),
  as float64 ``standard_normal`` values from PCG64 streams: a [D] vector from
  ``default_rng([seed, t])``; an [N, D] tensor in fixed blocks of
  ``rows_per_chunk(D)`` rows, block c from ``default_rng([seed, t, c])``.
  Blocks are independent streams, so they are drawn on several threads and
  the values do not depend on the thread count; a smaller N yields a prefix
  of the same rows. Seed 0 unless a test says otherwise.
* ``loc + scale * z`` is applied in float64, then the value is rounded to the
  storage type, round to nearest, ties to even: fp16 directly from float64
  (numpy converts float64 to float16 without passing through float32);
  float32 directly; bfloat16 from the float32 value, by rounding its bit
  pattern to the upper 16 bits (returned as uint16 bit patterns). The named
  workloads are fp16 throughout; tests of the other storage types pass
  ``act`` (X, R), ``cot`` (dY, dH) and ``param`` (gamma, beta) to the
  generators.
* The Modulated RMSNorm's scale and shift are [B, D] tensors drawn like an
  [N, D] one with B rows, in the activation storage type. The scalar
  parameters (Dynamic Tanh's alpha, PolyNorm's weights and bias) are fixed
  constants of the workload, not drawn.
* The fused norm + GEMV workloads draw X as an [M, K] tensor (M = N rows,
  K = D) and the weight W as a [K, Nout] tensor drawn like an [N, D] one with
  K rows, N(0, 0.02^2), in the activation storage type.
* GroupNorm draws X and dY as [N, C * L] tensors (one row per sample, viewed
  as [N, C, L]) and gamma, beta as [C] vectors.
* The Llama-shape RMSNorm workload marks 1 % of its 4096 channels as outliers:
  41 channels drawn without replacement from ``default_rng(1)`` and sorted;
  those X columns are multiplied by 20 before rounding.

The pages publish no dataset for this path; these synthetic tensors stand in
for activations and cotangents of the stated shapes and distributions.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Dict, Optional, Tuple

import numpy as np

# Elements per independently seeded block of an [N, D] tensor (a 32 MiB
# float64 temporary per block).
_CHUNK_ELEMS = 1 << 22
# Worker threads for drawing blocks (numpy releases the GIL while filling).
_THREADS = max(1, min(16, os.cpu_count() or 1))


@dataclass(frozen=True)
class TensorSpec:
    name: str
    per_row: bool          # True: shape [N, D]; False: shape [D]
    loc: float = 0.0
    scale: float = 1.0
    per_sample: bool = False   # shape [B, D] (the Modulated RMSNorm's scale and shift)
    matrix: bool = False       # shape [D, Nout] (the fused GEMV's weight W)
    per_channel: bool = False  # shape [C] (GroupNorm's gamma and beta)


@dataclass(frozen=True)
class Workload:
    name: str
    kind: str              # "rms", "ln", "add", "dyt", "poly", "mod", "rms_gemv", "ln_gemv"
    N: int
    D: int
    eps: float
    tensors: Tuple[TensorSpec, ...]
    outlier_frac: float = 0.0
    outlier_gain: float = 1.0
    outlier_seed: int = 1
    note: str = ""
    B: int = 1             # "mod": samples (N / B rows each)
    scalars: Tuple[float, ...] = ()   # "dyt": (alpha,); "poly": (w1, w2, w3, b)
    Nout: int = 0          # "*_gemv": output columns (N rows of X are the batch M, D is K)
    channels: int = 0      # "gn": C (rows of X are samples of C * L values, D = C * L)
    groups: int = 0        # "gn": G
    layout: str = "ncl"    # "gn": "ncl" channels-first, "nlc" channels-last (the
                           # generated values are the channels-first ones, transposed)

    def outlier_channels(self) -> np.ndarray:
        if self.outlier_frac <= 0.0:
            return np.zeros(0, dtype=np.int64)
        k = int(np.ceil(self.outlier_frac * self.D))
        rng = np.random.default_rng(self.outlier_seed)
        return np.sort(rng.choice(self.D, k, replace=False))


def _spec(kind: str, x=(0.0, 1.0), dy=(0.0, 1.0), r=(0.0, 2.0), dh=(0.0, 0.01),
          mod=(0.0, 0.1), w=(0.0, 0.02)):
    """Tensor list in draw order for one kind of norm."""
    X = TensorSpec("X", True, *x)
    G = TensorSpec("gamma", False, 1.0, 0.1)
    B = TensorSpec("beta", False, 0.0, 0.1)
    DY = TensorSpec("dY", True, *dy)
    if kind == "rms":
        return (X, G, DY)
    if kind in ("ln", "dyt"):
        return (X, G, B, DY)
    if kind == "add":
        return (X, TensorSpec("R", True, *r), G, DY, TensorSpec("dH", True, *dh))
    if kind == "poly":
        return (X, DY)
    if kind == "mod":
        return (X, G, TensorSpec("scale", False, *mod, per_sample=True),
                TensorSpec("shift", False, *mod, per_sample=True), DY)
    if kind == "gn":
        return (X, TensorSpec("gamma", False, 1.0, 0.1, per_channel=True),
                TensorSpec("beta", False, 0.0, 0.1, per_channel=True), DY)
    W = TensorSpec("W", False, *w, matrix=True)
    if kind == "rms_gemv":
        return (X, G, W)
    if kind == "ln_gemv":
        return (X, G, B, W)
    raise ValueError(kind)


# Fixed scalar parameters of the other norms: Dynamic Tanh's alpha (the
# initial value its paper uses), and PolyNorm's weights near their usual
# initial 1/3 with a small bias.
DYT_ALPHA = (0.5,)
POLY_PARAMS = (0.35, 0.3, 0.25, 0.05)


WORKLOADS: Dict[str, Workload] = {
    w.name: w
    for w in (
        Workload("rms_17x257", "rms", 17, 257, 1e-6, _spec("rms"),
                 note="ragged width RMSNorm"),
        Workload("ln_128x1024", "ln", 128, 1024, 1e-5, _spec("ln", x=(0.5, 1.0)),
                 note="LayerNorm, offset mean"),
        Workload("rms_16384x4096", "rms", 16384, 4096, 1e-5,
                 _spec("rms", dy=(0.0, 0.01)), outlier_frac=0.01, outlier_gain=20.0,
                 note="Llama-8B training shape (8 x 2048 tokens), 1 % outlier channels"),
        Workload("add_rms_32768x8192", "add", 32768, 8192, 1e-5,
                 _spec("add", dy=(0.0, 0.01), r=(0.0, 2.0), dh=(0.0, 0.01)),
                 note="fused residual-add + RMSNorm, both cotangents"),
        Workload("rms_1048576x128", "rms", 1048576, 128, 1e-6, _spec("rms"),
                 note="per-head QK-norm, B=8 x H=32 x S=4096 rows of 128"),
        Workload("ln_16384x4096", "ln", 16384, 4096, 1e-5, _spec("ln", x=(0.5, 1.0)),
                 note="supplemental LayerNorm at the Llama shape, offset-mean distributions"),
        Workload("dyt_16384x4096", "dyt", 16384, 4096, 0.0, _spec("dyt"), scalars=DYT_ALPHA,
                 note="Dynamic Tanh in place of the norm at the Llama shape"),
        Workload("poly_16384x4096", "poly", 16384, 4096, 1e-5, _spec("poly"),
                 scalars=POLY_PARAMS, note="PolyNorm on 16384 tokens of width 4096"),
        Workload("mod_rms_16384x3072", "mod", 16384, 3072, 1e-6, _spec("mod"), B=8,
                 note="Modulated RMSNorm: 8 samples x 2048 tokens of width 3072 (a "
                      "conditioned-transformer block)"),
        Workload("gn_32x320x4096_g32", "gn", 32, 320 * 4096, 1e-5, _spec("gn", x=(0.5, 1.0)),
                 channels=320, groups=32,
                 note="GroupNorm of a diffusion U-Net's first stage: 32 images, 320 channels "
                      "of 64 x 64 positions, 32 groups"),
        Workload("gn_32x320x16384_g32", "gn", 32, 320 * 16384, 1e-5, _spec("gn", x=(0.5, 1.0)),
                 channels=320, groups=32,
                 note="the same GroupNorm at 128 x 128 positions: slices of 163,840 values, "
                      "more than one workgroup holds in registers"),
        Workload("gn_nlc_32x4096x320_g32", "gn", 32, 320 * 4096, 1e-5, _spec("gn", x=(0.5, 1.0)),
                 channels=320, groups=32, layout="nlc",
                 note="the same GroupNorm on channels-last activations (32 images of 64 x 64 "
                      "positions, 320 channels each, 32 groups)"),
        Workload("rms_gemv_4x4096x12288", "rms_gemv", 4, 4096, 1e-5, _spec("rms_gemv"),
                 Nout=12288, note="decode step: RMSNorm of 4 tokens of width 4096 fused "
                                  "into the fused Q/K/V projection (3 x 4096 columns)"),
        Workload("ln_gemv_4x4096x12288", "ln_gemv", 4, 4096, 1e-5,
                 _spec("ln_gemv", x=(0.5, 1.0)), Nout=12288,
                 note="the same decode projection behind a LayerNorm, offset-mean X"),
        Workload("rms_gemv_1x4096x14336", "rms_gemv", 1, 4096, 1e-5, _spec("rms_gemv"),
                 Nout=14336, note="single-token decode: RMSNorm into an MLP up projection "
                                  "(4096 -> 14336)"),
    )
}

# The workload the benchmark's headline line is measured on.
HEADLINE = "rms_16384x4096"


# storage names -> numpy array type of the generated arrays (bfloat16 as bits)
STORAGE = {"f16": np.float16, "bf16": np.uint16, "f32": np.float32}


def to_storage(v: np.ndarray, storage: str) -> np.ndarray:
    """Round float64 values to ``storage`` (see the recipe above)."""
    if storage == "f16":
        return v.astype(np.float16)
    if storage == "f32":
        return v.astype(np.float32)
    if storage == "bf16":
        u = np.ascontiguousarray(v, dtype=np.float32).view(np.uint32)
        # nearest, ties to even, on the 16 bits kept (the generated values are finite)
        u = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
        return u.astype(np.uint16)
    raise ValueError(storage)


def rows_per_chunk(D: int) -> int:
    return max(1, _CHUNK_ELEMS // max(int(D), 1))


def _fill_rows(seed: int, t: int, out: np.ndarray, spec: TensorSpec, outliers: np.ndarray,
               gain: float):
    n, d = out.shape
    rows = rows_per_chunk(d)

    def block(c: int):
        r0 = c * rows
        r1 = min(n, r0 + rows)
        v = np.random.default_rng([seed, t, c]).standard_normal((r1 - r0, d))
        v *= spec.scale
        v += spec.loc
        if outliers.size:
            v[:, outliers] *= gain
        if out.dtype == np.uint16:
            out[r0:r1] = to_storage(v, "bf16")
        else:
            out[r0:r1] = v  # float64 -> float16/float32 assignment rounds to nearest even

    nblocks = (n + rows - 1) // rows
    if nblocks <= 1:
        for c in range(nblocks):
            block(c)
        return
    with ThreadPoolExecutor(max_workers=min(_THREADS, nblocks)) as ex:
        list(ex.map(block, range(nblocks)))


def generate(w: Workload, seed: int = 0, N: Optional[int] = None, act: str = "f16",
             param: Optional[str] = None, cot: Optional[str] = None) -> Dict[str, np.ndarray]:
    """Materialise every input tensor of ``w`` as contiguous numpy arrays:
    X and R in storage ``act``, the cotangents dY and dH in ``cot``, gamma
    and beta in ``param`` (both default to ``act``); fp16 and float32 as
    such, bfloat16 as uint16 bit patterns.

    ``N`` overrides the row count (same distributions; the rows are a prefix
    of the full workload's rows). The float64 draws do not depend on the
    storage types, so the same seed gives the same values rounded differently.
    """
    param = act if param is None else param
    cot = act if cot is None else cot
    n = w.N if N is None else int(N)
    outliers = w.outlier_channels()
    out: Dict[str, np.ndarray] = {}
    for t, spec in enumerate(w.tensors):
        if spec.per_channel:
            z = np.random.default_rng([seed, t]).standard_normal(w.channels)
            a = to_storage(spec.loc + spec.scale * z, param)
        elif spec.matrix:
            a = np.empty((w.D, w.Nout), dtype=STORAGE[act])
            _fill_rows(seed, t, a, spec, np.zeros(0, np.int64), 1.0)
        elif spec.per_sample:
            a = np.empty((w.B, w.D), dtype=STORAGE[act])
            _fill_rows(seed, t, a, spec, np.zeros(0, np.int64), 1.0)
        elif spec.per_row:
            a = np.empty((n, w.D), dtype=STORAGE[cot if spec.name in ("dY", "dH") else act])
            _fill_rows(seed, t, a, spec, outliers if spec.name == "X" else np.zeros(0, np.int64),
                       w.outlier_gain)
        else:
            z = np.random.default_rng([seed, t]).standard_normal(w.D)
            a = to_storage(spec.loc + spec.scale * z, param)
        out[spec.name] = a
    return out


def random_case(kind: str, N: int, D: int, seed: int, x_loc: float = 0.0, x_scale: float = 1.0,
                dy_scale: float = 1.0, r_scale: float = 2.0, dh_scale: float = 0.5,
                act: str = "f16", param: Optional[str] = None, cot: Optional[str] = None,
                B: int = 1, mod_scale: float = 0.1, Nout: int = 0,
                w_scale: float = 0.02, channels: int = 0,
                groups: int = 0) -> Dict[str, np.ndarray]:
    """Inputs for an arbitrary (kind, N, D) test case with the default recipe
    (B samples for "mod", Nout output columns for "*_gemv"; the scalar
    parameters are not drawn)."""
    w = Workload(f"case_{kind}_{N}x{D}", kind, N, D, 1e-5,
                 _spec(kind, x=(x_loc, x_scale), dy=(0.0, dy_scale), r=(0.0, r_scale),
                       dh=(0.0, dh_scale), mod=(0.0, mod_scale), w=(0.0, w_scale)), B=B,
                 Nout=Nout, channels=channels, groups=groups)
    return generate(w, seed, act=act, param=param, cot=cot)


def sample_rows(N: int, k: int, seed: int = 7) -> np.ndarray:
    """Sorted sample of ``k`` distinct row indices that always contains the
    first and last rows (ragged tails live there)."""
    if k >= N:
        return np.arange(N)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, N - 1), max(0, k - 2), replace=False)
    return np.unique(np.concatenate([[0, N - 1], mid]))
