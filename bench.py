#!/usr/bin/env python3
"""Benchmark: RMSNorm forward + backward at the Llama-8B training shape
(16384 rows x 4096 columns, fp16 storage, fp32 arithmetic) on one MI355X.

One step is one pass of the whole training pair over one batch: the forward
(Y, rstd) of one batch and the backward (dX, dgamma, via the row kernel and
the column reduce) of one batch. Inputs are resident in HBM before timing.
Several buffer sets rotate so that no kernel reads data another kernel has
touched recently: step k runs the forward on set k mod S and the backward on
set (k + S/2) mod S (S >= 4), whose forward ran S/2 steps earlier, with more
than the Infinity Cache's 256 MB of traffic in between. (A backward on the
set forwarded one step earlier was measured re-reading part of it from that
cache when the forward's loads allocate there.)

Printed: one JSON line with the whole-step throughput (algorithmic HBM bytes
per second: every tensor read or written once, workspace excluded), rows/s,
per-kernel device times from HIP events on the launch stream, the roofline of
the dominant kernel, and the CPU oracle timed on this host as a baseline.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import workloads  # noqa: E402

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E peak, GB/s
_CSRC = os.path.join(ROOT, "row_wise_normalization_amd", "csrc")
# the kernel sources behind each kind's launches (the row-kernel templates,
# launch tables and planner, and the kind's own instance files)
_ROW = ("mn_kernels.hpp", "mn_kernels.hip", "mn_tables.hpp", "mn_instances.hpp")
KERNEL_SRCS = {
    "pair": _ROW + ("mn_inst_f16.hip", "mn_inst_bf16.hip", "mn_inst_f32.hip"),
    "other": _ROW + ("mn_inst_ext_f16.hip", "mn_inst_ext_bf16.hip", "mn_inst_ext_f32.hip"),
    "gn": ("mn_kernels.hpp", "mn_kernels.hip", "mn_tables.hpp", "mn_groupnorm.hpp",
           "mn_gn_instances.hpp", "mn_gn_plan.hip", "mn_gn_fwd_f16.hip", "mn_gn_bwd_f16.hip",
           "mn_gn_fwd_bf16.hip", "mn_gn_bwd_bf16.hip", "mn_gn_fwd_f32.hip", "mn_gn_bwd_f32.hip"),
    "gnl": ("mn_kernels.hpp", "mn_kernels.hip", "mn_gnl.hip"),
    "gemv": ("mn_kernels.hpp", "mn_gemv.hip"),
}


def _src_group(kind: str, layout: str = "ncl") -> str:
    if kind == "gn" and layout == "nlc":
        return "gnl"
    if kind in ("rms", "ln", "add"):
        return "pair"
    if kind in ("dyt", "poly", "mod"):
        return "other"
    return "gn" if kind == "gn" else "gemv"
SIZE = {"f16": 2, "bf16": 2, "f32": 4}


def alg_bytes(kind: str, N: int, D: int, act: str = "f16", param: str = "f16",
              cot: str = "f16", dxt: str = "f16", B: int = 1, C: int = 0, G: int = 0):
    """Algorithmic bytes (each tensor read or written once) of the forward and
    the backward (row kernel and column reduce together): activations X, R,
    Y, H of `act`, gamma/beta of `param`, cotangents dY, dH of `cot`, dX of
    `dxt`, fp32 statistics and parameter gradients."""
    a, p, c, o = SIZE[act], SIZE[param], SIZE[cot], SIZE[dxt]
    nd = N * D
    if kind == "rms":
        fwd = 2 * a * nd + p * D + 4 * N                      # X, gamma -> Y, rstd
        bwd = (a + c + o) * nd + (p + 4) * D + 4 * N          # X, dY, gamma, rstd -> dX, dgamma
    elif kind == "ln":
        fwd = 2 * a * nd + 2 * p * D + 8 * N                  # + beta, mean
        bwd = (a + c + o) * nd + (p + 8) * D + 8 * N          # + mean, dbeta
    elif kind == "dyt":
        fwd = 2 * a * nd + 2 * p * D + 4                      # X, gamma, beta, alpha -> Y
        bwd = (a + c + o) * nd + (p + 8) * D + 8              # -> dX, dgamma, dbeta, dalpha
    elif kind == "poly":
        fwd = 2 * a * nd + 16 + 12 * N                        # X, params -> Y, rstd [N][3]
        bwd = (a + c + o) * nd + 32 + 12 * N                  # + rstd -> dX, dparams
    elif kind == "mod":
        fwd = 2 * a * nd + p * D + 2 * a * B * D + 4 * N      # + scale, shift [B][D]
        bwd = (a + c + o) * nd + (p + 4) * D + (a + 8) * B * D + 4 * N
    elif kind == "gn":                                        # N samples of D = C * L values
        fwd = 2 * a * nd + 2 * p * C + 8 * N * G              # X, gamma, beta -> Y, mean, rstd
        bwd = (a + c + o) * nd + p * C + 8 * N * G + 8 * C    # -> dX, dgamma, dbeta
    else:
        fwd = 4 * a * nd + p * D + 4 * N                      # X, R -> H, Y
        bwd = (2 * a + 2 * c + o) * nd + (p + 4) * D + 4 * N  # X, R, dY, dH -> dX
    return fwd, bwd


def gemv_bytes(M: int, K: int, N: int, act: str = "f16", param: str = "f16", ln: bool = False):
    """Algorithmic bytes of one fused norm + GEMV call: X [M, K], gamma (and
    beta) [K], W [K, N] read once, Y [M, N] written once; the fp32 partials
    of the K slices are workspace and not counted."""
    a, p = SIZE[act], SIZE[param]
    return a * (M * K + K * N + M * N) + p * K * (2 if ln else 1)


# Untimed steps before the counted warm-up: the GPU idles while the host
# generates the inputs, and its clocks take longer to come back up than a
# few steps last (20 timed steps after 5 warm-up steps measured 1-2 % below
# 200 after 50 on one box).
SETTLE_S = 0.2


def settle(run_step, torch) -> int:
    """Run untimed steps for at least SETTLE_S seconds; returns their count."""
    t0, n = time.perf_counter(), 0
    while True:
        for _ in range(8):
            run_step(n)
            n += 1
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= SETTLE_S:
            return n


WARMUP_NOTE = (f"the counted warm-up steps follow {SETTLE_S} s of untimed steps (clocks settle "
               "after the host-side input generation)")


def back_set(k: int, S: int) -> int:
    """Buffer set of step k's backward: the one forwarded S/2 steps ago."""
    return (k + S // 2) % S


def kernel_hash(kind: str = "rms", layout: str = "ncl") -> str:
    """Hash of the kernel sources behind `kind`'s launches."""
    h = hashlib.sha256()
    for name in KERNEL_SRCS[_src_group(kind, layout)]:
        with open(os.path.join(_CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, kernel):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    only if it was taken on the current kernel source; `kernel` is a label,
    or a tuple of labels whose bytes are added (a direction that runs as
    several kernels)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    w = workloads.WORKLOADS[workload]
    if t.get("kernel_source_sha256_16") != kernel_hash(w.kind, w.layout):
        return None
    names = (kernel,) if isinstance(kernel, str) else tuple(kernel)
    vals = [t.get("kernels", {}).get(n, {}).get("hbm_bytes_per_launch") for n in names]
    return None if any(v is None for v in vals) else sum(vals)


# GroupNorm backwards that run as three kernels and the column reduce (the
# channels-last layout, and slices larger than one workgroup holds)
GN_MULTI_BACKWARD = ("backward_sums", "backward_merge", "backward_apply", "reduce_partials")


def backward_traffic_labels(workload: str):
    """The profile labels whose HBM bytes make up one backward call's traffic
    in bench_other's roofline: the row kernel, or every kernel of a
    multi-kernel GroupNorm backward."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if os.path.exists(path):
        with open(path) as f:
            ks = json.load(f).get("kernels", {})
        if "backward_rows" not in ks and all(k in ks for k in GN_MULTI_BACKWARD):
            return GN_MULTI_BACKWARD
    return "backward_rows"


class HipEvent:
    """A HIP event created with hipEventDisableSystemFence through the HIP
    runtime this process already loaded: its record carries no system-scope
    cache writeback/invalidate, so bracketing a kernel does not slow the
    kernels around it (HIP documents the flag for timing-only events)."""

    _lib = None
    DISABLE_SYSTEM_FENCE = 0x20000000

    @classmethod
    def lib(cls):
        if cls._lib is None:
            path = None
            with open("/proc/self/maps") as f:
                for line in f:
                    if "libamdhip64" in line:
                        path = line.split()[-1]
                        break
            if path is None:
                raise RuntimeError("HIP runtime not loaded")
            L = ctypes.CDLL(path)
            L.hipEventCreateWithFlags.argtypes = [ctypes.POINTER(ctypes.c_void_p), ctypes.c_uint]
            L.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
            L.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                              ctypes.c_void_p]
            L.hipEventDestroy.argtypes = [ctypes.c_void_p]
            cls._lib = L
        return cls._lib

    def __init__(self):
        self.h = ctypes.c_void_p()
        rc = self.lib().hipEventCreateWithFlags(ctypes.byref(self.h), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")

    def record(self, stream):
        rc = self.lib().hipEventRecord(self.h, ctypes.c_void_p(stream.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"hipEventRecord failed ({rc})")

    def elapsed_ms(self, end: "HipEvent") -> float:
        ms = ctypes.c_float()
        rc = self.lib().hipEventElapsedTime(ctypes.byref(ms), self.h, end.h)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return float(ms.value)

    def __del__(self):
        if self._lib is not None and self.h:
            self._lib.hipEventDestroy(self.h)


def _oracle_pass(w, d, lo: int, hi: int):
    """The oracle's forward and backward over rows lo..hi-1 of the workload
    (for the Modulated RMSNorm whole samples, for GroupNorm samples);
    returns the parameter gradients of those rows."""
    import oracle

    X, g, dY = d["X"][lo:hi], d.get("gamma"), d["dY"][lo:hi]
    if w.kind == "dyt":
        oracle.dyt_forward(X, w.scalars[0], g, d["beta"])
        return oracle.dyt_backward(X, w.scalars[0], g, dY)[2]
    if w.kind == "poly":
        oracle.polynorm_forward(X, w.scalars[:3], w.scalars[3], w.eps)
        return oracle.polynorm_backward(X, w.scalars[:3], dY, w.eps)[1]
    if w.kind == "mod":
        S = w.N // w.B
        sc, sh = d["scale"][lo // S:hi // S], d["shift"][lo // S:hi // S]
        oracle.modrms_forward(X, g, sc, sh, w.eps)
        return oracle.modrms_backward(X, g, sc, dY, w.eps)[1]
    if w.kind == "gn":
        shp = (hi - lo, w.channels, w.D // w.channels)
        oracle.groupnorm_forward(X.reshape(shp), g, d["beta"], w.groups, w.eps)
        return oracle.groupnorm_backward(X.reshape(shp), g, dY.reshape(shp), w.groups, w.eps)[1]
    if w.kind == "rms":
        oracle.rmsnorm_forward(X, g, w.eps)
        return oracle.rmsnorm_backward(X, g, dY, w.eps)[1]
    if w.kind == "ln":
        oracle.layernorm_forward(X, g, d["beta"], w.eps)
        return oracle.layernorm_backward(X, g, dY, w.eps)[1]
    R = d["R"][lo:hi]
    oracle.add_rmsnorm_forward(X, R, g, w.eps)
    return oracle.add_rmsnorm_backward(X, R, g, dY, d["dH"][lo:hi], w.eps)[1]


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_threads() -> int:
    """Host threads for the threaded baseline: the CPUs this process may run
    on, at most 16 (one GPU's share of its host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline(w, d, budget_s: float, types=("f16",) * 4):
    """The oracle (C, fp64) on this host, timed on full forward + backward
    passes over all rows of the same workload: first on one core (a third of
    the budget), then with the rows split into static contiguous chunks over
    cpu_threads() host threads (the oracle's ctypes calls release the
    interpreter lock), the chunks' parameter gradients added in chunk order;
    each repeated until its share of the budget is spent (at least once).
    The threaded figure is the reported value, the one-core one sits beside
    it."""
    from concurrent.futures import ThreadPoolExecutor

    fwd_b, bwd_b = alg_bytes(w.kind, w.N, w.D, *types, B=w.B, C=w.channels, G=w.groups)
    align = w.N // w.B if w.kind == "mod" else 1

    def timed(fn, budget):
        t0 = time.perf_counter()
        reps = 0
        while True:
            fn()
            reps += 1
            el = time.perf_counter() - t0
            if el >= budget:
                return reps, el

    reps1, el1 = timed(lambda: _oracle_pass(w, d, 0, w.N), budget_s / 3)
    T = cpu_threads()
    per = -(-w.N // T)
    per = -(-per // align) * align
    chunks = [(lo, min(w.N, lo + per)) for lo in range(0, w.N, per)]
    with ThreadPoolExecutor(T) as ex:
        def threaded():
            parts = list(ex.map(lambda c: _oracle_pass(w, d, c[0], c[1]), chunks))
            total = parts[0]
            for p in parts[1:]:
                total = total + p
            return total
        repsT, elT = timed(threaded, budget_s - budget_s / 3)
    one = el1 / reps1
    many = elT / repsT
    return {
        "value": round((fwd_b + bwd_b) / many / 1e9, 4),
        "unit": "GB/s",
        "rows_per_s": round(w.N / many, 1),
        "cores": T,
        "cpu_model": _cpu_model(),
        "kind": "oracle",
        "sample": f"{repsT} full forward+backward passes over all {w.N}x{w.D} rows in "
                  f"{len(chunks)} contiguous row chunks on {T} threads ({elT:.1f} s), C fp64",
        "single_core": {"value": round((fwd_b + bwd_b) / one / 1e9, 4), "unit": "GB/s",
                        "rows_per_s": round(w.N / one, 1),
                        "sample": f"{reps1} full passes on one thread ({el1:.1f} s)"},
    }


# The shapes of the pages' binary32 LayerNorm forward timings (rows x width).
PAGES_SHAPES = [(1, 127), (17, 257), (128, 1024), (64, 4096)]


def pages_context(torch, mn):
    """Binary32 LayerNorm forward at the shapes the pages time, measured the
    way they describe their table: inputs resident on the device, output
    preallocated, 100 ms of warmup, then the median over 11 windows of
    100 ms of the host-wall time per synchronized call. Reported both
    through the Python binding (tensor checks included) and as a direct
    C-ABI call with prepared arguments, next to the device time per call
    from events. Context only: the pages measure another GPU and API."""
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    L = mn.lib()
    out = []
    for N, D in PAGES_SHAPES:
        d = workloads.random_case("ln", N, D, seed=0, x_loc=0.5, act="f32", param="f32")
        X = torch.from_numpy(d["X"]).to(dev)
        g = torch.from_numpy(d["gamma"]).to(dev)
        b = torch.from_numpy(d["beta"]).to(dev)
        Y = torch.empty_like(X)
        mean = torch.empty(N, dtype=torch.float32, device=dev)
        rstd = torch.empty(N, dtype=torch.float32, device=dev)
        eps = 1e-5

        def via_binding():
            mn.mn_layernorm_forward_ex(X, g, b, Y, mean, rstd, eps, stream)

        cargs = [ctypes.c_void_p(t.data_ptr()) for t in (X, g, b, Y, mean, rstd)]
        craw = (N, D, ctypes.c_float(eps), mn.MN_F32, mn.MN_F32, ctypes.c_void_p(stream.cuda_stream))
        fn = L.mn_layernorm_forward_ex

        def direct():
            if fn(*cargs, *craw) != 0:
                raise RuntimeError("mn_layernorm_forward_ex failed")

        def window(call, seconds=0.1):
            n = 0
            t0 = time.perf_counter()
            while True:
                call()
                stream.synchronize()
                n += 1
                el = time.perf_counter() - t0
                if el >= seconds:
                    return el / n

        res = {"rows": N, "width": D}
        for name, call in (("binding", via_binding), ("direct", direct)):
            window(call)
            res[f"host_wall_p50_us_{name}"] = round(
                float(np.median([window(call) for _ in range(11)])) * 1e6, 3)
        e0, e1 = HipEvent(), HipEvent()
        e0.record(stream)
        for _ in range(1000):
            direct()
        e1.record(stream)
        stream.synchronize()
        res["device_us_per_call_back_to_back"] = round(e0.elapsed_ms(e1), 3)
        out.append(res)
    print(json.dumps({
        "metric": "host-wall us per binary32 LayerNorm forward call (p50 of 11 x 100 ms windows, "
                  "synchronized calls)",
        "unit": "us", "higher_is_better": False, "data": "synthetic", "dtype": "f32",
        "shapes": out, "device": torch.cuda.get_device_name(dev),
    }), flush=True)


# --- rocprofv3 summaries ------------------------------------------------------

# Kernel-name fragments -> (label, which algorithmic byte count applies).
PROFILE_KERNELS = (("gnl_sum_kernel<0", "forward_sums"), ("gnl_stats_kernel", "forward_stats"),
                   ("gnl_apply_kernel<0", "forward_apply"), ("gnl_sum_kernel<1", "backward_sums"),
                   ("gnl_merge_kernel", "backward_merge"), ("gnl_apply_kernel<1", "backward_apply"),
                   ("gn_chunk_stats_kernel", "forward_stats"),
                   ("gn_stats_merge_kernel", "forward_merge"), ("gn_unit_y_kernel", "forward_apply"),
                   ("gn_unit_sums_kernel", "backward_sums"),
                   ("gn_unit_merge_kernel", "backward_merge"),
                   ("gn_unit_dx_kernel", "backward_apply"),
                   ("gn_fwd_kernel", "forward"), ("gn_bwd_kernel", "backward_rows"),
                   ("fwd_kernel", "forward"), ("bwd_kernel", "backward_rows"),
                   ("reduce_kernel", "reduce_partials"), ("gemv_mfma_kernel", "gemv"),
                   ("gemv_kernel", "gemv"))
COPY_KERNEL = "__amd_rocclr_copyBuffer"


def _csvs(root: str, suffix: str):
    """Every CSV under `root` whose name ends with `suffix` (rocprofv3 puts
    them in the output directory or in host/process subdirectories)."""
    import glob
    return sorted(glob.glob(os.path.join(root, "**", f"*{suffix}"), recursive=True))


def _read_csv(path: str):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def profile_commands(workload: str, prefix: str, extra: str = "--cpu-budget 0"):
    """The three rocprofv3 runs a summary is made from (run from /tmp with
    TMPDIR=/tmp; R is the repository root)."""
    b = f"python3 $R/bench.py --workload {workload}"
    return [
        f"rocprofv3 --kernel-trace --stats --output-format csv -d {prefix}_trace -o trace -- "
        f"{b} {extra}",
        f"rocprofv3 --pmc FETCH_SIZE --output-format csv -d {prefix}_fetch -o fetch -- "
        f"{b} --steps 4 --warmup 2 --cpu-budget 0",
        f"rocprofv3 --pmc WRITE_SIZE --output-format csv -d {prefix}_write -o write -- "
        f"{b} --steps 4 --warmup 2 --cpu-budget 0",
        f"python3 $R/bench.py --workload {workload} --summarize-profile {prefix}",
    ]


def summarize_profile(workload: str, prefix: str, out_dir: str = None):
    """Turn the three rocprofv3 runs of profile_commands() into
    profiles/traffic_<workload>.json and profiles/<workload>_trace_and_traffic.md.

    HBM bytes per launch come from the TCC counters FETCH_SIZE and
    WRITE_SIZE (KiB per dispatch, summed over the channels). They are
    calibrated against the HIP runtime's own device copy kernel, which
    bench.py issues when it clones its largest inputs (a copy of known size:
    N * D elements, or the weight matrix for the fused GEMV): the factor is
    the copied bytes over the counter's KiB * 1024. On gfx950 FETCH_SIZE
    reads half the copied bytes (factor about 2.0) and WRITE_SIZE all of
    them (factor 1.0)."""
    import statistics
    w = workloads.WORKLOADS[workload]
    out_dir = out_dir or os.path.join(ROOT, "profiles")
    stats_p = _csvs(prefix + "_trace", "kernel_stats.csv")
    trace_p = _csvs(prefix + "_trace", "kernel_trace.csv")
    fetch_p = _csvs(prefix + "_fetch", "counter_collection.csv")
    write_p = _csvs(prefix + "_write", "counter_collection.csv")
    if not (stats_p and fetch_p and write_p):
        raise SystemExit(f"rocprofv3 CSVs not found under {prefix}_trace/_fetch/_write")
    stats = _read_csv(stats_p[0])

    def counter(paths, name):
        d = {}
        for p in paths:
            for r in _read_csv(p):
                if r.get("Counter_Name") == name:
                    d.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return d

    fetch = counter(fetch_p, "FETCH_SIZE")
    write = counter(write_p, "WRITE_SIZE")
    gemv = w.kind.endswith("gemv")
    copy_bytes = w.D * w.Nout * SIZE["f16"] if gemv else w.N * w.D * SIZE["f16"]

    def calib(d):
        vals = [v for k, vs in d.items() if k.startswith(COPY_KERNEL) for v in vs]
        top = max(vals)
        return statistics.median([v for v in vals if v > 0.9 * top])

    cf, cw = calib(fetch), calib(write)
    sf, sw = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    if gemv:
        alg = {"gemv": gemv_bytes(w.N, w.D, w.Nout, ln=w.kind == "ln_gemv")}
    elif w.layout == "nlc":
        # channels-last GroupNorm: each direction is three kernels; the
        # algorithmic bytes belong to the direction, not to one of them
        alg = {k: None for k in ("forward_sums", "forward_stats", "forward_apply",
                                 "backward_sums", "backward_merge", "backward_apply",
                                 "reduce_partials")}
    else:
        fb, bb = alg_bytes(w.kind, w.N, w.D, B=w.B, C=w.channels, G=w.groups)
        alg = {"forward": fb, "backward_rows": bb, "reduce_partials": None}
        if w.kind == "gn":
            # slices larger than one workgroup holds: three kernels per
            # direction, the algorithmic bytes again the direction's
            alg.update({k: None for k in ("forward_stats", "forward_merge", "forward_apply",
                                          "backward_sums", "backward_merge", "backward_apply")})
    # resources of each kernel from the per-dispatch trace (first dispatch)
    res = {}
    for p in trace_p:
        for r in _read_csv(p):
            n = r.get("Kernel_Name", "")
            if n and n not in res:
                res[n] = {k: r[k] for k in ("VGPR_Count", "Accum_VGPR_Count", "SGPR_Count",
                                            "LDS_Block_Size", "Scratch_Size", "Workgroup_Size_X",
                                            "Grid_Size_X") if k in r}
    # the compiler's resource usage of each kernel, recorded by the build
    built = {}
    rpath = os.path.join(ROOT, "row_wise_normalization_amd", "_build", "kernel_resources.json")
    if os.path.exists(rpath):
        with open(rpath) as f:
            built = json.load(f)
    out = {"workload": workload, "kernel_source_sha256_16": kernel_hash(w.kind, w.layout),
           "calibration": {"kernel": COPY_KERNEL, "bytes_read": copy_bytes,
                           "bytes_written": copy_bytes, "FETCH_SIZE_KiB_median": cf,
                           "WRITE_SIZE_KiB_median": cw, "fetch_scale": sf, "write_scale": sw},
           "commands": profile_commands(workload, "$R/gpurun_out/prof_" + workload),
           "kernels": {}}
    for s in stats:
        n = s["Name"]
        label = next((lab for frag, lab in PROFILE_KERNELS if frag in n), None)
        if label is None or label not in alg:
            continue
        fv, wv = fetch.get(n, []), write.get(n, [])
        fr = statistics.median(fv) * 1024 * sf if fv else None
        wr = statistics.median(wv) * 1024 * sw if wv else None
        avg_ns = float(s["AverageNs"])
        a = alg[label]
        out["kernels"][label] = {
            "name": n, "calls": int(s["Calls"]), "avg_ns": avg_ns, "min_ns": int(s["MinNs"]),
            "max_ns": int(s["MaxNs"]), "fetch_bytes_per_launch": fr,
            "write_bytes_per_launch": wr,
            "hbm_bytes_per_launch": (fr + wr) if fr is not None and wr is not None else None,
            "algorithmic_bytes_per_launch": a,
            "algorithmic_GBps_at_avg": (a / (avg_ns * 1e-9) / 1e9) if a else None,
            "resources": res.get(n, {}),
            "compiler_resources": built.get(n, {}),
        }
    with open(os.path.join(out_dir, f"traffic_{workload}.json"), "w") as f:
        json.dump(out, f, indent=1)
    with open(stats_p[0]) as f:
        stats_text = f.read().strip()
    md = [f"# {workload}: rocprofv3 kernel trace and HBM traffic", "",
          f"Kernel sources: sha256[:16] = `{out['kernel_source_sha256_16']}` (the kernel templates, "
          "launch tables and instance files, as hashed by bench.py).", "",
          "## Commands (run from /tmp with TMPDIR=/tmp; R = repository root)", "", "```",
          *out["commands"], "```", "", "## Kernel statistics (trace_kernel_stats.csv)", "", "```",
          stats_text, "```", "", "## HBM traffic per launch (FETCH_SIZE, WRITE_SIZE)", "",
          f"Calibration: the runtime's device copy `{COPY_KERNEL}` of {copy_bytes:,} bytes reads "
          f"FETCH_SIZE = {cf:.1f} KiB and WRITE_SIZE = {cw:.1f} KiB per dispatch, so FETCH_SIZE is "
          f"scaled by {sf:.4f} and WRITE_SIZE by {sw:.4f} to bytes.", "",
          "| kernel | avg us | algorithmic bytes | fetched bytes | written bytes | measured / "
          "algorithmic | algorithmic GB/s at avg |", "|---|---:|---:|---:|---:|---:|---:|"]
    for label, k in out["kernels"].items():
        a, h, r = k["algorithmic_bytes_per_launch"], k["hbm_bytes_per_launch"], k["resources"]
        alg_s = f"{a:,}" if a else "-"
        ratio = f"{h / a:.4f}" if a and h else "-"
        gbs = f"{k['algorithmic_GBps_at_avg']:.0f}" if a else "-"
        fetched = f"{k['fetch_bytes_per_launch'] or 0:,.0f}"
        written = f"{k['write_bytes_per_launch'] or 0:,.0f}"
        md.append(f"| {label} (`{k['name'].split('(')[0]}`) | {k['avg_ns'] / 1000:.2f} | {alg_s} | "
                  f"{fetched} | {written} | {ratio} | {gbs} |")
    md += ["", "## Kernel resources (compiler remarks at build time; launch shape from the trace)",
           "", "| kernel | VGPRs | AGPRs | SGPRs | LDS bytes / block | scratch bytes / lane | "
           "occupancy (waves / SIMD) | workgroup | grid |", "|---|---:|---:|---:|---:|---:|---:|---:|---:|"]
    for label, k in out["kernels"].items():
        c, r = k["compiler_resources"], k["resources"]
        md.append(f"| {label} | {c.get('VGPRs', '?')} | {c.get('AGPRs', '?')} | "
                  f"{c.get('TotalSGPRs', '?')} | {c.get('LDS Size [bytes/block]', '?')} | "
                  f"{c.get('ScratchSize [bytes/lane]', '?')} | "
                  f"{c.get('Occupancy [waves/SIMD]', '?')} | {r.get('Workgroup_Size_X', '?')} | "
                  f"{r.get('Grid_Size_X', '?')} |")
    md.append("")
    with open(os.path.join(out_dir, f"{workload}_trace_and_traffic.md"), "w") as f:
        f.write("\n".join(md) + "\n")
    print("\n".join(md))


NORM_NAMES = {"rms": "RMSNorm", "ln": "LayerNorm", "add": "fused add + RMSNorm",
              "dyt": "Dynamic Tanh", "poly": "PolyNorm", "mod": "Modulated RMSNorm",
              "rms_gemv": "fused RMSNorm + GEMV", "ln_gemv": "fused LayerNorm + GEMV",
              "gn": "GroupNorm"}


def bench_gemv(args, w, torch, mn, act, param):
    """Fused RMSNorm / LayerNorm + GEMV (inference): one step is one fused
    call Y = Norm(X) @ W. Several copies of W rotate (each step reads a
    different one, more bytes than the Infinity Cache holds), events bracket
    every call on the launch stream."""
    M, K, N = w.N, w.D, w.Nout
    ln = w.kind == "ln_gemv"
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}
    print(f"[bench] {w.name}: generating inputs", file=sys.stderr, flush=True)
    d = workloads.generate(w, act=act, param=param)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    def upload(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    up = {k: upload(v) for k, v in d.items()}
    S = max(4, args.sets)
    nb = mn.norm_gemv_workspace_bytes(M, N, K)
    sets = [{"X": up["X"].clone(), "W": up["W"] if s == 0 else up["W"].clone(),
             "Y": torch.empty(M, N, dtype=tdt[act], device=dev),
             "ws": torch.zeros(nb // 4, dtype=torch.float32, device=dev)} for s in range(S)]
    beta = up.get("beta")

    def call(b):
        mn.mn_fused_norm_gemv_ex(b["X"], up["gamma"], b["W"], b["Y"], w.eps, b["ws"],
                                 beta=beta, stream=stream)

    Ks, Wu = args.steps, args.warmup
    nbytes = gemv_bytes(M, K, N, act, param, ln)
    settle(lambda k: call(sets[k % S]), torch)
    for k in range(Wu):
        call(sets[k % S])
    torch.cuda.synchronize()
    ev = [(HipEvent(), HipEvent()) for _ in range(Ks)]
    t0 = time.perf_counter()
    for k in range(Ks):
        ev[k][0].record(stream); call(sets[(Wu + k) % S]); ev[k][1].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / Ks
    call_ms = float(np.mean([a.elapsed_ms(b) for a, b in ev]))
    gbs = nbytes / (ms_step * 1e-3) / 1e9
    achieved = nbytes / (call_ms * 1e-3) / 1e9
    cpu = None
    if args.cpu_budget > 0:
        import oracle
        print(f"[bench] cpu baseline (oracle, {args.cpu_budget:.0f} s budget)", file=sys.stderr,
              flush=True)
        t = time.perf_counter()
        reps = 0
        while True:
            oracle.norm_gemv(d["X"], d["gamma"], d["W"], w.eps, beta=d.get("beta"))
            reps += 1
            el = time.perf_counter() - t
            if el >= args.cpu_budget:
                break
        cpu = {"value": round(nbytes * reps / el / 1e9, 4), "unit": "GB/s",
               "calls_per_s": round(reps / el, 3), "cores": 1, "kind": "oracle",
               "sample": f"{reps} full {M}x{K}x{N} calls ({el:.1f} s), single-threaded C fp64"}
    line = {
        "metric": f"achieved HBM GB/s (% of peak) for the fused norm + GEMV, "
                  f"{NORM_NAMES[w.kind]} {M}x{K} @ {K}x{N}",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": Ks, "warmup": Wu, "warmup_note": WARMUP_NOTE,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "M": M, "K": K, "N": N, "eps": w.eps, "io_dtype": act,
                   "param_dtype": param, "norm": NORM_NAMES[w.kind],
                   "step": "one fused call (a single launch: W tiles, the K slices of each "
                           "column tile added by its last block)", "weight_sets": S},
        "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "calls_per_s": round(1e3 / ms_step, 1),
        "kernels_ms": {"fused_call": round(call_ms, 5)},
        "roofline": {"bound": "hbm", "kernel": "fused norm + GEMV launch",
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": (measured_traffic(w.name, "gemv")
                                 if (act, param) == ("f16", "f16") else None),
                     "traffic_kernel": "gemv"},
        "cpu_baseline": cpu,
        "device": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(line), flush=True)


def bench_other(args, w, torch, mn, act, param, dxt):
    """Dynamic Tanh, PolyNorm, Modulated RMSNorm or GroupNorm: one step is the
    forward of one batch and the whole backward (row kernel and parameter
    reduction) of another, with rotating buffer sets as for the training
    pair; events bracket the forward and the backward call separately."""
    N, D, kind = w.N, w.D, w.kind
    C, G = w.channels, w.groups
    nlc = kind == "gn" and w.layout == "nlc"
    shp = ((N, D // C, C) if nlc else (N, C, D // C)) if kind == "gn" else (N, D)
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}
    print(f"[bench] {w.name}: generating inputs", file=sys.stderr, flush=True)
    d = workloads.generate(w, act=act, param=param)
    # the device copy of a channels-last workload holds X and dY transposed;
    # the oracle's CPU baseline keeps the channels-first arrays
    dd = dict(d)
    if nlc:
        for k in ("X", "dY"):
            dd[k] = np.ascontiguousarray(d[k].reshape(N, C, D // C).swapaxes(1, 2))
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    def upload(a):
        if a.dtype == np.uint16:
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    up = {k: upload(v) for k, v in dd.items()}
    scal = torch.tensor(np.asarray(w.scalars, np.float32), device=dev)
    S = max(4, args.sets)
    sets = []
    for s in range(S):
        b = {"X": (up["X"] if s == 0 else up["X"].clone()).view(shp),
             "dY": (up["dY"] if s == 0 else up["dY"].clone()).view(shp),
             "Y": torch.empty(shp, dtype=tdt[act], device=dev),
             "dX": torch.empty(shp, dtype=tdt[dxt], device=dev)}
        if kind == "gn":
            nb = (mn.groupnorm_nlc_workspace_bytes(N, D // C, C, G) if nlc
                  else mn.groupnorm_workspace_bytes(N, C, D // C, G))
            b["ws"] = torch.empty(nb // 4, dtype=torch.float32, device=dev)
        else:
            kcode = {"dyt": mn.MN_DYT, "poly": mn.MN_POLYNORM, "mod": mn.MN_MOD_RMSNORM}[kind]
            b["ws"] = mn.new_workspace(kcode, N, D, dev, B=w.B)
        if kind == "gn":
            b.update(mean=torch.empty(N, G, dtype=torch.float32, device=dev),
                     rstd=torch.empty(N, G, dtype=torch.float32, device=dev),
                     dg=torch.empty(C, dtype=torch.float32, device=dev),
                     db=torch.empty(C, dtype=torch.float32, device=dev))
        elif kind == "dyt":
            b.update(da=torch.empty(1, dtype=torch.float32, device=dev),
                     dg=torch.empty(D, dtype=torch.float32, device=dev),
                     db=torch.empty(D, dtype=torch.float32, device=dev))
        elif kind == "poly":
            b.update(rstd=torch.empty(N, 3, dtype=torch.float32, device=dev),
                     dp=torch.empty(4, dtype=torch.float32, device=dev))
        else:
            b.update(rstd=torch.empty(N, dtype=torch.float32, device=dev),
                     dg=torch.empty(D, dtype=torch.float32, device=dev),
                     dsc=torch.empty(w.B, D, dtype=torch.float32, device=dev),
                     dsh=torch.empty(w.B, D, dtype=torch.float32, device=dev))
        sets.append(b)

    def fwd(b):
        if nlc:
            mn.mn_groupnorm_nlc_forward_ex(b["X"], up["gamma"], up["beta"], b["Y"], b["mean"],
                                           b["rstd"], G, w.eps, b["ws"], stream)
        elif kind == "gn":
            mn.mn_groupnorm_forward_ex(b["X"], up["gamma"], up["beta"], b["Y"], b["mean"],
                                       b["rstd"], G, w.eps, stream)
        elif kind == "dyt":
            mn.mn_dyt_forward_ex(b["X"], scal, up["gamma"], up["beta"], b["Y"], stream)
        elif kind == "poly":
            mn.mn_polynorm_forward_ex(b["X"], scal, b["Y"], b["rstd"], w.eps, stream)
        else:
            mn.mn_mod_rmsnorm_forward_ex(b["X"], up["gamma"], up["scale"], up["shift"], b["Y"],
                                         b["rstd"], w.eps, stream)

    def bwd(b):
        if nlc:
            mn.mn_groupnorm_nlc_backward_ex(b["X"], up["gamma"], b["mean"], b["rstd"], b["dY"],
                                            b["dX"], b["dg"], b["db"], G, b["ws"], stream)
        elif kind == "gn":
            mn.mn_groupnorm_backward_ex(b["X"], up["gamma"], b["mean"], b["rstd"], b["dY"],
                                        b["dX"], b["dg"], b["db"], G, b["ws"], stream)
        elif kind == "dyt":
            mn.mn_dyt_backward_ex(b["X"], scal, up["gamma"], b["dY"], b["dX"], b["da"], b["dg"],
                                  b["db"], b["ws"], stream)
        elif kind == "poly":
            mn.mn_polynorm_backward_ex(b["X"], scal, b["rstd"], b["dY"], b["dX"], b["dp"],
                                       b["ws"], stream)
        else:
            mn.mn_mod_rmsnorm_backward_ex(b["X"], up["gamma"], up["scale"], b["rstd"], b["dY"],
                                          b["dX"], b["dg"], b["dsc"], b["dsh"], b["ws"], stream)

    K, W = args.steps, args.warmup
    fwd_b, bwd_b = alg_bytes(kind, N, D, act, param, act, dxt, B=w.B, C=C, G=G)
    for b in sets:
        fwd(b)
    settle(lambda k: (fwd(sets[k % S]), bwd(sets[back_set(k, S)])), torch)
    for k in range(W):
        fwd(sets[k % S]); bwd(sets[back_set(k, S)])
    torch.cuda.synchronize()
    ev = [[HipEvent() for _ in range(3)] for _ in range(K)]
    t0 = time.perf_counter()
    for k in range(K):
        e = ev[k]
        e[0].record(stream); fwd(sets[(W + k) % S]); e[1].record(stream)
        bwd(sets[back_set(W + k, S)]); e[2].record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / K
    fwd_ms = float(np.mean([e[0].elapsed_ms(e[1]) for e in ev]))
    bwd_ms = float(np.mean([e[1].elapsed_ms(e[2]) for e in ev]))
    gbs = (fwd_b + bwd_b) / (ms_step * 1e-3) / 1e9
    achieved = bwd_b / (bwd_ms * 1e-3) / 1e9
    cpu = None
    if args.cpu_budget > 0:
        print(f"[bench] cpu baseline (oracle, {args.cpu_budget:.0f} s budget)", file=sys.stderr,
              flush=True)
        cpu = cpu_baseline(w, d, args.cpu_budget, (act, param, act, dxt))
    tlab = backward_traffic_labels(w.name)
    line = {
        "metric": f"achieved HBM GB/s (% of peak) + rows/s for norm fwd+bwd, "
                  f"{NORM_NAMES[kind]} {'x'.join(str(v) for v in shp)}",
        "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W, "warmup_note": WARMUP_NOTE,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": w.name, "N": N, "D": D, "eps": w.eps, "io_dtype": act,
                   "param_dtype": param, "dx_dtype": dxt, "norm": NORM_NAMES[kind],
                   "samples": w.B, "scalars": list(w.scalars), "channels": C, "groups": G,
                   "layout": w.layout if kind == "gn" else None,
                   "step": "forward + backward (row kernel and parameter reduction)",
                   "buffer_sets": S},
        "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "rows_per_s": round(N / (ms_step * 1e-3), 1),
        "kernels_ms": {"forward": round(fwd_ms, 5), "backward": round(bwd_ms, 5)},
        "kernel_gbs": {"forward": round(fwd_b / (fwd_ms * 1e-3) / 1e9, 1),
                       "backward": round(bwd_b / (bwd_ms * 1e-3) / 1e9, 1)},
        "roofline": {"bound": "hbm",
                     "kernel": ("backward (row kernel + reduce)" if isinstance(tlab, str)
                                else "backward (sums, merge and apply kernels + reduce)"),
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": (measured_traffic(w.name, tlab)
                                 if (act, param, dxt) == ("f16",) * 3 else None),
                     "traffic_kernel": tlab if isinstance(tlab, str) else " + ".join(tlab)},
        "cpu_baseline": cpu,
        "device": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(line), flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=workloads.HEADLINE, choices=sorted(workloads.WORKLOADS))
    ap.add_argument("--sets", type=int, default=4, help="rotating buffer sets")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work for the CPU baseline (0: skip)")
    ap.add_argument("--act", default="f16", choices=sorted(SIZE),
                    help="storage of X, R, Y, H (default fp16, the workloads' own)")
    ap.add_argument("--param", default=None, choices=sorted(SIZE),
                    help="storage of gamma, beta (default: --act)")
    ap.add_argument("--cot", default=None, choices=sorted(SIZE),
                    help="storage of dY, dH (default: --act)")
    ap.add_argument("--dx", default=None, choices=sorted(SIZE),
                    help="storage of dX (default: --act)")
    ap.add_argument("--summarize-profile", metavar="PREFIX", default=None,
                    help="instead of running: summarize the rocprofv3 runs PREFIX_trace, "
                         "PREFIX_fetch and PREFIX_write of --workload into profiles/")
    ap.add_argument("--pages-context", action="store_true",
                    help="instead of the training step: host-wall time of the binary32 "
                         "LayerNorm forward at the shapes the pages time")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}): the normalization pair "
              "is row-local, so a multi-GPU run is this single-GPU path on each GPU's rows plus "
              "one dgamma all-reduce, which is not implemented here", file=sys.stderr)
        sys.exit(2)

    if args.summarize_profile:
        summarize_profile(args.workload, args.summarize_profile)
        return

    import torch
    import row_wise_normalization_amd as mn

    if args.pages_context:
        pages_context(torch, mn)
        return

    act = args.act
    param = args.param or act
    cot = args.cot or act
    dxt = args.dx or act
    typed = (act, param, cot, dxt) != ("f16",) * 4
    tdt = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}

    w = workloads.WORKLOADS[args.workload]
    N, D, kind = w.N, w.D, w.kind
    if kind in ("dyt", "poly", "mod", "gn"):
        bench_other(args, w, torch, mn, act, param, dxt)
        return
    if kind in ("rms_gemv", "ln_gemv"):
        bench_gemv(args, w, torch, mn, act, param)
        return
    print(f"[bench] {w.name}: generating inputs", file=sys.stderr, flush=True)
    d = workloads.generate(w, act=act, param=param, cot=cot)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    def upload(a):
        if a.dtype == np.uint16:  # bfloat16 bit patterns
            return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
        return torch.from_numpy(a).to(dev)

    S = max(4, args.sets)
    up = {k: upload(v) for k, v in d.items()}
    sets = []
    for s in range(S):
        b = {"X": up["X"] if s == 0 else up["X"].clone(),
             "dY": up["dY"] if s == 0 else up["dY"].clone(),
             "Y": torch.empty(N, D, dtype=tdt[act], device=dev),
             "dX": torch.empty(N, D, dtype=tdt[dxt], device=dev),
             "rstd": torch.empty(N, dtype=torch.float32, device=dev),
             "dgamma": torch.empty(D, dtype=torch.float32, device=dev)}
        if kind == "ln":
            b["mean"] = torch.empty(N, dtype=torch.float32, device=dev)
            b["dbeta"] = torch.empty(D, dtype=torch.float32, device=dev)
        if kind == "add":
            b["R"] = up["R"] if s == 0 else up["R"].clone()
            b["dH"] = up["dH"] if s == 0 else up["dH"].clone()
            b["H"] = torch.empty(N, D, dtype=tdt[act], device=dev)
        b["ws"] = mn.new_workspace({"rms": 0, "ln": 1, "add": 2}[kind], N, D, dev)
        sets.append(b)
    gamma = up["gamma"]
    beta = up.get("beta")
    kcode = {"rms": mn.MN_RMSNORM, "ln": mn.MN_LAYERNORM, "add": mn.MN_ADD_RMSNORM}[kind]
    x = "_ex" if typed else ""
    f_rms, f_ln, f_add = (getattr(mn, f"mn_{n}_forward{x}")
                          for n in ("rmsnorm", "layernorm", "add_rmsnorm"))
    b_rms, b_ln, b_add = (getattr(mn, f"mn_{n}_backward_rows{x}")
                          for n in ("rmsnorm", "layernorm", "add_rmsnorm"))
    g_rms, g_ln, g_add = (getattr(mn, f"mn_{n}_backward{x}")
                          for n in ("rmsnorm", "layernorm", "add_rmsnorm"))
    # small problems: the full backward is one launch (the row kernel adds
    # its own partial rows), so a step calls it instead of the two stages
    one_launch = mn.backward_launches(kcode, N, D) == 1

    def fwd(b):
        if kind == "rms":
            f_rms(b["X"], gamma, b["Y"], b["rstd"], w.eps, stream)
        elif kind == "ln":
            f_ln(b["X"], gamma, beta, b["Y"], b["mean"], b["rstd"], w.eps, stream)
        else:
            f_add(b["X"], b["R"], gamma, b["H"], b["Y"], b["rstd"], w.eps, stream)

    def bwd_rows(b):
        if kind == "rms":
            b_rms(b["X"], gamma, b["rstd"], b["dY"], b["dX"], b["ws"], stream)
        elif kind == "ln":
            b_ln(b["X"], gamma, b["mean"], b["rstd"], b["dY"], b["dX"], b["ws"], stream)
        else:
            b_add(b["X"], b["R"], gamma, b["rstd"], b["dY"], b["dH"], b["dX"], b["ws"], stream)

    def reduce(b):
        mn.mn_norm_reduce_partials(kcode, N, D, b["ws"], b["dgamma"], b.get("dbeta"), stream)

    def bwd_full(b):
        if kind == "rms":
            g_rms(b["X"], gamma, b["rstd"], b["dY"], b["dX"], b["dgamma"], b["ws"], stream)
        elif kind == "ln":
            g_ln(b["X"], gamma, b["mean"], b["rstd"], b["dY"], b["dX"], b["dgamma"], b["dbeta"],
                 b["ws"], stream)
        else:
            g_add(b["X"], b["R"], gamma, b["rstd"], b["dY"], b["dH"], b["dX"], b["dgamma"],
                  b["ws"], stream)

    if one_launch:
        bwd_rows, reduce = bwd_full, (lambda b: None)

    K, W = args.steps, args.warmup
    fwd_b, bwd_b = alg_bytes(kind, N, D, act, param, cot, dxt)
    # The dominant kernel (most algorithmic bytes per launch) is the backward
    # row kernel; the timed loop brackets only it with events, so that the
    # step wall time carries two event records per step.
    ev = [(HipEvent(), HipEvent()) for _ in range(K)]

    def step(k, rows_events=None):
        f = sets[k % S]
        bk = sets[back_set(k, S)]
        fwd(f)
        if rows_events: rows_events[0].record(stream)
        bwd_rows(bk)
        if rows_events: rows_events[1].record(stream)
        reduce(bk)

    print(f"[bench] warmup {W} steps", file=sys.stderr, flush=True)
    for b in sets:
        fwd(b)
    settle(step, torch)
    for k in range(W):
        step(k)
    torch.cuda.synchronize()
    print(f"[bench] timing {K} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for k in range(K):
        step(W + k, ev[k])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_step = (t1 - t0) * 1e3 / K
    rows_ms = float(np.mean([a.elapsed_ms(b) for a, b in ev]))

    # Launch-bound workloads (under 64 MB per step): back-to-back device
    # throughput, 1000 steps enqueued without synchronizing, once issued from
    # Python (host-issue bound) and once replayed from a HIP graph of 100
    # steps (device bound), events around each.
    b2b = None
    if fwd_b + bwd_b < (64 << 20):
        nb = 1000
        e0, e1 = HipEvent(), HipEvent()
        torch.cuda.synchronize()
        e0.record(stream)
        for k in range(nb):
            step(k)
        e1.record(stream)
        torch.cuda.synchronize()
        eager_us = e0.elapsed_ms(e1) * 1e3 / nb
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(side):
            step_stream = stream
            stream = side
            for k in range(4):
                step(k)
            side.synchronize()
            with torch.cuda.graph(graph, stream=side):
                for k in range(100):
                    step(k)
            stream = step_stream
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = HipEvent(), HipEvent()
        e0.record(stream)
        for _ in range(nb // 100):
            graph.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        graph_us = e0.elapsed_ms(e1) * 1e3 / nb
        b2b = {"steps": nb, "eager_us_per_step": round(eager_us, 3),
               "graph_us_per_step": round(graph_us, 3),
               "graph_rows_per_s": round(N / (graph_us * 1e-6), 1),
               "graph_GBps": round((fwd_b + bwd_b) / (graph_us * 1e-6) / 1e9, 1),
               "note": "1000 forward + backward steps back to back between two events: issued "
                       "from Python one call at a time, and replayed from a captured HIP graph "
                       "of 100 steps"}

    # Diagnostic pass (not the timed region): every kernel bracketed.
    dg = [[HipEvent() for _ in range(4)] for _ in range(K)]
    for k in range(K):
        f = sets[k % S]
        bk = sets[back_set(k, S)]
        dg[k][0].record(stream); fwd(f); dg[k][1].record(stream); bwd_rows(bk)
        dg[k][2].record(stream); reduce(bk); dg[k][3].record(stream)
    torch.cuda.synchronize()
    fwd_ms = float(np.mean([e[0].elapsed_ms(e[1]) for e in dg]))
    red_ms = 0.0 if one_launch else float(np.mean([e[2].elapsed_ms(e[3]) for e in dg]))

    step_bytes = fwd_b + bwd_b
    gbs = step_bytes / (ms_step * 1e-3) / 1e9
    kernels = {
        "forward": {"avg_ms": fwd_ms, "bytes": fwd_b},
        "backward_rows": {"avg_ms": rows_ms, "bytes": bwd_b},
        "reduce_partials": {"avg_ms": red_ms, "bytes": None},
    }
    dom = "backward_rows"
    achieved = bwd_b / (rows_ms * 1e-3) / 1e9
    roofline = {
        "bound": "hbm",
        "kernel": dom,
        "achieved": round(achieved, 1),
        "peak": HBM_PEAK_GBS,
        "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBS, 4),
        "traffic": measured_traffic(w.name, dom) if not typed else None,
    }

    cpu = None
    if args.cpu_budget > 0:
        print(f"[bench] cpu baseline (oracle, {args.cpu_budget:.0f} s budget)", file=sys.stderr,
              flush=True)
        cpu = cpu_baseline(w, d, args.cpu_budget, (act, param, cot, dxt))

    line = {
        "metric": f"achieved HBM GB/s (% of peak) + rows/s for norm fwd+bwd, "
                  f"{NORM_NAMES[kind]} {N}x{D}",
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "warmup_note": WARMUP_NOTE,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": w.name, "N": N, "D": D, "eps": w.eps, "io_dtype": act,
            "param_dtype": param, "cotangent_dtype": cot, "dx_dtype": dxt,
            "norm": NORM_NAMES[kind],
            "step": ("forward + backward (one launch: rows, then the column reduce by the "
                     "last workgroup)" if one_launch else
                     "forward + backward rows + column reduce"), "buffer_sets": S,
        },
        "pct_of_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "rows_per_s": round(N / (ms_step * 1e-3), 1),
        "kernels_ms": {k: round(v["avg_ms"], 5) for k, v in kernels.items()},
        "kernels_ms_note": "backward_rows from the timed loop; forward and reduce_partials "
                           "from an event-bracketed pass after it; HIP events without the "
                           "system-scope fence, recorded on the launch stream",
        "kernel_gbs": {k: (round(v["bytes"] / (v["avg_ms"] * 1e-3) / 1e9, 1) if v["bytes"] else None)
                       for k, v in kernels.items()},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "device": torch.cuda.get_device_name(dev),
    }
    if b2b is not None:
        line["back_to_back"] = b2b
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
