"""Build libmn_norm.so (gfx950) in-tree with hipcc.

Usage: python -m row_wise_normalization_amd.build  (or call build()).
"""
from __future__ import annotations

import json
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libmn_norm.so"
LIB_PATH = os.path.join(PKG, LIB_NAME)

# The kernel instances are split by activation storage type and kind group
# so that the sources compile in parallel.
SOURCES = ["mn_inst_f16.hip", "mn_inst_bf16.hip", "mn_inst_f32.hip", "mn_inst_ext_f16.hip",
           "mn_inst_ext_bf16.hip", "mn_inst_ext_f32.hip", "mn_gn_fwd_f16.hip", "mn_gn_bwd_f16.hip",
           "mn_gn_fwd_bf16.hip", "mn_gn_bwd_bf16.hip", "mn_gn_fwd_f32.hip", "mn_gn_bwd_f32.hip",
           "mn_gn_plan.hip", "mn_gnl.hip", "mn_gemv.hip", "mn_kernels.hip", "mn_noalloc.hip", "mn_api.cpp"]
ARCH = "gfx950"

# Device-code flags. Packed fp32 instructions are disabled on purpose; no
# fast-math and no denormal flushing (IEEE fp32 division and square root).
# No implicit contraction: the kernels write every fused multiply-add they
# use as fmaf, so each storage-type instance evaluates the same expressions
# with the same roundings.
HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libmn_norm.so)")


RESOURCES = os.path.join(PKG, "_build", "kernel_resources.json")


def _resources(remarks: str):
    """Per-kernel resource usage from the compiler's
    kernel-resource-usage remarks: {mangled name: {field: value}}."""
    out, cur = {}, None
    for line in remarks.splitlines():
        if "remark:" not in line:
            continue
        body = line.split("remark:", 1)[1].split("[-Rpass", 1)[0].strip()
        if body.startswith("Function Name:"):
            cur = body.split(":", 1)[1].strip()
            out[cur] = {}
        elif cur and ":" in body:
            k, v = body.split(":", 1)
            out[cur][k.strip()] = v.strip()
    return out


def build(verbose: bool = False) -> str:
    """Compile every source (in parallel) and link the shared library; always
    rebuilds. The compiler's per-kernel resource usage (VGPRs, AGPRs, LDS,
    scratch, occupancy) is kept in _build/kernel_resources.json, keyed by
    the demangled kernel name, for the profile summaries."""
    objs = []
    build_dir = os.path.join(PKG, "_build")
    os.makedirs(build_dir, exist_ok=True)
    cc = hipcc()
    procs = []
    for src in SOURCES:
        obj = os.path.join(build_dir, src + ".o")
        cmd = [cc, *HIPCC_FLAGS, "-Rpass-analysis=kernel-resource-usage", "-I", INCLUDE,
               "-I", CSRC, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stderr=subprocess.PIPE, text=True)))
        objs.append(obj)
    failed, resources = [], {}
    for src, p in procs:
        _, err = p.communicate()
        if p.returncode != 0:
            sys.stderr.write(err)
            failed.append(src)
        else:
            resources.update(_resources(err))
    if failed:
        raise RuntimeError(f"hipcc failed on {', '.join(failed)}")
    names = list(resources)
    dem = subprocess.run(["c++filt"], input="\n".join(names), capture_output=True, text=True)
    pretty = dem.stdout.splitlines() if dem.returncode == 0 else names
    with open(RESOURCES, "w") as f:
        json.dump({d: resources[m] for m, d in zip(names, pretty)}, f, indent=0)
    tmp = LIB_PATH + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
