"""Host memory-safety gates, CPU only.

* The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer runs
  the whole pin battery in a child process (the sanitizer runtimes preloaded
  into that interpreter); any report aborts it.
* A copy of the oracle with one planted heap overflow must be reported, so
  the gate above is known to be live.
* The library's host code -- argument validation (mn_api.cpp), the launch
  planners (mn_kernels.hip, mn_gn_plan.hip, mn_gnl.hip) and the no-allocation entry point
  (mn_noalloc.hip) -- is rebuilt with the sanitizers on the host side only
  (device code untouched) and linked with the other objects of the normal
  build; the plain-C caller tests/c/abi_check.c, built with the sanitizers,
  runs every validation path against it.
"""
import os
import shutil
import subprocess
import sys

import pytest

import oracle
import row_wise_normalization_amd as mn
from row_wise_normalization_amd import build as hip_build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
       "-g"]


def _gcc_runtime(name):
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True,
                       text=True).stdout.strip()
    return p if os.path.isabs(p) and os.path.exists(p) else None


def _san_env():
    libs = [_gcc_runtime("libasan.so"), _gcc_runtime("libubsan.so")]
    if None in libs:
        pytest.skip("gcc sanitizer runtimes not found")
    env = dict(os.environ)
    env["LD_PRELOAD"] = ":".join(libs)
    # the interpreter itself keeps allocations until exit by design
    env["ASAN_OPTIONS"] = "detect_leaks=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    return env


PINS = """
import sys
sys.path[:0] = [{root!r}, {tests!r}]
import oracle, oracle_pins
o = oracle.Oracle({lib!r})
for pin in oracle_pins.ALL_PINS:
    pin(o)
print("pins ok", len(oracle_pins.ALL_PINS))
"""


def _run_pins(lib):
    code = PINS.format(root=ROOT, tests=os.path.join(ROOT, "tests"), lib=lib)
    return subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                          env=_san_env(), timeout=600)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_pins_under_address_and_ub_sanitizers(tmp_path):
    lib = oracle.compile_library(oracle.SRC_PATH, str(tmp_path / "libmn_oracle_san.so"), SAN)
    r = _run_pins(lib)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "pins ok" in r.stdout


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_planted_heap_overflow_is_reported(tmp_path):
    with open(oracle.SRC_PATH) as f:
        src = f.read()
    # the fused add's row loop runs one element past its scratch row
    old = "for (int64_t j = 0; j < D; ++j) w->x[j] = w->x[j] + w->r[j];"
    assert old in src
    bad = tmp_path / "mn_oracle_overflow.c"
    bad.write_text(src.replace(old, old.replace("j < D", "j <= D")))
    lib = oracle.compile_library(str(bad), str(tmp_path / "libbad.so"), SAN)
    r = _run_pins(lib)
    assert r.returncode != 0
    assert "AddressSanitizer" in r.stderr and "heap-buffer-overflow" in r.stderr


HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
# sources holding the host-side validation and planning
HOST_SOURCES = ["mn_api.cpp", "mn_kernels.hip", "mn_gn_plan.hip", "mn_gnl.hip", "mn_noalloc.hip"]


@pytest.mark.skipif(not os.path.exists(mn.LIB_PATH), reason="libmn_norm.so not built")
def test_c_abi_validation_under_address_and_ub_sanitizers(tmp_path):
    build_dir = os.path.join(hip_build.PKG, "_build")
    others = [os.path.join(build_dir, s + ".o") for s in hip_build.SOURCES
              if s not in HOST_SOURCES]
    if not all(os.path.exists(o) for o in others):
        pytest.skip("objects of the normal build not present (run __graft_entry__.build())")
    cc = hip_build.hipcc()
    flags = [f for f in hip_build.HIPCC_FLAGS if f != "-O3"] + ["-O1", "-g"] + HOST_SAN
    procs, objs = [], []
    for s in HOST_SOURCES:
        o = str(tmp_path / (s + ".san.o"))
        cmd = [cc, *flags, "-I", hip_build.INCLUDE, "-I", hip_build.CSRC, "-c",
               os.path.join(hip_build.CSRC, s), "-o", o]
        procs.append((s, subprocess.Popen(cmd, stdout=subprocess.DEVNULL,
                                          stderr=subprocess.PIPE, text=True)))
        objs.append(o)
    for s, p in procs:
        _, err = p.communicate()
        assert p.returncode == 0, f"{s}: {err[-2000:]}"
    lib = str(tmp_path / "libmn_norm_san.so")
    subprocess.run([cc, f"--offload-arch={hip_build.ARCH}", "-shared", "-fPIC", "-o", lib,
                    *objs, *others], check=True, capture_output=True)
    undef = subprocess.run(["nm", "-D", "--undefined-only", lib], capture_output=True,
                           text=True, check=True).stdout
    assert "__asan_report" in undef, "host code was not instrumented"
    clang = os.path.join(os.path.dirname(os.path.realpath(cc)), "..", "llvm", "bin", "clang")
    clang = clang if os.path.exists(clang) else shutil.which("clang")
    if clang is None:
        pytest.skip("clang not available")
    exe = str(tmp_path / "abi_check_san")
    subprocess.run([clang, "-std=c99", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-I", hip_build.INCLUDE,
                    os.path.join(ROOT, "tests", "c", "abi_check.c"), lib,
                    f"-Wl,-rpath,{tmp_path}", "-o", exe], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stderr[-4000:]
    assert r.stdout.strip() == "ok"
