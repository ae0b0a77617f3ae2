"""Sanitizer builds of the host-side code, run on the CPU (no GPU needed).

* ``native/capi_checks.cpp``: the C ABI's planning and validation code
  (``nsa_capi.hip``, ``nsa_timing.hip``) compiled with the address and
  undefined-behaviour sanitizers on the host pass, linked with the library's
  kernel objects; every call returns before anything is launched.
* ``native/index_checks.cpp``: the selected-block index helpers that keep the
  backward pass inside rows 0 .. t for any selection list (signed overflow
  would abort under the sanitizer).
* ``native/oracle_checks.c``: the fp64 oracle under the same sanitizers on
  small layouts that reach every path.
"""
import glob
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
NATIVE = os.path.join(ROOT, "tests", "native")
CSRC = os.path.join(ROOT, "sparse_attention_long_nsa_amd", "csrc")
OUT = os.path.join(ROOT, "_build", "san")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CLANG = "/opt/rocm/lib/llvm/bin/clang++"
# host pass only: the device code of these programs is never run
SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]
HOST_ONLY = ["-x", "hip", "--offload-host-only", "--offload-arch=gfx950", "-O1", "-g", "-std=c++17"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="print_stacktrace=1", OMP_NUM_THREADS="4")


def run(cmd, **kw):
    r = subprocess.run(cmd, capture_output=True, text=True, **kw)
    assert r.returncode == 0, (" ".join(cmd), r.stdout[-4000:], r.stderr[-4000:])
    return r.stdout


@pytest.fixture(scope="module")
def outdir():
    os.makedirs(OUT, exist_ok=True)
    return OUT


def kernel_objects():
    """Normal (unsanitized) objects of the kernel sources, built by the
    package's build step; built here if absent."""
    objs = sorted(glob.glob(os.path.join(ROOT, "_build", "*.hip.o")))
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if len(objs) != len(srcs):
        from sparse_attention_long_nsa_amd import build as nsa_build
        nsa_build.build()
        objs = sorted(glob.glob(os.path.join(ROOT, "_build", "*.hip.o")))
    return objs


def test_capi_host_code_under_sanitizers(outdir):
    host_srcs = ("nsa_capi.hip", "nsa_timing.hip")
    san_objs = []
    for name in host_srcs:
        o = os.path.join(outdir, name + ".o")
        run([HIPCC, *HOST_ONLY, *SAN, "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-c",
             os.path.join(CSRC, name), "-o", o])
        san_objs.append(o)
    drv = os.path.join(outdir, "capi_checks.o")
    run([HIPCC, *HOST_ONLY, *SAN, "-I", os.path.join(ROOT, "include"), "-c",
         os.path.join(NATIVE, "capi_checks.cpp"), "-o", drv])
    others = [o for o in kernel_objects() if os.path.basename(o)[:-2] not in host_srcs]
    exe = os.path.join(outdir, "capi_checks")
    run([CLANG, "-fsanitize=address,undefined", drv, *san_objs, *others, "-L/opt/rocm/lib", "-lamdhip64",
         "-Wl,-rpath,/opt/rocm/lib", "-o", exe])
    assert run([exe], env=ENV).strip() == "ok"


def test_index_helpers_under_sanitizers(outdir):
    exe = os.path.join(outdir, "index_checks")
    run([HIPCC, *HOST_ONLY, *SAN, "-I", CSRC, os.path.join(NATIVE, "index_checks.cpp"), "-o", exe])
    assert run([exe], env=ENV).strip() == "ok"


def test_oracle_under_sanitizers(outdir):
    exe = os.path.join(outdir, "oracle_checks")
    run(["gcc", "-O1", "-g", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-fno-omit-frame-pointer", "-Wall", os.path.join(NATIVE, "oracle_checks.c"), "-o", exe, "-lm"])
    assert run([exe], env=dict(ENV, ASAN_OPTIONS="detect_leaks=1")).strip() == "ok"
