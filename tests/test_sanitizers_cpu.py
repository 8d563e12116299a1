"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer, on the CPU.

Three programs are built with both sanitizers (every finding aborts the program) and run:
  - tests/sanitize_abi.cpp linked against libattn's sources, compiled with the sanitizers on the host
    side only (the device code is compiled as usual and never runs): every entry point's argument
    validation, including sizes next to INT_MAX, NULL, misaligned and overlapping pointers, and the
    size helpers.  No call passes validation, so no HIP call is made and no GPU is needed.
  - tests/sanitize_oracle.c linked with oracle/attn_oracle.c (gcc): every oracle function on small
    edge-case inputs, compared across its routes and against softmax invariants.
  - tests/sched_check.cpp (g++): the work-item maps of csrc/attn_sched.h.
Objects are cached under _build/sanitize/ by a hash of sources and flags.
"""
import hashlib
import os
import shutil
import subprocess
from concurrent.futures import ThreadPoolExecutor

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(ROOT, "tiled_online_softmax_02_amd", "csrc")
INCLUDE = os.path.join(ROOT, "include")
ORACLE_C = os.path.join(ROOT, "oracle", "attn_oracle.c")
OUT = os.path.join(ROOT, "_build", "sanitize")
LIB_SOURCES = ["attn_api.hip", "attn_fwd.hip", "attn_bwd.hip", "attn_fwd_fp8.hip"]

# sanitizers on the host pass only (each flag behind its own -Xarch_host)
HOST_SAN = "-Xarch_host -fsanitize=address -Xarch_host -fsanitize=undefined -Xarch_host -fno-sanitize-recover=all".split()
HIP_FLAGS = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", "-fno-omit-frame-pointer",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument"]
# flags for host-only compilers (gcc, g++, clang++ on .c/.cpp files)
CPU_SAN = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", "-g", "-O1"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")


def tool(name, *fallbacks):
    for cand in (shutil.which(name), *fallbacks):
        if cand and os.path.exists(cand):
            return cand
    pytest.skip("%s not found" % name)


def digest(paths, flags):
    h = hashlib.sha256(" ".join(flags).encode())
    for p in paths:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def run(cmd, what, timeout=600):
    r = subprocess.run(cmd, capture_output=True, text=True, timeout=timeout)
    if r.returncode != 0:
        pytest.fail("%s failed:\n%s\n%s" % (what, " ".join(cmd), r.stderr[-4000:]))


def run_checked(exe):
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=ENV)
    print(r.stdout.strip())
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    return r.stdout


def headers():
    return [os.path.join(CSRC, f) for f in sorted(os.listdir(CSRC)) if f.endswith(".h")] + \
        [os.path.join(INCLUDE, "attn.h")]


def test_abi_validation_under_asan_and_ubsan():
    hipcc = tool("hipcc", "/opt/rocm/bin/hipcc")
    clangxx = tool("amdclang++", "/opt/rocm/llvm/bin/clang++")
    os.makedirs(OUT, exist_ok=True)

    def obj(src):
        path = os.path.join(CSRC, src)
        out = os.path.join(OUT, "%s.%s.o" % (src, digest([path, *headers()], HIP_FLAGS + HOST_SAN)))
        if not os.path.exists(out):
            run([hipcc, *HIP_FLAGS, *HOST_SAN, "-c", path, "-o", out + ".tmp"], "hipcc " + src)
            os.replace(out + ".tmp", out)
        return out

    with ThreadPoolExecutor(max_workers=len(LIB_SOURCES)) as ex:
        objs = list(ex.map(obj, LIB_SOURCES))
    drv = os.path.join(HERE, "sanitize_abi.cpp")
    exe = os.path.join(OUT, "abi_checks")
    run([clangxx, "-std=c++17", *CPU_SAN, "-I" + INCLUDE, drv, *objs, "-L/opt/rocm/lib", "-lamdhip64",
         "-Wl,-rpath,/opt/rocm/lib", "-o", exe], "link abi_checks")
    out = run_checked(exe)
    assert "0 mismatches" in out


def test_oracle_under_asan_and_ubsan():
    gcc = tool("gcc")
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "oracle_checks")
    run([gcc, "-std=c99", "-Wall", *CPU_SAN, "-pthread", os.path.join(HERE, "sanitize_oracle.c"), ORACLE_C, "-lm",
         "-o", exe], "gcc oracle_checks")
    out = run_checked(exe)
    assert "failed 0" in out


def test_work_item_maps_under_asan_and_ubsan():
    gxx = tool("g++")
    os.makedirs(OUT, exist_ok=True)
    exe = os.path.join(OUT, "sched_checks")
    run([gxx, "-std=c++17", *CPU_SAN, "-D__HIP_PLATFORM_AMD__", "-I/opt/rocm/include", "-I" + CSRC,
         os.path.join(HERE, "sched_check.cpp"), "-o", exe], "g++ sched_checks")
    run_checked(exe)
