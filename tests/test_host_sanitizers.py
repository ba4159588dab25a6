"""The C ABI shim (bsm_api.cpp) under host AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU.

tests/host_sanitize/ holds stand-ins for the kernel launchers (they record
the parameter blocks and launch nothing) and a driver that calls every entry
point of include/bsm.h with rejected and accepted arguments: it checks the
statuses and messages, that accepted calls reach a launcher, and that the
workspace parts the shim carves out lie inside the caller's workspace
without overlapping.  The shim is compiled with the sanitizers on its host
code only (the device code of the file, the static decoding array, is
compiled as usual); the objects are linked by clang++ with the sanitizer
runtimes and the HIP runtime, which finds no device here."""
import os
import shutil
import subprocess

import pytest

from block_sparse_masked_build_amd import build

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SOURCES = [os.path.join(ROOT, "block_sparse_masked_build_amd", "csrc", "bsm_api.cpp"),
           os.path.join(HERE, "host_sanitize", "stub_launchers.cpp"),
           os.path.join(HERE, "host_sanitize", "driver.cpp")]
HOST_SANITIZERS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                   "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer"]


def _clangxx():
    for cand in ("/opt/rocm/llvm/bin/clang++", shutil.which("clang++")):
        if cand and os.path.exists(cand):
            return cand
    pytest.skip("clang++ not found")


def test_shim_under_host_sanitizers(tmp_path):
    hipcc = build.hipcc()
    objs = []
    for src in SOURCES:
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        cmd = [hipcc, f"--offload-arch={build.ARCH}", "-O1", "-g", "-std=c++17", "-fPIC", *HOST_SANITIZERS,
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               "-I", os.path.join(ROOT, "include"), "-x", "hip", "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        objs.append(obj)
    exe = str(tmp_path / "driver")
    rocm_lib = os.path.join(os.path.dirname(os.path.dirname(hipcc)), "lib")
    link = [_clangxx(), "-fsanitize=address,undefined", *objs, "-L", rocm_lib, "-lamdhip64",
            f"-Wl,-rpath,{rocm_lib}", "-o", exe]
    r = subprocess.run(link, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    # the HIP runtime's own allocations at exit are not the shim's: no leak check
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "all checks passed" in r.stdout
