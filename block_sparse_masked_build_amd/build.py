"""Builds libbsm.so in-tree: the HIP kernels for gfx950 and the C ABI shim.

    python -m block_sparse_masked_build_amd.build [--verbose]

Every source is compiled with hipcc for gfx950 only.  Packed fp32 VALU
instructions are disabled for device code (-packed-fp32-ops); the host pass
warns that it does not know the feature, which is harmless.  The machine-code
verifier runs on every build.
"""
from __future__ import annotations

import hashlib
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_PATH = os.path.join(HERE, "libbsm.so")

# (source, object, extra flags): the attention sources are compiled once
# per element type (bf16, fp16) and, for the forward and backward, once per
# head dimension, so that the pieces build in parallel
ELEM_FLAGS = {"bf16": [], "f16": ["-DBSM_ELEM_FP16"]}
# (longest first)
HEAD_DIMS = {"fwd": (256, 128, 64), "bwd": (128, 256, 64)}
SOURCES = ([(f"attn_{p}.hip", f"attn_{p}_d{d}_{e}.o", [f"-DBSM_HEAD_DIM={d}", *ef])
            for p in ("fwd", "bwd") for d in HEAD_DIMS[p] for e, ef in ELEM_FLAGS.items()] +
           [("attn_decode.hip", f"attn_decode_{e}.o", ef) for e, ef in ELEM_FLAGS.items()] +
           [("mask_builder.hip", "mask_builder.o", []), ("gather_pages.hip", "gather_pages.o", []),
            ("bsm_api.cpp", "bsm_api.o", [])])
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def compile_flags():
    return [f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            # run the machine-code verifier: an instruction the backend builds
            # with an illegal operand is a build error, not silent bad code
            "-mllvm", "-verify-machineinstrs",
            "-I", os.path.join(HERE, "..", "include")]


def source_stamp(extra) -> str:
    """Hash of every source and header the objects are built from, the
    compiler flags and the object's own flags."""
    h = hashlib.sha256()
    for d in (CSRC, os.path.join(HERE, "..", "include")):
        for name in sorted(os.listdir(d)):
            path = os.path.join(d, name)
            if os.path.isfile(path):
                h.update(name.encode())
                with open(path, "rb") as f:
                    h.update(f.read())
    h.update(" ".join(compile_flags() + list(extra)).encode())
    return h.hexdigest()


def object_dir(obj_name: str) -> str:
    """Each object is built in a folder of its own, beside its temporary
    files: the device assembly (*-gfx950.s, with inline assembly marked)
    that the machine-code checks of the test suite read, and a stamp of
    the sources it came from."""
    return os.path.join(BUILD_DIR, os.path.splitext(obj_name)[0])


def _compile(entry, verbose: bool) -> str:
    src, obj_name, extra = entry
    d = object_dir(obj_name)
    os.makedirs(d, exist_ok=True)
    obj = os.path.join(d, obj_name)
    stamp = os.path.join(d, "stamp.txt")
    if os.path.exists(stamp):
        os.remove(stamp)
    cmd = [hipcc(), *compile_flags(), *extra, "-save-temps=obj", "-x", "hip", "-c", os.path.join(CSRC, src),
           "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    if verbose and r.stderr.strip():
        lines = [ln for ln in r.stderr.splitlines() if "packed-fp32-ops" not in ln]
        if lines:
            print("\n".join(lines), flush=True)
    with open(stamp, "w") as f:
        f.write(source_stamp(extra))
    return obj


def build(verbose: bool = False) -> str:
    """Compile every source and link libbsm.so (always rebuilds)."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
