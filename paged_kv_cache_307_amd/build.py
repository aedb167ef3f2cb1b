"""Compile libpa.so (the HIP kernels and the C ABI) for gfx950, in-tree.

    python -m paged_kv_cache_307_amd.build

Each ``csrc/*.hip`` file is compiled by hipcc, and each host-only
``csrc/*.cpp`` file (the block manager) by the host C++ compiler, to an object
in ``_build/`` in parallel; the objects are linked into
``paged_kv_cache_307_amd/libpa.so``.  Packed fp32 instructions are disabled
for every device compilation.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libpa.so")
SOURCES = ["api.hip", "cache_ops.hip", "decode_mfma.hip", "decode_simt.hip", "decode_merge.hip",
           "prefill.hip", "context_parallel.hip"]
HOST_SOURCES = ["block_manager.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC or install ROCm)")


# Per-source flags.  The decode kernel keeps its matrix-core accumulators in
# ordinary vector registers: left to itself the compiler moves them to the
# accumulation registers once the partition-record staging adds register
# pressure, and then copies them back and forth around every softmax rescale.
# The prefill kernel has the same pattern (its accumulators moved 960 times
# per loop iteration between register files without the flag; 0.98 -> 0.83
# ms on the 16-sequence chunked-prefill layer with it).
SOURCE_FLAGS = {
    "decode_mfma.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
    "prefill.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
}


def host_cxx() -> str:
    for cand in (os.environ.get("CXX"), shutil.which("g++"), shutil.which("c++")):
        if cand:
            return cand
    raise RuntimeError("no host C++ compiler found (set CXX)")


def host_flags() -> list:
    return ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE, "-I", CSRC]


def compile_flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wno-unused-function",
        "-I", INCLUDE, "-I", CSRC,
    ]


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the device-only feature; that note is harmless
    lines = [ln for ln in proc.stdout.splitlines() if "packed-fp32-ops" not in ln]
    if proc.returncode != 0:
        raise RuntimeError("command failed:\n  " + " ".join(cmd) + "\n" + "\n".join(lines))
    return "\n".join(lines)


def build(verbose: bool = False) -> str:
    """Compile every source and link libpa.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    jobs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        jobs.append((obj, [cc, *compile_flags(), *SOURCE_FLAGS.get(src, []), "-c",
                           os.path.join(CSRC, src), "-o", obj]))
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".cpp", ".o"))
        jobs.append((obj, [host_cxx(), *host_flags(), "-c", os.path.join(CSRC, src), "-o", obj]))
    workers = min(len(jobs), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(workers) as ex:
        for out in ex.map(lambda j: _run(j[1]), jobs):
            if verbose and out.strip():
                print(out)
    tmp = LIB_PATH + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *[j[0] for j in jobs], "-o", tmp])
    os.replace(tmp, LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
