"""Build libkq.so (the C-ABI library) in-tree for gfx950.

Host sources are compiled with g++ (the packer with -ffp-contract=off so every
step is one IEEE fp32 operation); HIP sources with hipcc for gfx950 only, with
packed-fp32 instructions disabled and kernel arguments preloaded into SGPRs
(the command processor writes the first kernel-argument dwords into scalar
registers before a wave starts, so a kernel does not wait on a scalar load of
its arguments before issuing its first memory loads; the code object keeps a
prologue that loads them for firmware without preloading). Objects go to
_build/, the library next to this file.

One HIP runtime per process: PyTorch-ROCm ships its own libamdhip64.so with
the same soname (libamdhip64.so.7) as ROCm's. The binding imports torch before
it loads libkq.so, so the loader matches this library's dependency to the
runtime torch already holds, and torch's streams and allocations are valid
handles here. Without torch in the process the RUNPATH finds ROCm's own.

    python -m block_quantized_gemv_kq_amd.build [-v]
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkq.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = os.path.join(ROCM, "bin", "hipcc")
ARCH = "gfx950"

HOST_SOURCES = ["kq_api.cpp", "kq_pack.cpp"]
HIP_SOURCES = ["kq_gemv.hip", "kq_mfma.hip", "kq_moe.hip", "kq_misc.hip", "kq_stack.hip", "kq_shortlist.hip"]
# Measurement only: a read-only streaming kernel for the benchmark's ceiling,
# in a library of its own that the GEMV library never loads.
PROBE_SOURCES = ["kq_probe.hip"]
PROBE_LIB = os.path.join(HERE, "libkq_probe.so")

HOST_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-ffp-contract=off", "-Wall", "-Wextra",
              "-Wno-unused-parameter"]
HIP_FLAGS = ["--offload-arch=" + ARCH, "-O3", "-fPIC", "-std=c++17",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
             "-Wno-unused-command-line-argument",
             "-mllvm", "-amdgpu-kernarg-preload-count=16"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{p.stdout}\n{p.stderr}")
    if verbose and p.stderr.strip():
        print(p.stderr, file=sys.stderr)


def _compile(src, verbose):
    path = os.path.join(CSRC, src)
    obj = os.path.join(BUILD, src + ".o")
    if src.endswith(".cpp"):
        cmd = [shutil.which("g++") or "g++", *HOST_FLAGS, "-c", path, "-o", obj]
    else:
        cmd = [HIPCC, *HIP_FLAGS, "-c", path, "-o", obj]
    _run(cmd, verbose)
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source and link libkq.so (and the benchmark's
    libkq_probe.so). Always rebuilds."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = [s for s in HOST_SOURCES + HIP_SOURCES if os.path.exists(os.path.join(CSRC, s))]
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    _run([shutil.which("g++") or "g++", "-shared", "-fPIC", "-o", tmp, *objs,
          "-L" + os.path.join(ROCM, "lib"), "-lamdhip64",
          "-Wl,-rpath," + os.path.join(ROCM, "lib"), "-lpthread"], verbose)
    os.replace(tmp, LIB)
    pobjs = [_compile(s, verbose) for s in PROBE_SOURCES]
    tmp = PROBE_LIB + ".tmp"
    _run([shutil.which("g++") or "g++", "-shared", "-fPIC", "-o", tmp, *pobjs,
          "-L" + os.path.join(ROCM, "lib"), "-lamdhip64", "-Wl,-rpath," + os.path.join(ROCM, "lib")], verbose)
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
