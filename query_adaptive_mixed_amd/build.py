"""Build libqam.so in-tree with hipcc for gfx950.

Every translation unit under ``csrc/`` is compiled separately (in parallel)
and linked into ``query_adaptive_mixed_amd/libqam.so``.  Flags:

* ``--offload-arch=gfx950``                 MI355X only
* ``-ffp-contract=off``                     no silent FMA contraction (the
                                            fp64 level map must match IEEE
                                            evaluation bit for bit)
* ``-Xclang -target-feature -Xclang -packed-fp32-ops``
                                            no packed-fp32 instructions
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqam.so")

ARCH = "gfx950"
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument", "-I", INCLUDE, "-I", CSRC,
]
# Per-file extras.  The matrix-core kernels keep their MFMA accumulators in
# ordinary VGPRs: with AGPR accumulators the register allocator rotates them
# through copies on every ring step of the unrolled loop.
EXTRA_FLAGS = {
    "qmm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
    "qmatvec.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"],
}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; libqam needs ROCm's hipcc to build")
    return path


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(OBJDIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *CFLAGS, *EXTRA_FLAGS.get(os.path.basename(src), []), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, jobs: int = 8) -> str:
    """Compile every csrc/*.hip and link libqam.so; returns the library path."""
    os.makedirs(OBJDIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
