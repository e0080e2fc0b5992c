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
    # the single-matrix kernel's first 12 argument dwords arrive in scalar registers
    "qmatvec.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1", "-mllvm", "-amdgpu-kernarg-preload-count=12"],
}


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; libqam needs ROCm's hipcc to build")
    return path


# Host code under AddressSanitizer (device code unchanged): a separate
# library, libqam_host_asan.so, for running the CPU tests against the
# host-side checks, layouts and file parsing with the sanitizer preloaded.
HOST_ASAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
OBJDIR_ASAN = os.path.join(HERE, "_build_asan")
LIB_ASAN = os.path.join(HERE, "libqam_host_asan.so")
# the timeline build: the batch-1 kernel stamps chosen launches (qam_timeline_*)
TIMELINE = ["-DQAM_TIMELINE"]
OBJDIR_TIMELINE = os.path.join(HERE, "_build_timeline")
LIB_TIMELINE = os.path.join(HERE, "libqam_timeline.so")


def _compile(src: str, verbose: bool, asan: bool = False, timeline: bool = False) -> str:
    objdir = OBJDIR_ASAN if asan else (OBJDIR_TIMELINE if timeline else OBJDIR)
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *CFLAGS, *EXTRA_FLAGS.get(os.path.basename(src), []), *(HOST_ASAN if asan else []),
           *(TIMELINE if timeline else []), "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, jobs: int = 8, host_asan: bool = False, timeline: bool = False) -> str:
    """Compile every csrc/*.hip and link libqam.so (host_asan: the host code
    under AddressSanitizer, into libqam_host_asan.so; timeline: the batch-1
    kernel with its timeline stamps, into libqam_timeline.so); returns the
    path."""
    if host_asan and timeline:
        raise ValueError("one variant at a time")
    objdir = OBJDIR_ASAN if host_asan else (OBJDIR_TIMELINE if timeline else OBJDIR)
    os.makedirs(objdir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if timeline:
        # only the batch-1 source carries stamps; the rest is the product build's
        stamped = [s for s in srcs if os.path.basename(s) == "qmatvec.hip"]
        rest = [os.path.join(OBJDIR, os.path.basename(s) + ".o") for s in srcs if s not in stamped]
        if any(not os.path.exists(o) for o in rest):
            build(verbose=verbose, jobs=jobs)
        objs = [_compile(stamped[0], verbose, timeline=True)] + rest
    else:
        with cf.ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
            objs = list(ex.map(lambda s: _compile(s, verbose, host_asan), srcs))
    out = LIB_ASAN if host_asan else (LIB_TIMELINE if timeline else LIB)
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if host_asan:
        cmd += ["-Xarch_host", "-fsanitize=address", "-shared-libasan"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, host_asan="--host-asan" in sys.argv, timeline="--timeline" in sys.argv))
