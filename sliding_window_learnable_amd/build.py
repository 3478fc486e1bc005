"""Build libswa_sink.so (the C-ABI HIP library) in-tree with hipcc for gfx950.

Each ``csrc/*.hip`` file is compiled to an object in ``_build/`` (in
parallel), then linked into ``sliding_window_learnable_amd/libswa_sink.so``.
A second, debug-only library ``libswa_sink_poison.so`` is built the same
way with ``-DSWA_LDS_POISON`` (objects in ``_build/poison/``): its kernels
start from NaN-filled LDS and poison every copy's destination first, so a
read of LDS that nothing has written yet shows up as NaN.  Only the tests
load it; the package always loads ``libswa_sink.so``.
Run as ``python -m sliding_window_learnable_amd.build``.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libswa_sink.so")
POISON_LIB_PATH = os.path.join(PKG, "libswa_sink_poison.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
    "-fvisibility=hidden", "-ffp-contract=fast", "-fno-strict-aliasing",
    # packed fp32 arithmetic stays off on this target
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # matrix-core accumulators in ordinary VGPRs: the AGPR form makes the
    # compiler copy scores between the two register files every tile
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


# Files built with type-based alias analysis: their LDS is filled by
# buffer->LDS copies, and without TBAA the compiler assumes every LDS read may
# alias an in-flight copy and waits for all of them before it.  LDS shared
# between lanes there is only read after an asm barrier (a full compiler
# memory barrier).
STRICT_ALIASING = {"backward_mfma.hip"}


def flags_for(src: str) -> list:
    if os.path.basename(src) in STRICT_ALIASING:
        return [f for f in HIPCC_FLAGS if f != "-fno-strict-aliasing"]
    return list(HIPCC_FLAGS)


def _compile(job) -> str:
    src, out_dir, extra = job
    obj = os.path.join(out_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *flags_for(src), *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, res.stderr))
    return obj


def _link(objs, path):
    tmp = path + ".tmp%d" % os.getpid()
    cmd = [hipcc(), "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError("link failed:\n%s" % res.stderr)
    os.replace(tmp, path)


def build(verbose: bool = False, poison: bool = True) -> str:
    """Compile every HIP source and link libswa_sink.so (and, unless
    poison=False, the LDS-poisoning debug library); returns the product
    library's path."""
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    poison_dir = os.path.join(BUILD_DIR, "poison")
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = [(src, BUILD_DIR, []) for src in sources]
    if poison:
        os.makedirs(poison_dir, exist_ok=True)
        jobs += [(src, poison_dir, ["-DSWA_LDS_POISON"]) for src in sources]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(jobs))) as ex:
        objs = list(ex.map(_compile, jobs))
    _link(objs[:len(sources)], LIB_PATH)
    if verbose:
        print("built", LIB_PATH)
    if poison:
        _link(objs[len(sources):], POISON_LIB_PATH)
        if verbose:
            print("built", POISON_LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
