"""Build libhybridattn.so (gfx950) in-tree with hipcc.

Usage: ``python -m sparse_hybrid_attention_amd.build_lib`` or ``build()``.
Every HIP source under csrc/ is compiled to an object file in parallel, then
linked into ``sparse_hybrid_attention_amd/libhybridattn.so``.  The device
measurement probes under probe/ (used by the benchmark only, not part of the
library or its interface) are linked into ``libshattn_probe.so`` beside it.
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
BUILD = os.path.join(PKG, "_build")
PROBE = os.path.join(PKG, "probe")
LIB = os.path.join(PKG, "libhybridattn.so")
PROBE_LIB = os.path.join(PKG, "libshattn_probe.so")
ARCH = "gfx950"

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden", f"--offload-arch={ARCH}",
    # keep packed-fp32 VALU forms out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; ROCm is required to build the library")
    return path


# per-source options: the attention kernels never hold NaN (scores are finite,
# masked keys are -inf), so their float max needs no NaN-quieting instructions
FILE_FLAGS = {
    "attention.hip": ["-fno-honor-nans"],
    # the MFMA rate probe: accumulators in ordinary VGPRs (the accumulator-
    # register form of its loop is compiled with register copies per round)
    "probes.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=true"],
}


def _compile(src: str, extra) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [hipcc(), *HIPCC_FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out):
    tmp = out + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False, extra=()) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    probe_srcs = sorted(glob.glob(os.path.join(PROBE, "*.hip")))
    jobs = min(len(srcs) + len(probe_srcs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, list(extra)), srcs + probe_srcs))
    _link(objs[:len(srcs)], LIB)
    _link(objs[len(srcs):], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
