"""Builds libsmla.so (the gfx950 kernels + C ABI) in-tree with hipcc, and its debug twin
libsmla_debug.so (the same sources with SMLA_DEBUG_CHECKS: device-side precondition
checks reported in the workspace's error word).

    python -m prefill_token_amd.build        # or prefill_token_amd.build.build()
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(HERE, "libsmla.so")
DEBUG_LIB_PATH = os.path.join(HERE, "libsmla_debug.so")
PROBE_LIB_PATH = os.path.join(HERE, "libsmla_probe.so")  # measured MFMA ceilings for bench.py

SOURCES = [os.path.join(CSRC, "smla_kernels.hip"), os.path.join(CSRC, "kv_insert.hip"),
           os.path.join(CSRC, "index_build.hip"), os.path.join(CSRC, "wo_a.hip"), os.path.join(CSRC, "noalloc.hip"),
           os.path.join(CSRC, "smla_api.cpp")]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no packed fp32 VALU ops in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA results in VGPRs: with two waves per SIMD every register a wave has is a
    # VGPR, and the P.V accumulators are rescaled in place by plain VALU multiplies
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if cand and (os.path.sep not in cand or os.path.exists(cand)):
            return cand
    return "hipcc"


def _build_one(path: str, extra, verbose: bool, sources=None) -> str:
    tmp = path + ".tmp"
    cmd = [hipcc(), *HIPCC_FLAGS, *extra, "-I", INCLUDE, "-I", CSRC, "-o", tmp, *(sources or SOURCES)]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    noise = ("packed-fp32-ops", "is not a recognized feature")
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if not any(n in ln for n in noise)]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, path)
    return path


def build(verbose: bool = False) -> str:
    """Compile the libraries (the hipcc runs go in parallel); returns libsmla.so's path."""
    import concurrent.futures as cf

    with cf.ThreadPoolExecutor(3) as ex:
        jobs = [ex.submit(_build_one, LIB_PATH, [], verbose),
                ex.submit(_build_one, DEBUG_LIB_PATH, ["-DSMLA_DEBUG_CHECKS"], verbose),
                ex.submit(_build_one, PROBE_LIB_PATH, [], verbose, [os.path.join(CSRC, "peak_probe.hip")])]
        for j in jobs:
            j.result()
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
