"""Builds libkvq.so for gfx950 with hipcc (in-tree, next to this file).

Every HIP source is compiled with packed-FP32 instructions disabled. The
append kernels are compiled with -ffp-contract=off so their fp32 formulas
(differences, true divisions, round-half-even) are never fused.
"""
from __future__ import annotations

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libkvq.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]
SOURCES = {
    "kvq_api.cpp": [],
    "kvq_append.hip": ["-ffp-contract=off"],
    "kvq_decode.hip": [],
}


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    # hipcc's host pass does not know the GPU target feature; that warning is harmless
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for src, extra in SOURCES.items():
        obj = os.path.join(BUILD, src + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        jobs.append((obj, [HIPCC, *COMMON, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]))
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        outs = list(ex.map(lambda j: _run(j[1]), jobs))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[j[0] for j in jobs]])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
