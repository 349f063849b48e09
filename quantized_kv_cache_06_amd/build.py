"""Builds libkvq.so for gfx950 with hipcc (in-tree, next to this file).

Every HIP source is compiled with packed-FP32 instructions disabled. The
append kernels are compiled with -ffp-contract=off so their fp32 formulas
(differences, true divisions, round-half-even) are never fused.

The compiler's per-kernel resource report (registers, occupancy, scratch) is
written to _build/resource_usage.txt; a kernel that uses scratch memory or
spills registers fails the build: scratch loads share the in-order vector
memory counter with the streamed cache loads, so one scratch access waits
for every load in flight.
"""
from __future__ import annotations

import os
import re
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


RESOURCE_REPORT = os.path.join(BUILD, "resource_usage.txt")


def parse_resource_usage(text: str) -> dict:
    """{kernel: {field: value}} from -Rpass-analysis=kernel-resource-usage
    remarks."""
    kernels, cur = {}, None
    for line in text.splitlines():
        m = re.search(r"remark:\s+Function Name: (\S+)", line)
        if m:
            cur = kernels.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z][^:]*): (\S+) \[-Rpass-analysis", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = m.group(2)
    return kernels


def check_resource_usage(kernels: dict) -> None:
    bad = [k for k, f in kernels.items()
           if int(f.get("ScratchSize [bytes/lane]", "0")) > 0 or int(f.get("VGPRs Spill", "0")) > 0
           or int(f.get("SGPRs Spill", "0")) > 0]
    if bad:
        raise RuntimeError("kernels use scratch memory or spill registers: " + ", ".join(bad))


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for src, extra in SOURCES.items():
        obj = os.path.join(BUILD, src + ".o")
        lang = ["-x", "hip", "-Rpass-analysis=kernel-resource-usage"] if src.endswith(".hip") else []
        jobs.append((obj, [HIPCC, *COMMON, *extra, *lang, "-c", os.path.join(CSRC, src), "-o", obj]))
    with ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        outs = list(ex.map(lambda j: _run(j[1]), jobs))
    kernels = {}
    for o in outs:
        kernels.update(parse_resource_usage(o))
    with open(RESOURCE_REPORT, "w") as f:
        for k in sorted(kernels):
            f.write(k + "\n" + "".join(f"    {a}: {b}\n" for a, b in kernels[k].items()))
    check_resource_usage(kernels)
    if verbose:
        for o in outs:
            rest = "\n".join(l for l in o.splitlines() if "kernel-resource-usage" not in l and l.strip()
                             and not l.lstrip().startswith(("|", "^")) and not re.match(r"\s*\d+ \|", l))
            if rest.strip():
                print(rest)
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[j[0] for j in jobs]])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
