"""Builds ``librr.so`` (the C-ABI library with the gfx950 HIP kernels) in place.

    python -m memory_bound_row_softmax_amd.build

Every source under ``csrc/`` is compiled with hipcc for gfx950 into ``_build/``,
then linked into ``librr.so`` next to this file.  The compiler's per-kernel
resource remarks are collected into ``_build/resources.txt``; the build fails
if any kernel needs scratch memory (register spills), since a spilling kernel
re-reads its own data from memory and is no longer one read plus one write.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "librr.so")

SOURCES = ["api.cpp", "plan.cpp", "softmax.hip", "rmsnorm.hip", "xent.hip", "xent_grad.hip",
           "softmax_bwd.hip", "rmsnorm_bwd.hip", "long_row.hip", "packed.hip", "copy.hip"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build librr)")


def _flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
            # packed fp32 instructions are kept out of every kernel on purpose
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-command-line-argument"]


def _compile(src: str, build_dir: str = BUILD, extra=()) -> tuple[str, str]:
    obj = os.path.join(build_dir, src + ".o")
    cmd = [hipcc(), *_flags(), *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd.append("-Rpass-analysis=kernel-resource-usage")
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{res.stderr[-6000:]}")
    return obj, res.stderr


def _resources(remarks: str) -> list[dict]:
    rows, cur = [], None
    for line in remarks.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = {"name": m.group(1)}
            rows.append(cur)
            continue
        m = re.search(r"remark:\s+([A-Za-z][A-Za-z ]*?)(?: \[[^\]]*\])?: (\S+) \[-Rpass", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = m.group(2)
    return rows


def build(verbose: bool = False, out: str = LIB, extra_flags=()) -> str:
    """Compile every source and link the library (``librr.so`` next to this file
    unless `out` names another path, e.g. a variant built with `extra_flags`
    such as -DRR_STREAM_STORE_POLICY=2 for a tuning run); returns its path."""
    build_dir = BUILD if out == LIB else out + ".build"
    os.makedirs(build_dir, exist_ok=True)
    jobs = max(1, min(len(SOURCES), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)), 16))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda s: _compile(s, build_dir, tuple(extra_flags)), SOURCES))
    objs = [o for o, _ in results]
    kernels = []
    for _, remarks in results:
        kernels.extend(_resources(remarks))
    with open(os.path.join(build_dir, "resources.txt"), "w") as f:
        f.write("kernel\tVGPRs\tAGPRs\tSGPRs\tSGPRspill\tScratchSize\tOccupancy\tLDS\n")
        for k in kernels:
            f.write("\t".join([k["name"], k.get("VGPRs", "?"), k.get("AGPRs", "?"),
                               k.get("TotalSGPRs", "?"), k.get("SGPRs Spill", "?"),
                               k.get("ScratchSize", "?"), k.get("Occupancy", "?"),
                               k.get("LDS Size", "?")]) + "\n")
    # Scalar registers spilled into vector-register lanes cost no memory traffic;
    # anything that reaches scratch memory does.
    spills = [k["name"] for k in kernels if int(k.get("ScratchSize", "0")) > 0
              or int(k.get("VGPRs Spill", "0")) > 0]
    if spills:
        raise RuntimeError(f"{len(spills)} kernels spill to scratch memory, e.g. {spills[:3]}")
    tmp = out + ".tmp"
    res = subprocess.run([hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs],
                         capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr[-4000:]}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out} ({len(kernels)} kernels, none spilling)")
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
