"""Build libskgemm.so (the HIP kernels and the C ABI) for gfx950 with hipcc.

Each ``csrc/*.hip`` file compiles to an object in ``_build/`` (in parallel),
then links into ``split_reduction_amd/libskgemm.so``. The build also reads the
compiler's kernel resource report and fails if any kernel uses scratch memory
(register spills): a spilling kernel is slower than the design assumes.

Flags: ``-Xclang -target-feature -Xclang -packed-fp32-ops`` keeps the compiler
from forming packed FP32 instructions, which are not used anywhere here.
"""

from __future__ import annotations

import concurrent.futures
import os
import re
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libskgemm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3",
    "-std=c++20",
    f"--offload-arch={ARCH}",
    "-fPIC",
    "-fvisibility=hidden",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


def sources() -> list[str]:
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def _compile(src: str) -> tuple[str, str]:
    obj = os.path.join(BUILD, os.path.basename(src)[:-4] + ".o")
    cmd = [HIPCC, *COMMON, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr[-6000:]}")
    return obj, r.stderr


def _scratch_report(remarks: str) -> list[str]:
    """Kernels whose resource report shows scratch (spill) memory."""
    bad = []
    current = None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            current = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > 0:
            bad.append(f"{current}: scratch {m.group(1)} B/lane")
    return bad


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libskgemm.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = min(len(srcs), max(1, min(8, os.cpu_count() or 1)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        results = list(ex.map(_compile, srcs))
    objs = [o for o, _ in results]
    remarks = "\n".join(r for _, r in results)
    with open(os.path.join(BUILD, "resource_usage.txt"), "w") as f:
        f.write(remarks)
    bad = _scratch_report(remarks)
    if bad:
        raise RuntimeError("kernels use scratch memory (spills):\n" + "\n".join(bad))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
