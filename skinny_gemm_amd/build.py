"""Build the gfx950 HIP library ``skinny_gemm_amd/libqmoe.so`` with hipcc.

Every translation unit under ``csrc/`` is compiled for gfx950 only, with
packed-FP32 instruction selection disabled, then linked into one shared
library exporting the C ABI of ``include/qmoe.h``.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc")
OBJ = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libqmoe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-Wall", "-Wno-unused-function",
]


def _compile(src: str, incremental: bool = False) -> str:
    obj = os.path.join(OBJ, os.path.basename(src) + ".o")
    if incremental and os.path.exists(obj):
        deps = [src] + glob.glob(os.path.join(SRC, "*.h*")) + glob.glob(os.path.join(ROOT, "include", "*.h"))
        deps = [d for d in deps if not d.endswith(".hip") or d == src]
        if all(os.path.getmtime(d) <= os.path.getmtime(obj) for d in deps):
            return obj
    cmd = [HIPCC, *CFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 0, verbose: bool = False, incremental: bool = False) -> str:
    """Compile every source (``incremental`` reuses up-to-date objects) and link."""
    os.makedirs(OBJ, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(SRC, "*.hip")))
    jobs = jobs or min(len(srcs), max(1, min(16, os.cpu_count() or 1)))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, incremental), srcs))
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", LIB + ".tmp", *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(LIB + ".tmp", LIB)
    if verbose:
        print(f"built {LIB} from {len(srcs)} sources")
    return LIB


if __name__ == "__main__":
    build(verbose=True, incremental="--incremental" in sys.argv)
    sys.exit(0)
