"""Build libmta.so (gfx950) from the HIP sources in csrc/.

Every translation unit is compiled in parallel with hipcc into ``_build/`` at the
repository root, then linked into ``token_attention_amd/libmta.so``. Run it as
``python -m token_attention_amd.build`` or call :func:`build`.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libmta.so")
BUILD_DIR = os.path.join(ROOT, "_build")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # no packed fp32 instructions in generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


# The two-phase kernels (convolution after softmax) schedule better with the backend's
# instruction-level-parallelism strategy; the other kernels keep the default.
EXTRA_FLAGS = {"_postconv.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    extra = [f for suffix, fl in EXTRA_FLAGS.items() if src.endswith(suffix) for f in fl]
    cmd = [HIPCC] + CFLAGS + extra + ["-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "not a recognized feature" not in ln]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {os.path.basename(src)}:\n" + "\n".join(msgs))
    return obj


def build(jobs: int = 0, verbose: bool = True) -> str:
    """Compile every csrc/*.hip and link libmta.so; returns the library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    if jobs <= 0:
        jobs = max(1, min(len(srcs), os.cpu_count() or 1, 16))
    t0 = time.time()
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT} from {len(srcs)} sources in {time.time() - t0:.1f}s", file=sys.stderr)
    return OUT


if __name__ == "__main__":
    build()
