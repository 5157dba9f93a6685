"""Build librv.so (the HIP library behind the C ABI in include/rv.h) in-tree.

    python -m ragged_verification_amd.build        # or build() from Python

Every source is compiled for gfx950 only.  Packed-fp32 instruction selection
is switched off for all device code, and the scheduler additionally disables
floating-point contraction so its fp64 arithmetic stays bit-exact.
"""

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(HERE, "librv.so")

SOURCES = ["rv_api.hip", "k_schedule.hip", "k_pack.hip", "k_attn.hip", "k_lm.hip", "k_scatter.hip",
           "k_calib.hip", "k_estimate.hip", "rv_noalloc.hip"]
EXTRA = {"k_schedule.hip": ["-ffp-contract=off"], "k_calib.hip": ["-ffp-contract=off"],
         "k_estimate.hip": ["-ffp-contract=off"]}
ARCH = "gfx950"


def hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: librv needs ROCm's hipcc to build")


def _flags():
    return ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", os.path.join(ROOT, "include")]


def _compile(src):
    obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
    cmd = [hipcc(), *_flags(), *EXTRA.get(src, []), "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose=False):
    """Compile every source and link librv.so next to this file."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = min(len(SOURCES), max(1, (os.cpu_count() or 2)))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = LIB_PATH + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB_PATH)
    if verbose:
        print(f"built {LIB_PATH}")
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
