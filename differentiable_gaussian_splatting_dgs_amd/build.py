"""Build ``libgs.so`` (the HIP library) in-tree with hipcc for gfx950.

    python -m differentiable_gaussian_splatting_dgs_amd.build

Arithmetic flags: no FMA contraction (the canonical fp32 order writes every
fma explicitly), IEEE-correct fp32 division and square root, fp32
subnormals kept, and the packed-fp32 instructions disabled.  The atomic
optimizer is off: every atomic here is issued by one lane or has lane-
varying addresses, so its wave-reduction rewrite only adds work.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libgs.so")
BUILD = os.path.join(ROOT, "_build")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["api.hip", "compact.hip", "preprocess.hip", "binsort.hip", "raster_fwd.hip", "raster_bwd.hip",
           "loss.hip", "adam.hip", "coupling.hip", "shard.hip", "densify.hip"]

FLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    "-ffp-contract=off", "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt", "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # single-lane atomics stay single instructions (no wave-reduction loop)
    "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
    "-Wall", "-Wno-unused-function",
    f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
]


def _compile(src: str, csrc: str = CSRC, build_dir: str = BUILD, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, f"-I{csrc}", *extra, "-c", os.path.join(csrc, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    return obj


def build(jobs: int | None = None, csrc: str = CSRC, out: str = OUT, build_dir: str = BUILD, extra=()) -> str:
    """Compile every kernel source of `csrc` and link `out` (libgs.so by
    default); returns its path."""
    os.makedirs(build_dir, exist_ok=True)
    jobs = jobs or min(8, len(SOURCES))
    with cf.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(lambda f: _compile(f, csrc, build_dir, extra), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(int(sys.argv[1]) if len(sys.argv) > 1 else None))
