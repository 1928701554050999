"""Build libsv.so (all HIP sources under csrc/) for gfx950 with hipcc, in-tree."""
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
LIB = os.path.join(PKG, "libsv.so")
OBJ_DIR = os.path.join(ROOT, "_build", "obj")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-I", INCLUDE, "-I", CSRC,
    # no packed fp32 instructions anywhere in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]
# Per-file additions.  The head_dim-128/256 attention kernel handles finite scores and -inf
# (masked keys) only; without NaN semantics its row maxima need no canonicalising
# moves before each v_max.
FILE_FLAGS = {"attn_mfma_w4.hip": ["-fno-honor-nans"]}


def _compile(src: str, extra: list[str], obj_dir: str) -> str:
    obj = os.path.join(obj_dir, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, *FILE_FLAGS.get(os.path.basename(src), []), *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build_library(extra: list[str] | None = None, jobs: int = 8, out: str = LIB,
                  obj_dir: str = OBJ_DIR) -> str:
    """Compile every csrc/*.hip and link libsv.so (next to this file by default)."""
    extra = extra or []
    os.makedirs(obj_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra, obj_dir), srcs))
    tmp = out + ".tmp"
    r = subprocess.run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build_library(sys.argv[1:]))
