"""Build libmoeq8.so (HIP for gfx950) in the package directory.

Every source under csrc/ is compiled with hipcc for gfx950 only, in parallel,
then linked into one shared library.  Floating-point flags: no contraction of
a*b+c into FMA (the reduction order and the separately rounded products are
part of the kernels' contract), correctly rounded fp32 division, no fast math,
packed fp32 instructions disabled.
"""

from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
LIB_NAME = "libmoeq8.so"
LIB_PATH = os.path.join(PKG_DIR, LIB_NAME)
BUILD_DIR = os.path.join(PKG_DIR, "_build")

ARCH = "gfx950"
COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return cand


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _compile(src: str, build_dir: str = BUILD_DIR, extra=()) -> str:
    obj = os.path.join(build_dir, os.path.basename(src) + ".o")
    cmd = [hipcc(), *COMMON_FLAGS, *extra, "-c", src, "-o", obj]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{res.stdout}\n{res.stderr}")
    return obj


def build(verbose: bool = False, out_path: str = LIB_PATH, extra_flags=()) -> str:
    """Compile every HIP source and link ``out_path``.  Always rebuilds.
    ``extra_flags`` (e.g. -D tuning macros) go to every compile."""
    build_dir = BUILD_DIR if out_path == LIB_PATH else out_path + ".build"
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()
    workers = max(1, min(len(srcs), int(os.environ.get("MAX_JOBS", "8"))))
    with cf.ThreadPoolExecutor(workers) as ex:
        objs = list(ex.map(lambda s: _compile(s, build_dir, tuple(extra_flags)), srcs))
    tmp = out_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}\n{res.stderr}")
    os.replace(tmp, out_path)
    if verbose:
        print(f"built {out_path} from {len(srcs)} sources", file=sys.stderr)
    return out_path


if __name__ == "__main__":
    build(verbose=True)
