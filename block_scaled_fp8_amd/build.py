"""Build the HIP library libmoe_w8a16.so in-tree for gfx950.

Usage: python -m block_scaled_fp8_amd.build  (or call build_library()).
Every HIP source under csrc/ is compiled with hipcc for gfx950 and linked into
one shared library next to this file.  Packed fp32 VALU instructions are
switched off for all device code.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libmoe_w8a16.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
BUILD_DIR = os.path.join(ROOT, "_build")

HIPCC_FLAGS = [
    "-O3", "-std=c++17", "-fPIC",
    "--offload-arch=gfx950",
    "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # fp32 division correctly rounded (the activation quantiser's quotient
    # must be the IEEE one); this is HIP's default, stated explicitly
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Wall", "-Wno-unused-result", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


def _hipcc() -> str:
    for cand in (shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: the HIP library cannot be built")


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))


def build_library(verbose: bool = False, jobs: int = 8, extra_flags=(), lib_path: str = LIB_PATH,
                  build_dir: str = BUILD_DIR) -> str:
    """Compiles every source and links lib_path.  extra_flags go to every
    compile (e.g. host-only sanitizer flags, each after -Xarch_host)."""
    hipcc = _hipcc()
    os.makedirs(build_dir, exist_ok=True)
    srcs = sources()

    def compile_one(src):
        obj = os.path.join(build_dir, os.path.basename(src) + ".o")
        cmd = [hipcc, *HIPCC_FLAGS, *extra_flags, "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(srcs)))) as ex:
        objs = list(ex.map(compile_one, srcs))
    tmp = lib_path + ".tmp"
    cmd = [hipcc, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build_library(verbose="-v" in sys.argv))
