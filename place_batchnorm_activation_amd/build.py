"""Build libiabn.so (HIP for gfx950) in-tree, next to this file."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libiabn.so")
BUILD_DIR = os.path.join(HERE, "_build")

SOURCES = ["fwd.hip", "bwd.hip", "fused_nchw.hip", "fused_nhwc.hip", "noalloc.hip", "api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-I" + INCLUDE, "-I" + CSRC,
] + os.environ.get("IABN_EXTRA_CFLAGS", "").split()
# Device code: gfx950 only.  Packed fp32 instructions are switched off (they are
# not needed by this bandwidth-bound code, and plain scalar fp32 is what we test).
# Code object v5: loadable by the HIP runtime that PyTorch-ROCm ships (the
# library binds to whichever libamdhip64 the process loaded first).
DEVICE = ["--offload-arch=" + ARCH, "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-mcode-object-version=5"]


def _compile(src: str, verbose: bool) -> str:
    out = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    cmd = [HIPCC] + COMMON
    if src.endswith(".hip"):
        cmd += DEVICE + ["-x", "hip"]
    cmd += ["-c", path, "-o", out]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    return out


def build(verbose: bool = False, out: str = LIB) -> str:
    """Always recompiles every source; returns the library path.  IABN_EXTRA_CFLAGS
    (environment) adds compiler flags, e.g. -D overrides of tiling constants."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
