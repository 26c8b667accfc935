"""Build libiabn.so (HIP for gfx950) in-tree, next to this file."""
from __future__ import annotations

import concurrent.futures
import hashlib
import os
import re
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libiabn.so")
BUILD_DIR = os.path.join(HERE, "_build")

SOURCES = ["fwd.hip", "bwd.hip", "fused_nchw.hip", "fused_nhwc.hip", "ckpt.hip", "noalloc.hip", "api.cpp"]

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


# Every kernel must run without scratch memory (no register spills): the
# compiler's per-kernel resource report is kept next to each object file and
# checked after every build.
REMARKS = ["-Rpass-analysis=kernel-resource-usage"]
_REMARK_FN = re.compile(r"remark: Function Name: (\S+)")
_REMARK_SCRATCH = re.compile(r"remark:\s+ScratchSize \[bytes/lane\]: (\d+)")


def source_digest() -> str:
    """Digest of every library source and header and of the device flags."""
    h = hashlib.sha256(" ".join(DEVICE + COMMON[:4]).encode())
    for d in (CSRC, INCLUDE):
        for f in sorted(os.listdir(d)):
            with open(os.path.join(d, f), "rb") as fh:
                h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def remarks_path(src: str) -> str:
    return os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".resource-usage.txt")


def scratch_use(text: str) -> dict:
    """{mangled kernel name: scratch bytes per lane} from a resource report."""
    out, name = {}, None
    for line in text.splitlines():
        m = _REMARK_FN.search(line)
        if m:
            name = m.group(1)
            continue
        m = _REMARK_SCRATCH.search(line)
        if m and name:
            out[name] = int(m.group(1))
    return out


def _compile(src: str, verbose: bool, digest: str) -> str:
    out = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    cmd = [HIPCC] + COMMON
    if src.endswith(".hip"):
        cmd += DEVICE + REMARKS + ["-x", "hip"]
    cmd += ["-c", path, "-o", out]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    r = subprocess.run(cmd, capture_output=True, text=True)
    other = "\n".join(l for l in r.stderr.splitlines() if "kernel-resource-usage" not in l and
                      not l.startswith(" ") and "packed-fp32-ops" not in l)
    if other.strip():
        print(other, file=sys.stderr)
    if r.returncode != 0:
        raise subprocess.CalledProcessError(r.returncode, cmd, r.stdout, r.stderr)
    if src.endswith(".hip"):
        with open(remarks_path(src), "w") as fh:
            fh.write("# source digest %s\n" % digest)
            fh.write(r.stderr)
    return out


def build(verbose: bool = False, out: str = LIB) -> str:
    """Always recompiles every source; returns the library path.  IABN_EXTRA_CFLAGS
    (environment) adds compiler flags, e.g. -D overrides of tiling constants.
    Raises if any kernel uses scratch memory."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    digest = source_digest()
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose, digest), SOURCES))
    spills = {}
    for src in SOURCES:
        if src.endswith(".hip"):
            with open(remarks_path(src)) as fh:
                spills.update({k: v for k, v in scratch_use(fh.read()).items() if v})
    if spills:
        raise RuntimeError("kernels using scratch memory (register spills): %s" % spills)
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
