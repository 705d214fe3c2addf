"""Build libdex.so (the HIP lattice-step library) for gfx950 with hipcc.

Usage: python -m lossless_depth_adaptive_amd.build  (or build() from Python).
The shared library lands next to this file; it is git-ignored but travels with
the source tree.
"""

import hashlib
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libdex.so")
SOURCES = ["gemm.hip", "layer.hip", "lattice.hip", "dex_capi.hip"]
ARCH = os.environ.get("DEX_OFFLOAD_ARCH", "gfx950")

# Packed fp32 VALU forms are disabled for every device compile.
FLAGS = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-result", f"-I{INCLUDE}", f"-I{CSRC}"]

# The GEMM and attention kernels keep their MFMA accumulators in ordinary
# VGPRs: the compiler otherwise rotates them through AGPRs with copies in every
# k-step, or spills into AGPRs.
SOURCE_FLAGS = {src: ["-mllvm", "-amdgpu-mfma-vgpr-form"] for src in ("gemm.hip", "layer.hip")}


def library_digest(path: str = LIB) -> str:
    """SHA-256 (16 hex digits) of a built library file. Measurements taken
    with one build (counter summaries) name it, so a later reader can tell
    whether they still describe the library it loads; builds of the same
    sources with the same flags are byte-identical."""
    h = hashlib.sha256()
    with open(path, "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def _hipcc():
    for c in ("/opt/rocm/bin/hipcc", "hipcc"):
        if os.path.exists(c) or c == "hipcc":
            return c


def _compile(src: str, outdir: str, defines=()) -> str:
    obj = os.path.join(outdir, os.path.splitext(src)[0] + ".o")
    cmd = [_hipcc(), *FLAGS, *SOURCE_FLAGS.get(src, []), *[f"-D{d}" for d in defines], "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-6000:]}")
    return obj


def build(verbose: bool = True, lib: str = LIB, defines=()) -> str:
    """Compile every source and link ``lib``; ``defines`` are extra -D flags
    (tuning macros of the sources)."""
    outdir = os.path.join(HERE, "_build" + ("_" + "_".join(d.replace("=", "") for d in defines) if defines else ""))
    os.makedirs(outdir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda s: _compile(s, outdir, defines), SOURCES))
    tmp = lib + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-6000:]}")
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    build()
    sys.exit(0)
