"""Build libpi_ffn.so (the gfx950 HIP library) in-tree with hipcc.

Every translation unit under csrc/ is compiled to an object in parallel, then
the objects are linked into one shared library.
"""

import glob
import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_NAME = "libpi_ffn.so"
ARCH = os.environ.get("PI_FFN_ARCH", "gfx950")
BUILD_DIR = os.path.join(PKG_DIR, "_build")

FLAGS = [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
         # no packed-fp32 instructions in generated code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-Wno-unused-command-line-argument"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}: {' '.join(cmd[-3:])}")
    return res


def build(verbose: bool = False, jobs: int = 0) -> str:
    """Compile every HIP source for gfx950 and link PKG_DIR/libpi_ffn.so; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    sources = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    cc = hipcc()
    objs = [os.path.join(BUILD_DIR, os.path.basename(src)[:-4] + ".o") for src in sources]
    jobs = jobs or max(1, min(len(sources), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(jobs) as pool:
        list(pool.map(lambda so: _run([cc] + FLAGS + ["-I", INCLUDE, "-I", CSRC, "-c", so[0], "-o", so[1]],
                                      verbose), zip(sources, objs)))
    out = os.path.join(PKG_DIR, LIB_NAME)
    tmp = out + ".tmp"
    _run([cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs, verbose)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
