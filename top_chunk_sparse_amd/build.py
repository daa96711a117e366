"""Build libtcsparse.so in-tree with hipcc for gfx950.

    python -m top_chunk_sparse_amd.build          # or __graft_entry__.build()

Every HIP translation unit is compiled with packed-fp32 instructions disabled
(``-target-feature -packed-fp32-ops``); the host pass of hipcc warns that it does not know
the feature, which is harmless.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(ROOT, "_build")
LIB = os.path.join(HERE, "libtcsparse.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = ["decode.hip", "prefill.hip", "prefill_bwd.hip", "gist_prefill.hip", "api.cpp",
           "noalloc.hip"]

COMMON = ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _compile(src, defines=(), objdir=OBJDIR):
    obj = os.path.join(objdir, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + list(defines) + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"hipcc failed on {src}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = False, defines=(), out=LIB, objdir=OBJDIR) -> str:
    """Compile and link.  ``defines`` (e.g. ["-DTCS_GIST_U=8"]) set the tuning macros."""
    os.makedirs(objdir, exist_ok=True)
    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(lambda f: _compile(f, defines, objdir), SOURCES))
    tmp = out + ".tmp"
    cmd = [HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print("built", out)
    return out


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
