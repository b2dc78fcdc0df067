"""Build ``libcoli_moe.so`` (HIP, gfx950 only) in-tree with hipcc.

Every ``csrc/*.hip`` file is compiled to an object in parallel, then linked
into ``quantized_moe_coli_amd/libcoli_moe.so``.  hipcc cross-compiles for
gfx950 without a GPU present.  Packed-fp32 instructions are disabled for the
device code (the host pass warns that it does not know the feature; that is
harmless).
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG, "libcoli_moe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

CFLAGS = ["-O3", "-std=c++17", "--offload-arch=gfx950", "-fPIC", "-I", INCLUDE, "-I", CSRC,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")))


def _headers():
    return sorted(glob.glob(os.path.join(CSRC, "*.hpp")) + glob.glob(os.path.join(INCLUDE, "*.h")))


def _compile(src: str, extra=(), suffix=".o") -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + suffix)
    cmd = [HIPCC, *CFLAGS, *extra, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    warn = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip())
    if warn.strip():
        sys.stderr.write(warn + "\n")
    return obj


def stale() -> bool:
    if not os.path.exists(LIB_PATH):
        return True
    t = os.path.getmtime(LIB_PATH)
    return any(os.path.getmtime(p) > t for p in sources() + _headers())


# The timeline build: the same library with the decode kernel's timeline
# records compiled in (only these sources differ).
TRACE_LIB_PATH = os.path.join(PKG, "libcoli_moe_trace.so")
TRACE_SOURCES = ("decode.hip", "api.hip")
TRACE_FLAGS = ["-DCOLI_DECODE_TRACE"]


def _link(objs, path):
    tmp = path + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, path)


def build(jobs: int | None = None) -> str:
    """Compile and link the library and its timeline build; returns the
    library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = sources()
    traced = [s for s in srcs if os.path.basename(s) in TRACE_SOURCES]
    jobs = jobs or min(8, len(srcs) + len(traced))
    with cf.ThreadPoolExecutor(jobs) as ex:
        futs = [ex.submit(_compile, s) for s in srcs]
        tfuts = {os.path.basename(s): ex.submit(_compile, s, TRACE_FLAGS, ".trace.o") for s in traced}
        objs = [f.result() for f in futs]
        tobj = {k: f.result() for k, f in tfuts.items()}
    _link(objs, LIB_PATH)
    _link([tobj.get(os.path.basename(s), o) for s, o in zip(srcs, objs)], TRACE_LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build())
