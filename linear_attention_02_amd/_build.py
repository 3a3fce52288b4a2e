"""Build the gfx950 HIP library ``liblinattn.so`` in-tree with hipcc.

Each source under ``csrc/`` is compiled to an object in parallel, then linked
into ``linear_attention_02_amd/liblinattn.so``.  The library exports the C ABI
declared in ``include/linattn.h``.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJDIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "liblinattn.so")
SOURCES = ("fwd.hip", "bwd.hip", "ncbwd.hip", "decode.hip", "favor.hip", "noalloc.hip", "api.cpp")
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found; the HIP library needs ROCm's hipcc")


def common_flags() -> list[str]:
    extra = os.environ.get("LINATTN_HIPCC_FLAGS", "").split()
    return extra + [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # no packed-fp32 instructions in device code
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE, "-I", CSRC,
    ]


def _compile(src: str) -> str:
    obj = os.path.join(OBJDIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc()] + common_flags() + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{out}")
    return obj


def build(jobs: int | None = None, verbose: bool = False, out: str | None = None) -> str:
    """Compile every HIP source for gfx950 and link liblinattn.so (or `out`); returns its path."""
    os.makedirs(OBJDIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), os.cpu_count() or 1)
    with cf.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(_compile, SOURCES))
    lib = out or LIB
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", tmp]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout)
    os.replace(tmp, lib)
    if verbose:
        print(f"built {lib}", file=sys.stderr)
    return lib


if __name__ == "__main__":
    build(verbose=True, out=sys.argv[1] if len(sys.argv) > 1 else None)
