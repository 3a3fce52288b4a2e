"""CPU sanitizer leg: AddressSanitizer + UndefinedBehaviorSanitizer over the host code.

* The fp64 oracle (oracle/la_oracle.c) runs every function on small seeded inputs
  in exactly-sized heap buffers (tests/sanitize/oracle_driver.c) and checks a few of
  its pins on the way.
* The C ABI's host half (csrc/api.cpp: validation, size arithmetic near the 2^31
  limits, workspace layout, launch sequencing) runs the documented cases of every
  entry point (tests/sanitize/abi_driver.cpp) with the kernel launchers replaced by
  stubs generated from csrc/launch.h, so no GPU or device code is involved.

Both are built with gcc / g++ for the host only and fail on the first report.
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "linear_attention_02_amd", "csrc")
SAN = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1", OMP_NUM_THREADS="2")


def need(tool):
    if shutil.which(tool) is None:
        pytest.skip(f"{tool} not available")


def run(cmd, **kw):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=600, **kw)
    assert r.returncode == 0, "\n".join([" ".join(cmd), r.stdout[-4000:]])
    return r.stdout


def launcher_stubs():
    """A definition for every kernel launcher declared in launch.h that only counts the call."""
    text = open(os.path.join(CSRC, "launch.h")).read()
    text = re.sub(r"//[^\n]*", "", text)
    decls = re.findall(r"hipError_t\s+(launch_\w+)\s*\(([^;]*?)\)\s*;", text, re.S)
    assert len(decls) >= 15, decls
    out = ['#include "launch.h"', "int g_stub_launches = 0;", "namespace la {"]
    for name, args in decls:
        args = re.sub(r"\s*=\s*[^,]+", "", " ".join(args.split()))  # drop default arguments
        out.append(f"hipError_t {name}({args}) {{ ++g_stub_launches; return hipSuccess; }}")
    out.append("}  // namespace la")
    return "\n".join(out) + "\n"


def test_oracle_under_sanitizers(tmp_path):
    need("gcc")
    exe = str(tmp_path / "oracle_san")
    run(["gcc", "-std=c11", "-fopenmp", "-ffp-contract=off", *SAN, "-I", os.path.join(ROOT, "oracle"),
         os.path.join(ROOT, "tests", "sanitize", "oracle_driver.c"), os.path.join(ROOT, "oracle", "la_oracle.c"),
         "-o", exe, "-lm"])
    assert "all checks passed" in run([exe], env=ENV)


def test_abi_host_code_under_sanitizers(tmp_path):
    need("g++")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    if not os.path.exists(os.path.join(rocm, "include", "hip", "hip_runtime.h")):
        pytest.skip("HIP headers not available")
    stubs = tmp_path / "launch_stubs.cpp"
    stubs.write_text(launcher_stubs())
    exe = str(tmp_path / "abi_san")
    run(["g++", "-std=c++17", "-Wno-unused-result", *SAN, "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(rocm, "include"),
         "-I", os.path.join(ROOT, "include"), "-I", CSRC, os.path.join(CSRC, "api.cpp"), str(stubs),
         os.path.join(ROOT, "tests", "sanitize", "abi_driver.cpp"), "-L", os.path.join(rocm, "lib"), "-lamdhip64",
         "-Wl,-rpath," + os.path.join(rocm, "lib"), "-o", exe])
    out = run([exe], env=ENV)
    assert "all cases as documented" in out
