"""Build libsfmla.so (gfx950 kernels + C ABI) in-tree with hipcc."""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libsfmla.so")
BUILD = os.path.join(HERE, "_build")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
# Packed fp32 ops stay off: hipcc would otherwise form v_pk_* fp32 ops.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC, "-Wall",
          "-Wno-unused-function"]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("build step failed: %s" % " ".join(cmd))
    noise = "packed-fp32-ops"
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if noise not in ln and ln.strip()]
    if msgs and verbose:
        print("\n".join(msgs))


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    k_obj = os.path.join(BUILD, "sfmla_kernels.o")
    a_obj = os.path.join(BUILD, "sfmla_api.o")
    _run([HIPCC, "-x", "hip", "--offload-arch=" + ARCH] + DEVICE_FLAGS + COMMON +
         ["-c", os.path.join(CSRC, "sfmla_kernels.hip"), "-o", k_obj], verbose)
    _run([HIPCC] + COMMON + ["-D__HIP_PLATFORM_AMD__", "-c", os.path.join(CSRC, "sfmla_api.cpp"),
                             "-o", a_obj], verbose)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=" + ARCH, "-shared", "-fPIC", k_obj, a_obj, "-o", tmp], verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
