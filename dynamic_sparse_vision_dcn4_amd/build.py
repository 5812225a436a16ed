"""Build libdcn4.so (the HIP library behind include/dcn4.h) for gfx950.

Flags: -O3; -ffp-contract=off so that every fp32 operation the kernels write
is one IEEE operation (the arithmetic order is part of the result); packed
fp32 instructions disabled (-packed-fp32-ops); no fast-math, so fp32
subnormals are kept."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
LIB = os.path.join(PKG, "libdcn4.so")
SOURCES = [os.path.join(PKG, "csrc", f) for f in ("dcn4_kernels.hip", "dcn4_linear.hip",
                                                   "dcn4_api.cpp")]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def command(out: str = LIB, extra=()) -> list:
    return [HIPCC, f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-shared", "-ffp-contract=off", "-fno-fast-math",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-I", os.path.join(ROOT, "include"),
            "-I", os.path.join(PKG, "csrc"), *extra, *SOURCES, "-o", out]


def build(out: str = LIB, verbose: bool = False) -> str:
    tmp = out + ".tmp"
    r = subprocess.run(command(tmp), capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError("hipcc failed to build libdcn4.so")
    if verbose:
        sys.stderr.write(r.stderr)
    os.replace(tmp, out)
    return out


C_CLIENT_SRC = os.path.join(ROOT, "tests", "c", "abi_forward.c")
C_CLIENT = os.path.join(ROOT, "tests", "c", "abi_forward")


def build_c_client(out: str = C_CLIENT) -> str:
    """A plain C program that uses only include/dcn4.h and the HIP runtime
    (gcc; links libdcn4.so and the system libamdhip64)."""
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           C_CLIENT_SRC, "-L", PKG, "-ldcn4", "-L", "/opt/rocm/lib", "-lamdhip64",
           f"-Wl,-rpath,{PKG}", "-Wl,-rpath,/opt/rocm/lib", "-o", out]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_c_client())
