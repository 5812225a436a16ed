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
CSRC = os.path.join(PKG, "csrc")
SOURCES = [os.path.join(CSRC, f) for f in ("dcn4_kernels.hip", "dcn4_linear.hip",
                                           "dcn4_api.cpp")]
# the tiled forward kernels of each (dtype, sampling mode) pair compile in a
# translation unit of their own (dcn4_tile_part.hip), in parallel
TILE_PART = os.path.join(CSRC, "dcn4_tile_part.hip")
TILE_PAIRS = [(dt, mode) for dt in range(3) for mode in range(3)]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"


def flags(extra=()) -> list:
    return [f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
            "-ffp-contract=off", "-fno-fast-math",
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function", "-I", os.path.join(ROOT, "include"),
            "-I", CSRC, *extra]


def compile_units(tmpdir: str, extra=()) -> list:
    """(command, object) per translation unit."""
    units = []
    for src in SOURCES:
        obj = os.path.join(tmpdir, os.path.basename(src) + ".o")
        units.append(([HIPCC, *flags(extra), "-c", src, "-o", obj], obj))
    for dt, mode in TILE_PAIRS:
        obj = os.path.join(tmpdir, f"dcn4_tile_part_{dt}_{mode}.o")
        units.append(([HIPCC, *flags(extra), f"-DDCN4_TILE_PART_DT={dt}",
                       f"-DDCN4_TILE_PART_MODE={mode}", "-c", TILE_PART, "-o", obj], obj))
    return units


def build(out: str = LIB, verbose: bool = False, jobs: int = 0) -> str:
    import shutil
    import tempfile
    from concurrent.futures import ThreadPoolExecutor
    tmpdir = tempfile.mkdtemp(prefix="dcn4_build_")
    try:
        units = compile_units(tmpdir)
        jobs = jobs or min(len(units), max(1, min(os.cpu_count() or 1, 16)))
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            results = list(ex.map(lambda u: subprocess.run(u[0], capture_output=True,
                                                           text=True), units))
        failed = False
        for (cmd, _), r in zip(units, results):
            if r.returncode != 0 or verbose:
                sys.stderr.write(r.stdout + r.stderr)
            failed |= r.returncode != 0
        if failed:
            raise RuntimeError("hipcc failed to build libdcn4.so")
        tmp = out + ".tmp"
        link = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC",
                *[obj for _, obj in units], "-o", tmp]
        r = subprocess.run(link, capture_output=True, text=True)
        if r.returncode != 0:
            sys.stderr.write(r.stdout + r.stderr)
            raise RuntimeError("hipcc failed to link libdcn4.so")
        os.replace(tmp, out)
    finally:
        shutil.rmtree(tmpdir, ignore_errors=True)
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
