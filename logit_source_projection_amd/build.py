"""Build step for libsb.so (gfx950): hipcc, in-tree, always recompiles."""
import os
import subprocess

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libsb.so")
SOURCES = ["kernels.hip", "sb_api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # packed fp32 VALU forms are kept out of every kernel
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    # every symbol resolved at link time: a kernel template that failed to
    # instantiate is an error here, not a library that fails to load
    "-Wl,-z,defs",
    # export the sb_* calls of include/sb.h and nothing else
    "-Wl,--version-script=" + os.path.join(CSRC, "libsb.map"),
]


def build(verbose=False):
    """Compile libsb.so beside this file and return its path."""
    tmp = LIB + ".tmp"
    cmd = [HIPCC] + FLAGS + [os.path.join(CSRC, s) for s in SOURCES] + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


DRIVER_SRC = os.path.join(ROOT, "tests", "abi_driver.c")
DRIVER = os.path.join(ROOT, "tests", "abi_driver")


def build_abi_driver(verbose=False):
    """Compile the plain C program that drives libsb.so through include/sb.h
    and the HIP runtime alone (a test of the C ABI); C99, gcc.  It finds
    libsb.so through an rpath relative to itself.  Call after build()."""
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    tmp = DRIVER + ".tmp"
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(rocm, "include"), "-I", os.path.join(ROOT, "include"),
           DRIVER_SRC, "-o", tmp, "-L", HERE, "-lsb", "-L", os.path.join(rocm, "lib"),
           "-lamdhip64", "-Wl,-rpath,$ORIGIN/../logit_source_projection_amd",
           "-Wl,-rpath," + os.path.join(rocm, "lib")]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, DRIVER)
    return DRIVER


if __name__ == "__main__":
    print(build(verbose=True))
    print(build_abi_driver(verbose=True))
