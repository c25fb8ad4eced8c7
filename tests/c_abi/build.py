"""Build ``tests/c_abi/ew_c_client``: a plain C11 program that includes
``include/ew.h``, links ``libew.so``, the HIP runtime and the CPU oracle, and
checks a few calls end to end (test infrastructure).  Warnings are errors, so
the header is also checked to be clean C11."""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
PKG = os.path.join(ROOT, "memory_bound_elementwise_amd")
ORACLE = os.path.join(ROOT, "oracle")
ROCM_LIB = "/opt/rocm/lib"
SRC = os.path.join(HERE, "ew_c_client.c")
EXE = os.path.join(HERE, "ew_c_client")


def build(out: str = EXE, verbose: bool = False) -> str:
    cmd = ["gcc", "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror",
           "-I", os.path.join(ROOT, "include"), "-I", "/opt/rocm/include",
           "-o", out, SRC,
           "-L", PKG, "-lew", "-L", ORACLE, "-loracle", "-L", ROCM_LIB, "-lamdhip64",
           # found relative to the executable, wherever the tree is copied
           "-Wl,-rpath,$ORIGIN/../../memory_bound_elementwise_amd:$ORIGIN/../../oracle:"
           + ROCM_LIB]
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
