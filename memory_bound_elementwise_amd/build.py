"""Build ``libew.so`` (the C-ABI library in ``include/ew.h``) for gfx950.

    python memory_bound_elementwise_amd/build.py          # build in-tree
    python memory_bound_elementwise_amd/build.py --asm D  # also dump device asm to D

It is a standalone script: importing the package itself requires the built
library.

The library is built in-tree next to this file so that it travels with the
source tree.  Flags: no fast-math (IEEE results with subnormals preserved),
and packed-fp32 instruction forms disabled for every device pass.
"""
import argparse
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libew.so")
ARCH = "gfx950"

KERNEL_SOURCES = [os.path.join(CSRC, f) for f in
                  ("ew_stream.hip", "ew_batch.hip", "ew_gather.hip", "ew_view.hip")]
SOURCES = [os.path.join(CSRC, "ew_api.cpp"), *KERNEL_SOURCES]

DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Wall", "-Wextra", "-Wno-unused-parameter",
    "-I", INCLUDE, "-I", CSRC,
] + DEVICE_FLAGS


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), file=sys.stderr)
    res = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in res.stdout.splitlines()
                    if "packed-fp32-ops' is not a recognized feature" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"build failed ({res.returncode}):\n{' '.join(cmd)}\n{out}")
    if verbose and out.strip():
        print(out, file=sys.stderr)


def build(verbose: bool = False, extra_flags=(), out: str = LIB) -> str:
    """Compile every HIP source of the library for gfx950; returns the .so path."""
    tmp = out + ".tmp"
    cmd = [hipcc(), *COMMON_FLAGS, *extra_flags, "-shared", "-o", tmp, *SOURCES]
    _run(cmd, verbose)
    os.replace(tmp, out)
    return out


def device_asm(dest_dir: str, verbose: bool = False, extra_flags=()) -> str:
    """Write the gfx950 assembly of every kernel source to ``dest_dir``, one
    file per source plus their concatenation; returns the concatenation's path."""
    os.makedirs(dest_dir, exist_ok=True)
    parts = []
    for src in KERNEL_SOURCES:
        stem = os.path.splitext(os.path.basename(src))[0]
        path = os.path.join(dest_dir, f"{stem}-{ARCH}.s")
        cmd = [hipcc(), *COMMON_FLAGS, *extra_flags, "--cuda-device-only", "-S", "-o", path, src]
        _run(cmd, verbose)
        with open(path) as f:
            parts.append(f.read())
    path = os.path.join(dest_dir, f"ew_kernels-{ARCH}.s")
    with open(path, "w") as f:
        f.write("\n".join(parts))
    return path


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--asm", metavar="DIR", help="also write device assembly to DIR")
    ap.add_argument("-v", "--verbose", action="store_true")
    args = ap.parse_args(argv)
    print(build(verbose=args.verbose))
    if args.asm:
        print(device_asm(args.asm, verbose=args.verbose))


if __name__ == "__main__":
    main()
