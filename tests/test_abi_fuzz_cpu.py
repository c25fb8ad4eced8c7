"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

The library is rebuilt into a temporary directory with its host code
instrumented (the device code is compiled as usual), and the plain-C driver
``tests/c_abi/ew_fuzz.c``, instrumented the same way, makes a few hundred
thousand randomised calls of every host-side path: argument validation of
every entry point, the three plan functions, batch table images (sizes,
layout, too-small and misaligned buffers, plans that were not built), launch
rows and configurations, malformed launch-table files and status strings.
Device addresses are fabricated: the host code only does arithmetic on them,
and with no GPU visible every call that passes validation ends with
EW_ERR_NO_DEVICE before a launch (the driver refuses to run if a GPU is
visible).  Any sanitizer report, a status the header does not define, or a
plan or table image that breaks the header's identities fails the test.
"""
import os
import shutil
import subprocess

import pytest

from memory_bound_elementwise_amd import build as libbuild
from tests.conftest import ROOT

CLANG = "/opt/rocm/llvm/bin/clang"
SRC = os.path.join(ROOT, "tests", "c_abi", "ew_fuzz.c")
# host-side instrumentation only: each sanitizer flag is preceded by -Xarch_host
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]  # noqa: E501


@pytest.fixture(scope="module")
def fuzz_exe(tmp_path_factory):
    if not (os.path.exists(CLANG) and shutil.which("hipcc") or os.path.exists("/opt/rocm/bin/hipcc")):
        pytest.skip("the ROCm clang and hipcc are needed")
    d = tmp_path_factory.mktemp("san")
    lib = libbuild.build(extra_flags=HOST_SAN, out=str(d / "libew_san.so"))
    exe = str(d / "ew_fuzz")
    cmd = [CLANG, "-std=c11", "-O1", "-g", "-Wall", "-Wextra", "-Werror",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           "-fno-omit-frame-pointer", "-I", os.path.join(ROOT, "include"),
           "-o", exe, SRC, lib, "-L/opt/rocm/lib", "-lamdhip64",
           f"-Wl,-rpath,{d}:/opt/rocm/lib"]
    subprocess.run(cmd, check=True)
    return exe


@pytest.mark.parametrize("seed", [1, 2])
def test_host_code_is_clean_under_sanitizers(fuzz_exe, tmp_path, seed):
    env = dict(os.environ)
    env.update({
        # the HIP runtime is not instrumented: its allocations at exit are
        # not this library's leaks; the process may have a preloaded library
        "ASAN_OPTIONS": "detect_leaks=0:verify_asan_link_order=0:abort_on_error=0:"
                        "halt_on_error=1",
        "UBSAN_OPTIONS": "print_stacktrace=1:halt_on_error=1",
        # no GPU for the fabricated addresses, even on a machine that has one
        "HIP_VISIBLE_DEVICES": "-1", "ROCR_VISIBLE_DEVICES": "-1",
    })
    r = subprocess.run([fuzz_exe, "150000", str(seed), str(tmp_path / "table.txt")],
                       capture_output=True, text=True, timeout=600, env=env)
    if r.returncode == 77:
        pytest.skip("a GPU is visible")
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "ERROR: AddressSanitizer" not in out and "runtime error" not in out, out[-4000:]
    assert " 0 failures" in r.stdout, out[-2000:]
    print(r.stdout.strip())
    # every kind of outcome occurred, and no HIP call was reached
    counts = dict(kv.rsplit(" ", 1) for kv in r.stdout.split("statuses ")[1].split(", "))
    for name in ("OK", "INVALID_ARG", "MISALIGNED", "OVERLAP", "NO_DEVICE", "TOO_LARGE"):
        assert int(counts[name]) > 0, (name, r.stdout)
    assert int(counts["HIP"]) == 0, r.stdout
