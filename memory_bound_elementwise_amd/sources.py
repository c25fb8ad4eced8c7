"""Which kernel sources each measured workload runs, and their hashes.

A committed rocprofv3 summary (kernel durations, HBM traffic) stays valid as
long as the sources of the kernels it measured are unchanged.  The kernels
live in one file per family; a family's hash covers its own file, the files
its kernels call into, and the shared device headers.  bench.py prints each
record's family hash, and a summary is used only while the hash it was taken
on matches the current one.  The host file (ew_api.cpp) is not hashed: what
it decides for a launch -- grid, block, unroll, the split -- is part of every
record's key.
"""
import hashlib
import os

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "csrc")
COMMON = ("ew_internal.h", "ew_device.h")
FAMILIES = {
    "stream": ("ew_stream.hip",),
    "batch": ("ew_batch_args.h", "ew_batch.hip"),
    "gather": ("ew_gather_args.h", "ew_gather.hip"),
    # the x[::s] views run the gather's kernels
    "view": ("ew_view_args.h", "ew_view.hip", "ew_gather_args.h", "ew_gather.hip"),
}


def family(op: str, batch: bool = False) -> str:
    """The kernel family of a libew operation (a batched call: "batch")."""
    if batch:
        return "batch"
    if op in ("gather_f32", "gather_walk_f32"):
        return "gather"
    if op == "copy2d_f32":
        return "view"
    return "stream"


def source_hash(fam: str) -> str:
    """sha256[:16] over the shared headers and the family's files, in order."""
    h = hashlib.sha256()
    for name in COMMON + FAMILIES[fam]:
        with open(os.path.join(CSRC, name), "rb") as f:
            data = f.read()
        h.update(name.encode() + b"\0" + len(data).to_bytes(8, "little") + data)
    return h.hexdigest()[:16]


def all_hashes() -> dict:
    return {fam: source_hash(fam) for fam in FAMILIES}
