"""Launch-configuration tuner for libew on the current GPU.

    python -m memory_bound_elementwise_amd.tune [--out PATH] [--repeats R]

For every operation and two size classes -- small (n = 2^20, launch- and
cache-bound) and large (n = 2^28 elements; 2^26 for the copy and the
gather) -- time each (block, blocks_per_cu, unroll) of the sweep with HIP
events recorded on the launch stream: the median over R repeats of K
back-to-back launches.  The fastest shape of each class becomes a row
"op min_n block blocks_per_cu unroll" of the table written to PATH (by
default the package's launch_table.txt, which the binding loads at import).

blocks_per_cu = 1024 caps the grid far above any tile count used here, so it
means "one block per tile" (no grid-stride rounds); smaller values give a
persistent grid of that many blocks per compute unit.
"""
import argparse
import itertools
import json
import os
import statistics
import sys

import torch

import memory_bound_elementwise_amd as ew

BLOCKS = (64, 128, 256, 512, 1024)
BPC = (1, 2, 4, 8, 1024)
UNROLLS = (1, 2, 4)
LARGE_MIN_N = 1 << 22
SIZES = {"small": 1 << 20, "large": 1 << 28}
LARGE_N = {"copy_f32": 1 << 26, "gather_f32": 1 << 26}
BYTES_PER_ELEM = {"add_f32": 12, "add_f16": 6, "add_bf16": 6, "saxpy_f32": 12,
                  "relu_f32": 8, "copy_f32": 8, "gather_f32": 8}


def _launcher(op, n, bufs, stream):
    a, b, c = bufs
    s = stream.cuda_stream
    if op in ("add_f32", "add_f16", "add_bf16"):
        fn = getattr(ew, "ew_" + op)
        return lambda: fn(a.data_ptr(), b.data_ptr(), c.data_ptr(), n=n, stream=s)
    if op == "saxpy_f32":
        return lambda: ew.ew_saxpy_f32(0.5, a.data_ptr(), c.data_ptr(), n=n, stream=s)
    if op == "relu_f32":
        return lambda: ew.ew_relu_f32(a.data_ptr(), c.data_ptr(), n=n, stream=s)
    if op == "copy_f32":
        return lambda: ew.ew_copy_f32(a.data_ptr(), c.data_ptr(), n=n, stream=s)
    return lambda: ew.ew_gather_f32(a.data_ptr(), c.data_ptr(), 2, n=n, stream=s)


def _time(launch, stream, launches, repeats):
    for _ in range(3):
        launch()
    torch.cuda.synchronize()
    out = []
    for _ in range(repeats):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(launches):
            launch()
        e1.record(stream)
        torch.cuda.synchronize()
        out.append(e0.elapsed_time(e1) / launches)
    return statistics.median(out)


def tune(ops=ew.OPS, repeats=3, log=None):
    """Returns {op: {"small": (block, bpc, unroll, GB/s), "large": (...)}}."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream()
    # 1 GiB per buffer covers 2^28 fp32 elements; 16-bit ops use the same bytes.
    bufs = tuple(torch.rand(1 << 28, device=dev) for _ in range(3))
    best = {}
    for op in ops:
        best[op] = {}
        for cls, n in SIZES.items():
            if cls == "large":
                n = LARGE_N.get(op, n)
            launch = _launcher(op, n, bufs, stream)
            launches = 20 if n >= (1 << 24) else 200
            results = []
            for block, bpc, unroll in itertools.product(BLOCKS, BPC, UNROLLS):
                for m in (0, LARGE_MIN_N):
                    ew.ew_set_launch_config(op, m, block, bpc, unroll)
                ms = _time(launch, stream, launches, repeats)
                gbs = BYTES_PER_ELEM[op] * n / (ms / 1e3) / 1e9
                results.append((gbs, block, bpc, unroll))
                if log:
                    log.write(json.dumps({"op": op, "class": cls, "n": n, "block": block,
                                          "bpc": bpc, "unroll": unroll, "gbs": gbs}) + "\n")
            results.sort(reverse=True)
            gbs, block, bpc, unroll = results[0]
            best[op][cls] = (block, bpc, unroll, round(gbs, 1))
            print(f"[tune] {op:10s} {cls:5s} n={n}: block {block} bpc {bpc} unroll {unroll} "
                  f"-> {gbs:.0f} GB/s", flush=True)
        ew.ew_reset_launch_config()
    return best


def write_table(best, path):
    dev = torch.cuda.get_device_name(0)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    lines = [
        "# Launch configuration per operation and size class, loaded by the Python",
        "# binding at import (ew_load_launch_table).  Columns:",
        "#   op  min_n  block  blocks_per_cu  unroll",
        "# A row applies to n >= min_n up to the next row's min_n.",
        f"# Written by memory_bound_elementwise_amd/tune.py on {dev} ({cus} CUs); the",
        "# trailing comment is the median GB/s measured for that row.",
    ]
    for op, rows in best.items():
        for cls, min_n in (("small", 0), ("large", LARGE_MIN_N)):
            block, bpc, unroll, gbs = rows[cls]
            lines.append(f"{op:<11s} {min_n:<8d} {block:<5d} {bpc:<5d} {unroll:<2d} # {gbs} GB/s")
    with open(path, "w") as f:
        f.write("\n".join(lines) + "\n")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--out", default=ew.LAUNCH_TABLE)
    ap.add_argument("--repeats", type=int, default=3)
    ap.add_argument("--ops", default=",".join(ew.OPS))
    ap.add_argument("--log", help="write every measurement as JSON lines here")
    args = ap.parse_args(argv)
    log = open(args.log, "w") if args.log else None
    best = tune(ops=args.ops.split(","), repeats=args.repeats, log=log)
    write_table(best, args.out)
    print(f"[tune] wrote {args.out}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
