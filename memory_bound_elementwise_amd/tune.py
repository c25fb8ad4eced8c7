"""Launch-configuration tuner for libew on the current GPU.

    python -m memory_bound_elementwise_amd.tune [--out PATH] [--repeats R]

For every operation and two size classes -- small (n = 2^20, launch- and
cache-bound) and large (n = 2^28 elements, a working set far beyond the
256 MB Infinity Cache, so the timing reflects HBM) -- time each (block, blocks_per_cu, unroll) of the sweep with HIP
events recorded on the launch stream: the median over R repeats of K
back-to-back launches, then the six fastest re-timed round-robin over seven
rounds (so drift hits all finalists alike).  The large fp32 add is timed with
input A one element past an aligned allocation, the misaligned workload its
headline figure is quoted on.  The fastest shape of each class becomes a row
"op min_n block blocks_per_cu unroll" of the table written to PATH (by
default the package's launch_table.txt, which the binding loads at import).

blocks_per_cu = 1024 caps the grid far above any tile count used here, so it
means "one block per tile" (no grid-stride rounds); smaller values give a
persistent grid of that many blocks per compute unit.
"""
import argparse
import itertools
import json
import statistics
import sys

import torch

import memory_bound_elementwise_amd as ew

BLOCKS = (64, 128, 256, 512, 1024)
BPC = (1, 2, 4, 8, 1024)
UNROLLS = (1, 2, 4)
LARGE_MIN_N = 1 << 22
SIZES = {"small": 1 << 20, "large": 1 << 28}
BYTES_PER_ELEM = {"add_f32": 12, "add_f16": 6, "add_bf16": 6, "saxpy_f32": 12,
                  "relu_f32": 8, "copy_f32": 8, "gather_f32": 8, "add_relu_f32": 12,
                  "saxpy_relu_f32": 12, "bias_relu_f32": 8, "saxpy_f16": 6, "saxpy_bf16": 6,
                  "relu_f16": 4, "relu_bf16": 4, "copy2d_f32": 8,
                  # in place on normal(0, 1) data: every 64-byte span changes
                  "relu_inplace_f32": 8,
                  **{f"{m}_{d}": 8 if d == "f32" else 4
                     for m in ew.SCALAR_MAPS + ew.UNARY_MAPS for d in ew.MAP_DTYPES}}
BIAS_COLS = 4096
# copy2d is tuned on a submatrix view: 16384 rows of 16380 columns out of
# 16384-wide rows (the row-contiguous path, which uses the table).
C2D_ROWS, C2D_COLS, C2D_PITCH = 16384, 16380, 16384


# Element offset of input A for the large fp32 add: the misaligned-input
# workload (A one element past an aligned allocation) is the one the headline
# is quoted on, and misaligned loads favour larger tiles (fewer tile
# boundaries whose split cache lines are fetched twice).
LARGE_OFFSETS = {"add_f32": 1}


def _launcher(op, n, bufs, stream, off_a=0):
    a, b, c = bufs
    s = stream.cuda_stream
    pa = a.data_ptr() + 4 * off_a
    if op in ("add_f32", "add_f16", "add_bf16", "add_relu_f32"):
        fn = getattr(ew, "ew_" + op)
        return lambda: fn(pa, b.data_ptr(), c.data_ptr(), n=n, stream=s)
    if op in ("saxpy_f32", "saxpy_relu_f32", "saxpy_f16", "saxpy_bf16"):
        fn = getattr(ew, "ew_" + op)
        return lambda: fn(0.5, pa, c.data_ptr(), n=n, stream=s)
    if op in ("relu_f16", "relu_bf16") or op.rsplit("_", 1)[0] in ew.UNARY_MAPS:
        fn = getattr(ew, "ew_" + op)
        return lambda: fn(pa, c.data_ptr(), n=n, stream=s)
    if op.rsplit("_", 1)[0] in ew.SCALAR_MAPS:
        fn = getattr(ew, "ew_" + op)
        return lambda: fn(2.5, pa, c.data_ptr(), n=n, stream=s)
    if op == "copy2d_f32":
        return lambda: ew.ew_copy2d_f32(pa + 4, C2D_PITCH, 1, c.data_ptr(), C2D_ROWS, C2D_COLS,
                                        stream=s)
    if op == "bias_relu_f32":
        return lambda: ew.ew_bias_relu_f32(pa, b.data_ptr(), c.data_ptr(), n // BIAS_COLS,
                                           BIAS_COLS, stream=s)
    if op == "relu_f32":
        return lambda: ew.ew_relu_f32(pa, c.data_ptr(), n=n, stream=s)
    if op == "copy_f32":
        return lambda: ew.ew_copy_f32(pa, c.data_ptr(), n=n, stream=s)
    return lambda: ew.ew_gather_f32(pa, c.data_ptr(), 2, n=n, stream=s)


def _time(launch, stream, launches, repeats, restore=None):
    """Median over `repeats` of the mean launch time in ms.  With `restore`
    (an in-place op's input must be put back before each launch) every launch
    is timed by its own events, the restore outside them."""
    for _ in range(3):
        if restore is not None:
            restore()
        launch()
    torch.cuda.synchronize()
    out = []
    if restore is not None:
        with torch.cuda.stream(stream):
            for _ in range(repeats):
                evs = []
                for _ in range(launches):
                    restore()
                    e0 = torch.cuda.Event(enable_timing=True)
                    e1 = torch.cuda.Event(enable_timing=True)
                    e0.record(stream)
                    launch()
                    e1.record(stream)
                    evs.append((e0, e1))
                torch.cuda.synchronize()
                out.append(sum(a.elapsed_time(b) for a, b in evs) / launches)
        return statistics.median(out)
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


def _set(op, block, bpc, unroll):
    """Force one shape on every size class of op (every min_n of the loaded
    table's rows, plus 0 and LARGE_MIN_N), so the timed size uses it."""
    mins = {0, LARGE_MIN_N} | {r[0] for r in _read_rows(ew.LAUNCH_TABLE).get(op, [])}
    for m in sorted(mins):
        ew.ew_set_launch_row(op, m, block, bpc, unroll)


def tune(ops=ew.OPS, repeats=3, finalists=6, rounds=7, log=None):
    """Returns {op: {"small": (block, bpc, unroll, GB/s), "large": (...)}}.

    Stage 1 times every shape (median of `repeats`); stage 2 re-times the
    `finalists` fastest shapes round-robin for `rounds` rounds, so slow drift
    of clocks or temperature affects all finalists alike, and picks the best
    median."""
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream()
    # 1 GiB (+ one element) per buffer covers 2^28 fp32 elements at an offset.
    bufs = tuple(torch.rand((1 << 28) + 64, device=dev) for _ in range(3))
    best = {}
    for op in ops:
        best[op] = {}
        for cls, n in SIZES.items():
            off_a = LARGE_OFFSETS.get(op, 0) if cls == "large" else 0
            launch = _launcher(op, n, bufs, stream, off_a)
            launches = 20 if n >= (1 << 24) else 200
            nbytes = BYTES_PER_ELEM[op] * n
            if op == "copy2d_f32":
                if cls == "small":
                    launch = lambda: ew.ew_copy2d_f32(bufs[0].data_ptr() + 4, 1024, 1,
                                                      bufs[2].data_ptr(), 1024, 1020,
                                                      stream=stream.cuda_stream)
                    nbytes = 8 * 1024 * 1020
                else:
                    nbytes = 8 * C2D_ROWS * C2D_COLS
            restore = None
            if op == "relu_inplace_f32":
                # mixed signs (normal data), put back before every launch
                x = bufs[2][:n]
                pristine = torch.randn(n, device=dev)
                launch = lambda: ew.ew_relu_inplace_f32(x, n=n, stream=stream.cuda_stream)
                restore = lambda: x.copy_(pristine)
            results = []
            for block, bpc, unroll in itertools.product(BLOCKS, BPC, UNROLLS):
                _set(op, block, bpc, unroll)
                ms = _time(launch, stream, launches, repeats, restore)
                results.append((nbytes / (ms / 1e3) / 1e9, block, bpc, unroll))
                if log:
                    log.write(json.dumps({"op": op, "class": cls, "n": n, "stage": 1,
                                          "block": block, "bpc": bpc, "unroll": unroll,
                                          "gbs": results[-1][0]}) + "\n")
            results.sort(reverse=True)
            shapes = [r[1:] for r in results[:finalists]]
            times = {sh: [] for sh in shapes}
            for _ in range(rounds):
                for sh in shapes:
                    _set(op, *sh)
                    times[sh].append(_time(launch, stream, launches, 1, restore))
            final = sorted(((nbytes / (statistics.median(t) / 1e3) / 1e9,) + sh
                            for sh, t in times.items()), reverse=True)
            if log:
                for f in final:
                    log.write(json.dumps({"op": op, "class": cls, "n": n, "stage": 2,
                                          "block": f[1], "bpc": f[2], "unroll": f[3],
                                          "gbs": f[0]}) + "\n")
            gbs, block, bpc, unroll = final[0]
            best[op][cls] = (block, bpc, unroll, round(gbs, 1))
            print(f"[tune] {op:10s} {cls:5s} n={n}: block {block} bpc {bpc} unroll {unroll} "
                  f"-> {gbs:.0f} GB/s", flush=True)
        ew.ew_reset_launch_config()
    return best


def _read_rows(path):
    """Existing rows {op: [(min_n, block, bpc, unroll, comment)]} of a table file."""
    rows = {}
    try:
        lines = open(path).read().splitlines()
    except OSError:
        return rows
    for line in lines:
        body, _, comment = line.partition("#")
        f = body.split()
        if len(f) == 5:
            rows.setdefault(f[0], []).append(
                (int(f[1]), int(f[2]), int(f[3]), int(f[4]), comment.strip()))
    return rows


def write_table(best, path, merge_from=None):
    """Write the table.  Ops not in `best` keep their rows from `merge_from`.
    A tuned op gets its small row (min_n 0) and its large row, which replaces
    the op's last existing row at or above LARGE_MIN_N (so a large row that
    starts at 2^25, above a mid-size row, stays there); any other existing row
    of the op -- a mid-size row measured cold by a separate sweep -- is kept."""
    dev = torch.cuda.get_device_name(0)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    old = _read_rows(merge_from) if merge_from else {}
    lines = [
        "# Launch configuration per operation and size class, loaded by the Python",
        "# binding at import (ew_load_launch_table).  Columns:",
        "#   op  min_n  block  blocks_per_cu  unroll",
        "# A row applies to n >= min_n up to the next row's min_n.",
        f"# Written by memory_bound_elementwise_amd/tune.py on {dev} ({cus} CUs); the",
        "# trailing comment is the median GB/s measured for that row.",
    ]
    for op in ew.OPS:
        if op in best:
            kept = {r[0]: r for r in old.get(op, [])}
            large_min = max((m for m in kept if m >= LARGE_MIN_N), default=LARGE_MIN_N)
            rows = {m: r for m, r in kept.items() if m not in (0, large_min)}
            for cls, min_n in (("small", 0), ("large", large_min)):
                block, bpc, unroll, gbs = best[op][cls]
                rows[min_n] = (min_n, block, bpc, unroll, f"{gbs} GB/s")
            for (min_n, block, bpc, unroll, comment) in (rows[m] for m in sorted(rows)):
                tail = f" # {comment}" if comment else ""
                lines.append(f"{op:<15s} {min_n:<8d} {block:<5d} {bpc:<5d} {unroll:<2d}{tail}")
        else:
            for (min_n, block, bpc, unroll, comment) in old.get(op, []):
                tail = f" # {comment}" if comment else ""
                lines.append(f"{op:<15s} {min_n:<8d} {block:<5d} {bpc:<5d} {unroll:<2d}{tail}")
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
    write_table(best, args.out, merge_from=ew.LAUNCH_TABLE)
    print(f"[tune] wrote {args.out}")
    return 0


if __name__ == "__main__":
    sys.exit(main())
