"""Summarise rocprofv3 CSV output of bench.py runs into short text records.

Kernel durations (from ``rocprofv3 --kernel-trace --stats -f csv``):

    python -m memory_bound_elementwise_amd.rocprof_summary trace \\
        --stats DIR/NAME_kernel_stats.csv --kernel REGEX --bytes B \\
        --bench-json BENCH_OUTPUT_OF_THE_PROFILED_RUN \\
        --command "the rocprofv3 command line" --out profiles/FILE.txt

Every configuration's kernel durations from the kernel trace of one default
bench run (per-dispatch median, matched by kernel name, grid and block):

    python -m memory_bound_elementwise_amd.rocprof_summary configs \\
        --trace DIR/NAME_kernel_trace.csv --bench-json BENCH_OUTPUT \\
        --command "the rocprofv3 command line" --out profiles/FILE.txt

HBM traffic (from two ``rocprofv3 --pmc`` runs per kernel, FETCH_SIZE then
WRITE_SIZE, each in KiB per dispatch).  The counters are calibrated on the
plain copy kernel of known size: scale = algorithmic bytes / counted bytes,
per counter.  The result is written as text and merged into
profiles/traffic.json, which bench.py reads (keyed by workload, kernel
source hash and launch shape):

    python -m memory_bound_elementwise_amd.rocprof_summary traffic \\
        --workload NAME --kernel REGEX --bytes B \\
        --fetch DIR/..._counter_collection.csv --write DIR/..._counter_collection.csv \\
        --calib-kernel REGEX --calib-bytes-read R --calib-bytes-written W \\
        --calib-fetch CSV --calib-write CSV --launch '{"block": .., "grid": .., "unroll": ..}' \\
        --bench-json FETCH_RUN_OUTPUT --bench-json-write WRITE_RUN_OUTPUT \\
        --command-fetch "..." --command-write "..." --command-calib "..." --out profiles/FILE.txt

The kernel source hash written into every record is the one the profiled
bench.py run printed (env.kernel_source_sha256_16), never the hash of the
source as it is when the summary is written.
"""
import argparse
import csv
import json
import os
import re
import statistics
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")


def bench_record(path):
    """The JSON line bench.py printed in the profiled run (its last line)."""
    with open(path) as f:
        return json.loads(f.read().strip().splitlines()[-1])


def profiled_hash(bench_json):
    """The kernel source hash the profiled run was built from: taken from the
    bench line it printed, so that a summary written later, after the source
    has changed, cannot claim the new hash.  Refuses a bench line without one."""
    rec = bench_record(bench_json)
    h = rec.get("env", {}).get("kernel_source_sha256_16")
    if not h:
        raise SystemExit(f"{bench_json}: no env.kernel_source_sha256_16")
    return h


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def kernel_stats(path, kernel_re):
    """(name, calls, average ns, min ns, max ns) of the kernel matching the regex."""
    rx = re.compile(kernel_re)
    for r in _rows(path):
        if rx.search(r["Name"]):
            return (r["Name"], int(r["Calls"]), float(r["AverageNs"]), float(r["MinNs"]),
                    float(r["MaxNs"]))
    raise SystemExit(f"no kernel matching {kernel_re!r} in {path}")


def counter_per_dispatch(path, kernel_re, counter):
    """Median over dispatches of the counter summed within each dispatch."""
    rx = re.compile(kernel_re)
    per = {}
    for r in _rows(path):
        if r.get("Counter_Name") != counter or not rx.search(r.get("Kernel_Name", "")):
            continue
        per.setdefault(r.get("Dispatch_Id") or r.get("Correlation_Id"), 0.0)
        per[r.get("Dispatch_Id") or r.get("Correlation_Id")] += float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} rows for kernel {kernel_re!r} in {path}")
    return statistics.median(per.values()), len(per)


def dispatch_durations(path, kernel_re):
    """Per-dispatch durations in ns of the kernel matching the regex, from a
    rocprofv3 kernel_trace.csv."""
    rx = re.compile(kernel_re)
    return [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in _rows(path)
            if rx.search(r.get("Kernel_Name", ""))]


def cmd_trace(a):
    name, calls, avg, mn, mx = kernel_stats(a.stats, a.kernel)
    gbs = a.bytes / avg
    src_hash = profiled_hash(a.bench_json)
    bench_ms = bench_record(a.bench_json).get("ms_per_step")
    text = [
        f"# {a.title}",
        "",
        f"command: {a.command}",
        f"source:  rocprofv3 kernel_stats.csv ({os.path.basename(a.stats)})",
        "",
        f"kernel:          {name}",
        f"dispatches:      {calls}",
        f"average:         {avg / 1000:.3f} us   (min {mn / 1000:.3f}, max {mx / 1000:.3f})",
    ]
    if a.trace:
        d = sorted(dispatch_durations(a.trace, a.kernel))
        text.append(f"median:          {statistics.median(d) / 1000:.3f} us   (p10 "
                    f"{d[len(d) // 10] / 1000:.3f}, p90 {d[(9 * len(d)) // 10] / 1000:.3f}; "
                    f"{len(d)} dispatches in {os.path.basename(a.trace)})")
    text += [
        f"algorithmic:     {a.bytes} bytes per launch",
        f"achieved:        {gbs:.1f} GB/s = {100 * gbs / 8000:.2f} % of 8000 GB/s",
        f"kernel source:   ew_kernels.hip sha256[:16] {src_hash} (of the profiled run)",
    ]
    if bench_ms:
        text.append(f"bench.py events: {bench_ms:.5f} ms per step "
                    f"({100 * (bench_ms * 1e6 - avg) / avg:+.2f} % vs the trace average)")
    with open(a.out, "w") as f:
        f.write("\n".join(text) + "\n")
    print("\n".join(text))


def cmd_traffic(a):
    fetch_kib, nd_f = counter_per_dispatch(a.fetch, a.kernel, "FETCH_SIZE")
    write_kib, nd_w = counter_per_dispatch(a.write, a.kernel, "WRITE_SIZE")
    cal_f, _ = counter_per_dispatch(a.calib_fetch, a.calib_kernel, "FETCH_SIZE")
    cal_w, _ = counter_per_dispatch(a.calib_write, a.calib_kernel, "WRITE_SIZE")
    scale_f = a.calib_bytes_read / (cal_f * 1024)
    scale_w = a.calib_bytes_written / (cal_w * 1024)
    fetch_b = fetch_kib * 1024 * scale_f
    write_b = write_kib * 1024 * scale_w
    total = fetch_b + write_b
    launch = json.loads(a.launch)
    src_hash = profiled_hash(a.bench_json)
    if profiled_hash(a.bench_json_write) != src_hash:
        raise SystemExit("the FETCH_SIZE and WRITE_SIZE runs were built from different sources")
    text = [
        f"# HBM traffic: {a.workload}",
        "",
        f"fetch command: {a.command_fetch}",
        f"write command: {a.command_write}",
        f"calibration:   {a.command_calib}",
        "",
        f"kernel:            {a.kernel}  launch {launch}",
        f"FETCH_SIZE:        {fetch_kib:.0f} KiB per dispatch (median of {nd_f})",
        f"WRITE_SIZE:        {write_kib:.0f} KiB per dispatch (median of {nd_w})",
        f"calibration copy:  FETCH {cal_f:.0f} KiB for {a.calib_bytes_read} B read -> scale "
        f"{scale_f:.4f};  WRITE {cal_w:.0f} KiB for {a.calib_bytes_written} B written -> scale "
        f"{scale_w:.4f}",
        f"HBM bytes/launch:  fetch {fetch_b:.0f} + write {write_b:.0f} = {total:.0f}",
        f"algorithmic bytes: {a.bytes}  (traffic / algorithmic = {total / a.bytes:.4f})",
        f"kernel source:     ew_kernels.hip sha256[:16] {src_hash} (of the profiled runs)",
    ]
    with open(a.out, "w") as f:
        f.write("\n".join(text) + "\n")
    print("\n".join(text))
    try:
        with open(TRAFFIC_JSON) as f:
            data = json.load(f)
    except (OSError, ValueError):
        data = {"about": "HBM bytes per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                         "scaled by the copy-kernel calibration; see the .txt summaries",
                "workloads": {}}
    data["workloads"][a.workload] = {
        "kernel": a.kernel, "launch": launch, "kernel_source_sha256_16": src_hash,
        "fetch_kib": fetch_kib, "write_kib": write_kib, "scale_fetch": scale_f,
        "scale_write": scale_w, "hbm_bytes_per_launch": round(total),
        "algorithmic_bytes": a.bytes, "summary": os.path.basename(a.out)}
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")


# Kernel of each operation in a kernel trace (template operator name).
OP_KERNEL = {"add_f32": "OpAddF32", "add_f16": "OpAddF16", "add_bf16": "OpAddBF16",
             "saxpy_f32": "OpSaxpyF32", "relu_f32": "OpReluF32", "copy_f32": "OpCopyF32"}
BYTES_PER_ELEM = {"add_f32": 12, "add_f16": 6, "add_bf16": 6, "saxpy_f32": 12, "relu_f32": 8,
                  "copy_f32": 8, "gather_f32": 8}


def cmd_configs(a):
    """Per-dispatch durations of every configuration's kernel in one traced
    default bench run: each record of the bench line (main workload and
    other_configs) whose op is a streaming op or the gather is matched to the
    trace by kernel name, grid and block."""
    line = bench_record(a.bench_json)
    src_hash = line.get("env", {}).get("kernel_source_sha256_16")
    main = {"workload": line["config"]["name"], "op": line["config"]["op"],
            "n": line["config"]["n"], "launch": line["config"]["launch"],
            "split": line["config"]["split"], "gbs": line["value"], "timing": "back-to-back, mean"}
    recs = [main] + [r for r in line.get("other_configs", [])
                     if r.get("op") in BYTES_PER_ELEM and r.get("workload", "").startswith(("cfg", "headline"))]
    rows = _rows(a.trace)
    text = [
        "# Kernel durations of the five configurations and the headline (rocprofv3 kernel trace)",
        "",
        f"command: {a.command}",
        f"source:  per-dispatch durations (End - Start) in {os.path.basename(a.trace)}, each "
        "configuration's kernel matched by name, grid and block",
        "note:    for the cold workloads (<= 1 GiB) the dispatches include the rotated launches "
        "that bench.py times, the flushed per-launch ones and the warm ones; all include the "
        "parity launch",
        "         the bench.py column is that profiled run's own figure: the tracer adds host-side "
        "cost to every launch, which shows only where back-to-back launches are bound by the "
        "host (the 2^20 add)",
        f"kernel source: ew_kernels.hip sha256[:16] {src_hash} (of the profiled run)",
        "",
        "| workload | kernel | grid x block | dispatches | median us (p10, p90) | GB/s at the median "
        "| bench.py GB/s (its timing) |",
        "|---|---|---|---|---|---|---|",
    ]
    for r in sorted(recs, key=lambda r: r["workload"]):
        op, n, lc = r["op"], r["n"], r["launch"]
        if op == "gather_f32":
            rx = re.compile(r"ew_gather(2|_passes)?_kernel")
        else:
            co = ["true" if c else "false" for c in r["split"]["in_coaligned"]]
            rx = re.compile(re.escape(f"ew_stream_kernel<ew::{OP_KERNEL[op]}, {lc['unroll']}, "
                                      f"{co[0]}, {co[1]}>"))
        d = sorted(int(x["End_Timestamp"]) - int(x["Start_Timestamp"]) for x in rows
                   if rx.search(x["Kernel_Name"])
                   and int(x["Workgroup_Size_X"]) == lc["block"]
                   and int(x["Grid_Size_X"]) == lc["block"] * lc["grid"])
        if not d:
            raise SystemExit(f"no dispatch of {r['workload']}'s kernel in {a.trace}")
        med = statistics.median(d)
        name = next(x["Kernel_Name"] for x in rows if rx.search(x["Kernel_Name"]))
        name = name.replace("void ew::", "").split("(")[0]
        gbs = BYTES_PER_ELEM[op] * n / med
        text.append(f"| {r['workload']} | {name} | {lc['grid']} x {lc['block']} | {len(d)} | "
                    f"{med / 1000:.2f} ({d[len(d) // 10] / 1000:.2f}, {d[(9 * len(d)) // 10] / 1000:.2f}) | "
                    f"{gbs:.1f} | {r['gbs']} ({r['timing']}) |")
    with open(a.out, "w") as f:
        f.write("\n".join(text) + "\n")
    print("\n".join(text))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("trace")
    t.add_argument("--stats", required=True)
    t.add_argument("--kernel", required=True)
    t.add_argument("--bytes", type=int, required=True)
    t.add_argument("--command", required=True)
    t.add_argument("--title", default="Kernel duration")
    t.add_argument("--trace", help="the run's kernel_trace.csv: also report the per-dispatch "
                                   "median")
    t.add_argument("--bench-json", required=True,
                   help="the bench.py output of the profiled run (events and source hash)")
    t.add_argument("--out", required=True)
    r = sub.add_parser("traffic")
    r.add_argument("--workload", required=True)
    r.add_argument("--kernel", required=True)
    r.add_argument("--bytes", type=int, required=True)
    r.add_argument("--fetch", required=True)
    r.add_argument("--write", required=True)
    r.add_argument("--calib-kernel", required=True)
    r.add_argument("--calib-bytes-read", type=int, required=True)
    r.add_argument("--calib-bytes-written", type=int, required=True)
    r.add_argument("--calib-fetch", required=True)
    r.add_argument("--calib-write", required=True)
    r.add_argument("--launch", required=True)
    r.add_argument("--command-fetch", required=True)
    r.add_argument("--command-write", required=True)
    r.add_argument("--command-calib", required=True)
    r.add_argument("--bench-json", required=True,
                   help="bench.py output of the FETCH_SIZE run (source hash)")
    r.add_argument("--bench-json-write", required=True,
                   help="bench.py output of the WRITE_SIZE run")
    r.add_argument("--out", required=True)
    c = sub.add_parser("configs")
    c.add_argument("--trace", required=True, help="kernel_trace.csv of a default bench run")
    c.add_argument("--bench-json", required=True, help="that run's bench.py output")
    c.add_argument("--command", required=True)
    c.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    {"trace": cmd_trace, "traffic": cmd_traffic, "configs": cmd_configs}[a.cmd](a)
    return 0


if __name__ == "__main__":
    sys.exit(main())
