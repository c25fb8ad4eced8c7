"""Summarise rocprofv3 CSV output of bench.py runs into short text records.

Kernel durations of every workload in one traced bench run (per-dispatch
average, median, p10 and p90, each workload's kernel matched by the kernel
instance its record names, grid and block), written as a text table and
merged into profiles/kernel_trace.json, which bench.py reads back for the
main workload's ``roofline.profiled``:

    rocprofv3 --kernel-trace --stats -f csv -d DIR -o run -- python3 bench.py ... > OUT
    python -m memory_bound_elementwise_amd.rocprof_summary configs \
        --trace DIR/run_kernel_trace.csv --bench-json OUT \
        --command "the rocprofv3 command line" --out profiles/FILE.txt

HBM traffic (from two ``rocprofv3 --pmc`` runs per workload, FETCH_SIZE then
WRITE_SIZE, each in KiB per dispatch).  The counters are calibrated on the
plain copy kernel of known size: scale = algorithmic bytes / counted bytes,
per counter.  The result is written as text and merged into
profiles/traffic.json, which bench.py reads (keyed by workload, kernel
source hash and launch shape):

    python -m memory_bound_elementwise_amd.rocprof_summary traffic \
        --workload NAME --family FAMILY \
        --fetch DIR/..._counter_collection.csv --write DIR/..._counter_collection.csv \
        --calib-workload COPY_WORKLOAD --calib-fetch CSV --calib-write CSV \
        --calib-bench-json COPY_FETCH_RUN_OUTPUT \
        --bench-json FETCH_RUN_OUTPUT --bench-json-write WRITE_RUN_OUTPUT \
        --command-fetch "..." --command-write "..." --command-calib "..." --out profiles/FILE.txt

Each run's dispatches are matched by the kernel instance and launch shape
that its bench.py record names.

The launch shape, the algorithmic bytes and the kernel source hash written
into every record are the ones the profiled bench.py run printed for that
workload (its record's ``source_sha256_16``: the hash of its kernel family's
sources), never the hash of the source as it is when the summary is written.
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
KERNEL_TRACE_JSON = os.path.join(ROOT, "profiles", "kernel_trace.json")


def bench_records(path):
    """Every record a bench.py run printed: the other workloads' lines and
    the final line (the main workload), as {workload: record}.  The final
    line's record carries the kernel fields of the main workload under its
    own keys; it is keyed by config.name."""
    out = {}
    with open(path) as f:
        lines = [ln for ln in f.read().splitlines() if ln.startswith("{")]
    for ln in lines[:-1]:
        r = json.loads(ln)
        if "workload" in r:
            out[r["workload"]] = r
    last = json.loads(lines[-1])
    cfg = last.get("config", {})
    main = {"workload": cfg.get("name"), "op": cfg.get("op"), "n": cfg.get("n"),
            "launch": cfg.get("launch"), "gbs": last.get("value"), "ms": last.get("ms_per_step"),
            "timing": last.get("timing"),
            "kernel": (last.get("roofline") or {}).get("kernel"),
            "algorithmic_bytes": (last.get("roofline") or {}).get("algorithmic_bytes_per_launch"),
            "source_sha256_16": last.get("env", {}).get("kernel_source_sha256_16"),
            "final_line": True}
    out[main["workload"]] = main
    return out


def bench_record(path, workload):
    """The record of one workload in a bench.py output file."""
    recs = bench_records(path)
    if workload not in recs:
        raise SystemExit(f"{path}: no record of workload {workload!r}")
    return recs[workload]


def profiled_hash(bench_json, workload):
    """The kernel-source hash (of the workload's kernel family) that the
    profiled run was built from: taken from the record bench.py printed, so
    that a summary written later, after the source has changed, cannot claim
    the new hash.  Refuses a record without one."""
    h = bench_record(bench_json, workload).get("source_sha256_16")
    if not h:
        raise SystemExit(f"{bench_json}: no source hash for {workload}")
    return h


def _merge(path, about, workload, rec):
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        data = {"about": about, "workloads": {}}
    data["workloads"][workload] = rec
    with open(path, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
        f.write("\n")


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


def counter_per_dispatch(path, kernel, counter, launch=None):
    """Median over dispatches of the counter summed within each dispatch, for
    the dispatches of one kernel instance (see kernel_matches) -- and, given
    its launch, of that grid and block only."""
    per = {}
    for r in _rows(path):
        if r.get("Counter_Name") != counter or not kernel_matches(kernel, r.get("Kernel_Name", "")):
            continue
        if launch and (int(r["Workgroup_Size"]) != launch["block"]
                       or int(r["Grid_Size"]) != launch["block"] * launch["grid"]):
            continue
        key = r.get("Dispatch_Id") or r.get("Correlation_Id")
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    if not per:
        raise SystemExit(f"no {counter} rows for kernel {kernel!r} in {path}")
    return statistics.median(per.values()), len(per)


def dispatch_durations(path, kernel_re):
    """Per-dispatch durations in ns of the kernel matching the regex, from a
    rocprofv3 kernel_trace.csv."""
    rx = re.compile(kernel_re)
    return [int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in _rows(path)
            if rx.search(r.get("Kernel_Name", ""))]


def cmd_traffic(a):
    rec = bench_record(a.bench_json, a.workload)
    cal = bench_record(a.calib_bench_json, a.calib_workload)
    fetch_kib, nd_f = counter_per_dispatch(a.fetch, rec["kernel"], "FETCH_SIZE", rec["launch"])
    write_kib, nd_w = counter_per_dispatch(a.write, rec["kernel"], "WRITE_SIZE", rec["launch"])
    cal_f, _ = counter_per_dispatch(a.calib_fetch, cal["kernel"], "FETCH_SIZE", cal["launch"])
    cal_w, _ = counter_per_dispatch(a.calib_write, cal["kernel"], "WRITE_SIZE", cal["launch"])
    # the calibration is a copy: half its algorithmic bytes read, half written
    scale_f = (cal["algorithmic_bytes"] // 2) / (cal_f * 1024)
    scale_w = (cal["algorithmic_bytes"] // 2) / (cal_w * 1024)
    fetch_b = fetch_kib * 1024 * scale_f
    write_b = write_kib * 1024 * scale_w
    total = fetch_b + write_b
    launch = rec["launch"]
    src_hash = profiled_hash(a.bench_json, a.workload)
    if profiled_hash(a.bench_json_write, a.workload) != src_hash:
        raise SystemExit("the FETCH_SIZE and WRITE_SIZE runs were built from different sources")
    alg = rec["algorithmic_bytes"]
    cal_bytes = cal["algorithmic_bytes"]
    text = [
        f"# HBM traffic: {a.workload}",
        "",
        f"fetch command: {a.command_fetch}",
        f"write command: {a.command_write}",
        f"calibration:   {a.command_calib}",
        "",
        f"kernel:            {rec['kernel']}  launch {json.dumps(launch)}",
        f"FETCH_SIZE:        {fetch_kib:.0f} KiB per dispatch (median of {nd_f})",
        f"WRITE_SIZE:        {write_kib:.0f} KiB per dispatch (median of {nd_w})",
        f"calibration copy:  {a.calib_workload}: FETCH {cal_f:.0f} KiB for {cal_bytes // 2} B "
        f"read -> scale {scale_f:.4f};  WRITE {cal_w:.0f} KiB for {cal_bytes // 2} B written "
        f"-> scale {scale_w:.4f}",
        f"HBM bytes/launch:  fetch {fetch_b:.0f} + write {write_b:.0f} = {total:.0f}",
        f"algorithmic bytes: {alg}  (traffic / algorithmic = {total / alg:.4f})",
        f"kernel sources:    {a.family} family sha256[:16] {src_hash} (of the profiled runs)",
    ]
    with open(a.out, "w") as f:
        f.write("\n".join(text) + "\n")
    print("\n".join(text))
    _merge(a.index or TRAFFIC_JSON, "HBM bytes per launch from rocprofv3 FETCH_SIZE + WRITE_SIZE, "
                                    "scaled by the copy-kernel calibration; see the .txt "
                                    "summaries", a.workload, {
        "kernel": rec["kernel"], "launch": launch,
        "kernel_source_sha256_16": src_hash,
        "fetch_kib": fetch_kib, "write_kib": write_kib, "scale_fetch": scale_f,
        "scale_write": scale_w, "hbm_bytes_per_launch": round(total),
        "algorithmic_bytes": alg, "summary": os.path.basename(a.out)})


def _mangled_pattern(instance):
    """A regex for the Itanium-mangled name of a kernel instance: rocprofv3
    leaves names mangled when it cannot demangle them (template arguments of
    type _Float16 or __bf16).  The identifiers, the 16-bit types and the
    integer and boolean template arguments must appear in order."""
    toks = []
    for t in re.findall(r"[A-Za-z_][A-Za-z_0-9]*|\d+", instance.replace("ew::", "")):
        if t == "_Float16":
            toks.append("DF16_")
        elif t == "__bf16":
            toks.append("DF16b")
        elif t in ("true", "false"):
            toks.append("Lb1E" if t == "true" else "Lb0E")
        elif t.isdigit():
            toks.append(f"Li{t}E")
        else:
            toks.append(f"{len(t)}{t}")
    return re.compile("^_ZN2ew" + ".*?".join(map(re.escape, toks)))


def kernel_matches(instance, name):
    """Whether a trace's kernel name is the given instance (demangled, or
    mangled where the profiler left it so)."""
    if name.startswith("_Z"):
        return bool(_mangled_pattern(instance).search(name))
    return ("ew::" + instance + "(") in name.replace("void ", "")


def cmd_configs(a):
    """Per-dispatch durations of every workload's kernel in one traced bench
    run: each record that names its kernel instance is matched to the trace
    by kernel name, grid and block.  Writes the text table and one record per
    workload to profiles/kernel_trace.json (keyed by workload, kernel source
    hash and launch shape, which bench.py reads back)."""
    recs = bench_records(a.bench_json)
    rows = _rows(a.trace)
    text = [
        "# Kernel durations per workload (rocprofv3 kernel trace of one bench.py run)",
        "",
        f"command: {a.command}",
        f"source:  per-dispatch durations (End - Start) in {os.path.basename(a.trace)}, each "
        "workload's kernel matched by name, grid and block",
        "note:    for the cold workloads (<= 1 GiB) the dispatches include the rotated launches "
        "that bench.py times, the flushed per-launch ones and the warm ones; all include the "
        "parity launch",
        "         the bench.py column is that profiled run's own figure (its timing method in "
        "the record): the tracer adds host-side cost to every launch, which shows only where "
        "back-to-back launches are bound by the host (small arrays)",
        "",
        "| workload | kernel | grid x block | dispatches | average us | median us (p10, p90) "
        "| GB/s at the average | bench.py GB/s | sources sha256[:16] |",
        "|---|---|---|---|---|---|---|---|---|",
    ]
    wanted = [w for w in a.workloads.split(",")] if a.workloads else sorted(recs)
    # two workloads with the same kernel instance and launch shape cannot be
    # told apart in the trace: neither is reported
    shape = {}
    for name, r in recs.items():
        if r.get("kernel") and r.get("launch"):
            key = (r["kernel"], r["launch"].get("block"), r["launch"].get("grid"))
            shape.setdefault(key, []).append(name)
    ambiguous = {n for names in shape.values() if len(names) > 1 for n in names}
    names_seen = {}
    for name in wanted:
        r = recs.get(name)
        if not r or not r.get("kernel") or not r.get("gbs"):
            continue
        if name in ambiguous:
            text.append(f"| {name} | {r['kernel']} | (same kernel and launch as another "
                        "workload of the run: not separable in the trace) | | | | | | |")
            continue
        lc = r["launch"]
        if r["kernel"] not in names_seen:
            names_seen[r["kernel"]] = {x["Kernel_Name"] for x in rows
                                       if kernel_matches(r["kernel"], x["Kernel_Name"])}
        knames = names_seen[r["kernel"]]
        d = sorted(int(x["End_Timestamp"]) - int(x["Start_Timestamp"]) for x in rows
                   if x["Kernel_Name"] in knames
                   and int(x["Workgroup_Size_X"]) == lc["block"]
                   and int(x["Grid_Size_X"]) == lc["block"] * lc["grid"])
        if not d:
            print(f"no dispatch of {name}'s kernel {r['kernel']} in {a.trace}", file=sys.stderr)
            continue
        avg, med = statistics.fmean(d), statistics.median(d)
        p10, p90 = d[len(d) // 10], d[(9 * len(d)) // 10]
        alg = r["algorithmic_bytes"]
        text.append(f"| {name} | {r['kernel']} | {lc['grid']} x {lc['block']} | {len(d)} | "
                    f"{avg / 1000:.2f} | {med / 1000:.2f} ({p10 / 1000:.2f}, {p90 / 1000:.2f}) | "
                    f"{alg / avg:.1f} | {r['gbs']} | {r['source_sha256_16']} |")
        _merge(a.index or KERNEL_TRACE_JSON, "rocprofv3 kernel-trace durations per workload, "
                                             "from the summary named in each record", name, {
            "kernel": r["kernel"], "launch": lc, "kernel_source_sha256_16": r["source_sha256_16"],
            "dispatches": len(d), "avg_ns": round(avg, 1), "median_ns": med, "p10_ns": p10,
            "p90_ns": p90, "algorithmic_bytes": alg, "summary": os.path.basename(a.out)})
    with open(a.out, "w") as f:
        f.write("\n".join(text) + "\n")
    print("\n".join(text))


# MI355X: 8 XCDs, 16 L2 (TCC) channels each.  rocprofv3 reports a TCC
# counter summed over all 128 channels and GRBM_GUI_ACTIVE summed over the
# XCDs (a 0.49 ms kernel reads about 8 x 0.49 ms x 2.4 GHz).
XCDS, CHANNELS_PER_XCD = 8, 16


def memory_side_lines(med):
    """Derived figures of the L2-to-memory interface counters, when
    collected: mean request latency (requests in flight summed per cycle /
    requests, as the counters' definitions state), the requests in flight
    per L2 channel, and the share of the channels' busy cycles in which the
    interface had no DRAM credits left."""
    out = []
    busy = med.get("GRBM_GUI_ACTIVE")
    cycles = busy / XCDS if busy else None          # busy cycles of one XCD
    channels = XCDS * CHANNELS_PER_XCD
    for kind, what in (("RD", "read"), ("WR", "write")):
        level, req = med.get(f"TCC_EA0_{kind}REQ_LEVEL"), med.get(f"TCC_EA0_{kind}REQ")
        if level and req:
            out.append(f"mean {what} request latency, L2 to memory: {level / req:.0f} cycles "
                       f"(TCC_EA0_{kind}REQ_LEVEL / TCC_EA0_{kind}REQ)")
            if cycles:
                out.append(f"{what} requests in flight per L2 channel: "
                           f"{level / cycles / channels:.0f} (TCC_EA0_{kind}REQ_LEVEL / "
                           f"busy cycles / {channels} channels)")
    for c, what in (("TCC_EA0_RDREQ_DRAM_CREDIT_STALL", "read"),
                    ("TCC_EA0_WRREQ_DRAM_CREDIT_STALL", "write")):
        if c in med and cycles:
            out.append(f"{what} interface out of DRAM credits: "
                       f"{med[c] / (cycles * channels):.3f} of the L2 channels' busy cycles")
    return out


def cmd_counters(a):
    """Per-dispatch medians of the counters of one rocprofv3 --pmc pass for
    the workload's kernel (e.g. the LDS counters of the kernels that stage
    data in LDS), with bank-conflict cycles as a share of LDS-active cycles
    when both were collected."""
    rec = bench_record(a.bench_json, a.workload)
    kernel = a.kernel or rec["kernel"]
    rows = [r for r in _rows(a.csv) if kernel_matches(kernel, r.get("Kernel_Name", ""))]
    if not rows:
        raise SystemExit(f"no dispatch of {kernel!r} in {a.csv}")
    per = {}
    for r in rows:
        key = (r["Counter_Name"], r.get("Dispatch_Id") or r.get("Correlation_Id"))
        per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    names = sorted({k[0] for k in per})
    med = {c: statistics.median(v for (n, _), v in per.items() if n == c) for c in names}
    dispatches = len({k[1] for k in per})
    text = [
        f"# {a.title}",
        "",
        f"command: {a.command}",
        f"source:  {os.path.basename(a.csv)}, kernel {rows[0]['Kernel_Name'].split('(')[0]}, "
        f"{dispatches} dispatches (median per dispatch; each counter summed over its "
        f"hardware instances)",
        f"launch:  {json.dumps(rec.get('launch'))}",
        "",
    ]
    text += [f"{c:22s} {med[c]:.6g}" for c in names]
    if "SQ_LDS_BANK_CONFLICT" in med and med.get("SQ_LDS_IDX_ACTIVE"):
        text.append(f"bank-conflict cycles / LDS-active cycles: "
                    f"{med['SQ_LDS_BANK_CONFLICT'] / med['SQ_LDS_IDX_ACTIVE']:.3f}")
    text += memory_side_lines(med)
    text.append(f"kernel sources: {a.family} family sha256[:16] "
                f"{profiled_hash(a.bench_json, a.workload)} (of the profiled run)")
    with open(a.out, "w") as f:
        f.write("\n".join(text) + "\n")
    print("\n".join(text))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__,
                                 formatter_class=argparse.RawDescriptionHelpFormatter)
    sub = ap.add_subparsers(dest="cmd", required=True)
    r = sub.add_parser("traffic")
    r.add_argument("--workload", required=True)
    r.add_argument("--fetch", required=True)
    r.add_argument("--write", required=True)
    r.add_argument("--calib-workload", required=True,
                   help="the copy workload whose known bytes calibrate both counters")
    r.add_argument("--calib-fetch", required=True)
    r.add_argument("--calib-write", required=True)
    r.add_argument("--calib-bench-json", required=True,
                   help="bench.py output of the calibration's FETCH_SIZE run")
    r.add_argument("--family", required=True, help="kernel family of the workload "
                                                   "(stream, batch, gather, view)")
    r.add_argument("--command-fetch", required=True)
    r.add_argument("--command-write", required=True)
    r.add_argument("--command-calib", required=True)
    r.add_argument("--bench-json", required=True,
                   help="bench.py output of the FETCH_SIZE run (source hash)")
    r.add_argument("--bench-json-write", required=True,
                   help="bench.py output of the WRITE_SIZE run")
    r.add_argument("--out", required=True)
    r.add_argument("--index", help="profile index to merge into (default profiles/traffic.json)")
    c = sub.add_parser("configs")
    c.add_argument("--trace", required=True, help="kernel_trace.csv of a default bench run")
    c.add_argument("--bench-json", required=True, help="that run's bench.py output")
    c.add_argument("--command", required=True)
    c.add_argument("--workloads", help="comma-separated workloads (default: every record "
                                       "naming its kernel)")
    c.add_argument("--out", required=True)
    c.add_argument("--index", help="profile index to merge into (default "
                                   "profiles/kernel_trace.json)")
    k = sub.add_parser("counters")
    k.add_argument("--csv", required=True, help="counter_collection.csv of one --pmc pass")
    k.add_argument("--kernel", help="kernel instance (default: the workload record's)")
    k.add_argument("--workload", required=True)
    k.add_argument("--family", required=True)
    k.add_argument("--bench-json", required=True)
    k.add_argument("--command", required=True)
    k.add_argument("--title", default="Hardware counters")
    k.add_argument("--out", required=True)
    a = ap.parse_args(argv)
    {"traffic": cmd_traffic, "configs": cmd_configs, "counters": cmd_counters}[a.cmd](a)
    return 0


if __name__ == "__main__":
    sys.exit(main())
