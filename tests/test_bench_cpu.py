"""bench.py's host-side bookkeeping, without a GPU: byte formulas, the
in-place ReLU's store counts, the traffic record lookup and the one-GPU
contract."""
import json
import os
import subprocess
import sys

import numpy as np

import bench
from tests.conftest import ROOT


def test_algorithmic_bytes_follow_the_read_plus_write_rule():
    n = (1 << 28) + 3
    assert bench.algorithmic_bytes("add_f32", n) == 12 * n         # headline: 3221225508
    assert bench.algorithmic_bytes("add_f32", n) == 3221225508
    assert bench.algorithmic_bytes("add_f16", 10) == 60
    assert bench.algorithmic_bytes("relu_f32", 10) == 80
    assert bench.algorithmic_bytes("bias_relu_f32", 4096 * 3, 4096) == 8 * 4096 * 3 + 4 * 4096
    # in place: every element read, only the changed ones written
    assert bench.algorithmic_bytes("relu_inplace_f32", 100, 0, 0) == 400
    assert bench.algorithmic_bytes("relu_inplace_f32", 100, 0, 37) == 400 + 4 * 37


def test_relu_store_counts_follow_the_reading_of_the_relu():
    """Changed: sign bit set and not a NaN (so -0 and -inf count, negative
    NaNs do not); spans are 16 elements (64 bytes)."""
    bits = np.zeros(40, np.uint32)                      # +0: unchanged
    bits[3] = 0x80000000                                # -0 -> +0
    bits[17] = 0xFF800000                               # -inf
    bits[20] = 0xFFC00000                               # negative NaN: kept
    bits[39] = 0xBF800000                               # -1
    changed, spans = bench.relu_store_counts(bits.view(np.float32), np)
    assert changed == 3
    assert spans == 3                                   # spans 0, 1 and 2 (elements 32..39)
    assert bench.relu_store_counts(np.abs(np.arange(-5, 5, dtype=np.float32)), np) == (0, 0)


def test_traffic_is_reported_only_for_the_current_kernel_source(tmp_path, monkeypatch):
    rec = {"workloads": {"w": {"kernel_source_sha256_16": bench.kernel_source_hash("add_f32"),
                               "launch": {"block": 1024, "grid": 7, "unroll": 1},
                               "hbm_bytes_per_launch": 123}}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(f))
    assert bench.traffic_for("w", {"block": 1024, "grid": 7, "unroll": 1}) == 123
    assert bench.traffic_for("w", {"block": 512, "grid": 7, "unroll": 1}) is None
    assert bench.traffic_for("other", {"block": 1024, "grid": 7, "unroll": 1}) is None
    # a record taken on another family's sources does not apply
    assert bench.traffic_for("w", {"block": 1024, "grid": 7, "unroll": 1},
                             bench.kernel_source_hash("gather_f32")) is None
    rec["workloads"]["w"]["kernel_source_sha256_16"] = "0" * 16
    f.write_text(json.dumps(rec))
    assert bench.traffic_for("w", {"block": 1024, "grid": 7, "unroll": 1}) is None


def test_source_hashes_cover_each_family_and_the_shared_headers(tmp_path, monkeypatch):
    """A family's hash changes with its own file and with the shared device
    headers, and not with another family's file."""
    import shutil
    from memory_bound_elementwise_amd import sources
    for name in os.listdir(sources.CSRC):
        shutil.copy(os.path.join(sources.CSRC, name), tmp_path / name)
    monkeypatch.setattr(sources, "CSRC", str(tmp_path))
    before = sources.all_hashes()
    assert len(set(before.values())) == len(before)
    with open(tmp_path / "ew_view.hip", "a") as f:
        f.write("\n// edit\n")
    after = sources.all_hashes()
    assert after["view"] != before["view"]
    assert all(after[k] == before[k] for k in ("stream", "batch", "gather"))
    with open(tmp_path / "ew_gather.hip", "a") as f:
        f.write("\n// edit\n")
    again = sources.all_hashes()
    assert again["gather"] != after["gather"] and again["view"] != after["view"]
    with open(tmp_path / "ew_device.h", "a") as f:
        f.write("\n// edit\n")
    last = sources.all_hashes()
    assert all(last[k] != again[k] for k in last)
    assert sources.family("gather_walk_f32") == "gather"
    assert sources.family("copy2d_f32") == "view"
    assert sources.family("add_f32", batch=True) == "batch"
    assert sources.family("sqrt_bf16") == "stream"


def test_kernel_instance_names_match_the_profiler_s_demangled_names():
    import synth
    W = synth.WORKLOADS
    split = {"in_coaligned": [1, 1]}
    assert (bench.kernel_instance(W["headline_add_f32_2e28"], {"unroll": 1}, split)
            == "ew_stream_kernel<ew::OpAddF32, 1, true, true>")
    assert (bench.kernel_instance(W["cfg2_add_f32_2e28p3_offA1"], {"unroll": 1},
                                  {"in_coaligned": [0, 1]})
            == "ew_stream_kernel<ew::OpAddF32, 1, false, true>")
    assert (bench.kernel_instance(W["sqrt_bf16_2e28"], {"unroll": 1}, split)
            == "ew_stream_kernel<ew::OpMap16<__bf16, ew::FnSqrtWidenedBF16>, 1, true, true>")
    assert (bench.kernel_instance(W["relu_inplace_f32_2e28_nonneg"], {"unroll": 1}, split)
            == "ew_relu_inplace_kernel<1>")
    import memory_bound_elementwise_amd as ew

    class Prep:            # the workload's device buffers, as made-up addresses
        def __init__(self, src):
            self.view_src = src
            self.ptrs = (None, type("T", (), {"data_ptr": lambda self_: src})(), None)

    base, out = 1 << 40, 1 << 42
    walk = ew.ew_make_plan("gather_walk_f32", out, base, 0, 1 << 26, 256)
    assert (bench.kernel_instance(W["gather_walk_f32_2e26_s2"], {"unroll": 1}, split, walk, ew,
                                  Prep(base)) == "ew_gather_kernel<1>")
    spans = ew.ew_make_gather_plan(out, base, 1 << 26, 2, 256)
    assert (bench.kernel_instance(W["cfg5b_gather_f32_2e26_s2"], {"unroll": 1}, split, spans,
                                  ew, Prep(base)) == "ew_gather2_kernel<1, true>")
    assert (bench.kernel_instance(W["cfg5b_gather_f32_2e26_s2"], {"unroll": 1}, split, spans,
                                  ew, Prep(base + 4)) == "ew_gather2_kernel<1, false>")
    passes = ew.ew_make_gather_plan(out, base, 1 << 26, 3, 256)
    assert (bench.kernel_instance(W["gather_f32_2e26_s3"], {"unroll": 1}, split, passes, ew,
                                  Prep(base)) == "ew_gather_passes_kernel<3, 1>")
    six = ew.ew_make_gather_plan(out, base, 1 << 26, 6, 256)          # gcd 2: span 6, step 2
    assert (bench.kernel_instance(W["gather_f32_2e26_s3"], {"unroll": 1}, split, six, ew,
                                  Prep(base)) == "ew_gather_passes_kernel<6, 2>")
    view = ew.ew_make_copy2d_plan(base, 0, 3, out, 1, 1 << 24, 256)
    assert (bench.kernel_instance(W["strided_view_f32_2e24_s3"], {"unroll": 1}, split, view, ew,
                                  Prep(base)) == "ew_gather_passes_kernel<3, 3>")
    tr = ew.ew_make_copy2d_plan(base, 1, 16384, out, 16384, 16384, 256)
    assert (bench.kernel_instance(W["transpose_f32_16384x16384"], {"unroll": 1}, split, tr, ew,
                                  Prep(base)) == "ew_transpose_kernel")
    # the tiled transposition: whole rows below stride 68, else 128 x 128 tiles below
    # 1024 rows of the stride and 256 x 64 from there on
    import dataclasses
    for name, stride, mode in (("gather_f32_2e26_s33", 33, 1), ("gather_f32_2e26_s1000", 1000, 3),
                               ("gather_f32_2e26_s33", 65537 * 3, 2), ("gather_f32_2e26_s33", 36, 4)):
        w = dataclasses.replace(W[name], stride=stride)
        tiles = ew.ew_make_gather_plan(out, base, w.n, stride, 256)
        assert ew.PATHS[tiles.path] == "gather_tiles"
        assert (bench.kernel_instance(w, {"unroll": 1}, split, tiles, ew, Prep(base))
                == f"ew_gather_tiles_kernel<{mode}>")
    assert (bench.kernel_instance(W["fused_bias_relu_f32_65536x4096"], {"unroll": 1},
                                  {"in_coaligned": [1, 1], "head": 0})
            == "ew_bias_relu_kernel<1, true, true>")
    assert (bench.kernel_instance(W["batch_add_f32_1024x1024"], {"unroll": 2}, split)
            == "ew_batch_table_kernel<ew::OpAddF32, 2>")


def _fake_record(name, op, n, gbs, **kw):
    ms = bench.algorithmic_bytes(op, n) / (gbs * 1e9) * 1e3
    rec = {"workload": name, "op": op, "n": n, "gbs": gbs, "ms": round(ms, 5),
           "parity": "PASS", "mismatches": 0, "kernel": f"k<{op}>",
           "launch": {"block": 1024, "grid": 65536, "unroll": 1},
           "split": {"head": 0, "vectors": n // 4, "tail": 0, "in_coaligned": [1, 1]},
           "source_sha256_16": "0" * 16, "algorithmic_bytes": bench.algorithmic_bytes(op, n),
           "timing": "back-to-back, mean"}
    rec.update(kw)
    return rec


def test_final_line_is_one_compact_json_record_with_roofline_and_cpu_baseline():
    """The driver reads the last stdout line alone: it must parse on its own,
    stay well under 4 KB, and carry the metric, roofline (with the attainable
    streams and the strided comparison) and cpu_baseline."""
    import argparse
    import synth
    w = synth.WORKLOADS[bench.DEFAULT_WORKLOAD]
    assert (w.op, w.n, w.seed, w.offsets) == ("add_f32", 1 << 28, 100, {})
    sample = "add_f32 on the first 67108864 elements of the workload's inputs, 9 passes " \
             "in 12.3 s (scalar C loop, one thread)"
    res = _fake_record(w.name, "add_f32", w.n, 6500.0, cpu_baseline={
        "value": 30.1, "unit": "GB/s", "cores": 1, "kind": "oracle", "sample": sample,
        "cpu": "AMD EPYC", "all_cores": {"value": 220.0, "unit": "GB/s", "cores": 16,
                                         "sample": "x" * 200}},
        torch_context={"op": "torch.add", "gbs": 6000.0})
    others = [_fake_record(name, synth.WORKLOADS[name].op, synth.WORKLOADS[name].n, 6400.0)
              for name in synth.WORKLOADS if name != w.name]
    others[3]["parity"] = "FAIL"
    args = argparse.Namespace(steps=20, warmup=5)
    env = {"device": "AMD Instinct MI355X", "arch": "gfx950:sramecc+:xnack-", "cus": 256,
           "clocks": {"sclk": "2400Mhz", "mclk": "2000Mhz"}, "torch": "2.10", "hip": "7.0",
           "numpy": "2.2", "kernel_source_sha256_16": "0" * 16,
           "sources_sha256_16": {k: "0" * 16 for k in ("stream", "batch", "gather", "view")},
           "input_sha256": {"a": "1" * 16, "b": "2" * 16}}
    line = bench.final_line(args, w, res, others, env)
    text = json.dumps(line, separators=(",", ":"))
    assert len(text) < 3000, len(text)
    out = "\n".join([json.dumps(r) for r in others] + [text])
    last = json.loads(out.splitlines()[-1])
    for key in ("metric", "value", "unit", "n_gpus", "steps", "warmup", "ms_per_step",
                "higher_is_better", "scaling", "vs_baseline", "dtype", "data", "config",
                "parity", "roofline", "cpu_baseline", "cpu_baseline_all_cores"):
        assert key in last, key
    assert last["metric"] == ("achieved HBM GB/s (read+write bytes/time) and % of MI355X peak, "
                              "N=2^28")
    assert last["value"] == 6500.0 and last["unit"] == "GB/s" and last["dtype"] == "f32"
    rl = last["roofline"]
    assert rl["bound"] == "hbm" and rl["peak"] == 8000.0 and rl["unit"] == "GB/s"
    assert rl["frac"] == round(6500.0 / 8000, 4)
    assert rl["algorithmic_bytes_per_launch"] == 12 * (1 << 28)
    assert rl["attainable"]["copy_gbs"] == 6400.0
    assert rl["attainable"]["value_over_copy"] == round(6500 / 6400, 4)
    so = last["strided_over_coalesced"]
    assert so["walk"]["over_copy"] == 1.0 and so["gather"]["over_copy"] == 1.0
    assert last["cpu_baseline"]["kind"] == "oracle" and "all_cores" not in last["cpu_baseline"]
    assert last["cpu_baseline_all_cores"]["cores"] == 16
    assert last["others"]["not_passing"] == [others[3]["workload"]]
    assert last["config"]["name"] == "headline_add_f32_2e28"


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_committed_traffic_records_name_existing_summaries():
    import os
    with open(bench.TRAFFIC_JSON) as fh:
        data = json.load(fh)
    for name, rec in data["workloads"].items():
        assert os.path.exists(os.path.join(ROOT, "profiles", rec["summary"])), name
        assert rec["hbm_bytes_per_launch"] > 0


def test_sweep_resume_skips_recorded_points(tmp_path, monkeypatch):
    """An interrupted sweep resumes: points already in the output file with
    parity PASS are skipped, the rest are measured and appended."""
    out = tmp_path / "sweep.jsonl"
    out.write_text(json.dumps({"op": "add_f32", "n": 5, "parity": "PASS"}) + "\n"
                   + json.dumps({"op": "add_f32", "n": 7, "parity": "FAIL"}) + "\n")
    monkeypatch.setattr(bench, "SWEEP_OPS", (("add_f32", "uniform"),))
    monkeypatch.setattr(bench, "SWEEP_SIZES", [5, 7, 9])
    measured = []

    def fake_measure(w, *a, **k):
        measured.append(w.n)
        return {"op": w.op, "n": w.n, "parity": "PASS"}, None, 1.0
    monkeypatch.setattr(bench, "measure", fake_measure)

    class FakeCuda:
        @staticmethod
        def empty_cache():
            pass

    class FakeTorch:
        cuda = FakeCuda

    import synth
    assert bench.run_sweep(FakeTorch, np, None, synth, None, 256, None, str(out)) == 0
    assert measured == [7, 9]
    lines = [json.loads(x) for x in out.read_text().splitlines()]
    assert [(r["n"], r["parity"]) for r in lines] == [(5, "PASS"), (7, "FAIL"), (7, "PASS"),
                                                      (9, "PASS")]


def test_rotation_puts_a_gibibyte_of_other_traffic_between_two_uses():
    """Cold timing over R buffer copies used in turn: the R - 1 launches
    between two uses of one copy move at least 1 GiB, and R is the smallest
    count that does (at least 2)."""
    gib = 1 << 30
    for nbytes in (12 << 20, 402653184, 536870912, 805306368, gib, 3 * gib):
        r = bench.rotation_sets(nbytes)
        assert r >= 2
        assert (r - 1) * nbytes >= gib
        assert r == 2 or (r - 2) * nbytes < gib
    assert bench.rotation_sets(12 * (1 << 20)) == 87       # the 2^20 fp32 add
    assert bench.rotation_sets(12 * (1 << 25)) == 4        # SAXPY 2^25
    assert bench.rotation_sets(8 * (1 << 26)) == 3         # copy and gather 2^26


def test_clocks_come_from_sysfs_without_a_child_process(tmp_path, monkeypatch):
    """The DPM level marked '*' of the device's PCI address is reported; a
    missing directory gives None.  No process is spawned."""
    dev = tmp_path / "0000:75:00.0"
    dev.mkdir()
    (dev / "pp_dpm_sclk").write_text("0: 500Mhz\n1: 2400Mhz *\n")
    (dev / "pp_dpm_mclk").write_text("0: 900Mhz\n1: 2000Mhz *\n")

    class Props:
        pci_domain_id, pci_bus_id, pci_device_id = 0, 0x75, 0

    real_join = bench.os.path.join
    monkeypatch.setattr(bench.os.path, "join",
                        lambda a, *b: real_join(str(tmp_path), *b) if a == "/sys/bus/pci/devices"
                        else real_join(a, *b))
    monkeypatch.setattr(subprocess, "run", None)
    assert bench._clocks(Props) == {"sclk": "2400Mhz", "mclk": "2000Mhz"}

    class Other:
        pci_domain_id, pci_bus_id, pci_device_id = 0, 0x11, 0
    assert bench._clocks(Other) is None


def test_rocprof_summaries_read_the_bench_output_and_the_profiler_csv(tmp_path):
    """The kernel-trace summary matches each record's kernel instance, grid
    and block in the trace and writes an index bench.py can read back; the
    counter summary takes per-dispatch medians."""
    import argparse
    import csv
    import synth
    from memory_bound_elementwise_amd import rocprof_summary as rs
    w = synth.WORKLOADS[bench.DEFAULT_WORKLOAD]
    res = _fake_record(w.name, "add_f32", w.n, 6500.0)
    res["kernel"] = "ew_stream_kernel<ew::OpAddF32, 1, true, true>"
    other = _fake_record("copy_f32_2e28", "copy_f32", 1 << 28, 6600.0,
                         kernel="ew_stream_kernel<ew::OpCopyF32, 1, true, true>",
                         launch={"block": 256, "grid": 262144, "unroll": 1})
    env = {"kernel_source_sha256_16": "0" * 16}
    line = bench.final_line(argparse.Namespace(steps=20, warmup=5), w, res, [other], env)
    out = tmp_path / "bench.out"
    out.write_text(json.dumps(other) + "\n" + json.dumps(line) + "\n")
    trace = tmp_path / "run_kernel_trace.csv"
    with open(trace, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Kernel_Name", "Workgroup_Size_X", "Grid_Size_X", "Start_Timestamp",
                     "End_Timestamp"])
        for k, d in enumerate((490000, 500000, 495000)):
            wr.writerow(["void ew::ew_stream_kernel<ew::OpAddF32, 1, true, true>(ew::StreamArgs)",
                         1024, 1024 * 65536, 1000 * k, 1000 * k + d])
        wr.writerow(["void ew::ew_stream_kernel<ew::OpAddF32, 1, false, true>(ew::StreamArgs)",
                     1024, 1024 * 65536, 0, 1])          # another instance: not matched
        for k in range(4):
            wr.writerow(["void ew::ew_stream_kernel<ew::OpCopyF32, 1, true, true>(ew::StreamArgs)",
                         256, 256 * 262144, 0, 320000 + k])
    index = tmp_path / "kernel_trace.json"
    rs.main(["configs", "--trace", str(trace), "--bench-json", str(out), "--command", "cmd",
             "--out", str(tmp_path / "kt.txt"), "--index", str(index)])
    idx = json.loads(index.read_text())["workloads"]
    assert idx[w.name]["dispatches"] == 3 and idx[w.name]["median_ns"] == 495000
    assert idx[w.name]["launch"] == res["launch"]
    assert idx["copy_f32_2e28"]["dispatches"] == 4
    rec = bench._committed(str(index), w.name, "0" * 16, res["launch"])
    assert rec and rec["avg_ns"] == 495000.0
    # counters: two dispatches, a counter summed over its rows per dispatch
    cc = tmp_path / "run_counter_collection.csv"
    with open(cc, "w", newline="") as f:
        wr = csv.writer(f)
        wr.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for d, (bank, active) in enumerate(((30, 100), (50, 100))):
            wr.writerow([d, "void ew::ew_transpose_kernel(ew::Copy2dArgs)",
                         "SQ_LDS_BANK_CONFLICT", bank / 2])
            wr.writerow([d, "void ew::ew_transpose_kernel(ew::Copy2dArgs)",
                         "SQ_LDS_BANK_CONFLICT", bank / 2])
            wr.writerow([d, "void ew::ew_transpose_kernel(ew::Copy2dArgs)",
                         "SQ_LDS_IDX_ACTIVE", active])
    rs.main(["counters", "--csv", str(cc), "--kernel", "ew_transpose_kernel", "--workload",
             w.name, "--family", "view", "--bench-json", str(out), "--command", "cmd",
             "--out", str(tmp_path / "c.txt")])
    text = (tmp_path / "c.txt").read_text()
    assert "SQ_LDS_BANK_CONFLICT   40" in text and "LDS-active cycles: 0.400" in text


def test_kernel_names_match_in_demangled_and_mangled_form():
    """rocprofv3 leaves kernels with _Float16 / __bf16 template arguments
    mangled; the summary still finds each instance, and only that one."""
    from memory_bound_elementwise_amd.rocprof_summary import kernel_matches
    relu_f16 = "_ZN2ew16ew_stream_kernelINS_8OpRelu16IDF16_EELi1ELb1ELb1EEEvNS_10StreamArgsE"
    sqrt_bf16 = ("_ZN2ew16ew_stream_kernelINS_7OpMap16IDF16bNS_17FnSqrtWidenedBF16EEELi1ELb1E"
                 "Lb1EEEvNS_10StreamArgsE")
    assert kernel_matches("ew_stream_kernel<ew::OpRelu16<_Float16>, 1, true, true>", relu_f16)
    assert not kernel_matches("ew_stream_kernel<ew::OpRelu16<__bf16>, 1, true, true>", relu_f16)
    assert not kernel_matches("ew_stream_kernel<ew::OpRelu16<_Float16>, 2, true, true>", relu_f16)
    assert not kernel_matches("ew_stream_kernel<ew::OpRelu16<_Float16>, 1, false, true>",
                              relu_f16)
    assert kernel_matches(
        "ew_stream_kernel<ew::OpMap16<__bf16, ew::FnSqrtWidenedBF16>, 1, true, true>", sqrt_bf16)
    name = "void ew::ew_stream_kernel<ew::OpAddF32, 1, true, true>(ew::StreamArgs)"
    assert kernel_matches("ew_stream_kernel<ew::OpAddF32, 1, true, true>", name)
    assert not kernel_matches("ew_stream_kernel<ew::OpAddF32, 1, false, true>", name)
    assert kernel_matches("ew_transpose_kernel", "ew::ew_transpose_kernel(ew::Copy2dArgs)")


def test_memory_side_counter_figures():
    """Latency = requests in flight summed per cycle / requests; in flight per
    channel = that sum / one XCD's busy cycles / 128 channels; credit stalls
    as a share of the channels' busy cycles (GRBM_GUI_ACTIVE is summed over
    the 8 XCDs, the TCC counters over the 128 channels)."""
    from memory_bound_elementwise_amd import rocprof_summary as rs
    med = {"GRBM_GUI_ACTIVE": 8 * 1000.0, "TCC_EA0_RDREQ": 500.0,
           "TCC_EA0_RDREQ_LEVEL": 128 * 1000 * 300.0,
           "TCC_EA0_RDREQ_DRAM_CREDIT_STALL": 128 * 1000 * 0.25}
    lines = rs.memory_side_lines(med)
    assert any("latency" in ln and f"{128 * 1000 * 300 / 500:.0f} cycles" in ln for ln in lines)
    assert any("in flight per L2 channel: 300 " in ln for ln in lines)
    assert any("read interface out of DRAM credits: 0.250" in ln for ln in lines)
    assert rs.memory_side_lines({"GRBM_GUI_ACTIVE": 1.0}) == []
