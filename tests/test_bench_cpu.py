"""bench.py's host-side bookkeeping, without a GPU: byte formulas, the
in-place ReLU's store counts, the traffic record lookup and the one-GPU
contract."""
import json
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
    rec = {"workloads": {"w": {"kernel_source_sha256_16": bench.kernel_source_hash(),
                               "launch": {"block": 1024, "grid": 7, "unroll": 1},
                               "hbm_bytes_per_launch": 123}}}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_JSON", str(f))
    assert bench.traffic_for("w", {"block": 1024, "grid": 7, "unroll": 1}) == 123
    assert bench.traffic_for("w", {"block": 512, "grid": 7, "unroll": 1}) is None
    assert bench.traffic_for("other", {"block": 1024, "grid": 7, "unroll": 1}) is None
    rec["workloads"]["w"]["kernel_source_sha256_16"] = "0" * 16
    f.write_text(json.dumps(rec))
    assert bench.traffic_for("w", {"block": 1024, "grid": 7, "unroll": 1}) is None


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
