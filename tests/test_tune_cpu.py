"""The tuner's table writer, without a GPU: a tuned op gets new small and
large rows, keeps any other row (a mid-size row measured cold by a separate
sweep), and its large row replaces the op's last row at or above 2^22; ops
not tuned keep every row."""
import memory_bound_elementwise_amd.tune as tune


def test_write_table_keeps_rows_it_does_not_measure(tmp_path, monkeypatch):
    old = tmp_path / "old.txt"
    old.write_text(
        "add_f32     0        512   1     2  # old small\n"
        "add_f32     4194304  512   1024  2  # mid, cold sweep\n"
        "add_f32     33554432 1024  1024  1  # old large\n"
        "copy_f32    0        256   8     1  # copy small\n"
        "copy_f32    4194304  256   1024  1  # copy large\n")

    class FakeCuda:
        @staticmethod
        def get_device_name(i):
            return "test device"

        @staticmethod
        def get_device_properties(i):
            class P:
                multi_processor_count = 256
            return P

    class FakeTorch:
        cuda = FakeCuda

    monkeypatch.setattr(tune, "torch", FakeTorch)
    out = tmp_path / "new.txt"
    tune.write_table({"add_f32": {"small": (256, 2, 1, 3000.0), "large": (1024, 1024, 1, 6600.0)},
                      "relu_f32": {"small": (64, 4, 4, 2000.0), "large": (256, 1024, 1, 6700.0)}},
                     str(out), merge_from=str(old))
    rows = tune._read_rows(str(out))
    assert [r[:4] for r in rows["add_f32"]] == [(0, 256, 2, 1), (1 << 22, 512, 1024, 2),
                                                (1 << 25, 1024, 1024, 1)]
    assert rows["add_f32"][1][4] == "mid, cold sweep"
    assert [r[:4] for r in rows["copy_f32"]] == [(0, 256, 8, 1), (1 << 22, 256, 1024, 1)]
    assert [r[:4] for r in rows["relu_f32"]] == [(0, 64, 4, 4), (1 << 22, 256, 1024, 1)]
