"""The C-ABI library without a GPU: it loads, exports every symbol the header
declares, and rejects bad arguments before any HIP call.

No test here launches a kernel.  Every call with made-up addresses fails
validation first; the one test that passes validation runs only when no GPU
is visible (it then gets EW_ERR_NO_DEVICE).
"""
import ctypes
import os
import re

import pytest

import memory_bound_elementwise_amd as ew
from tests.conftest import ROOT, _gpu_visible

HEADER = os.path.join(ROOT, "include", "ew.h")

(EW_OK, EW_ERR_INVALID_ARG, EW_ERR_MISALIGNED, EW_ERR_OVERLAP, EW_ERR_NO_DEVICE, EW_ERR_HIP,
 EW_ERR_TOO_LARGE) = (0, -1, -2, -3, -4, -5, -6)

BASE = 0x7F0000000000          # a made-up, 256-byte aligned device address
MiB = 1 << 20


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ew_[a-z0-9_]+)\s*\(", text)))


def _raw():
    return ctypes.CDLL(ew.library_path())


def test_header_declares_the_operations():
    names = _declared_functions()
    for op in ("ew_add_f32", "ew_add_f16", "ew_add_bf16", "ew_saxpy_f32", "ew_relu_f32",
               "ew_copy_f32", "ew_gather_f32"):
        assert op in names


def test_library_exports_every_declared_symbol():
    lib = _raw()
    missing = [n for n in _declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_binding_names_match_the_c_abi():
    for name in _declared_functions():
        assert hasattr(ew, name), name


def test_abi_version_and_status_strings():
    assert ew.ew_abi_version() == 14
    for code in (EW_OK, EW_ERR_INVALID_ARG, EW_ERR_MISALIGNED, EW_ERR_OVERLAP,
                 EW_ERR_NO_DEVICE, EW_ERR_HIP, EW_ERR_TOO_LARGE):
        s = ew.ew_status_string(code)
        assert s.startswith("EW_")
    assert ew.ew_status_string(12345) == "EW_ERR_UNKNOWN"
    assert ew.ew_last_hip_error() == 0


def _status(fn, *args):
    try:
        fn(*args)
    except ew.EwError as e:
        return e.status
    return EW_OK


def test_n_zero_is_a_no_op_even_with_null_pointers():
    assert _status(ew.ew_add_f32, 0, 0, 0, 0, 0) == EW_OK
    assert _status(ew.ew_add_f16, 0, 0, 0, 0, 0) == EW_OK
    assert _status(ew.ew_add_bf16, 0, 0, 0, 0, 0) == EW_OK
    assert _status(ew.ew_saxpy_f32, 2.5, 0, 0, 0, 0) == EW_OK
    assert _status(ew.ew_relu_f32, 0, 0, 0, 0) == EW_OK
    assert _status(ew.ew_copy_f32, 0, 0, 0, 0) == EW_OK
    assert _status(ew.ew_gather_f32, 0, 0, 2, 0, 0) == EW_OK


def test_null_pointers_are_invalid():
    n = 16
    assert _status(ew.ew_add_f32, 0, BASE, BASE + MiB, n, 0) == EW_ERR_INVALID_ARG
    assert _status(ew.ew_add_f32, BASE, 0, BASE + MiB, n, 0) == EW_ERR_INVALID_ARG
    assert _status(ew.ew_add_f32, BASE, BASE + MiB, 0, n, 0) == EW_ERR_INVALID_ARG
    assert _status(ew.ew_saxpy_f32, 1.0, 0, BASE, n, 0) == EW_ERR_INVALID_ARG
    assert _status(ew.ew_relu_f32, BASE, 0, n, 0) == EW_ERR_INVALID_ARG
    assert _status(ew.ew_copy_f32, 0, BASE, n, 0) == EW_ERR_INVALID_ARG
    assert _status(ew.ew_gather_f32, 0, BASE, 2, n, 0) == EW_ERR_INVALID_ARG


def test_zero_stride_and_size_overflow_are_invalid():
    assert _status(ew.ew_gather_f32, BASE, BASE + MiB, 0, 16, 0) == EW_ERR_INVALID_ARG
    # n * 4 overflows size_t
    assert _status(ew.ew_add_f32, BASE, BASE + MiB, BASE + 2 * MiB, (1 << 63), 0) == \
        EW_ERR_INVALID_ARG
    # n at or above 2^62 elements
    assert _status(ew.ew_add_f16, BASE, BASE + MiB, BASE + 2 * MiB, (1 << 62), 0) == \
        EW_ERR_INVALID_ARG
    # the range would wrap around the address space
    top = (1 << 64) - 64
    assert _status(ew.ew_relu_f32, top, BASE, 1024, 0) == EW_ERR_INVALID_ARG


def test_element_misalignment_is_rejected():
    n = 16
    assert _status(ew.ew_add_f32, BASE + 2, BASE + MiB, BASE + 2 * MiB, n, 0) == \
        EW_ERR_MISALIGNED
    assert _status(ew.ew_add_f32, BASE, BASE + MiB, BASE + 2 * MiB + 1, n, 0) == \
        EW_ERR_MISALIGNED
    assert _status(ew.ew_add_f16, BASE + 1, BASE + MiB, BASE + 2 * MiB, n, 0) == \
        EW_ERR_MISALIGNED
    assert _status(ew.ew_add_bf16, BASE, BASE + MiB + 3, BASE + 2 * MiB, n, 0) == \
        EW_ERR_MISALIGNED
    assert _status(ew.ew_saxpy_f32, 2.5, BASE + 6, BASE + MiB, n, 0) == EW_ERR_MISALIGNED
    assert _status(ew.ew_gather_f32, BASE + 2, BASE + MiB, 2, n, 0) == EW_ERR_MISALIGNED


def test_partial_overlap_is_rejected():
    n = 1024
    # output starts one element into input a
    assert _status(ew.ew_add_f32, BASE, BASE + MiB, BASE + 4, n, 0) == EW_ERR_OVERLAP
    assert _status(ew.ew_add_f32, BASE + 4, BASE + MiB, BASE, n, 0) == EW_ERR_OVERLAP
    assert _status(ew.ew_add_f16, BASE + MiB, BASE, BASE + 2, n, 0) == EW_ERR_OVERLAP
    assert _status(ew.ew_saxpy_f32, 2.5, BASE, BASE + 8, n, 0) == EW_ERR_OVERLAP
    assert _status(ew.ew_relu_f32, BASE, BASE + 4 * n - 4, n, 0) == EW_ERR_OVERLAP
    assert _status(ew.ew_copy_f32, BASE + 4, BASE, n, 0) == EW_ERR_OVERLAP
    # the gather forbids any overlap, exact aliasing included
    assert _status(ew.ew_gather_f32, BASE, BASE, 2, n, 0) == EW_ERR_OVERLAP
    assert _status(ew.ew_gather_f32, BASE, BASE + 4 * n - 4, 2, n, 0) == EW_ERR_OVERLAP


def test_fused_ops_validation():
    n = 1024
    assert _status(ew.ew_add_relu_f32, 0, 0, 0, 0, 0) == EW_OK
    assert _status(ew.ew_add_relu_f32, 0, BASE, BASE + MiB, n, 0) == EW_ERR_INVALID_ARG
    assert _status(ew.ew_add_relu_f32, BASE + 2, BASE + MiB, BASE + 2 * MiB, n, 0) == \
        EW_ERR_MISALIGNED
    assert _status(ew.ew_add_relu_f32, BASE, BASE + MiB, BASE + 4, n, 0) == EW_ERR_OVERLAP
    assert _status(ew.ew_saxpy_relu_f32, 1.0, BASE, BASE + 8, n, 0) == EW_ERR_OVERLAP
    assert _status(ew.ew_saxpy_relu_f32, 1.0, 0, BASE, n, 0) == EW_ERR_INVALID_ARG
    # bias + ReLU: rows or cols 0 is a no-op; null bias; rows*cols overflow;
    # misaligned bias; bias overlapping y; x partially overlapping y
    assert _status(ew.ew_bias_relu_f32, 0, 0, 0, 0, 16, 0) == EW_OK
    assert _status(ew.ew_bias_relu_f32, 0, 0, 0, 16, 0, 0) == EW_OK
    assert _status(ew.ew_bias_relu_f32, BASE, 0, BASE + MiB, 4, 4, 0) == EW_ERR_INVALID_ARG
    assert _status(ew.ew_bias_relu_f32, BASE, BASE + 8 * MiB, BASE + MiB, 1 << 40, 1 << 40,
                   0) == EW_ERR_INVALID_ARG
    assert _status(ew.ew_bias_relu_f32, BASE, BASE + 8 * MiB + 2, BASE + MiB, 4, 4, 0) == \
        EW_ERR_MISALIGNED
    assert _status(ew.ew_bias_relu_f32, BASE, BASE + MiB + 16, BASE + MiB, 4, 4, 0) == \
        EW_ERR_OVERLAP
    assert _status(ew.ew_bias_relu_f32, BASE + 4, BASE + 8 * MiB, BASE, 4, 4, 0) == \
        EW_ERR_OVERLAP


def test_copy2d_validation():
    c2 = ew.ew_copy2d_f32
    assert _status(c2, 0, 1, 1, 0, 0, 5, 0) == EW_OK                      # rows 0
    assert _status(c2, BASE, 1, 1, BASE + MiB, 5, 0, 0) == EW_OK           # cols 0
    assert _status(c2, 0, 1, 1, BASE, 4, 4, 0) == EW_ERR_INVALID_ARG
    assert _status(c2, BASE, 1, 1, 0, 4, 4, 0) == EW_ERR_INVALID_ARG
    assert _status(c2, BASE, 1, 1, BASE + MiB, 1 << 40, 1 << 40, 0) == EW_ERR_INVALID_ARG
    # a view reaching below address 0 or past the top of the address space
    assert _status(c2, 0x1000, -4096, 1, BASE, 4, 4, 0) == EW_ERR_INVALID_ARG
    assert _status(c2, (1 << 64) - 4096, 1 << 20, 1, BASE, 4, 4, 0) == EW_ERR_INVALID_ARG
    assert _status(c2, BASE + 2, 1, 4, BASE + MiB, 4, 4, 0) == EW_ERR_MISALIGNED
    assert _status(c2, BASE, 1, 4, BASE + MiB + 1, 4, 4, 0) == EW_ERR_MISALIGNED
    # out overlapping the touched span, including through a negative stride
    assert _status(c2, BASE, 4, 1, BASE + 4 * 15, 4, 4, 0) == EW_ERR_OVERLAP
    assert _status(c2, BASE + 4096, -256, 1, BASE + 4096 - 256 * 3 * 4, 4, 4, 0) == \
        EW_ERR_OVERLAP


def test_adjacent_ranges_do_not_overlap_and_copy_onto_itself_is_a_no_op():
    n = 1024
    # [BASE, BASE+4n) and [BASE+4n, ...) touch but do not overlap: validation
    # passes, so check through the planner (which launches nothing).
    p = ew.ew_make_plan("copy_f32", BASE + 4 * n, BASE, 0, n, 256)
    assert p.vectors == n // 4
    # copy with out == in returns EW_OK without a launch or a device
    assert _status(ew.ew_copy_f32, BASE, BASE, n, 0) == EW_OK


@pytest.mark.skipif(_gpu_visible(), reason="only meaningful where no GPU is visible")
def test_valid_call_without_a_device_reports_no_device():
    assert _status(ew.ew_add_f32, BASE, BASE + MiB, BASE + 2 * MiB, 1000, 0) == EW_ERR_NO_DEVICE
    assert _status(ew.ew_gather_f32, BASE, BASE + MiB, 2, 1000, 0) == EW_ERR_NO_DEVICE
    # exact aliasing is allowed for add, so it also gets as far as the device check
    assert _status(ew.ew_add_f32, BASE, BASE + MiB, BASE, 1000, 0) == EW_ERR_NO_DEVICE
    assert _status(ew.ew_saxpy_f32, 2.5, BASE, BASE, 1000, 0) == EW_ERR_NO_DEVICE


def test_launch_rows_set_get_reset_and_load(tmp_path):
    """Size-class rows: ew_set_launch_row / ew_get_launch_row."""
    try:
        ew.ew_reset_launch_config()
        default = ew.ew_get_launch_row("add_f32", 1 << 28)
        ew.ew_set_launch_row("add_f32", 1 << 26, 512, 4, 4)
        assert ew.ew_get_launch_row("add_f32", 1 << 28) == (512, 4, 4)
        assert ew.ew_get_launch_row("add_f32", (1 << 26) - 1) != (512, 4, 4)
        # replacing a row
        ew.ew_set_launch_row("add_f32", 1 << 26, 1024, 2, 8)
        assert ew.ew_get_launch_row("add_f32", 1 << 26) == (1024, 2, 8)
        # invalid values
        for bad in ((100, 8, 1), (0, 8, 1), (2048, 8, 1), (256, 0, 1), (256, 8, 3)):
            with pytest.raises(ew.EwError):
                ew.ew_set_launch_row("add_f32", 0, *bad)
        with pytest.raises(ew.EwError):
            ew.ew_set_launch_row("no_such_op", 0, 256, 8, 1)
        with pytest.raises(ew.EwError):
            ew.ew_get_launch_row("no_such_op", 0)
        ew.ew_reset_launch_config()
        assert ew.ew_get_launch_row("add_f32", 1 << 28) == default
        # table file
        f = tmp_path / "table.txt"
        f.write_text("# op min_n block bpc unroll\n\nrelu_f32 0 128 16 1  # small\n"
                     "relu_f32 1048576 512 2 4\n")
        ew.ew_load_launch_table(str(f))
        assert ew.ew_get_launch_row("relu_f32", 10) == (128, 16, 1)
        assert ew.ew_get_launch_row("relu_f32", 1 << 21) == (512, 2, 4)
        bad = tmp_path / "bad.txt"
        bad.write_text("relu_f32 0 128\n")
        with pytest.raises(ew.EwError):
            ew.ew_load_launch_table(str(bad))
        with pytest.raises(ew.EwError):
            ew.ew_load_launch_table(str(tmp_path / "missing.txt"))
    finally:
        ew.ew_reset_launch_config()
        if os.path.exists(ew.LAUNCH_TABLE):
            ew.ew_load_launch_table(ew.LAUNCH_TABLE)


def test_set_launch_config_replaces_every_size_class():
    """ew_set_launch_config(op, block, blocks_per_cu, unroll): one row for
    every n of that operation; other operations keep their rows."""
    try:
        ew.ew_reset_launch_config()
        relu = [ew.ew_get_launch_row("relu_f32", n) for n in (1, 1 << 22, 1 << 28)]
        ew.ew_set_launch_config("add_f32", 256, 4, 2)
        for n in (0, 1, 1 << 20, 1 << 22, 1 << 25, 1 << 28, (1 << 62) - 1):
            assert ew.ew_get_launch_row("add_f32", n) == (256, 4, 2), n
        assert [ew.ew_get_launch_row("relu_f32", n) for n in (1, 1 << 22, 1 << 28)] == relu
        p = ew.ew_make_plan("add_f32", BASE, BASE + 8 * MiB, BASE + 16 * MiB, 1 << 20, 256)
        assert (p.block, p.blocks_per_cu, p.unroll) == (256, 4, 2)
        assert p.grid == min(4 * 256, -(-(1 << 18) // 512))
        for bad in ((100, 8, 1), (0, 8, 1), (2048, 8, 1), (256, 0, 1), (256, 1025, 1),
                    (256, 8, 3)):
            with pytest.raises(ew.EwError):
                ew.ew_set_launch_config("add_f32", *bad)
        with pytest.raises(ew.EwError):
            ew.ew_set_launch_config("no_such_op", 256, 8, 1)
        with pytest.raises(ew.EwError):
            ew.ew_get_launch_config("no_such_op", 1)
    finally:
        ew.ew_reset_launch_config()
        ew.ew_load_launch_table(ew.LAUNCH_TABLE)


@pytest.mark.skipif(_gpu_visible(), reason="only meaningful where no GPU is visible")
def test_get_launch_config_needs_a_device():
    """The grid depends on the current device's compute-unit count."""
    with pytest.raises(ew.EwError) as e:
        ew.ew_get_launch_config("add_f32", 1 << 28)
    assert e.value.status == EW_ERR_NO_DEVICE


def test_compiled_defaults_match_the_shipped_table():
    """The library's built-in rows are the tuned table it ships with, so a
    caller that never loads the file gets the same launches."""
    rows = []
    for line in open(ew.LAUNCH_TABLE):
        f = line.split("#")[0].split()
        if f:
            rows.append((f[0], int(f[1]), tuple(int(v) for v in f[2:5])))
    assert {r[0] for r in rows} == set(ew.OPS)
    try:
        ew.ew_reset_launch_config()
        for op, min_n, cfg in rows:
            assert ew.ew_get_launch_row(op, min_n) == cfg, (op, min_n)
    finally:
        ew.ew_load_launch_table(ew.LAUNCH_TABLE)


def test_planning_and_the_table_are_thread_safe():
    """Several threads plan, read and rewrite the launch table at once (the
    ctypes calls release the GIL); every plan stays self-consistent and the
    process survives.  Rows are rewritten with values every row can take."""
    import threading
    errors = []

    def planner(seed):
        try:
            for k in range(400):
                n = (seed * 7919 + k * 104729) % (1 << 24) + 1
                p = ew.ew_make_plan("add_f32", BASE + 4 * (k % 4), BASE + 2 * MiB * 64,
                                    BASE + 4 * MiB * 64, n, 256)
                assert p.head + 4 * p.vectors + p.tail == n
                assert p.tiles == -(-p.vectors // (p.block * p.unroll))
                g = ew.ew_make_gather_plan(BASE + 8 * MiB * 64, BASE, n, 3, 256)
                assert g.n == n
        except Exception as e:   # noqa: BLE001 - reported below
            errors.append(repr(e))

    def writer():
        try:
            for k in range(400):
                ew.ew_set_launch_row("add_f32", 1 << 22, (64, 256, 1024)[k % 3], 1024, 1)
                ew.ew_get_launch_row("add_f32", 1 << 23)
                if k % 50 == 0:
                    ew.ew_reset_launch_config()
        except Exception as e:   # noqa: BLE001
            errors.append(repr(e))

    threads = [threading.Thread(target=planner, args=(s,)) for s in range(6)]
    threads.append(threading.Thread(target=writer))
    try:
        for t in threads:
            t.start()
        for t in threads:
            t.join()
    finally:
        ew.ew_reset_launch_config()
        ew.ew_load_launch_table(ew.LAUNCH_TABLE)
    assert not errors, errors[:3]


def test_header_is_clean_c11_and_a_c_program_links_against_the_library(tmp_path):
    """A plain C11 program (no C++, no torch) includes ew.h with warnings as
    errors and links libew.so, the HIP runtime and the oracle."""
    import importlib.util
    spec = importlib.util.spec_from_file_location(
        "_c_client_build", os.path.join(ROOT, "tests", "c_abi", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    exe = mod.build(out=str(tmp_path / "client"))
    assert os.path.exists(exe)


def _batch(op, items, alpha=0.0):
    """ew_batch on raw (out, in0, in1, n) tuples; returns the status."""
    arr = (ew.EwBatchItem * max(len(items), 1))(*[ew.EwBatchItem(*it) for it in items])
    return ew._c["ew_batch"](op.encode(), alpha, arr, len(items), None)


def test_batch_validation():
    n = 1024
    a, b, c = BASE, BASE + MiB, BASE + 2 * MiB
    assert _batch("add_f32", []) == EW_OK
    assert _batch("add_f32", [(c, a, b, 0), (0, 0, 0, 0)]) == EW_OK          # all n == 0
    assert ew._c["ew_batch"](b"add_f32", 0.0, None, 3, None) == EW_ERR_INVALID_ARG
    for op in ("gather_f32", "bias_relu_f32", "copy2d_f32", "relu_inplace_f32", "nope"):
        assert _batch(op, [(c, a, b, n)]) == EW_ERR_INVALID_ARG, op
    # each item is validated like its single call
    assert _batch("add_f32", [(c, a, b, n), (c + 4 * MiB, 0, b, n)]) == EW_ERR_INVALID_ARG
    assert _batch("add_f16", [(c, a + 1, b, n)]) == EW_ERR_MISALIGNED
    assert _batch("relu_f32", [(a + 4, a, None, n)]) == EW_ERR_OVERLAP
    # across items: an output may not meet another item's input or output
    assert _batch("add_f32", [(c, a, b, n), (c + 4 * n - 4, a, b, n)]) == EW_ERR_OVERLAP
    assert _batch("add_f32", [(c, a, b, n), (a + 8, c + 8 * MiB, b, 4)]) == EW_ERR_OVERLAP
    assert _batch("saxpy_f32", [(b, a, None, n), (a, b, None, n)]) == EW_ERR_OVERLAP
    # exact aliasing inside one item stays allowed, as for the single call
    assert _batch("relu_f32", [(a, a, None, n), (b, b, None, n)]) in (EW_OK, EW_ERR_NO_DEVICE,
                                                                      EW_ERR_HIP)


@pytest.mark.skipif(_gpu_visible(), reason="only meaningful where no GPU is visible")
def test_valid_batch_without_a_device_reports_no_device():
    n = 1024
    a, b = BASE, BASE + MiB
    outs = [BASE + (2 + k) * MiB for k in range(100)]
    # 100 items reading the same two inputs (shared reads are fine)
    items = [(o, a, b, n + k) for k, o in enumerate(outs)]
    assert _batch("add_f32", items) == EW_ERR_NO_DEVICE
    assert _batch("scale_bf16", [(o, a, None, n) for o in outs], 2.5) == EW_ERR_NO_DEVICE


def _build(op, items, table=None, table_bytes=0):
    """ew_batch_build on raw (out, in0, in1, n) tuples; returns (status, plan)."""
    arr = (ew.EwBatchItem * max(len(items), 1))(*[ew.EwBatchItem(*it) for it in items])
    plan = ew.EwBatchPlan()
    st = ew._c["ew_batch_build"](op.encode(), arr, len(items), table, table_bytes,
                                 ctypes.byref(plan))
    return st, plan


def test_batch_build_validates_like_the_host_array_call():
    """Every item list that ew_batch rejects, ew_batch_build rejects with the
    same status (the two share their validation)."""
    n = 1024
    a, b, c = BASE, BASE + MiB, BASE + 2 * MiB
    cases = [("add_f32", [(c, a, b, n), (c + 4 * MiB, 0, b, n)]),
             ("add_f16", [(c, a + 1, b, n)]),
             ("relu_f32", [(a + 4, a, None, n)]),
             ("add_f32", [(c, a, b, n), (c + 4 * n - 4, a, b, n)]),
             ("add_f32", [(c, a, b, n), (a + 8, c + 8 * MiB, b, 4)]),
             ("saxpy_f32", [(b, a, None, n), (a, b, None, n)])]
    cases += [(op, [(c, a, b, n)]) for op in ("gather_f32", "gather_walk_f32", "bias_relu_f32",
                                               "copy2d_f32", "relu_inplace_f32", "nope")]
    for op, items in cases:
        want = _batch(op, items)
        assert want != EW_OK
        assert _build(op, items)[0] == want, (op, items)
    st = ew._c["ew_batch_build"](b"add_f32", None, 3, None, 0, ctypes.byref(ew.EwBatchPlan()))
    assert st == EW_ERR_INVALID_ARG
    assert ew._c["ew_batch_build"](b"add_f32", None, 0, None, 0, None) == EW_ERR_INVALID_ARG


def _batch_shape(op, items, es):
    """The documented launch shape of a batched call: the row for the total
    n (unroll at most 4), the tile halved -- unroll first, then the block,
    down to 64 threads -- while half of it still covers the mean item's
    vectors, and one block per tile (blocks_per_cu 1024) once shrunk."""
    total = sum(it[3] for it in items)
    block, bpc, unroll = ew.ew_get_launch_row(op, total)
    unroll = min(unroll, 4)
    live = [it[3] for it in items if it[3] > 0]
    mean = -(-sum(n // (16 // es) for n in live) // len(live))
    shrunk = False
    while unroll > 1 and block * unroll // 2 >= mean:
        unroll //= 2
        shrunk = True
    while block > 64 and block // 2 >= mean:
        block //= 2
        shrunk = True
    return block, 1024 if shrunk else bpc, unroll


def test_batch_tiles_shrink_to_small_items():
    """1024 items of 1024 fp32 elements (256 vectors each): the row for 2^20
    elements has 1024-vector tiles, so the tile shrinks to 256 vectors, one
    item per tile and one block per tile; large items keep the row's shape."""
    small = [(BASE + 3 * k * 8192, BASE + (3 * k + 1) * 8192, BASE + (3 * k + 2) * 8192, 1024)
             for k in range(1024)]
    st, plan = _build("add_f32", small)
    assert st == EW_OK
    assert plan.block * plan.unroll == 256 and plan.tiles == 1024 and plan.blocks_per_cu == 1024
    big = [(BASE + 3 * k * (1 << 22), BASE + (3 * k + 1) * (1 << 22),
            BASE + (3 * k + 2) * (1 << 22), 1 << 20) for k in range(4)]
    st, plan = _build("add_f32", big)
    assert st == EW_OK
    block, bpc, unroll = ew.ew_get_launch_row("add_f32", 1 << 22)
    assert (plan.block, plan.blocks_per_cu, plan.unroll) == (block, bpc, min(4, unroll))


def _expected_tiles(out, n, es, block, unroll):
    head = min(((16 - out % 16) % 16) // es, n)
    vectors = (n - head) // (16 // es)
    return max(1, -(-vectors // (block * unroll)))


@pytest.mark.parametrize("op,es", [("add_f32", 4), ("add_bf16", 2), ("saxpy_f32", 4),
                                   ("relu_f16", 2), ("sqrt_f32", 4)])
def test_batch_build_writes_the_documented_image(op, es):
    """The image holds one 40-byte record per item with n > 0 (in0, in1, out,
    n, first tile) and one 32-bit item index per tile; the tile counts are the
    single call's (head aligning the output to 16 bytes), at least one per
    item; a size query (no table) gives the same plan."""
    import random
    rnd = random.Random(7 + es)
    items = []
    for k in range(300):
        n = rnd.choice([0, 1, 3, 7, 8, 15, 1000, 4096, 65536 + 5, rnd.randrange(1, 200000)])
        base = BASE + k * 4 * MiB
        out = base + es * rnd.randrange(0, 8)
        in0 = base + MiB + es * rnd.randrange(0, 8)
        in1 = base + 2 * MiB + es * rnd.randrange(0, 8)
        if op == "saxpy_f32":
            in1 = None                       # the second input is out itself
        elif op in ("relu_f16", "sqrt_f32"):
            in1 = None
        items.append((out, in0, in1, n))
    st, plan = _build(op, items)
    assert st == EW_OK
    total = sum(it[3] for it in items)
    block, bpc, unroll = _batch_shape(op, items, es)
    assert (plan.block, plan.unroll, plan.blocks_per_cu) == (block, unroll, bpc)
    live = [it for it in items if it[3] > 0]
    tiles = [_expected_tiles(it[0], it[3], es, block, unroll) for it in live]
    assert plan.items == len(live) and plan.tiles == sum(tiles) and plan.total_n == total
    assert plan.bytes == -(-(40 * len(live) + 4 * sum(tiles)) // 8) * 8
    img = (ctypes.c_uint64 * (plan.bytes // 8))()
    st, plan2 = _build(op, items, ctypes.addressof(img), plan.bytes)
    assert st == EW_OK and bytes(plan2) == bytes(plan)
    raw = bytes(img)
    import struct
    first = 0
    for k, (it, nt) in enumerate(zip(live, tiles)):
        in0, in1, out, n, ft = struct.unpack_from("<5Q", raw, 40 * k)
        second = it[0] if op == "saxpy_f32" else (it[2] or 0)
        assert (in0, in1, out, n, ft) == (it[1], second, it[0], it[3], first), k
        idx = struct.unpack_from(f"<{nt}I", raw, 40 * len(live) + 4 * first)
        assert set(idx) == {k}
        first += nt
    assert raw[40 * len(live) + 4 * first:] == b"\0" * (plan.bytes - 40 * len(live) - 4 * first)
    # too small a table, or a misaligned one
    assert _build(op, items, ctypes.addressof(img), plan.bytes - 8)[0] == EW_ERR_INVALID_ARG
    big = (ctypes.c_uint64 * (plan.bytes // 8 + 1))()
    assert _build(op, items, ctypes.addressof(big) + 4, plan.bytes)[0] == EW_ERR_MISALIGNED


def test_batch_build_of_nothing_and_run_checks_the_plan():
    st, plan = _build("add_f32", [(BASE, BASE + MiB, BASE + 2 * MiB, 0)])
    assert st == EW_OK and plan.items == 0 and plan.tiles == 0 and plan.bytes == 0
    run = ew._c["ew_batch_run"]
    assert run(ctypes.byref(plan), 0.0, None, None) == EW_OK          # nothing to launch
    assert run(None, 0.0, BASE, None) == EW_ERR_INVALID_ARG
    st, plan = _build("add_f32", [(BASE + 2 * MiB * k, BASE + 2 * MiB * k + MiB,
                                   BASE + 2 * MiB * k + MiB + 4096, 1000) for k in range(4)])
    assert st == EW_OK and plan.items == 4
    assert run(ctypes.byref(plan), 0.0, None, None) == EW_ERR_INVALID_ARG
    assert run(ctypes.byref(plan), 0.0, BASE + 4, None) == EW_ERR_MISALIGNED
    for field, value in (("op", 999), ("op", 6), ("block", 100), ("unroll", 8), ("items", 0),
                         ("tiles", 3), ("bytes", 8), ("blocks_per_cu", 0)):
        bad = ew.EwBatchPlan.from_buffer_copy(plan)
        setattr(bad, field, value)
        assert run(ctypes.byref(bad), 0.0, BASE, None) == EW_ERR_INVALID_ARG, field
    if not _gpu_visible():
        assert run(ctypes.byref(plan), 0.0, BASE, None) == EW_ERR_NO_DEVICE


def test_gather_walk_validation():
    walk = ew._c["ew_gather_walk_f32"]
    assert walk(None, None, 0, 0, None) == EW_OK                        # n == 0
    assert walk(BASE, BASE + MiB, 1000, 0, None) == EW_ERR_INVALID_ARG   # stride 0
    assert walk(None, BASE + MiB, 1000, 2, None) == EW_ERR_INVALID_ARG
    assert walk(BASE + 2, BASE + MiB, 1000, 2, None) == EW_ERR_MISALIGNED
    assert walk(BASE, BASE + 3996, 1000, 2, None) == EW_ERR_OVERLAP
    assert walk(BASE, BASE, 1000, 1, None) == EW_ERR_OVERLAP             # no exact alias either
    if not _gpu_visible():
        assert walk(BASE, BASE + MiB, 1000, 2, None) == EW_ERR_NO_DEVICE


def test_batch_run_static_checks_before_any_hip_call():
    """The allocation-free run: a table larger than the static array is
    refused with its own status, before any device is touched; the plan is
    checked as for ew_batch_run."""
    run = ew._c["ew_batch_run_static"]
    img = (ctypes.c_uint64 * 4)()
    st, empty = _build("add_f32", [(BASE, BASE + MiB, BASE + 2 * MiB, 0)])
    assert st == EW_OK and run(ctypes.byref(empty), 0.0, None, None) == EW_OK
    # about 6000 single-tile items: a table over 256 KiB
    items = [(BASE + 3 * k * 4096, BASE + (3 * k + 1) * 4096, BASE + (3 * k + 2) * 4096, 1000)
             for k in range(6000)]
    st, big = _build("add_f32", items)
    assert st == EW_OK and big.bytes > ew.BATCH_SCRATCH_BYTES
    assert run(ctypes.byref(big), 0.0, ctypes.addressof(img), None) == EW_ERR_TOO_LARGE
    st, small = _build("add_f32", items[:100])
    assert st == EW_OK and small.bytes <= ew.BATCH_SCRATCH_BYTES
    assert run(None, 0.0, ctypes.addressof(img), None) == EW_ERR_INVALID_ARG
    assert run(ctypes.byref(small), 0.0, None, None) == EW_ERR_INVALID_ARG
    bad = ew.EwBatchPlan.from_buffer_copy(small)
    bad.bytes += 8
    assert run(ctypes.byref(bad), 0.0, ctypes.addressof(img), None) == EW_ERR_INVALID_ARG
    if not _gpu_visible():
        assert run(ctypes.byref(small), 0.0, ctypes.addressof(img), None) == EW_ERR_NO_DEVICE
