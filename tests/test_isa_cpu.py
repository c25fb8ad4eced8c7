"""Static checks on the gfx950 assembly of every kernel (no GPU needed).

The library's numerics rest on instruction choices the compiler could change
silently; these checks fail the build's tests if it does:

* no LDS (except the transpose's tile and the pass gather's staging) and no
  scratch (register spills);
* float denormal modes "preserve" for binary32 and binary16/64;
* no packed-fp32 instructions (the library is built without them);
* no single-rounding mixed-precision fma into a 16-bit result
  (v_fma_mixlo/mixhi_f16): the 16-bit SAXPY is defined as a binary32 fma
  followed by a separate round-to-nearest-even;
* no round-toward-zero conversions (v_cvt_pkrtz_*);
* the ReLU kernels select with a compare (no v_max_*, whose NaN rule returns
  the other operand);
* the square-root kernels take a refined binary32 root (the hardware
  estimate followed by fma residual corrections), never a native 16-bit
  root, and the scalar maps multiply / add in binary32;
* the pass-decomposed gather loads each wave's input span straight into LDS,
  all loads in flight together;
* the streaming kernels move 16 bytes per lane (global_load_dwordx4 /
  global_store_dwordx4) and store non-temporally; the single-input ones
  (copy, ReLU, in-place ReLU, bias + ReLU, the scalar and unary maps) and the
  strided-view kernel store their body
  with a compiler-emitted buffer store carrying the device-scope and
  non-temporal bits (buffer_store_dwordx4 ... nt sc1).
"""
import importlib.util
import os
import re

import pytest

from tests.conftest import ROOT


@pytest.fixture(scope="module")
def asm(tmp_path_factory):
    spec = importlib.util.spec_from_file_location(
        "_ew_build", os.path.join(ROOT, "memory_bound_elementwise_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    path = mod.device_asm(str(tmp_path_factory.mktemp("asm")))
    return open(path).read()


def _kernels(text):
    """{mangled name: (body, metadata)} for every kernel in the assembly."""
    # a function's label is followed by its first basic block; a data label
    # (the batch scratch array) is not
    bodies = dict(re.findall(r"\n(_ZN2ew\w+):[^\n]*\n(; %bb\.0:.*?)\n\.Lfunc_end", text, re.S))
    meta = dict(re.findall(r"\.amdhsa_kernel (\w+)(.*?)\.end_amdhsa_kernel", text, re.S))
    assert bodies and set(bodies) == set(meta), "could not split the assembly into kernels"
    return {k: (bodies[k], meta[k]) for k in bodies}


def _pass_lds(stride, step):
    # staging: 4 waves x stride loads of 1 KiB, each followed by 16 bytes of
    # padding when the stride is even
    staging = 4 * (65 if stride % 2 == 0 else 64) * stride * 16
    if step == stride:          # one run: the staging only
        return staging
    blocks_per_cu = 4 if stride == 2 else 2 if stride <= 5 else 1
    lds = max(staging, 160 * 1024 // blocks_per_cu - 1024)
    assert lds * (blocks_per_cu + 1) > 160 * 1024 >= lds * blocks_per_cu
    return lds


def test_every_kernel_has_no_lds_no_scratch_and_preserves_denormals(asm):
    """Only the transpose (one 128 x 132 fp32 tile), the gather's tiled
    transposition (its largest tile, 256 x 68 words, plus 128 run starts of
    8 bytes) and the
    pass-decomposed gather stage data in LDS.  A pass block that writes several runs (256
    threads, 16 * stride bytes per lane) reserves just over 1/(k + 1) of the
    CU's 160 KiB so that at most k blocks share a CU: k = 4 for stride 2, 2
    for 3..5, 1 for 6..32.  A single run (step == span: the x[::s] view, or a
    gather whose stride divides n) reserves its staging only."""
    ks = _kernels(asm)
    assert len(ks) > 100
    for name, (_, meta) in ks.items():
        d = dict(re.findall(r"\.amdhsa_(\w+) (\S+)", meta))
        lds = "67584" if "transpose" in name else "70656" if "gather_tiles" in name else (
            str(_pass_lds(*map(int, re.search(r"passes_kernelILi(\d+)ELi(\d+)E", name).groups())))
            if "gather_passes" in name else "0")
        assert d["group_segment_fixed_size"] == lds, name
        assert d["private_segment_fixed_size"] == "0", name
        assert d["float_denorm_mode_32"] == "3", name
        assert d["float_denorm_mode_16_64"] == "3", name


def test_wide_tile_instances_fit_two_blocks_per_cu(asm):
    """The gather's 128 x 128 and 256 x 64 tile instances run two 1024-thread
    blocks per CU: 32 waves, 8 per SIMD, so each wave may hold at most 64 of
    a SIMD's 512 VGPRs per lane, and two blocks' LDS must fit in the CU's
    160 KiB.  (The whole-row instances hold more registers and run one block
    per CU.)"""
    seen = 0
    for name, (_, meta) in _kernels(asm).items():
        m = re.search(r"gather_tiles_kernelILi(\d)E", name)
        if not m or m.group(1) not in ("2", "3"):
            continue
        d = dict(re.findall(r"\.amdhsa_(\w+) (\S+)", meta))
        assert int(d["next_free_vgpr"]) <= 64, (name, d["next_free_vgpr"])
        assert 2 * int(d["group_segment_fixed_size"]) <= 160 * 1024, name
        seen += 1
    assert seen == 2


def test_no_forbidden_instructions(asm):
    for pat in (r"\bv_pk_(add|mul|fma)_f32\b", r"\bv_fma_mix(lo|hi)_f16\b",
                r"\bv_mad_mix(lo|hi)_f16\b", r"\bv_cvt_pkrtz"):
        assert not re.search(pat, asm), pat


def test_relu_kernels_select_rather_than_max(asm):
    for name, (body, _) in _kernels(asm).items():
        if "Relu" in name:
            assert not re.search(r"\bv_(pk_)?max_(f32|f16|num_f32|num_f16|bf16)", body), name


def test_saxpy_kernels_use_a_fused_multiply_add(asm):
    for name, (body, _) in _kernels(asm).items():
        if "Saxpy" in name:
            assert re.search(r"\bv_fma(c)?_(mix_)?f32", body), name
            assert not re.search(r"\bv_mul_f32\b", body), name


SINGLE_INPUT_OPS = ("OpReluF32", "OpCopyF32", "OpRelu16", "OpMapF32", "OpMap16", "OpAbs")


def test_stream_kernels_move_16_bytes_per_lane_with_nt_stores(asm):
    """The batched kernels (item table in the kernel arguments or in device
    memory) follow the same store policy as the single ones."""
    n_single = n_batch = n_table = 0
    for name, (body, _) in _kernels(asm).items():
        n_batch += "ew_batch_kernel" in name
        n_table += "ew_batch_table_kernel" in name
        if ("ew_stream_kernel" in name or "relu_inplace" in name or "ew_batch_kernel" in name
                or "ew_batch_table_kernel" in name):
            assert re.search(r"global_load_dwordx4 .* nt\b", body), name
            if ("relu_inplace" in name or any(op in name for op in SINGLE_INPUT_OPS)):
                n_single += 1
                assert re.search(r"buffer_store_dwordx4 .* nt sc1\b", body), name
                assert not re.search(r"global_store_dwordx4", body), name
            else:
                assert re.search(r"global_store_dwordx4 .* nt\b", body), name
    assert n_single > 0
    assert n_batch == 23 * 3           # every batchable operator kernel x unroll 1, 2, 4
    assert n_table == 23 * 3


def test_strided_view_and_bias_relu_kernels_store_at_device_scope(asm):
    ks = [v[0] for k, v in _kernels(asm).items()
          if "ew_copy2d_kernel" in k or "ew_bias_relu_kernel" in k]
    assert ks
    for body in ks:
        assert re.search(r"buffer_store_dwordx4 .* nt sc1\b", body)


def test_device_scope_stores_come_from_the_compiler(asm):
    """The sc1 bit is set only through the buffer-store builtin: a global
    store with sc1 could only come from inline assembly, whose data registers
    the compiler does not protect after issue (that once stored stale data)."""
    assert not re.search(r"global_store_dword\S* .*\bsc1\b", asm)


def test_transpose_moves_16_bytes_per_lane_through_lds(asm):
    """Regression: a brace-initialised HIP float4 once collapsed the tile load
    into one 4-byte load broadcast to four lanes.  The full-tile path must
    load 16 bytes per lane, write them to LDS as one 128-bit store, and write
    16 bytes per lane to the output."""
    bodies = [v[0] for k, v in _kernels(asm).items() if "transpose" in k]
    assert len(bodies) == 1
    for body in bodies:
        assert re.search(r"global_load_dwordx4 .* nt\b", body)
        assert re.search(r"\bds_write_b128\b", body)
        assert re.search(r"global_store_dwordx4 .* nt\b", body)


def test_pass_gather_loads_its_span_straight_into_lds(asm):
    """Regression: staged through VGPRs, the span loads of the pass gather
    were issued one at a time (each waited for before the next) once the
    instance ran short of registers (s >= 23), at 0.6 x the speed.  Every
    instance must issue its S loads into LDS (buffer_load_dwordx4 ... lds)
    back to back, with no wait on the vector memory counter between them, and
    wait for them (vmcnt(0)) before its first LDS read."""
    ks = {k: v[0] for k, v in _kernels(asm).items() if "gather_passes_kernel" in k}
    assert len(ks) > 31
    for name, body in ks.items():
        S = int(re.search(r"passes_kernelILi(\d+)ELi", name).group(1))
        lines = [l.strip() for l in body.splitlines()
                 if l.strip() and not l.strip().startswith((";", "."))]
        loads = [i for i, l in enumerate(lines) if re.match(r"buffer_load_dwordx4 .*\blds$", l)]
        assert len(loads) == S, name
        assert loads[-1] - loads[0] < 8 * S, name          # one run of instructions
        assert not any(l.startswith("s_waitcnt") and "vmcnt" in l
                       for l in lines[loads[0]:loads[-1]]), name
        first_read = next(i for i in range(loads[-1], len(lines)) if lines[i].startswith("ds_read"))
        waits = [l for l in lines[loads[-1]:first_read] if l.startswith("s_waitcnt")]
        assert any("vmcnt(0)" in l for l in waits), name
        assert not re.search(r"\bglobal_load_dwordx4\b", body.split("ds_read")[0]), name


def test_inplace_relu_decides_stores_with_a_wave_vote(asm):
    """The in-place ReLU stores a 64-byte span whole or not at all: each lane's
    decision combines the wave's compare mask (a vote) with a 4-lane group
    mask shifted by the lane index."""
    ks = [v for k, v in _kernels(asm).items() if "relu_inplace" in k]
    assert len(ks) == 4
    for body, _ in ks:
        assert re.search(r"\bv_mbcnt_(lo|hi)_u32_b32\b", body)     # lane index
        assert re.search(r"\bv_lshlrev_b64\b", body)               # group mask << lane group


def test_sqrt_kernels_round_the_binary32_root_correctly(asm):
    """Neither hardware estimate (v_sqrt_f32, v_rsq_f32) is correctly rounded
    alone: for fp32 data and the binary16 map it is refined with fma
    residuals (the root's neighbours are tested and one is selected).  The
    bfloat16 map needs no refinement (every bfloat16 root is at least 32
    binary32 ulps from a bfloat16 rounding boundary; pinned in
    test_rounding_margins_cpu.py).  No form may use a native 16-bit root."""
    ks = {k: v[0] for k, v in _kernels(asm).items() if "FnSqrt" in k}
    # 3 formats x (4 unrolls x 2 alignments of the single kernel + 3 unrolls
    # of each batched kernel)
    assert len(ks) == 3 * (4 * 2 + 3 + 3)
    assert sum("FnSqrtWidenedF16" in k for k in ks) == 8 + 3 + 3
    assert sum("FnSqrtWidenedBF16" in k for k in ks) == 8 + 3 + 3
    for name, body in ks.items():
        assert not re.search(r"\bv_(sqrt|rsq|rcp)_f16", body), name
        if "FnSqrtWidenedBF16" in name:
            # no refinement needed (rounding margin >= 32 ulps): the hardware
            # root, tiny inputs scaled by 2^32 (0x4f800000) and back by 2^-16
            assert re.search(r"\bv_sqrt_f32", body), name
            assert re.search(r"0x4f800000", body) and re.search(r"0x37800000", body), name
            assert not re.search(r"\bv_rsq_f32", body), name
            continue
        assert re.search(r"\bv_(sqrt|rsq)_f32", body), name
        assert re.search(r"\bv_fma(_mix)?_f32\b.*-v", body), name


def test_scalar_maps_compute_in_binary32(asm):
    ks = {k: v[0] for k, v in _kernels(asm).items() if "FnScale" in k or "FnAddScalar" in k}
    assert len(ks) == 2 * 3 * (4 * 2 + 3 + 3)
    for name, body in ks.items():
        op = "v_mul_f32" if "FnScale" in name else "v_add_f32"
        assert re.search(r"\b" + op, body), name
