"""HIP path against the CPU oracle through the C ABI, element by element.

* brute force: every n in 0..17 plus ragged sizes, every pointer offset class,
  every op; inputs mix special values (NaN, +-inf, +-0, subnormals, extremes)
  with random bit patterns and the config distributions; every output region
  sits in one arena whose untouched bytes must keep their sentinel (guard
  bands catch any out-of-bounds head / tail / body write);
* every kernel instantiation: each op under block sizes 64..1024, unroll
  1..8 and co-aligned / misaligned inputs, at a size spanning several tiles
  with a ragged tail;
* exact aliasing where the ABI allows it.
"""
import functools
import math
import os

import numpy as np
import pytest
import torch

import memory_bound_elementwise_amd as ew
import oracle
import synth
from tests.gpu_util import DEV, ELEM, NP_DTYPE, download, mismatches, upload

pytestmark = pytest.mark.gpu

GUARD = 64
SENTINEL = 0xA5
SIZES = list(range(0, 18)) + [31, 32, 33, 63, 64, 65, 127, 129, 1000, 4099]

SPECIAL_F32 = np.array(
    [0.0, -0.0, 1.0, -1.0, np.inf, -np.inf, np.nan, -np.nan, 1e-45, -1e-45, 1e-40, -3e-39,
     1.1754944e-38, -1.1754942e-38, 3.4028235e38, -3.4028235e38, 0.5, 2.5, -2.5, 65504.0,
     1e30, -1e-30, 16777217.0, 0.1],
    dtype=np.float32)


@functools.lru_cache(maxsize=8)
def _f32_pool(length, seed):
    """Thirds of uniform[-1,1), normal(0,1) and random bit patterns (every
    class: NaN, inf, subnormal, zero), interleaved, with the special values
    written at random positions and at the very start."""
    g = synth.rng(seed)
    pool = np.empty(length, np.float32)
    pool[0::3] = synth.uniform_pm1(g, len(pool[0::3]))
    pool[1::3] = synth.normal01(g, len(pool[1::3]))
    pool[2::3] = g.integers(0, 1 << 32, size=len(pool[2::3]), dtype=np.uint32).view(np.float32)
    k = min(length, SPECIAL_F32.size)
    pool[:k] = SPECIAL_F32[:k]
    pos = g.integers(0, length, size=max(length // 64, 1))
    pool[pos] = SPECIAL_F32[np.arange(pos.size) % SPECIAL_F32.size]
    pool.setflags(write=False)
    return pool


U16_SPECIAL = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x03FF, 0x0400, 0x3C00, 0x7BFF,
                        0x7C00, 0xFC00, 0x7E00, 0x7C01, 0x7F80, 0xFF80, 0x7FC0, 0x7F81,
                        0x0080, 0x007F, 0x3F80, 0xBF80], dtype=np.uint16)


@functools.lru_cache(maxsize=8)
def _u16_pool(length, seed):
    """Random 16-bit patterns (every binary16 / bfloat16 class) with the
    special patterns at the start and at random positions."""
    g = synth.rng(seed)
    pool = g.integers(0, 1 << 16, size=length, dtype=np.uint16)
    k = min(length, U16_SPECIAL.size)
    pool[:k] = U16_SPECIAL[:k]
    pos = g.integers(0, length, size=max(length // 64, 1))
    pool[pos] = U16_SPECIAL[np.arange(pos.size) % U16_SPECIAL.size]
    pool.setflags(write=False)
    return pool


# Bit patterns at the in-place ReLU's decision boundary: -0, -inf and the
# most negative finite change; negative NaNs and +0 do not.
RELU_EDGE_BITS = np.array([0x80000000, 0xFF800000, 0xFF800001, 0xFFC00000, 0xFFFFFFFF,
                           0x7F800000, 0x00000000, 0x80000001, 0xFF7FFFFF, 0x7FFFFFFF],
                          dtype=np.uint32)


@functools.lru_cache(maxsize=8)
def _sparse_negative_pool(length, seed):
    """The f32 pool with every sign cleared, then about one element in 40
    negated (so most 64-byte spans hold no element to clear and many hold
    exactly one), with the decision-boundary bit patterns at the start."""
    pool = np.abs(_f32_pool(length, seed))
    g = synth.rng(seed + 17)
    pos = g.integers(0, length, size=max(length // 40, 1))
    pool[pos] = -pool[pos]
    k = min(length, RELU_EDGE_BITS.size)
    pool[:k] = RELU_EDGE_BITS[:k].view(np.float32)
    pool.setflags(write=False)
    return pool


def _pool(op, length, seed):
    if op == "relu_inplace_f32":
        return _sparse_negative_pool(length, seed)
    return _u16_pool(length, seed) if ELEM[op] == 2 else _f32_pool(length, seed)


SCALAR_MAPS = tuple(f"{m}_{d}" for m in ew.SCALAR_MAPS for d in ew.MAP_DTYPES)
UNARY_MAPS = tuple(f"{m}_{d}" for m in ew.UNARY_MAPS for d in ew.MAP_DTYPES)


def _oracle(op, ins, n, alpha=2.5, stride=2):
    if op in SCALAR_MAPS:
        return getattr(oracle, op)(alpha, ins[0])
    if op in UNARY_MAPS:
        return getattr(oracle, op)(ins[0])
    if op in ("add_f32", "add_f16", "add_bf16", "add_relu_f32"):
        return getattr(oracle, op)(ins[0], ins[1])
    if op in ("saxpy_f32", "saxpy_relu_f32", "saxpy_f16", "saxpy_bf16"):
        return getattr(oracle, op)(alpha, ins[0], ins[1])
    if op in ("relu_f32", "relu_f16", "relu_bf16"):
        return getattr(oracle, op)(ins[0])
    if op == "relu_inplace_f32":
        return oracle.relu_f32(ins[0])
    if op == "copy_f32":
        return oracle.copy_f32(ins[0])
    return oracle.gather_f32(ins[0], stride)


def _call(op, out_ptr, in_ptrs, n, alpha=2.5, stride=2):
    s = torch.cuda.current_stream().cuda_stream
    if op in SCALAR_MAPS:
        getattr(ew, "ew_" + op)(alpha, in_ptrs[0], out_ptr, n=n, stream=s)
    elif op in UNARY_MAPS:
        getattr(ew, "ew_" + op)(in_ptrs[0], out_ptr, n=n, stream=s)
    elif op in ("add_f32", "add_f16", "add_bf16", "add_relu_f32"):
        getattr(ew, "ew_" + op)(in_ptrs[0], in_ptrs[1], out_ptr, n=n, stream=s)
    elif op in ("saxpy_f32", "saxpy_relu_f32", "saxpy_f16", "saxpy_bf16"):
        getattr(ew, "ew_" + op)(alpha, in_ptrs[0], out_ptr, n=n, stream=s)
    elif op in ("relu_f32", "relu_f16", "relu_bf16"):
        getattr(ew, "ew_" + op)(in_ptrs[0], out_ptr, n=n, stream=s)
    elif op == "relu_inplace_f32":
        ew.ew_relu_inplace_f32(out_ptr, n=n, stream=s)
    elif op == "copy_f32":
        ew.ew_copy_f32(in_ptrs[0], out_ptr, n=n, stream=s)
    elif op == "gather_walk_f32":
        ew.ew_gather_walk_f32(in_ptrs[0], out_ptr, stride, n=n, stream=s)
    else:
        ew.ew_gather_f32(in_ptrs[0], out_ptr, stride, n=n, stream=s)


def _run_cases(op, cases, seed, alpha=2.5):
    """cases: list of (n, off_out, [off_in...], stride).  All outputs live in
    one sentinel-filled arena; returns a list of failure descriptions."""
    es = ELEM[op]
    dt = NP_DTYPE[es]
    n_in = 1 if op in ONE_INPUT else 2
    max_n = max(c[0] for c in cases)
    pool_len = max_n + 32
    pools = [_pool(op, pool_len, seed + k) for k in range(n_in)]
    dev_pools = [upload(p)[1] for p in pools]          # base tensors, offset 0
    for d in dev_pools:
        assert d.data_ptr() % 256 == 0

    layout, cursor = [], 0
    for (n, off_out, offs_in, stride) in cases:
        start = -(-(cursor + GUARD) // 256) * 256
        out_byte = start + off_out * es
        layout.append(out_byte)
        cursor = out_byte + n * es + GUARD
    total = -(-(cursor + 256) // 256) * 256
    host = np.full(total, SENTINEL, np.uint8)
    if op in IN_PLACE:   # y is updated in place: seed each output span with y
        for (n, off_out, offs_in, stride), ob in zip(cases, layout):
            host[ob:ob + n * es] = pools[1][offs_in[1]:offs_in[1] + n].view(np.uint8)
    if op == "relu_inplace_f32":   # x is the output span itself
        for (n, off_out, offs_in, stride), ob in zip(cases, layout):
            host[ob:ob + n * es] = pools[0][offs_in[0]:offs_in[0] + n].view(np.uint8)
    arena = torch.from_numpy(host).to(DEV)
    base = arena.data_ptr()
    assert base % 256 == 0

    for (n, off_out, offs_in, stride), ob in zip(cases, layout):
        assert ob + n * es <= total
        in_ptrs = []
        for k in range(n_in):
            assert offs_in[k] + n <= pool_len
            in_ptrs.append(dev_pools[k].data_ptr() + offs_in[k] * es)
        _call(op, base + ob, in_ptrs, n, alpha=alpha, stride=stride)
    torch.cuda.synchronize()
    res = arena.cpu().numpy()

    failures = []
    written = np.zeros(total, bool)
    for (n, off_out, offs_in, stride), ob in zip(cases, layout):
        written[ob:ob + n * es] = True
        got = res[ob:ob + n * es].view(dt)
        ins = [pools[k][offs_in[k]:offs_in[k] + n] for k in range(n_in)]
        ref = _oracle(op, ins, n, alpha=alpha, stride=stride)
        bad = mismatches(op, got, ref)
        if bad.size:
            failures.append(f"{op} n={n} off_out={off_out} offs_in={offs_in} stride={stride}: "
                            f"{bad.size} mismatches, first at {bad[0]}")
    outside = res[~written]
    if np.any(outside != SENTINEL):
        failures.append(f"{op}: {np.count_nonzero(outside != SENTINEL)} bytes written outside "
                        "the output ranges (guard band)")
    return failures


IN_PLACE = ("saxpy_f32", "saxpy_relu_f32", "saxpy_f16", "saxpy_bf16")
ONE_INPUT = ("relu_f32", "copy_f32", "gather_f32", "gather_walk_f32", "relu_f16", "relu_bf16",
             "relu_inplace_f32") + SCALAR_MAPS + UNARY_MAPS
TWO_INPUT = ("add_f32", "add_f16", "add_bf16", "add_relu_f32") + IN_PLACE


def _offset_cases(op):
    es = ELEM[op]
    vec = 16 // es
    cases = []
    for n in SIZES:
        if op in TWO_INPUT:
            offs_b = range(vec) if es == 4 else (0, 3, 7)
            for oo in range(vec):
                for oa in range(vec):
                    for ob in offs_b:
                        if op in IN_PLACE:
                            ob = oo          # y is the output itself
                        cases.append((n, oo, [oa, ob], 0))
        elif op == "relu_inplace_f32":
            for oo in range(32):        # every head length of the 64-byte alignment, twice
                cases.append((n, oo, [(5 * oo) % 29], 2))
        else:
            for oo in range(vec):
                for oa in range(vec):
                    cases.append((n, oo, [oa], 2))
    # saxpy produced duplicates (ob forced to oo); drop them
    seen, uniq = set(), []
    for c in cases:
        key = (c[0], c[1], tuple(c[2]), c[3])
        if key not in seen:
            seen.add(key)
            uniq.append(c)
    return uniq


ALL_STREAM_OPS = ["add_f32", "add_f16", "add_bf16", "saxpy_f32", "relu_f32", "copy_f32",
                  "gather_f32", "gather_walk_f32", "add_relu_f32", "saxpy_relu_f32", "saxpy_f16", "saxpy_bf16",
                  "relu_f16", "relu_bf16", "relu_inplace_f32"] + list(SCALAR_MAPS + UNARY_MAPS)


@pytest.mark.parametrize("alpha", [np.float32(1.0) / np.float32(3.0), -7.5e-39, np.inf, np.nan,
                                   -0.0, 3e38])
def test_scalar_maps_other_alphas(alpha):
    """The scalar-broadcast maps with an inexact alpha, a subnormal one, inf,
    NaN, -0 and one that overflows most products, over ragged sizes and
    offsets (the brute-force test covers alpha = 2.5)."""
    print(f"[parity] scalar maps alpha={alpha}", flush=True)
    for op in SCALAR_MAPS:
        vec = 16 // ELEM[op]
        cases = [(n, oo, [(oo + k) % vec], 0) for n in (1, 7, 33, 1000, 4099, 65537)
                 for k, oo in enumerate(range(vec))]
        failures = _run_cases(op, cases, seed=305, alpha=float(np.float32(alpha)))
        assert not failures, failures[:5]


@pytest.mark.parametrize("op", ALL_STREAM_OPS)
def test_brute_force_small_all_offsets(op):
    print(f"[parity] brute force {op}", flush=True)
    failures = _run_cases(op, _offset_cases(op), seed=300)
    assert not failures, failures[:10]


@pytest.mark.parametrize("op", ["gather_f32", "gather_walk_f32"])
def test_gather_brute_force_strides(op):
    """Both gathers (the library's, with its segment / pass / contiguous-span
    plans, and the per-output index walk) on every small n with strides up
    to 2^64 - 1, and the plans' boundary cases."""
    print(f"[parity] gather strides {op}", flush=True)
    cases = []
    for n in range(1, 18):
        for stride in sorted({1, 2, 3, max(n - 1, 1), n, n + 1, 2 * n + 5, (1 << 63) + 5,
                              (1 << 64) - 1}):
            for oo in range(4):
                cases.append((n, oo, [(oo + 1) % 4], stride))
    for n in (1000, 4099, 65537):
        for stride in (1, 2, 3, 7, n - 1, n + 1, 1 << 40):
            cases.append((n, 1, [2], stride))
    # replicated-segment plans (gcd(stride, n) in 2..8) and their neighbours
    for n, stride in (((1 << 20), 2), ((1 << 20) + 4, 2), (3 << 18, 6), ((1 << 20), 8),
                      ((1 << 20), 4), (3 << 18, 3), (5 * 4096, 5), ((1 << 20) + 1, 2),
                      ((1 << 20), (1 << 20) + 2)):
        for oo in (0, 1, 3):
            cases.append((n, oo, [0], stride))
    failures = _run_cases(op, cases, seed=310)
    assert not failures, failures[:10]


def test_gather_pass_decomposition_small_strides():
    """Strides 2..32 take the pass-decomposed kernel, with g = gcd(s, n) equal
    segments of s/g runs (stride 2 on n/2 a multiple of 4 aside, which takes
    the contiguous-span kernel): every such stride at every n up to 80 and at
    ragged and highly composite larger n, with aligned and misaligned input
    and output."""
    print("[parity] gather passes", flush=True)
    cases = []
    for n in list(range(3, 81)) + [1000, 4099, 65537, (1 << 20) + 1, 3 * 5 * 7 * 4096 + 1,
                                   (1 << 20), 720720, 3 * (1 << 18) + 24]:
        for s in range(2, 33):
            if s >= n:
                continue
            for oo, oi in ((0, 0), (1, 0), (0, 3), (3, 2)):
                cases.append((n, oo, [oi], s))
    failures = _run_cases("gather_f32", cases, seed=315)
    assert not failures, failures[:10]


def _tile_cases():
    """(n, stride) pairs on the tiled transposition: whole-row tiles
    (33..67), 128 x 128 and 256 x 64 ones (partial column bands), g = gcd
    1..31, exactly 128 rows, ragged last rows and bands."""
    cus = 256
    pairs = []
    for n in (4225, 20011, 100003, 1 << 20, (1 << 20) + 5, 3 << 18, 720720 + 1):
        for s in (33, 34, 36, 37, 40, 44, 48, 52, 63, 64, 65, 67, 68, 97, 100, 126, 127):
            pairs.append((n, s))
    for n in ((1 << 20), (1 << 20) + 1, 1000003, 3 * 5 * 7 * 4096 + 1, 4 << 20):
        for s in (129, 130, 135, 136, 200, 255, 259, 1000, 1281, 4097, 8191):
            pairs.append((n, s))
    pairs += [(16511, 129), (33 * 127 + 1, 33), (128 * 1000 + 3, 1000), (31 * 4099, 62),
              (1 << 20, 80), ((1 << 20) + 48, 176)]
    # more than one window of 128 tiles dealt to the XCDs in runs of 16
    # (whole rows, and a single row band of wide tiles)
    pairs += [(2200000, 35), (4 << 20, 33), (4 << 20, 60), (128 * 16385 - 3, 16385)]
    out = []
    for n, s in pairs:
        p = ew.ew_make_gather_plan(1 << 40, 1 << 42, n, s, cus)
        if ew.PATHS[p.path] == "gather_tiles":
            out.append((n, s))
    return out


def test_gather_tiled_transposition_large_strides():
    """Strides above 32 (with g = gcd(s, n) < 32 and at least 128 rows of s
    elements) take the tiled transposition: narrow and wide tiles, every g
    from 1 to 31 that the sizes produce, with aligned and misaligned input
    and output."""
    print("[parity] gather tiles", flush=True)
    pairs = _tile_cases()
    assert len(pairs) > 80
    assert {math.gcd(n, s) for n, s in pairs} >= {1, 2, 4, 8, 16, 31}
    # all four tile shapes: whole rows (s < 68; one word apart in LDS when
    # s is a multiple of 4), 128 x 128 (fewer than 1024 rows of s elements)
    # and 256 x 64
    modes = {(4 if s % 4 == 0 else 1) if s < 68 else 2 if -(-n // s) < 1024 else 3
             for n, s in pairs}
    assert modes == {1, 2, 3, 4}
    cases = []
    for k, (n, s) in enumerate(pairs):
        oo, oi = ((0, 0), (1, 0), (0, 3), (3, 2))[k % 4]
        cases.append((n, oo, [oi], s))
    failures = _run_cases("gather_f32", cases, seed=345)
    assert not failures, failures[:10]


def test_gather_walk_long_replicated_segments():
    """Strides sharing a factor of 32 or more with n take the per-output walk
    over one segment stored g times once the segment holds at least 2^14
    elements (below that, the walk over all n)."""
    print("[parity] gather replicated walk", flush=True)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    cases = []
    for n, s, reps in ((1 << 20, 64, 64), (1 << 21, 128, 128), (3 << 20, 96, 96),
                       (5 << 20, 320, 320), (1 << 20, 16 * 1025, 16),
                       (1 << 20, 128, 1), (1 << 20, 1 << 16, 1)):
        p = ew.ew_make_gather_plan(1 << 40, 1 << 42, n, s, cus)
        assert ew.PATHS[p.path] == "gather_walk" and p.reps == reps, (n, s, p.reps)
        cases += [(n, 0, [0], s), (n, 1, [3], s)]
    failures = _run_cases("gather_f32", cases, seed=355)
    assert not failures, failures[:10]


def test_gather_tiled_transposition_launch_variants():
    """The tiled transposition with its grid capped below the tile count (the
    launch table's blocks per CU), so that blocks stride over several tiles
    and reuse their LDS tile and run starts: whole-row tiles (s = 33, 34),
    256 x 64 (s = 200) and 128 x 128 (s = 16385, fewer than 1024 rows).
    Between them they take each tile order: XCD runs of 16 tiles over many
    windows (whole rows; s = 16385 with 6 and 9 row bands) and two adjacent
    row bands per XCD in full groups (s = 200, 246 and 738 row bands)."""
    print("[parity] gather tiles variants", flush=True)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    try:
        for bpc in (1, 3):
            _force_launch("gather_f32", 128, bpc, 1)
            cases = []
            for n, s in ((cus * bpc * 3 * 16384 + 11, 33), (cus * bpc * 3 * 16384 + 7, 200),
                         (cus * bpc * 3 * 16384 + 4, 34), (cus * bpc * 3 * 16384 + 1, 16385)):
                p = ew.ew_make_gather_plan(1 << 40, 1 << 42, n, s, cus)
                assert ew.PATHS[p.path] == "gather_tiles" and p.tiles > 2 * p.grid, \
                    (n, s, p.tiles, p.grid)
                cases += [(n, 1, [2], s), (n, 0, [0], s)]
            failures = _run_cases("gather_f32", cases, seed=350)
            assert not failures, (bpc, failures[:5])
    finally:
        ew.ew_reset_launch_config()
        if os.path.exists(ew.LAUNCH_TABLE):
            ew.ew_load_launch_table(ew.LAUNCH_TABLE)


def test_gather_pass_decomposition_launch_variants():
    """The pass-decomposed gather under forced grid caps (its block shape is
    fixed), at sizes where the grid-stride loop runs three rounds and the
    last tile is partial."""
    print("[parity] gather passes variants", flush=True)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    try:
        for (block, bpc, unroll) in LAUNCHES:
            _force_launch("gather_f32", block, bpc, unroll)
            cases = []
            if bpc > 8:
                continue      # the kernel's block shape is fixed: only the grid cap varies
            for s, gcd in ((3, 1), (8, 1), (29, 1), (6, 2), (24, 8), (12, 12)):
                # one group (four outputs per pass) per thread of the fixed block
                threads = ew.ew_make_gather_plan(1 << 40, 1 << 42, 1000003, s, cus).block
                n = (2 * bpc * cus + 1) * threads * 4 * s - 7
                while math.gcd(n, s) != gcd:
                    n += 1
                p = ew.ew_make_gather_plan(1 << 40, 1 << 42, n, s, cus)
                assert (p.passes, p.reps) == (s // gcd, gcd) and p.tiles > 2 * p.grid, \
                    (s, p.tiles, p.grid)
                cases += [(n, 1, [2], s), (n, 0, [0], s)]
            failures = _run_cases("gather_f32", cases, seed=330)
            assert not failures, (block, bpc, unroll, failures[:5])
    finally:
        ew.ew_reset_launch_config()
        if os.path.exists(ew.LAUNCH_TABLE):
            ew.ew_load_launch_table(ew.LAUNCH_TABLE)


def _table_min_ns(op):
    """Every size-class boundary of op in the default and the loaded table."""
    mins = {0, 1 << 22}
    if os.path.exists(ew.LAUNCH_TABLE):
        for line in open(ew.LAUNCH_TABLE):
            f = line.split("#")[0].split()
            if len(f) == 5 and f[0] == op:
                mins.add(int(f[1]))
    return sorted(mins)


def _force_launch(op, block, bpc, unroll):
    for m in _table_min_ns(op):
        ew.ew_set_launch_row(op, m, block, bpc, unroll)


LAUNCHES = [(64, 1, 1), (64, 3, 8), (256, 8, 1), (256, 8, 2), (256, 2, 4), (512, 2, 4),
            (1024, 1, 2), (1024, 1, 8), (128, 16, 1)]


@pytest.mark.parametrize("op", ALL_STREAM_OPS)
def test_every_kernel_variant_several_tiles_ragged(op):
    """Each (block, unroll) and alignment variant, at a size of a few tiles
    plus a ragged tail, with a grid smaller than the tile count so the
    grid-stride loop runs several rounds."""
    print(f"[parity] kernel variants {op}", flush=True)
    es = ELEM[op]
    vec = 16 // es
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    try:
        for (block, bpc, unroll) in LAUNCHES:
            _force_launch(op, block, bpc, unroll)
            # 2 * grid + 1 tiles: the grid-stride loop runs three rounds and
            # the last tile is partial
            n = (2 * bpc * cus + 1) * block * unroll * vec - 3 * vec + 13
            plan = ew.ew_make_plan(op, 1 << 40, 1 << 41, (1 << 42) if op in (
                "add_f32", "add_f16", "add_bf16", "add_relu_f32") else (
                1 << 40 if op in IN_PLACE else 0), n, cus)
            assert plan.tiles > 2 * plan.grid, (plan.tiles, plan.grid)
            if op == "relu_inplace_f32":
                offs = [(0, [0]), (1, [1]), (17, [3]), (31, [2])]
            elif op not in TWO_INPUT:
                offs = [(1, [1]), (1, [0]), (0, [3])]
            elif op in IN_PLACE:
                offs = [(1, [2, 1]), (0, [0, 0]), (3, [1, 3])]
            else:
                offs = [(1, [1, 1]), (1, [0, 1]), (1, [1, 2]), (0, [3, 5 % vec])]
            cases = [(n, oo, oi, 2) for (oo, oi) in offs]
            if op == "gather_f32":
                # stride 2 with two equal segments: the contiguous-load kernel
                m = (2 * bpc * cus + 1) * block * unroll * 4
                gp = ew.ew_make_gather_plan(1 << 40, 1 << 41, 2 * m, 2, cus)
                assert gp.reps == 2 and gp.tiles > 2 * gp.grid, (gp.reps, gp.tiles, gp.grid)
                cases += [(2 * m, 1, [1], 2), (2 * m, 0, [3], 2), (2 * m, 2, [0], 2)]
            failures = _run_cases(op, cases, seed=320)
            assert not failures, (block, bpc, unroll, failures[:5])
    finally:
        ew.ew_reset_launch_config()
        if os.path.exists(ew.LAUNCH_TABLE):
            ew.ew_load_launch_table(ew.LAUNCH_TABLE)


def _bias_case(rows, cols, off_x, off_y, off_b, seed, in_place=False):
    """One bias+ReLU launch with guard bands around y; returns failures."""
    n = rows * cols
    x = _f32_pool(n + 8, seed)[:n]
    bias = _f32_pool(cols + 8, seed + 1)[:cols]
    tx, _kx = upload(x, off_x)
    tb, _kb = upload(bias, off_b)
    if in_place:
        ty = tx
    else:
        base = torch.full((n + off_y + 32,), -7.0, device=DEV)
        ty = base[off_y:off_y + n]
    ew.ew_bias_relu_f32(tx, tb, ty, rows, cols)
    torch.cuda.synchronize()
    got = download(ty, 4)
    ref = oracle.bias_relu_f32(x, bias, rows, cols)
    bad = mismatches("bias_relu_f32", got, ref)
    out = [f"rows={rows} cols={cols} offs=({off_x},{off_y},{off_b}): {bad.size} mismatches"] \
        if bad.size else []
    if not in_place:
        guard = base.cpu().numpy()
        if np.any(guard[:off_y] != -7.0) or np.any(guard[off_y + n:] != -7.0):
            out.append(f"rows={rows} cols={cols}: guard band written")
    return out


def test_bias_relu_shapes_and_offsets():
    print("[parity] bias_relu", flush=True)
    failures = []
    shapes = [(1, 1), (1, 3), (2, 5), (3, 7), (5, 4), (4, 16), (7, 33), (1, 1000), (1000, 1),
              (33, 127), (64, 129), (129, 64), (256, 1024), (3, 100003)]
    for k, (rows, cols) in enumerate(shapes):
        for off_x, off_y, off_b in ((0, 0, 0), (1, 0, 3), (0, 3, 1), (2, 1, 0), (3, 3, 2)):
            failures += _bias_case(rows, cols, off_x, off_y, off_b, 340 + k)
    failures += _bias_case(64, 129, 1, 1, 0, 360, in_place=True)
    assert not failures, failures[:10]


def test_bias_relu_every_kernel_variant():
    print("[parity] bias_relu variants", flush=True)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    try:
        for (block, bpc, unroll) in LAUNCHES:
            _force_launch("bias_relu_f32", block, bpc, unroll)
            vecs = (2 * bpc * cus + 1) * block * unroll
            for cols in (4096, 3):
                rows = -(-4 * vecs // cols) + 1
                failures = _bias_case(rows, cols, 1, 0, 1, 370) + \
                    _bias_case(rows, cols, 0, 0, 0, 371)
                assert not failures, (block, bpc, unroll, cols, failures[:3])
    finally:
        ew.ew_reset_launch_config()
        if os.path.exists(ew.LAUNCH_TABLE):
            ew.ew_load_launch_table(ew.LAUNCH_TABLE)


def _copy2d_case(rows, cols, sr, sc, seed, off_out=0):
    """One strided-view copy with guard bands around the output; the view
    starts inside a base buffer so that every touched element exists."""
    lo = min(0, (rows - 1) * sr) + min(0, (cols - 1) * sc)
    hi = max(0, (rows - 1) * sr) + max(0, (cols - 1) * sc)
    offset = -lo + 3
    base_len = offset + hi + 8
    base = _f32_pool(base_len, seed)
    tb, _kb = upload(base)
    n = rows * cols
    obuf = torch.full((n + off_out + 32,), -5.0, device=DEV)
    out = obuf[off_out:off_out + n]
    ew.ew_copy2d_f32(tb.data_ptr() + 4 * offset, sr, sc, out.data_ptr(), rows, cols)
    torch.cuda.synchronize()
    got = download(out, 4)
    ref = oracle.copy2d_f32(base, offset, sr, sc, rows, cols)
    bad = mismatches("copy_f32", got, ref)
    fails = [f"copy2d rows={rows} cols={cols} sr={sr} sc={sc} off={off_out}: "
             f"{bad.size} mismatches"] if bad.size else []
    g = obuf.cpu().numpy()
    if np.any(g[:off_out] != -5.0) or np.any(g[off_out + n:] != -5.0):
        fails.append(f"copy2d rows={rows} cols={cols} sr={sr} sc={sc}: guard band written")
    return fails


def test_copy2d_paths_shapes_and_strides():
    print("[parity] copy2d", flush=True)
    failures = []
    k = 0
    for rows, cols in ((1, 1), (1, 7), (3, 5), (64, 64), (65, 63), (1, 1000), (130, 129),
                       (200, 7), (7, 300), (513, 257), (128, 128), (127, 129), (256, 385)):
        for sr, sc in ((cols, 1), (cols + 5, 1), (1, rows), (1, rows + 3), (1, -rows),
                       (-cols, 1), (2 * cols, 2), (3, 7 * rows), (0, 1), (cols, 0), (1, 1),
                       (1, 0), (1, 2 * rows), (-1, rows), (1, -2 * rows)):
            for off_out in (0, 1):
                k += 1
                failures += _copy2d_case(rows, cols, sr, sc, 400 + k, off_out)
    # 1-D stride-2 views (x[::2]): every length up to 40 and every output
    # alignment, so the head, the shortened body and the 1-4 element tail
    # all occur
    for cols in range(1, 41):
        for off_out in range(4):
            k += 1
            failures += _copy2d_case(1, cols, 0, 2, 400 + k, off_out)
    # 1-D views x[::s], s = 3..32 (one element kept per s of a contiguously
    # read span): short and ragged lengths, every output alignment
    for sc in range(3, 33):
        for cols in list(range(1, 21)) + [255, 256, 257, 1000, 4099]:
            for off_out in (0, 1, 3):
                k += 1
                failures += _copy2d_case(1, cols, 0, sc, 400 + k, off_out)
    assert not failures, failures[:10]


def test_copy2d_large_tiles_and_variants():
    """Several grid-stride rounds for the output-ordered kernel and for the
    transpose, and edge tiles for the transpose, at moderate sizes."""
    print("[parity] copy2d variants", flush=True)
    failures = []
    failures += _copy2d_case(2050, 3001, 1, 2050, 450)          # transpose, ragged tiles
    failures += _copy2d_case(3001, 2050, 1, 3001 + 64, 451, 1)  # transpose of a padded matrix
    failures += _copy2d_case(1, 1 << 22, 0, 2, 452, 1)          # x[::2]
    failures += _copy2d_case(1, (1 << 21) + 5, 0, 3, 455, 2)    # x[::3], many tiles
    failures += _copy2d_case(1, (1 << 20) + 3, 0, 8, 456)       # x[::8]
    failures += _copy2d_case(1, (1 << 20) + 7, 0, 13, 457, 1)   # x[::13]
    failures += _copy2d_case(1, (1 << 19) + 1, 0, 16, 458)      # x[::16]
    failures += _copy2d_case(1, (1 << 18) + 9, 0, 32, 459, 2)   # x[::32]
    failures += _copy2d_case(1500, 1999, 2111, 1, 453, 3)       # submatrix, misaligned rows
    failures += _copy2d_case(999, 1001, -1001, 1, 454)          # rows in reverse order
    try:
        for (block, bpc, unroll) in LAUNCHES:
            _force_launch("copy2d_f32", block, bpc, unroll)
            failures += _copy2d_case(333, 4097, 4099, 1, 460 + unroll, 1)
            failures += _copy2d_case(2, 3 * 4096 + 5, 5 * 4096, 3, 470 + unroll)
            # transpose: 17 x 24 tiles of 128, more than one block per CU's
            # worth when blocks_per_cu is 1, so blocks stride over tiles
            failures += _copy2d_case(2050, 3001, 1, 2050, 480 + unroll, 1)
    finally:
        ew.ew_reset_launch_config()
        if os.path.exists(ew.LAUNCH_TABLE):
            ew.ew_load_launch_table(ew.LAUNCH_TABLE)
    assert not failures, failures[:10]


def test_exact_aliasing_in_place():
    print("[parity] aliasing", flush=True)
    n = 100003
    s = torch.cuda.current_stream().cuda_stream
    g = synth.rng(330)
    a = _f32_pool(n, 331)
    b = synth.uniform_pm1(g, n)
    # c == a
    ta, _ka = upload(a, 1)
    tb, _kb = upload(b, 0)
    ew.ew_add_f32(ta, tb, ta, stream=s)
    torch.cuda.synchronize()
    assert mismatches("add_f32", download(ta, 4), oracle.add_f32(a, b)).size == 0
    # c == b, 16-bit
    a16 = _u16_pool(n, 332)
    b16 = _u16_pool(n, 333)
    ta, _ka = upload(a16, 3)
    tb, _kb = upload(b16, 5)
    ew.ew_add_bf16(ta, tb, tb, stream=s)
    torch.cuda.synchronize()
    assert mismatches("add_bf16", download(tb, 2), oracle.add_bf16(a16, b16)).size == 0
    # relu in place
    x = _f32_pool(n, 334)
    tx, _kx = upload(x, 2)
    ew.ew_relu_f32(tx, tx, stream=s)
    torch.cuda.synchronize()
    assert mismatches("relu_f32", download(tx, 4), oracle.relu_f32(x)).size == 0
    # saxpy with x == y: y = fma(alpha, y, y)
    y = synth.normal01(g, n)
    ty, _ky = upload(y, 1)
    ew.ew_saxpy_f32(2.5, ty, ty, stream=s)
    torch.cuda.synchronize()
    assert mismatches("saxpy_f32", download(ty, 4), oracle.saxpy_f32(2.5, y, y)).size == 0
    # the maps in place, y == x
    for op, pool, es in (("sqrt_f32", x, 4), ("scale_bf16", a16, 2), ("add_scalar_f16", b16, 2),
                         ("abs_f32", x, 4)):
        tm, _km = upload(pool, 1)
        args = (2.5, tm, tm) if op in SCALAR_MAPS else (tm, tm)
        getattr(ew, "ew_" + op)(*args, stream=s)
        torch.cuda.synchronize()
        ref = _oracle(op, [pool], n)
        assert mismatches(op, download(tm, es), ref).size == 0, op
    # copy onto itself leaves the data unchanged
    tz, _kz = upload(x, 0)
    ew.ew_copy_f32(tz, tz, stream=s)
    torch.cuda.synchronize()
    assert np.array_equal(download(tz, 4).view(np.uint32), x.view(np.uint32))


def test_one_hip_runtime_in_the_process():
    """libew and torch must share one HIP runtime (streams and pointers from
    torch are only valid inside the runtime that created them)."""
    with open("/proc/self/maps") as f:
        paths = {line.split()[-1] for line in f if "libamdhip64" in line}
    assert len(paths) == 1, paths


def test_errors_surface_as_exceptions_on_device():
    t = torch.zeros(1024, device=DEV)
    with pytest.raises(ew.EwError) as e:
        ew.ew_add_f32(t[1:], t, t[:-1])
    assert e.value.status == -3
    with pytest.raises(ew.EwError):
        ew.ew_gather_f32(t, t, 2)


def test_non_default_stream_orders_with_the_stream():
    """Work on a user stream is ordered after earlier work on that stream."""
    n = 1 << 22
    s = torch.cuda.Stream()
    x = torch.arange(n, dtype=torch.float32, device=DEV)
    y = torch.empty_like(x)
    z = torch.empty_like(x)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        ew.ew_copy_f32(x, y)            # defaults to the current (user) stream
        ew.ew_relu_f32(y, z)
    s.synchronize()
    assert torch.equal(z, x)


def test_launch_log_names_each_plan():
    """EW_LOG=1 prints one line per launch with the plan and the chosen path
    (a child process: the setting is read once per process)."""
    import subprocess
    import sys
    code = (
        "import torch, memory_bound_elementwise_amd as ew\n"
        "a = torch.zeros(1003, device='cuda'); b = torch.zeros(1003, device='cuda')\n"
        "c = torch.zeros(1003, device='cuda')\n"
        "ew.ew_add_f32(a[1:], b[1:], c[1:])\n"
        "ew.ew_gather_f32(a, c, 3)\n"
        "ew.ew_copy2d_f32(a, 1, 17, c, 17, 59)\n"
        "torch.cuda.synchronize()\n")
    env = dict(os.environ, EW_LOG="1")
    r = subprocess.run([sys.executable, "-c", code], cwd=os.path.dirname(os.path.dirname(
        os.path.abspath(__file__))), env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    lines = [ln for ln in r.stderr.splitlines() if ln.startswith("[ew] ")]
    assert len(lines) == 3, r.stderr[-2000:]
    assert lines[0].startswith("[ew] add_f32 n=1002 ") and "path=stream" in lines[0]
    assert lines[1].startswith("[ew] gather_f32 n=1003 ") and "path=passes" in lines[1]
    assert lines[2].startswith("[ew] copy2d_f32 n=1003 ") and "path=transpose tiles" in lines[2]


def test_binding_checks_gpu_tensors_before_the_call():
    """GPU tensors of the right width and length pass; a shorter input, a
    wrong width or a non-contiguous view is refused before any launch, and
    the output is left untouched."""
    x = torch.randn(1000, device=DEV)
    y = torch.full((1000,), 7.0, device=DEV)
    with pytest.raises(ValueError, match="999 elements"):
        ew.ew_relu_f32(x[:999], y)
    with pytest.raises(TypeError):
        ew.ew_scale_f16(2.0, x, y)
    with pytest.raises(ValueError, match="not contiguous"):
        ew.ew_abs_f32(x[::2], y[:500])
    torch.cuda.synchronize()
    assert bool((y == 7.0).all())
    ew.ew_relu_f32(x, y)
    torch.cuda.synchronize()
    assert torch.equal(y, torch.clamp(x, min=0.0))
