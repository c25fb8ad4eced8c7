"""Maximum sizes: arrays past 2^32 elements.

Element indices, byte offsets and the gather's index products must all be
64-bit (the pages' kernels use 32-bit `int` indices).  Inputs are
deterministic integer patterns generated on the GPU; results are checked two
ways:

* properties that hold at any size, on every element, on the device, chunk
  by chunk (A + (-0) == A bitwise; copy == input; the stride-2 gather's two
  halves are equal; no sign bit left after the in-place ReLU);
* sampled elements (first, last, around the 2^31 and 2^32 element
  boundaries, and random positions) against the oracle computed one by one
  on the host.
"""
import numpy as np
import pytest
import torch

import memory_bound_elementwise_amd as ew
import oracle
from tests.gpu_util import DEV, mismatches

pytestmark = pytest.mark.gpu

CHUNK = 1 << 27
GiB = 1 << 30


def _need(nbytes):
    free, _ = torch.cuda.mem_get_info()
    if free < nbytes + 4 * GiB:
        pytest.skip(f"needs {nbytes / GiB:.0f} GiB of free device memory")


def _fill_f32(t, mul, mod, scale):
    """t[i] = ((i * mul) mod mod) * scale, exact in binary32 (mod <= 2^24)."""
    n = t.numel()
    for s in range(0, n, CHUNK):
        e = min(n, s + CHUNK)
        i = torch.arange(s, e, device=DEV, dtype=torch.int64)
        t[s:e] = ((i * mul) % mod).to(torch.float32) * scale


def _fill_bits(t, mul, bits):
    """Integer view of t gets ((i * mul) >> 7) mod 2^bits, as signed ints."""
    n = t.numel()
    for s in range(0, n, CHUNK):
        e = min(n, s + CHUNK)
        i = torch.arange(s, e, device=DEV, dtype=torch.int64)
        v = ((i * mul) >> 7) & ((1 << bits) - 1)
        v = torch.where(v >= (1 << (bits - 1)), v - (1 << bits), v)
        t[s:e] = v.to(t.dtype)


def _samples(n, seed=5):
    g = np.random.Generator(np.random.PCG64(seed))
    edges = [0, 1, 2, 3, n - 4, n - 3, n - 2, n - 1]
    for b in (1 << 31, 1 << 32):
        if b < n:
            edges += list(range(max(0, b - 5), min(n, b + 5)))
    idx = np.concatenate([np.array(edges, np.int64), g.integers(0, n, size=1 << 18)])
    return np.unique(idx)


def _take(t, idx):
    return t[torch.from_numpy(idx).to(DEV)].cpu().numpy()


def _chunked_equal(x, y):
    n = x.numel()
    for s in range(0, n, CHUNK):
        e = min(n, s + CHUNK)
        if not torch.equal(x[s:e], y[s:e]):
            return False
    return True


def test_add_f32_past_2_pow_32_elements():
    n = (1 << 32) + 5
    _need(3 * 4 * n)
    print(f"[large] add_f32 n={n}", flush=True)
    a = torch.empty(n, dtype=torch.float32, device=DEV)
    b = torch.empty(n, dtype=torch.float32, device=DEV)
    c = torch.empty(n, dtype=torch.float32, device=DEV)
    _fill_f32(a, 40503, 65521, 2.0 ** -8)
    b.fill_(-0.0)
    ew.ew_add_f32(a, b, c)
    torch.cuda.synchronize()
    assert _chunked_equal(c.view(torch.int32), a.view(torch.int32))   # A + (-0) == A
    _fill_f32(b, 7919, 1021, 2.0 ** -10)
    ew.ew_add_f32(a, b, c)
    torch.cuda.synchronize()
    idx = _samples(n)
    ref = oracle.add_f32(_take(a, idx), _take(b, idx))
    assert mismatches("add_f32", _take(c, idx), ref).size == 0
    del a, b, c
    torch.cuda.empty_cache()


def test_add_bf16_past_2_pow_32_elements_misaligned():
    n = (1 << 32) + 9
    _need(3 * 2 * (n + 8))
    print(f"[large] add_bf16 n={n}", flush=True)
    abase = torch.empty(n + 8, dtype=torch.int16, device=DEV)
    b = torch.empty(n, dtype=torch.int16, device=DEV)
    cbase = torch.empty(n + 8, dtype=torch.int16, device=DEV)
    a, c = abase[3:3 + n], cbase[1:1 + n]
    _fill_bits(a, 2654435761, 16)
    _fill_bits(b, 40503 * 65537, 16)
    ew.ew_add_bf16(a, b, c)
    torch.cuda.synchronize()
    idx = _samples(n)
    got = _take(c, idx).view(np.uint16)
    ref = oracle.add_bf16(_take(a, idx).view(np.uint16), _take(b, idx).view(np.uint16))
    assert mismatches("add_bf16", got, ref).size == 0
    del abase, b, cbase, a, c
    torch.cuda.empty_cache()


def test_copy_and_saxpy_past_2_pow_32_elements():
    n = (1 << 32) + 7
    _need(2 * 4 * (n + 4))
    print(f"[large] copy / saxpy n={n}", flush=True)
    xbase = torch.empty(n + 4, dtype=torch.float32, device=DEV)
    y = torch.empty(n, dtype=torch.float32, device=DEV)
    x = xbase[1:1 + n]
    _fill_f32(x, 40503, 65521, 2.0 ** -8)
    ew.ew_copy_f32(x, y)
    torch.cuda.synchronize()
    assert _chunked_equal(y.view(torch.int32), x.view(torch.int32))
    _fill_f32(y, 7919, 1021, 2.0 ** -10)
    idx = _samples(n)
    y0 = _take(y, idx)
    ew.ew_saxpy_f32(2.5, x, y)
    torch.cuda.synchronize()
    ref = oracle.saxpy_f32(2.5, _take(x, idx), y0)
    assert mismatches("saxpy_f32", _take(y, idx), ref).size == 0
    del xbase, x, y
    torch.cuda.empty_cache()


def test_gather_wide_index_products():
    """stride = n - 1 with n > 2^32: stride * (n - 1) exceeds 2^64, so each
    lane's first index takes the exact double-and-add path."""
    n = (1 << 32) + 8
    _need(2 * 4 * n)
    print(f"[large] gather stride n-1, n={n}", flush=True)
    src = torch.empty(n, dtype=torch.int32, device=DEV)
    out = torch.empty(n, dtype=torch.int32, device=DEV)
    _fill_bits(src, 2654435761, 32)
    plan = ew.ew_make_gather_plan(out.data_ptr(), src.data_ptr(), n, n - 1,
                                  torch.cuda.get_device_properties(0).multi_processor_count)
    assert plan.reps == 1
    ew.ew_gather_f32(src.data_ptr(), out.data_ptr(), n - 1, n=n)
    torch.cuda.synchronize()
    idx = _samples(n)
    j = np.array([oracle.gather_index(n, n - 1, int(i)) for i in idx], np.int64)
    assert np.array_equal(_take(out, idx), _take(src, j))
    del src, out
    torch.cuda.empty_cache()


def test_gather_stride_2_replicated_segments_past_2_pow_32():
    n = (1 << 33) + 16          # two segments of 2^32 + 8 elements
    _need(2 * 4 * n)
    print(f"[large] gather stride 2, n={n}", flush=True)
    src = torch.empty(n, dtype=torch.int32, device=DEV)
    out = torch.empty(n, dtype=torch.int32, device=DEV)
    _fill_bits(src, 2654435761, 32)
    plan = ew.ew_make_gather_plan(out.data_ptr(), src.data_ptr(), n, 2,
                                  torch.cuda.get_device_properties(0).multi_processor_count)
    assert plan.reps == 2 and plan.segment == n // 2
    ew.ew_gather_f32(src.data_ptr(), out.data_ptr(), 2, n=n)
    torch.cuda.synchronize()
    assert _chunked_equal(out[: n // 2], out[n // 2:])
    idx = _samples(n)
    j = np.array([oracle.gather_index(n, 2, int(i)) for i in idx], np.int64)
    assert np.array_equal(_take(out, idx), _take(src, j))
    del src, out
    torch.cuda.empty_cache()


def test_gather_passes_past_2_pow_32_elements():
    """The pass-decomposed gather with 64-bit slots, runs and segments: stride
    6 on n = 2^32 + 2^20 (gcd 2: two segments of three runs each) and stride
    31 (coprime: 31 runs), sampled against the oracle's index, the two
    segments of stride 6 equal on every element."""
    n = (1 << 32) + (1 << 20)
    _need(2 * 4 * n)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    src = torch.empty(n, dtype=torch.int32, device=DEV)
    out = torch.empty(n, dtype=torch.int32, device=DEV)
    _fill_bits(src, 2654435761, 32)
    for stride, reps, runs in ((6, 2, 3), (31, 1, 31)):
        print(f"[large] gather stride {stride}, n={n}", flush=True)
        plan = ew.ew_make_gather_plan(out.data_ptr(), src.data_ptr(), n, stride, cus)
        assert ew.PATHS[plan.path] == "gather_passes"
        assert (plan.reps, plan.passes, plan.segment) == (reps, runs, n // reps)
        ew.ew_gather_f32(src.data_ptr(), out.data_ptr(), stride, n=n)
        torch.cuda.synchronize()
        if reps == 2:
            assert _chunked_equal(out[: n // 2], out[n // 2:])
        idx = _samples(n)
        j = np.array([oracle.gather_index(n, stride, int(i)) for i in idx], np.int64)
        assert np.array_equal(_take(out, idx), _take(src, j)), stride
    del src, out
    torch.cuda.empty_cache()


def test_relu_inplace_past_2_pow_32_elements_misaligned():
    n = (1 << 32) + 21
    _need(4 * (n + 8))
    print(f"[large] relu_inplace n={n}", flush=True)
    base = torch.empty(n + 8, dtype=torch.float32, device=DEV)
    x = base[5:5 + n]                                   # head of 11 elements to 64 bytes
    _fill_f32(x, 40503, 65521, 2.0 ** -8)               # non-negative ...
    xi = x.view(torch.int32)
    for s in range(0, n, CHUNK):                        # ... then every 7th element negated
        e = min(n, s + CHUNK)
        i = torch.arange(s, e, device=DEV, dtype=torch.int64)
        xi[s:e] = torch.where(i % 7 == 3, xi[s:e] | (-(1 << 31)), xi[s:e])
    idx = _samples(n)
    before = _take(x, idx)
    ew.ew_relu_inplace_f32(x)
    torch.cuda.synchronize()
    assert mismatches("relu_f32", _take(x, idx), oracle.relu_f32(before)).size == 0
    for s in range(0, n, CHUNK):                        # property on every element
        assert not bool(torch.signbit(x[s:min(n, s + CHUNK)]).any())
    del base, x, xi
    torch.cuda.empty_cache()


def test_gather_tiles_past_2_pow_32_elements():
    """The tiled transposition with 64-bit rows, run starts and segments on
    n = 2^32 + 2^20 = 2^20 * 4097: stride 33 (coprime, narrow tiles of whole
    rows), 100 (gcd 4: four segments of 25 runs, narrow), 1000 (gcd 8: eight
    segments of 125 runs, 128 x 128 tiles) and 65537 (coprime, wide),
    sampled against the oracle's index, replicated segments equal on every
    element."""
    n = (1 << 32) + (1 << 20)
    _need(2 * 4 * n)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    src = torch.empty(n, dtype=torch.int32, device=DEV)
    out = torch.empty(n, dtype=torch.int32, device=DEV)
    _fill_bits(src, 2654435761, 32)
    for stride, reps, runs in ((33, 1, 33), (100, 4, 25), (1000, 8, 125), (65537, 1, 65537)):
        print(f"[large] gather tiles stride {stride}, n={n}", flush=True)
        plan = ew.ew_make_gather_plan(out.data_ptr(), src.data_ptr(), n, stride, cus)
        assert ew.PATHS[plan.path] == "gather_tiles"
        assert (plan.reps, plan.passes, plan.segment) == (reps, runs, n // reps)
        ew.ew_gather_f32(src.data_ptr(), out.data_ptr(), stride, n=n)
        torch.cuda.synchronize()
        seg = n // reps
        for k in range(1, reps):
            assert _chunked_equal(out[:seg], out[k * seg:(k + 1) * seg]), (stride, k)
        idx = _samples(n)
        for k in (1, runs // 2, runs - 1):              # around run starts
            b = -(-k * seg // runs)
            idx = np.unique(np.concatenate([idx, np.arange(b - 6, b + 6)]))
        j = np.array([oracle.gather_index(n, stride, int(i)) for i in idx], np.int64)
        assert np.array_equal(_take(out, idx), _take(src, j)), stride
    del src, out
    torch.cuda.empty_cache()


def test_gather_passes_stride3_past_2_pow_32_elements():
    """Stride 3 with gcd(3, n) == 1 and n > 2^32: the pass kernel's slot and
    destination arithmetic in 64 bits (host planning in 128)."""
    n = (1 << 32) + 1
    _need(2 * 4 * n)
    print(f"[large] gather passes stride 3, n={n}", flush=True)
    src = torch.empty(n, dtype=torch.int32, device=DEV)
    out = torch.empty(n, dtype=torch.int32, device=DEV)
    _fill_bits(src, 2654435761, 32)
    plan = ew.ew_make_gather_plan(out.data_ptr(), src.data_ptr(), n, 3,
                                  torch.cuda.get_device_properties(0).multi_processor_count)
    assert plan.passes == 3
    ew.ew_gather_f32(src.data_ptr(), out.data_ptr(), 3, n=n)
    torch.cuda.synchronize()
    idx = _samples(n)
    for k in (1, 2):                                    # around each pass boundary
        b = -(-k * n // 3)
        idx = np.unique(np.concatenate([idx, np.arange(b - 6, b + 6)]))
    j = np.array([oracle.gather_index(n, 3, int(i)) for i in idx], np.int64)
    assert np.array_equal(_take(out, idx), _take(src, j))
    del src, out
    torch.cuda.empty_cache()


def test_transpose_past_2_pow_32_elements():
    """A 65536 x 65540 transposed view (2^32 + 2^18 elements): tile and row
    offsets past 32 bits, ragged edge tiles on one side."""
    rows, cols = 65536, 65540
    n = rows * cols
    _need(2 * 4 * n)
    print(f"[large] transpose {rows} x {cols}", flush=True)
    src = torch.empty(n, dtype=torch.int32, device=DEV)    # (cols x rows) row-major
    out = torch.empty(n, dtype=torch.int32, device=DEV)
    _fill_bits(src, 2654435761, 32)
    ew.ew_copy2d_f32(src.data_ptr(), 1, rows, out.data_ptr(), rows, cols)
    torch.cuda.synchronize()
    idx = _samples(n)
    r, c = idx // cols, idx % cols
    assert np.array_equal(_take(out, idx), _take(src, c * rows + r))
    del src, out
    torch.cuda.empty_cache()


def test_bias_relu_past_2_pow_32_elements():
    """rows x cols > 2^32 with a column count that is not a multiple of 4
    (the per-element bias walk) and a misaligned output."""
    rows, cols = 1048063, 4099
    n = rows * cols
    assert n > 1 << 32
    _need(2 * 4 * (n + 8))
    print(f"[large] bias_relu {rows} x {cols}", flush=True)
    x = torch.empty(n, dtype=torch.float32, device=DEV)
    ybase = torch.empty(n + 8, dtype=torch.float32, device=DEV)
    y = ybase[3:3 + n]
    _fill_f32(x, 40503, 65521, 2.0 ** -8)
    x.sub_(128.0)                                      # mixed signs, exact in binary32
    bias = ((torch.arange(cols, device=DEV, dtype=torch.float32) % 509) - 254.0) * 0.25
    ew.ew_bias_relu_f32(x, bias, y, rows, cols)
    torch.cuda.synchronize()
    idx = _samples(n)
    hb = bias.cpu().numpy()
    ref = oracle.relu_f32(oracle.add_f32(_take(x, idx), hb[idx % cols]))
    assert mismatches("bias_relu_f32", _take(y, idx), ref).size == 0
    del x, ybase, y
    torch.cuda.empty_cache()


def test_submatrix_view_past_2_pow_32_elements():
    """A 65537 x 65536 sub-matrix of a 65540-wide array, starting 3 elements
    in: the rows-contiguous path with row and column walks past 32 bits."""
    rows, cols, pitch = 65537, 65536, 65540
    n = rows * cols
    base_n = (rows - 1) * pitch + cols + 3
    _need(4 * (n + base_n))
    print(f"[large] submatrix {rows} x {cols}", flush=True)
    src = torch.empty(base_n, dtype=torch.int32, device=DEV)
    out = torch.empty(n, dtype=torch.int32, device=DEV)
    _fill_bits(src, 2654435761, 32)
    ew.ew_copy2d_f32(src.data_ptr() + 4 * 3, pitch, 1, out.data_ptr(), rows, cols)
    torch.cuda.synchronize()
    idx = _samples(n)
    r, c = idx // cols, idx % cols
    assert np.array_equal(_take(out, idx), _take(src, 3 + r * pitch + c))
    del src, out
    torch.cuda.empty_cache()


def test_batch_table_with_an_item_past_2_pow_32_elements():
    """The device-table batch with one bf16 item of 2^32 + 7 elements (its
    output one element off alignment) between two small items: 64-bit tile
    and element arithmetic inside the table kernel, sampled against the
    oracle, the small items on every element."""
    n = (1 << 32) + 7
    _need(3 * 2 * (n + 8))
    print(f"[large] batch table, bf16 item n={n}", flush=True)
    abase = torch.empty(n + 8, dtype=torch.int16, device=DEV)
    b = torch.empty(n, dtype=torch.int16, device=DEV)
    cbase = torch.empty(n + 8, dtype=torch.int16, device=DEV)
    a, c = abase[2:2 + n], cbase[1:1 + n]
    _fill_bits(a, 2654435761, 16)
    _fill_bits(b, 40503 * 65537, 16)
    sa, sb = abase[-6:], b[:5]        # small items: abase past a's end, b's first elements
    sc1 = torch.empty(5, dtype=torch.int16, device=DEV)
    sc2 = torch.empty(3, dtype=torch.int16, device=DEV)
    batch = ew.EwBatch("add_bf16", [(sc1, sa[:5], sb, 5), (c, a, b, n), (sc2, sa[1:4], sb[2:5], 3)])
    assert batch.plan.items == 3 and batch.plan.tiles > (1 << 16)
    batch()
    torch.cuda.synchronize()
    idx = _samples(n)
    got = _take(c, idx).view(np.uint16)
    ref = oracle.add_bf16(_take(a, idx).view(np.uint16), _take(b, idx).view(np.uint16))
    assert mismatches("add_bf16", got, ref).size == 0
    h = lambda t: t.cpu().numpy().view(np.uint16)          # noqa: E731
    assert mismatches("add_bf16", h(sc1), oracle.add_bf16(h(sa[:5]), h(sb))).size == 0
    assert mismatches("add_bf16", h(sc2), oracle.add_bf16(h(sa[1:4]), h(sb[2:5]))).size == 0
    del abase, b, cbase, a, c, batch
    torch.cuda.empty_cache()
