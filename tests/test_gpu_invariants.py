"""Closed forms and invariants checked on the HIP path's own outputs, with no
oracle involved: identities that the operations' definitions fix, so a slip
in a kernel shows here even if the oracle shared it.

* add: -0 is the additive identity (bitwise), addition commutes, a + (-a)
  is +0 for finite a (fp32, and the 16-bit formats with -0 = 0x8000);
* SAXPY: alpha = 0 and x = +0 return y; alpha = 2 equals the add of the
  exact 2x and y (both round 2x + y once);
* ReLU ([PerfNotes] 5.2, read as IEEE maximum(x, +0)): no sign bit on a
  non-NaN result, x > 0 passes unchanged, everything else non-NaN becomes +0,
  NaN passes bitwise, idempotent, relu(x) - relu(-x) = x for finite x != 0;
* in-place ReLU and the fused chains equal their unfused compositions;
* copy is bitwise (signalling NaN payloads included); the gather with stride
  1 or n + 1 is the copy, with stride 2 and even n its halves are equal, and
  with a stride coprime with n it is a permutation;
* a transposed view of a transposed view is the identity, and a view with
  contiguous strides is the copy;
* the scalar and unary maps: scale by 1, -1 and 2, adding -0, abs as a
  sign-bit clear, the roots of exact squares.

Sizes span several tiles with a ragged tail; pointers are misaligned.
"""
import math

import numpy as np
import pytest
import torch

import memory_bound_elementwise_amd as ew
import synth
from tests.gpu_util import download, upload

pytestmark = pytest.mark.gpu

N = (1 << 20) + 13


def _pool_f32(n, seed):
    """Uniform, normal and random bit patterns in thirds, with special values."""
    g = synth.rng(seed)
    x = np.empty(n, np.float32)
    x[0::3] = synth.uniform_pm1(g, len(x[0::3]))
    x[1::3] = synth.normal01(g, len(x[1::3]))
    x[2::3] = g.integers(0, 1 << 32, size=len(x[2::3]), dtype=np.uint32).view(np.float32)
    sp = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-45, -1e-45, 1e-40, -3e-39,
                   3.4028235e38, -3.4028235e38, 0.5, -2.5], np.float32)
    x[:sp.size] = sp
    return x


def _bits(x):
    return x.view(np.uint32)


def _nan32(x):
    return (_bits(x) & 0x7FFFFFFF) > 0x7F800000


def _same_f32(got, want):
    """Bitwise, except that any NaN matches any NaN."""
    gn, wn = _nan32(got), _nan32(want)
    return bool(np.all((_bits(got) == _bits(want)) | (gn & wn)) and np.all(gn == wn))


def _run(fn, *arrays, offs=(1, 0, 3), out_like=None):
    """Upload arrays at the given element offsets, call fn(*views) and
    return the host copies of every view after the call."""
    views, keep = [], []
    for a, o in zip(arrays, offs):
        v, b = upload(a, o)
        views.append(v)
        keep.append(b)
    fn(*views)
    torch.cuda.synchronize()
    return [download(v, a.dtype.itemsize) for v, a in zip(views, arrays)]


def test_add_negative_zero_is_the_identity_and_addition_commutes():
    a = _pool_f32(N, 401)
    b = _pool_f32(N, 402)
    mz = np.full(N, -0.0, np.float32)
    _, _, c = _run(ew.ew_add_f32, a, mz, np.zeros(N, np.float32))
    assert _same_f32(c, a)
    _, _, ab = _run(ew.ew_add_f32, a, b, np.zeros(N, np.float32))
    _, _, ba = _run(ew.ew_add_f32, b, a, np.zeros(N, np.float32), offs=(2, 3, 0))
    assert _same_f32(ab, ba)
    fin = a[np.isfinite(a)]
    _, _, z = _run(ew.ew_add_f32, fin, -fin, np.zeros(fin.size, np.float32))
    assert np.all(_bits(z) == 0)               # a + (-a) = +0 in round-to-nearest


@pytest.mark.parametrize("op,nan_mask", [
    ("add_f16", lambda u: ((u & 0x7C00) == 0x7C00) & ((u & 0x03FF) != 0)),
    ("add_bf16", lambda u: ((u & 0x7F80) == 0x7F80) & ((u & 0x007F) != 0))])
def test_16bit_add_negative_zero_is_the_identity(op, nan_mask):
    g = synth.rng(403)
    a = g.integers(0, 1 << 16, size=N, dtype=np.uint16)
    mz = np.full(N, 0x8000, np.uint16)
    _, _, c = _run(getattr(ew, "ew_" + op), a, mz, np.zeros(N, np.uint16))
    an, cn = nan_mask(a), nan_mask(c)
    assert np.all(an == cn)
    assert np.all((c == a) | an)


def test_saxpy_closed_forms():
    g = synth.rng(404)
    x = synth.normal01(g, N) * np.float32(1e3)
    y = _pool_f32(N, 405)
    y[_bits(y) == 0x80000000] = np.float32(1.0)        # fma(., ., -0) may give +0
    y[~np.isfinite(y)] = np.float32(2.0)
    _, y0 = _run(lambda xv, yv: ew.ew_saxpy_f32(0.0, xv, yv), x, y.copy())
    assert np.all(_bits(y0) == _bits(y))               # alpha = 0: y, bitwise
    _, y1 = _run(lambda xv, yv: ew.ew_saxpy_f32(2.5, xv, yv), np.zeros(N, np.float32), y.copy())
    assert np.all(_bits(y1) == _bits(y))               # x = +0: y, bitwise
    # alpha = 2: 2x is exact, so fma(2, x, y) and the add of 2x and y both
    # round the same exact sum once
    _, y2 = _run(lambda xv, yv: ew.ew_saxpy_f32(2.0, xv, yv), x, y.copy())
    _, _, s = _run(ew.ew_add_f32, np.float32(2) * x, y, np.zeros(N, np.float32))
    assert np.all(_bits(y2) == _bits(s))


def test_relu_properties():
    x = _pool_f32(N, 406)
    _, y = _run(ew.ew_relu_f32, x, np.zeros(N, np.float32))
    nan = _nan32(x)
    assert np.all(_bits(y[nan]) == _bits(x[nan]))       # NaN passes bitwise
    assert not np.any(np.signbit(y[~nan]))              # never a sign bit otherwise
    pos = ~nan & (x > 0)
    assert np.all(_bits(y[pos]) == _bits(x[pos]))       # x > 0 unchanged
    assert np.all(_bits(y[~nan & ~pos]) == 0)           # the rest is +0
    _, yy = _run(ew.ew_relu_f32, y, np.zeros(N, np.float32))
    assert np.all(_bits(yy) == _bits(y))                # idempotent
    fin = np.isfinite(x) & (x != 0)
    neg = (_bits(x) ^ np.uint32(0x80000000)).view(np.float32)
    _, yn = _run(ew.ew_relu_f32, neg, np.zeros(N, np.float32))
    assert np.all(y[fin] - yn[fin] == x[fin])           # relu(x) - relu(-x) = x, exactly


def test_inplace_relu_and_fused_chains_equal_their_compositions():
    x = _pool_f32(N, 407)
    _, y = _run(ew.ew_relu_f32, x, np.zeros(N, np.float32))
    (xi,) = _run(ew.ew_relu_inplace_f32, x.copy(), offs=(5,))
    assert np.all(_bits(xi) == _bits(y))
    absx = np.abs(synth.normal01(synth.rng(408), N))
    (ai,) = _run(ew.ew_relu_inplace_f32, absx.copy(), offs=(2,))
    assert np.all(_bits(ai) == _bits(absx))             # nothing to change, nothing changed

    a, b = _pool_f32(N, 409), _pool_f32(N, 410)
    _, _, fused = _run(ew.ew_add_relu_f32, a, b, np.zeros(N, np.float32))
    _, _, s = _run(ew.ew_add_f32, a, b, np.zeros(N, np.float32))
    _, r = _run(ew.ew_relu_f32, s, np.zeros(N, np.float32))
    assert _same_f32(fused, r)
    _, fs = _run(lambda xv, yv: ew.ew_saxpy_relu_f32(2.5, xv, yv), a, b.copy())
    _, sx = _run(lambda xv, yv: ew.ew_saxpy_f32(2.5, xv, yv), a, b.copy())
    _, rs = _run(ew.ew_relu_f32, sx, np.zeros(N, np.float32))
    assert _same_f32(fs, rs)


def test_copy_and_gather_closed_forms():
    g = synth.rng(411)
    x = g.integers(0, 1 << 32, size=N, dtype=np.uint32).view(np.float32)
    x[:4] = np.array([0x7F800001, 0xFF800001, 0x7FA00000, 0x80000000], np.uint32).view(np.float32)
    _, c = _run(ew.ew_copy_f32, x, np.zeros(N, np.float32))
    assert np.all(_bits(c) == _bits(x))                  # signalling NaNs included
    for stride in (1, N + 1, 2 * N + 1):
        _, gth = _run(lambda i, o: ew.ew_gather_f32(i, o, stride), x, np.zeros(N, np.float32))
        assert np.all(_bits(gth) == _bits(x)), stride
    even = x[:N - 1] if (N - 1) % 2 == 0 else x[:N]
    n = even.size
    _, ge = _run(lambda i, o: ew.ew_gather_f32(i, o, 2), even, np.zeros(n, np.float32))
    assert np.all(_bits(ge[:n // 2]) == _bits(ge[n // 2:]))   # outputs i and i + n/2 agree
    assert np.all(_bits(ge[:n // 2]) == _bits(even[0::2]))
    for stride in (2, 3, 5, 7, 8, 1000003):
        m = N if math.gcd(stride, N) == 1 else N - 2
        assert math.gcd(stride, m) == 1
        _, gp = _run(lambda i, o: ew.ew_gather_f32(i, o, stride), x[:m], np.zeros(m, np.float32))
        assert np.array_equal(np.sort(_bits(gp)), np.sort(_bits(x[:m]))), stride   # permutation
        i = np.arange(0, m, 997, dtype=np.uint64)
        assert np.all(_bits(gp)[i] == _bits(x[:m])[(np.uint64(stride) * i) % np.uint64(m)])


def test_double_transpose_is_the_identity_and_contiguous_strides_copy():
    rows, cols = 1031, 1029                     # edge tiles on both axes
    x = _pool_f32(rows * cols, 412)
    xv, xb = upload(x, 1)
    t, tb = upload(np.zeros(rows * cols, np.float32), 3)
    z, zb = upload(np.zeros(rows * cols, np.float32), 2)
    ew.ew_copy2d_f32(xv, 1, cols, t, cols, rows)          # t = x^T (cols x rows)
    ew.ew_copy2d_f32(t, 1, rows, z, rows, cols)           # z = t^T
    c, cb = upload(np.zeros(rows * cols, np.float32), 0)
    ew.ew_copy2d_f32(xv, cols, 1, c, rows, cols)          # contiguous strides
    torch.cuda.synchronize()
    assert np.all(_bits(download(z, 4)) == _bits(x))
    assert np.all(_bits(download(c, 4)) == _bits(x))
    tt = download(t, 4).reshape(cols, rows)
    assert np.all(_bits(tt) == _bits(x.reshape(rows, cols).T))


def test_scalar_and_unary_map_closed_forms():
    """scale by 1 is the identity, by -1 flips the sign bit and by 2 equals
    the add of x and x; adding -0 is the identity; abs clears exactly the sign
    bit; the root of an exact square k^2 (k < 2^12) is k, and of 4^j is 2^j."""
    x = _pool_f32(N, 413)
    x = x[~_nan32(x)]
    n = x.size
    z = np.zeros(n, np.float32)
    _, s1 = _run(lambda xv, yv: ew.ew_scale_f32(1.0, xv, yv), x, z)
    assert np.all(_bits(s1) == _bits(x))
    _, sm = _run(lambda xv, yv: ew.ew_scale_f32(-1.0, xv, yv), x, z)
    assert np.all(_bits(sm) == (_bits(x) ^ np.uint32(0x80000000)))
    _, s2 = _run(lambda xv, yv: ew.ew_scale_f32(2.0, xv, yv), x, z)
    _, _, xx = _run(ew.ew_add_f32, x, x, np.zeros(n, np.float32))
    assert np.all(_bits(s2) == _bits(xx))
    _, a0 = _run(lambda xv, yv: ew.ew_add_scalar_f32(-0.0, xv, yv), x, z)
    assert np.all(_bits(a0) == _bits(x))
    _, ab = _run(ew.ew_abs_f32, x, z)
    assert np.all((_bits(ab) | (_bits(x) & np.uint32(0x80000000))) == _bits(x))
    assert not np.any(_bits(ab) & np.uint32(0x80000000))
    k = np.arange(1, 4096, dtype=np.float32)
    sq = np.concatenate([k * k, np.ldexp(np.float32(1), np.arange(-74, 64, 2)).astype(np.float32)])
    _, r = _run(ew.ew_sqrt_f32, sq, np.zeros(sq.size, np.float32))
    want = np.concatenate([k, np.ldexp(np.float32(1), np.arange(-37, 32)).astype(np.float32)])
    assert np.all(_bits(r) == _bits(want))
