"""Pins for the CPU oracle: library routines, exact arithmetic, closed forms,
invariants and brute force -- never the oracle against itself.

Each test is chosen so that a plausible slip in ``oracle/oracle.c`` (a wrong
rounding rule, an unfused SAXPY, a dropped NaN case, a signed-zero mistake,
a wrong gather index) fails at least one of them.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
import synth
from tests.pins import exact, f16c

F32_SPECIALS = np.array(
    [0.0, -0.0, 1.0, -1.0, 0.5, -0.5, 2.0, 3.0, 1.5, np.inf, -np.inf, np.nan,
     np.finfo(np.float32).max, -np.finfo(np.float32).max,
     np.finfo(np.float32).tiny, -np.finfo(np.float32).tiny,
     1e-45, -1e-45, 2.8e-45, 1.1754942e-38, 65504.0, 65520.0, 65519.99,
     6.1035156e-05, 5.9604645e-08, 2.9802322e-08, 2.9802326e-08,
     3.3895314e38, 1.0000001, 0.99999994, 16777216.0, 16777217.0, 1e10, -1e-10,
     0.1, -0.3, 1e-40, -1e-38],
    dtype=np.float32)


def _nan_class_equal(got_bits, ref_bits, got_is_nan, ref_is_nan):
    """Bitwise equality, except NaN positions compare by class (both NaN)."""
    same = (got_bits == ref_bits) | (got_is_nan & ref_is_nan)
    return bool(np.all(same)) and bool(np.all(got_is_nan == ref_is_nan))


def _random_f32_bits(n, seed, finite=True):
    g = np.random.Generator(np.random.PCG64(seed))
    u = g.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
    if finite:
        exp = (u >> 23) & 0xFF
        u = np.where(exp == 0xFF, u & ~np.uint32(0x40000000), u).astype(np.uint32)
    return u.view(np.float32)


def test_fpenv_is_ieee_default():
    assert oracle.fpenv_ok()


# --------------------------------------------------------------------------
# binary16 conversions
# --------------------------------------------------------------------------

@pytest.mark.skipif(not f16c.available(), reason="host CPU lacks F16C")
def test_f32_to_f16_exhaustive_vs_f16c():
    """All 2^32 binary32 patterns narrowed by the oracle == VCVTPS2PH (RNE).
    NaNs compare by class and sign (payload rules differ).  The loop runs in
    the C pin helper, calling the oracle's conversion through its address."""
    import ctypes
    fn = ctypes.cast(oracle._load().oracle_f32_to_f16, ctypes.c_void_p).value
    assert f16c.count_mismatches(fn, 0, 1 << 32) == 0
    # the helper itself must see a planted difference: the bfloat16
    # conversion disagrees with binary16 narrowing almost everywhere
    other = ctypes.cast(oracle._load().oracle_f32_to_bf16, ctypes.c_void_p).value
    assert f16c.count_mismatches(other, 0x3F800000, 1 << 16) > 60000


def test_f32_to_f16_vs_numpy_sample():
    """A second library (numpy's own software conversion) on random patterns
    and specials."""
    x = np.concatenate([_random_f32_bits(1 << 18, 7, finite=True), F32_SPECIALS])
    got = oracle.f32_to_f16(x)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    nan = np.isnan(x)
    assert np.array_equal(got[~nan], ref[~nan])


def test_f16_rounding_closed_forms():
    cases = {
        65504.0: 0x7BFF, 65519.99: 0x7BFF, 65520.0: 0x7C00, -65520.0: 0xFC00,
        5.9604645e-08: 0x0001,           # 2^-24, smallest subnormal
        2.9802322e-08: 0x0000,           # 2^-25 exactly: tie -> even (0)
        2.9802326e-08: 0x0001,           # just above 2^-25
        8.940697e-08: 0x0002,            # 1.5 * 2^-24: tie -> even (2)
        6.1035156e-05: 0x0400,           # 2^-14, smallest normal
        1.0: 0x3C00, -2.0: 0xC000, 1.0009766: 0x3C01,
        1.00048828125: 0x3C00,           # 1 + 2^-11: tie -> even (1.0)
        1.00146484375: 0x3C02,           # 1 + 3*2^-11: tie -> even (1+2^-9)
        -0.0: 0x8000, np.inf: 0x7C00,
    }
    for v, bits in cases.items():
        assert oracle._load().oracle_f32_to_f16(float(np.float32(v))) == bits, v


def test_f16_widen_all_patterns():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.f16_to_f32(h)
    if f16c.available():
        ref = f16c.widen(h)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    ref2 = h.view(np.float16).astype(np.float32)
    nan = np.isnan(ref2)
    assert np.array_equal(got.view(np.uint32)[~nan], ref2.view(np.uint32)[~nan])
    assert np.all(np.isnan(got[nan]))


def test_f16_round_trip_identity():
    """Every non-NaN binary16 survives widen -> narrow unchanged."""
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    back = oracle.f32_to_f16(oracle.f16_to_f32(h))
    nan = ((h & 0x7C00) == 0x7C00) & ((h & 0x03FF) != 0)
    assert np.array_equal(back[~nan], h[~nan])


# --------------------------------------------------------------------------
# bfloat16 conversions
# --------------------------------------------------------------------------

def _torch_bf16_bits(x):
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_f32_to_bf16_structured_sweep_vs_torch():
    """Every upper half-word (sign, exponent, top 7 fraction bits) crossed
    with every low-half pattern class that decides RNE rounding (zero, just
    above zero, below / at / above one half, all ones), plus random patterns.
    Rounding depends only on the low 16 bits against 0x8000 and on the parity
    and carry of the upper half, so this covers every rounding decision."""
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0x0000, 0x0001, 0x0002, 0x3FFF, 0x7FFE, 0x7FFF, 0x8000,
                     0x8001, 0x8002, 0xBFFF, 0xFFFE, 0xFFFF], dtype=np.uint32)
    bits = (hi[:, None] | lows[None, :]).reshape(-1)
    bits = np.concatenate([bits, _random_f32_bits(1 << 20, 11, finite=False).view(np.uint32)])
    x = bits.view(np.float32)
    got = oracle.f32_to_bf16(x)
    ref = _torch_bf16_bits(x)
    nan = (bits & 0x7FFFFFFF) > 0x7F800000
    assert np.array_equal(got[~nan], ref[~nan])
    gn = got[nan]
    assert np.all((gn & 0x7F80) == 0x7F80) and np.all((gn & 0x007F) != 0)
    assert np.all((gn >> 15) == (bits[nan] >> 31))


def test_bf16_widen_all_patterns():
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.bf16_to_f32(h)
    ref = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_bf16_closed_forms():
    f = oracle._load().oracle_f32_to_bf16
    assert f(1.0) == 0x3F80
    assert f(float(np.float32(1.0 + 2.0 ** -8))) == 0x3F80     # tie -> even
    assert f(float(np.float32(1.0 + 3 * 2.0 ** -8))) == 0x3F82  # tie -> even (up)
    assert f(float(np.finfo(np.float32).max)) == 0x7F80         # carries to inf
    assert f(float(np.float32(-0.0))) == 0x8000
    assert f(float(np.float32(1e-45))) == 0x0000                # tiny subnormal -> +0


# --------------------------------------------------------------------------
# add f32
# --------------------------------------------------------------------------

def test_add_f32_vs_numpy():
    g = synth.rng(1)
    a = np.concatenate([synth.uniform_pm1(g, 1 << 18), _random_f32_bits(1 << 18, 2, False)])
    b = np.concatenate([synth.uniform_pm1(g, 1 << 18), _random_f32_bits(1 << 18, 3, False)])
    sa, sb = np.meshgrid(F32_SPECIALS, F32_SPECIALS)
    a = np.concatenate([a, sa.ravel()])
    b = np.concatenate([b, sb.ravel()])
    got = oracle.add_f32(a, b)
    with np.errstate(all="ignore"):
        ref = a + b
    assert _nan_class_equal(got.view(np.uint32), ref.view(np.uint32),
                            np.isnan(got), np.isnan(ref))
    tref = (torch.from_numpy(a) + torch.from_numpy(b)).numpy()
    assert _nan_class_equal(got.view(np.uint32), tref.view(np.uint32),
                            np.isnan(got), np.isnan(tref))


def test_add_f32_exact_rational():
    a = np.concatenate([_random_f32_bits(1500, 21), synth.uniform_pm1(synth.rng(22), 1500)])
    b = np.concatenate([_random_f32_bits(1500, 23), synth.uniform_pm1(synth.rng(24), 1500)])
    # make some pairs cancel heavily and some share exponents
    b[:200] = -a[:200] * np.float32(1.0000001)
    got = oracle.add_f32(a, b)
    for x, y, r in zip(a, b, got):
        q = exact.f32_to_fraction(x) + exact.f32_to_fraction(y)
        both_neg = math.copysign(1, x) < 0 and math.copysign(1, y) < 0
        ref = exact.round_rne(q, exact.BINARY32, zero_sign_negative=both_neg)
        assert exact.f32_bits(ref) == exact.f32_bits(float(r)), (x, y)


def test_add_f32_invariants():
    g = synth.rng(5)
    a = np.concatenate([synth.uniform_pm1(g, 4096), _random_f32_bits(4096, 6, False), F32_SPECIALS])
    b = np.concatenate([synth.uniform_pm1(g, 4096), _random_f32_bits(4096, 7, False),
                        F32_SPECIALS[::-1]])
    nz = np.full_like(a, -0.0)
    # A + (-0) == A bitwise (also for A = -0 and NaN payloads of quiet NaNs)
    s = oracle.add_f32(a, nz)
    finite_or_inf = ~np.isnan(a)
    assert np.array_equal(s.view(np.uint32)[finite_or_inf], a.view(np.uint32)[finite_or_inf])
    # commutativity, bitwise (NaN by class)
    ab, ba = oracle.add_f32(a, b), oracle.add_f32(b, a)
    assert _nan_class_equal(ab.view(np.uint32), ba.view(np.uint32), np.isnan(ab), np.isnan(ba))
    # a + (-a) == +0 for finite a
    fin = np.isfinite(a)
    z = oracle.add_f32(a[fin], -a[fin])
    assert np.all(z.view(np.uint32) == 0)
    # small integers add exactly
    ia = np.arange(-4096, 4096, dtype=np.float32)
    assert np.array_equal(oracle.add_f32(ia, ia[::-1]), np.zeros_like(ia) - 1)
    # overflow, subnormals kept (no FTZ), NaN propagates
    big = np.float32(np.finfo(np.float32).max)
    assert np.isposinf(oracle.add_f32(np.array([big]), np.array([big]))[0])
    den = np.array([1e-45, 3e-44, -1e-40], np.float32)
    assert np.array_equal(oracle.add_f32(den, np.zeros_like(den)).view(np.uint32),
                          den.view(np.uint32))
    assert oracle.add_f32(np.array([1e-45], np.float32),
                          np.array([1e-45], np.float32))[0] == np.float32(2.8e-45)
    assert np.isnan(oracle.add_f32(np.array([np.nan], np.float32), np.array([1.0], np.float32))[0])
    assert np.isnan(oracle.add_f32(np.array([np.inf], np.float32), np.array([-np.inf], np.float32))[0])


# --------------------------------------------------------------------------
# add f16 / bf16
# --------------------------------------------------------------------------

def _special_f16_bits():
    v = np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x03FF, 0x0400, 0x3C00, 0xBC00,
                  0x7BFF, 0xFBFF, 0x7C00, 0xFC00, 0x7E00, 0x7C01, 0x3BFF, 0x3C01,
                  0x5640, 0x1400, 0x7BFE, 0x0200], dtype=np.uint16)
    return v


def test_add_f16_vs_numpy():
    g = np.random.Generator(np.random.PCG64(31))
    a = g.integers(0, 1 << 16, size=1 << 20, dtype=np.uint32).astype(np.uint16)
    b = g.integers(0, 1 << 16, size=1 << 20, dtype=np.uint32).astype(np.uint16)
    u = synth.make_inputs("add_f16", 1 << 16, 104)
    sa, sb = np.meshgrid(_special_f16_bits(), _special_f16_bits())
    a = np.concatenate([a, u["a"], sa.ravel()])
    b = np.concatenate([b, u["b"], sb.ravel()])
    got = oracle.add_f16(a, b)
    with np.errstate(all="ignore"):
        ref = (a.view(np.float16) + b.view(np.float16)).view(np.uint16)
    gnan = np.isnan(got.view(np.float16))
    rnan = np.isnan(ref.view(np.float16))
    assert _nan_class_equal(got, ref, gnan, rnan)


def test_add_f16_exact_rational():
    """The fp32 detour gives the correctly rounded binary16 sum."""
    g = np.random.Generator(np.random.PCG64(32))
    a = g.integers(0, 1 << 16, size=3000, dtype=np.uint32).astype(np.uint16)
    b = g.integers(0, 1 << 16, size=3000, dtype=np.uint32).astype(np.uint16)
    fin = ((a & 0x7C00) != 0x7C00) & ((b & 0x7C00) != 0x7C00)
    a, b = a[fin], b[fin]
    got = oracle.add_f16(a, b)
    for x, y, r in zip(a, b, got):
        fx, fy = float(np.uint16(x).view(np.float16)), float(np.uint16(y).view(np.float16))
        q = exact.f32_to_fraction(fx) + exact.f32_to_fraction(fy)
        both_neg = math.copysign(1, fx) < 0 and math.copysign(1, fy) < 0
        ref = exact.round_rne(q, exact.BINARY16, zero_sign_negative=both_neg)
        assert exact.f16_bits(ref) == int(r), (hex(x), hex(y))


def test_add_f16_overflow_threshold():
    def add(x, y):
        return int(oracle.add_f16(np.array([x], np.uint16), np.array([y], np.uint16))[0])
    h = lambda v: int(np.array([v], np.float16).view(np.uint16)[0])
    assert add(h(65504.0), h(8.0)) == h(65504.0)      # 65512 < 65520 -> 65504
    assert add(h(65504.0), h(16.0)) == 0x7C00          # 65520 is the tie -> inf
    assert add(h(-65504.0), h(-16.0)) == 0xFC00
    assert add(0x0001, 0x0001) == 0x0002               # subnormals kept
    assert add(0x0001, 0x8001) == 0x0000               # x + (-x) == +0
    assert add(0x8000, 0x8000) == 0x8000               # -0 + -0 == -0


def test_add_bf16_vs_torch():
    g = np.random.Generator(np.random.PCG64(33))
    a = g.integers(0, 1 << 16, size=1 << 20, dtype=np.uint32).astype(np.uint16)
    b = g.integers(0, 1 << 16, size=1 << 20, dtype=np.uint32).astype(np.uint16)
    u = synth.make_inputs("add_bf16", 1 << 16, 105)
    a = np.concatenate([a, u["a"]])
    b = np.concatenate([b, u["b"]])
    got = oracle.add_bf16(a, b)
    ta = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    tb = torch.from_numpy(b.view(np.int16)).view(torch.bfloat16)
    ref = (ta + tb).view(torch.int16).numpy().view(np.uint16)
    gnan = ((got & 0x7F80) == 0x7F80) & ((got & 0x7F) != 0)
    rnan = ((ref & 0x7F80) == 0x7F80) & ((ref & 0x7F) != 0)
    assert _nan_class_equal(got, ref, gnan, rnan)


def test_add_bf16_exact_rational():
    g = np.random.Generator(np.random.PCG64(34))
    a = g.integers(0, 1 << 16, size=3000, dtype=np.uint32).astype(np.uint16)
    b = g.integers(0, 1 << 16, size=3000, dtype=np.uint32).astype(np.uint16)
    fin = ((a & 0x7F80) != 0x7F80) & ((b & 0x7F80) != 0x7F80)
    a, b = a[fin], b[fin]
    got = oracle.add_bf16(a, b)
    for x, y, r in zip(a, b, got):
        fx = float((np.uint32(x) << 16).view(np.float32))
        fy = float((np.uint32(y) << 16).view(np.float32))
        q = exact.f32_to_fraction(fx) + exact.f32_to_fraction(fy)
        both_neg = math.copysign(1, fx) < 0 and math.copysign(1, fy) < 0
        ref = exact.round_rne(q, exact.BFLOAT16, zero_sign_negative=both_neg)
        ref_bits = exact.f32_bits(ref) >> 16
        assert ref_bits == int(r), (hex(x), hex(y))


# --------------------------------------------------------------------------
# SAXPY
# --------------------------------------------------------------------------

def test_saxpy_exact_rational():
    """fmaf(alpha, x, y) == alpha*x + y computed exactly, rounded once."""
    g = synth.rng(41)
    x = np.concatenate([synth.normal01(g, 2000), _random_f32_bits(1000, 42)])
    y = np.concatenate([synth.normal01(g, 2000), _random_f32_bits(1000, 43)])
    # heavy cancellation near y = -2.5 x, where an unfused multiply-add drifts
    y[:300] = -(np.float32(2.5) * x[:300])
    for alpha in (np.float32(2.5), np.float32(-0.7), np.float32(3.0e-30)):
        got = oracle.saxpy_f32(alpha, x, y)
        for xi, yi, r in zip(x, y, got):
            p = exact.f32_to_fraction(alpha) * exact.f32_to_fraction(xi)
            q = p + exact.f32_to_fraction(yi)
            prod_neg = (math.copysign(1, float(alpha)) * math.copysign(1, float(xi))) < 0
            both_neg = prod_neg and math.copysign(1, float(yi)) < 0
            ref = exact.round_rne(q, exact.BINARY32, zero_sign_negative=both_neg)
            if math.isinf(ref) and math.isinf(float(r)):
                assert (ref > 0) == (float(r) > 0)
                continue
            assert exact.f32_bits(ref) == exact.f32_bits(float(r)), (alpha, xi, yi)


def test_saxpy_is_fused_not_two_roundings():
    """On the SAXPY config's inputs an unfused multiply-then-add differs from
    the single-rounding result on many elements; the oracle must be fused."""
    inp = synth.make_inputs("saxpy_f32", 1 << 18, 103, "normal")
    x, y = inp["x"], inp["y"]
    got = oracle.saxpy_f32(2.5, x, y)
    unfused = (np.float32(2.5) * x) + y
    assert np.count_nonzero(got != unfused) > 1000
    # the double-precision evaluation rounded once to binary32 agrees here
    dbl = (np.float64(2.5) * x.astype(np.float64) + y.astype(np.float64)).astype(np.float32)
    assert np.array_equal(got, dbl)


def test_saxpy_closed_forms():
    g = synth.rng(44)
    x = synth.normal01(g, 4096)
    y = synth.normal01(g, 4096)
    # alpha = 0 returns y (finite x, y != -0)
    assert np.array_equal(oracle.saxpy_f32(0.0, x, y).view(np.uint32), y.view(np.uint32))
    # x = 0 returns y
    assert np.array_equal(oracle.saxpy_f32(2.5, np.zeros_like(x), y).view(np.uint32),
                          y.view(np.uint32))
    # y = +0 gives the correctly rounded product alpha*x
    assert np.array_equal(oracle.saxpy_f32(2.5, x, np.zeros_like(y)),
                          np.float32(2.5) * x)
    # alpha = 2: the product is exact, so SAXPY equals the add of (2x, y)
    assert np.array_equal(oracle.saxpy_f32(2.0, x, y), oracle.add_f32(np.float32(2) * x, y))
    # y is not modified by the wrapper
    y0 = y.copy()
    oracle.saxpy_f32(2.5, x, y)
    assert np.array_equal(y, y0)


# --------------------------------------------------------------------------
# ReLU, copy, gather
# --------------------------------------------------------------------------

def test_relu_vs_numpy_maximum():
    g = synth.rng(51)
    x = np.concatenate([synth.normal01(g, 1 << 18), _random_f32_bits(1 << 18, 52, False),
                        F32_SPECIALS, np.array([-np.nan], np.float32)])
    got = oracle.relu_f32(x)
    ref = np.maximum(x, np.float32(0))
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_relu_invariants():
    g = synth.rng(53)
    x = np.concatenate([synth.normal01(g, 1 << 16), _random_f32_bits(1 << 16, 54, True),
                        np.array([-0.0, 0.0, -np.inf, np.inf], np.float32)])
    y = oracle.relu_f32(x)
    assert np.all(y >= 0) and np.all((y.view(np.uint32) >> 31) == 0)
    pos = x > 0
    assert np.array_equal(y[pos].view(np.uint32), x[pos].view(np.uint32))
    assert np.array_equal(oracle.relu_f32(y).view(np.uint32), y.view(np.uint32))
    fin = np.isfinite(x) & (x != 0)
    assert np.array_equal(oracle.relu_f32(x[fin]) - oracle.relu_f32(-x[fin]), x[fin])
    assert oracle.relu_f32(np.array([-0.0], np.float32)).view(np.uint32)[0] == 0
    n = oracle.relu_f32(np.array([np.nan, -np.nan], np.float32))
    assert np.all(np.isnan(n)) and (n.view(np.uint32)[1] >> 31) == 1


def test_add_relu_vs_numpy():
    """maximum(a + b, 0) with numpy's own add and maximum, bitwise."""
    g = synth.rng(55)
    a = np.concatenate([synth.uniform_pm1(g, 1 << 18), _random_f32_bits(1 << 18, 56, False),
                        F32_SPECIALS, np.array([-0.0, 1.0, np.nan], np.float32)])
    b = np.concatenate([synth.uniform_pm1(g, 1 << 18), _random_f32_bits(1 << 18, 57, False),
                        F32_SPECIALS[::-1], np.array([-0.0, -1.0, 1.0], np.float32)])
    with np.errstate(all="ignore"):
        ref = np.maximum(a + b, np.float32(0))
    got = oracle.add_relu_f32(a, b)
    assert np.array_equal(got.view(np.uint32)[~np.isnan(ref)], ref.view(np.uint32)[~np.isnan(ref)])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    # -0 + -0 = -0, whose ReLU is +0; 1 + -1 = +0
    assert got.view(np.uint32)[-3] == 0 and got.view(np.uint32)[-2] == 0


def test_saxpy_relu_exact_rational():
    g = synth.rng(58)
    x = np.concatenate([synth.normal01(g, 1500), _random_f32_bits(500, 59)])
    y = np.concatenate([synth.normal01(g, 1500), _random_f32_bits(500, 60)])
    y[:200] = -(np.float32(2.5) * x[:200])          # results near zero, both signs
    got = oracle.saxpy_relu_f32(2.5, x, y)
    for xi, yi, r in zip(x, y, got):
        q = exact.f32_to_fraction(np.float32(2.5)) * exact.f32_to_fraction(xi) + \
            exact.f32_to_fraction(yi)
        v = exact.round_rne(q, exact.BINARY32)
        ref = v if v > 0 else 0.0
        if math.isinf(ref):
            assert math.isinf(float(r)) and float(r) > 0
            continue
        assert exact.f32_bits(ref) == exact.f32_bits(float(r)), (xi, yi)


def test_bias_relu_vs_numpy_broadcast():
    g = synth.rng(61)
    for rows, cols in ((1, 1), (3, 7), (64, 129), (1000, 4), (17, 1)):
        x = synth.normal01(g, rows * cols)
        bias = synth.normal01(g, cols)
        ref = np.maximum(x.reshape(rows, cols) + bias[None, :], np.float32(0)).reshape(-1)
        got = oracle.bias_relu_f32(x, bias, rows, cols)
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    # bias of zeros reduces to the plain ReLU (x + 0 keeps x except -0 -> +0)
    x = synth.normal01(g, 4096)
    assert np.array_equal(oracle.bias_relu_f32(x, np.zeros(64, np.float32), 64, 64),
                          oracle.relu_f32(x))


def _bf16_value(bits):
    return float((np.uint32(bits) << np.uint32(16)).view(np.float32))


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_saxpy16_exact_rational(fmt):
    """One binary32 fma of the widened operands, then one rounding to the
    16-bit format: the exact rational alpha*x + y rounded twice."""
    g = np.random.Generator(np.random.PCG64(81 if fmt == "f16" else 82))
    x = g.integers(0, 1 << 16, size=2500, dtype=np.uint16)
    y = g.integers(0, 1 << 16, size=2500, dtype=np.uint16)
    if fmt == "f16":
        fin = ((x & 0x7C00) != 0x7C00) & ((y & 0x7C00) != 0x7C00)
        val = lambda b: float(np.uint16(b).view(np.float16))
        to_bits, fmt16 = exact.f16_bits, exact.BINARY16
        fn = oracle.saxpy_f16
    else:
        fin = ((x & 0x7F80) != 0x7F80) & ((y & 0x7F80) != 0x7F80)
        val = _bf16_value
        to_bits = lambda v: exact.f32_bits(v) >> 16
        fmt16 = exact.BFLOAT16
        fn = oracle.saxpy_bf16
    x, y = x[fin], y[fin]
    for alpha in (np.float32(2.5), np.float32(-0.3), np.float32(1.0)):
        got = fn(alpha, x, y)
        for xi, yi, r in zip(x, y, got):
            q = exact.f32_to_fraction(alpha) * exact.f32_to_fraction(val(xi)) + \
                exact.f32_to_fraction(val(yi))
            prod_neg = (math.copysign(1, float(alpha)) * math.copysign(1, val(xi))) < 0
            both_neg = prod_neg and math.copysign(1, val(yi)) < 0
            v32 = exact.round_rne(q, exact.BINARY32, zero_sign_negative=both_neg)
            if math.isinf(v32):
                ref = v32
            else:
                ref = exact.round_rne(exact.f32_to_fraction(v32), fmt16,
                                      zero_sign_negative=math.copysign(1, v32) < 0)
            assert to_bits(ref) == int(r), (fmt, alpha, hex(xi), hex(yi))


def test_relu16_vs_library_maximum():
    """numpy float16 and torch bfloat16 maximum agree on every input except
    the zeros (both return -0 for maximum(-0, +0), where IEEE 754-2019 gives
    +0) and NaN payloads (torch returns a canonical NaN): those are pinned by
    closed forms."""
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    zero = (h & 0x7FFF) == 0
    f16_nan = ((h & 0x7C00) == 0x7C00) & ((h & 0x03FF) != 0)
    got = oracle.relu_f16(h)
    ref = np.maximum(h.view(np.float16), np.float16(0)).view(np.uint16)
    ok = ~zero & ~f16_nan
    assert np.array_equal(got[ok], ref[ok])
    assert np.all(got[zero] == 0) and np.array_equal(got[f16_nan], h[f16_nan])
    bf_nan = ((h & 0x7F80) == 0x7F80) & ((h & 0x007F) != 0)
    got = oracle.relu_bf16(h)
    t = torch.from_numpy(h.view(np.int16)).view(torch.bfloat16)
    ref = torch.maximum(t, torch.zeros_like(t)).view(torch.int16).numpy().view(np.uint16)
    ok = ~zero & ~bf_nan
    assert np.array_equal(got[ok], ref[ok])
    assert np.all(got[zero] == 0) and np.array_equal(got[bf_nan], h[bf_nan])


def test_relu16_keeps_positive_subnormals():
    """Closed form at the edge a flushing environment would break: every
    positive subnormal of both 16-bit formats (bfloat16 subnormals are
    binary32 subnormals once widened) is kept bit for bit, every negative
    one becomes +0."""
    for fn, mant in ((oracle.relu_f16, 0x03FF), (oracle.relu_bf16, 0x007F)):
        pos = np.arange(1, mant + 1, dtype=np.uint16)
        neg = pos | np.uint16(0x8000)
        assert np.array_equal(fn(pos), pos)
        assert not np.any(fn(neg))


def test_copy_bitwise_including_nan_payloads():
    g = np.random.Generator(np.random.PCG64(61))
    bits = g.integers(0, 1 << 32, size=1 << 16, dtype=np.uint64).astype(np.uint32)
    bits[:8] = [0x7F800001, 0xFF800001, 0x7FA00000, 0x7FC00001, 0xFFFFFFFF,
                0x00000001, 0x80000000, 0x7F800000]   # signalling NaNs etc.
    x = bits.view(np.float32)
    assert np.array_equal(oracle.copy_f32(x).view(np.uint32), bits)
    assert oracle.copy_f32(np.zeros(0, np.float32)).size == 0


def _gather_brute(x_bits, stride):
    n = len(x_bits)
    return np.array([x_bits[(stride * i) % n] for i in range(n)], dtype=np.uint32)


def test_gather_brute_force_small():
    g = np.random.Generator(np.random.PCG64(71))
    for n in range(1, 18):
        bits = g.integers(0, 1 << 32, size=n, dtype=np.uint64).astype(np.uint32)
        for stride in sorted({1, 2, 3, n - 1 if n > 1 else 1, n, n + 1, 2 * n + 5,
                              (1 << 63) + 7, (1 << 64) - 1}):
            got = oracle.gather_f32(bits.view(np.float32), stride).view(np.uint32)
            assert np.array_equal(got, _gather_brute(bits, stride)), (n, stride)


def test_gather_closed_forms():
    x = synth.uniform_pm1(synth.rng(72), 1 << 16)
    # stride 1 is the contiguous copy
    assert np.array_equal(oracle.gather_f32(x, 1).view(np.uint32), x.view(np.uint32))
    # even n, stride 2: out[i] == out[i + n/2] == x[2i]
    n = x.size
    o = oracle.gather_f32(x, 2)
    assert np.array_equal(o[: n // 2], o[n // 2:])
    assert np.array_equal(o[: n // 2], x[0::2])
    # odd n, stride 2: a permutation of the input
    xo = x[: n - 1]
    oo = oracle.gather_f32(xo, 2)
    assert np.array_equal(np.sort(oo.view(np.uint32)), np.sort(xo.view(np.uint32)))
    # stride == n reads element 0 everywhere
    assert np.all(oracle.gather_f32(x, n) == x[0])


def test_gather_large_index_products_exact():
    """Index products beyond 2^64 must still be reduced exactly."""
    n = 1000003
    x = np.arange(n, dtype=np.uint32).view(np.float32)
    stride = (1 << 64) - 3
    o = oracle.gather_f32(x, stride).view(np.uint32)
    for i in (0, 1, 2, 999, 123456, n - 1):
        assert o[i] == (stride * i) % n


def test_gather_index_matches_python_integers():
    g = np.random.Generator(np.random.PCG64(73))
    for _ in range(2000):
        n = int(g.integers(1, 1 << 62))
        stride = int(g.integers(0, 1 << 63)) * 2 + int(g.integers(0, 2))
        i = int(g.integers(0, n))
        assert oracle.gather_index(n, stride, i) == (stride * i) % n
    n = (1 << 32) + 8
    assert oracle.gather_index(n, n - 1, 5) == n - 5
    assert oracle.gather_index(n, n - 1, 0) == 0


def test_gather_index_agrees_with_the_array_gather():
    x = np.arange(997, dtype=np.uint32).view(np.float32)
    for stride in (1, 2, 5, 996, 997, (1 << 64) - 1):
        o = oracle.gather_f32(x, stride).view(np.uint32)
        assert all(int(o[i]) == oracle.gather_index(997, stride, i) for i in range(997))


def _as_strided_ref(base, offset, sr, sc, rows, cols):
    """numpy's own strided view of the same memory, copied (bitwise)."""
    from numpy.lib.stride_tricks import as_strided
    b = base.view(np.uint32)
    v = as_strided(b[offset:], shape=(rows, cols), strides=(4 * sr, 4 * sc)) if sr >= 0 and \
        sc >= 0 else None
    if v is None:
        # negative strides: index explicitly (a different code path from the oracle's loop)
        r = np.arange(rows)[:, None]
        c = np.arange(cols)[None, :]
        v = b[offset + r * sr + c * sc]
    return np.ascontiguousarray(v).reshape(-1)


def test_copy2d_vs_numpy_strided_views():
    g = np.random.Generator(np.random.PCG64(91))
    base = g.integers(0, 1 << 32, size=1 << 16, dtype=np.uint32).view(np.float32)
    cases = [(0, 1, 1, 1, 1), (5, 7, 1, 3, 7), (0, 1, 2, 1, 1000),      # 1-D x[::2]
             (3, 64, 1, 10, 50),                                         # submatrix
             (0, 1, 128, 128, 96), (1, 1, 200, 150, 199),                # transposed views
             (17, 300, 3, 20, 40), (0, 0, 1, 5, 9),                      # broadcast rows
             (8000, -64, 1, 100, 64), (9000, 1, -3, 7, 500), (40000, -129, -1, 33, 64)]
    for off, sr, sc, rows, cols in cases:
        got = oracle.copy2d_f32(base, off, sr, sc, rows, cols).view(np.uint32)
        ref = _as_strided_ref(base, off, sr, sc, rows, cols)
        assert np.array_equal(got, ref), (off, sr, sc, rows, cols)


def test_copy2d_closed_forms():
    x = synth.uniform_pm1(synth.rng(92), 96 * 80)
    # contiguous strides are a plain copy
    assert np.array_equal(oracle.copy2d_f32(x, 0, 80, 1, 96, 80), x)
    # transposing twice gives the original back
    t = oracle.copy2d_f32(x, 0, 1, 80, 80, 96)            # (80 x 96) = x^T
    assert np.array_equal(oracle.copy2d_f32(t, 0, 1, 96, 96, 80), x)
    assert np.array_equal(t.reshape(80, 96), x.reshape(96, 80).T)
    # rows = 1 with stride 2 is x[::2]
    assert np.array_equal(oracle.copy2d_f32(x, 0, 0, 2, 1, x.size // 2), x[::2])
    with pytest.raises(ValueError):
        oracle.copy2d_f32(x, 0, 80, 1, 97, 80)


# --------------------------------------------------------------------------
# ulp distance
# --------------------------------------------------------------------------

def test_ulp_distance_closed_forms():
    u = oracle.ulp_distance_f32
    one = np.float32(1.0)
    assert u(one, np.nextafter(one, np.float32(2))) == 1
    assert u(0.0, -0.0) == 0
    assert u(np.float32(1e-45), np.float32(-1e-45)) == 2
    assert u(np.finfo(np.float32).max, np.float32(np.inf)) == 1
    assert u(one, one) == 0
    assert u(one, np.float32(2.0)) == 1 << 23


# --------------------------------------------------------------------------
# Scalar-broadcast and unary maps
# --------------------------------------------------------------------------

MAP_ALPHAS = (np.float32(2.5), np.float32(-0.3), np.float32(1.0) / np.float32(3.0),
              np.float32(1e-30), np.float32(-3e38))


def test_scale_and_add_scalar_f32_vs_numpy():
    g = synth.rng(91)
    x = np.concatenate([synth.uniform_pm1(g, 1 << 16), _random_f32_bits(1 << 16, 92, False),
                        F32_SPECIALS])
    for alpha in MAP_ALPHAS + (np.float32(np.inf), np.float32(np.nan), np.float32(-0.0)):
        with np.errstate(all="ignore"):
            for got, ref in ((oracle.scale_f32(alpha, x), alpha * x),
                             (oracle.add_scalar_f32(alpha, x), x + alpha)):
                assert _nan_class_equal(got.view(np.uint32), ref.view(np.uint32),
                                        np.isnan(got), np.isnan(ref)), alpha


def test_scale_and_add_scalar_f32_exact_rational():
    x = np.concatenate([_random_f32_bits(1200, 93), synth.uniform_pm1(synth.rng(94), 800)])
    for alpha in MAP_ALPHAS:
        fa = exact.f32_to_fraction(alpha)
        for xi, r in zip(x, oracle.scale_f32(alpha, x)):
            neg = (math.copysign(1, float(alpha)) * math.copysign(1, float(xi))) < 0
            ref = exact.round_rne(fa * exact.f32_to_fraction(xi), exact.BINARY32,
                                  zero_sign_negative=neg)
            assert exact.f32_bits(ref) == exact.f32_bits(float(r)), (alpha, xi)
        for xi, r in zip(x, oracle.add_scalar_f32(alpha, x)):
            both_neg = math.copysign(1, float(alpha)) < 0 and math.copysign(1, float(xi)) < 0
            ref = exact.round_rne(fa + exact.f32_to_fraction(xi), exact.BINARY32,
                                  zero_sign_negative=both_neg)
            assert exact.f32_bits(ref) == exact.f32_bits(float(r)), (alpha, xi)


def test_scalar_map_closed_forms():
    """scale by 1 is the identity and by -1 flips the sign bit; scale by 2 is
    the exact doubling x + x; adding -0 is the identity (all non-NaN x)."""
    x = np.concatenate([_random_f32_bits(1 << 16, 95, False), F32_SPECIALS])
    x = x[~np.isnan(x)]
    b = x.view(np.uint32)
    assert np.array_equal(oracle.scale_f32(1.0, x).view(np.uint32), b)
    assert np.array_equal(oracle.scale_f32(-1.0, x).view(np.uint32), b ^ np.uint32(0x80000000))
    assert np.array_equal(oracle.scale_f32(2.0, x).view(np.uint32),
                          oracle.add_f32(x, x).view(np.uint32))
    assert np.array_equal(oracle.add_scalar_f32(-0.0, x).view(np.uint32), b)


def test_sqrt_f32_vs_numpy_and_exact_root():
    """numpy's float32 sqrt (correctly rounded, as IEEE 754 requires) on random
    patterns of every class, and the exact rational root on positive samples
    including subnormals."""
    x = np.concatenate([_random_f32_bits(1 << 18, 96, False), F32_SPECIALS,
                        np.abs(_random_f32_bits(1 << 12, 97))])
    got = oracle.sqrt_f32(x)
    with np.errstate(all="ignore"):
        ref = np.sqrt(x)
    assert _nan_class_equal(got.view(np.uint32), ref.view(np.uint32), np.isnan(got), np.isnan(ref))
    pos = np.abs(_random_f32_bits(2000, 98))
    pos = np.concatenate([pos, (np.arange(1, 200, dtype=np.uint32) * 40503).view(np.float32)])
    for xi, r in zip(pos, oracle.sqrt_f32(pos)):
        ref = exact.sqrt_rne(exact.f32_to_fraction(xi), exact.BINARY32)
        assert exact.f32_bits(ref) == exact.f32_bits(float(r)), xi
    neg0 = oracle.sqrt_f32(np.array([-0.0, np.inf, -1.0, -np.inf], np.float32))
    assert neg0.view(np.uint32)[0] == 0x80000000 and neg0[1] == np.inf
    assert np.isnan(neg0[2]) and np.isnan(neg0[3])


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_sqrt16_every_pattern_is_the_correctly_rounded_root(fmt):
    """Every 16-bit pattern: a positive finite x gives the exact root rounded
    once to the 16-bit format (so the binary32 detour never double-rounds
    wrongly), -0 gives -0, +inf gives +inf, negatives and NaNs give NaN."""
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    if fmt == "f16":
        got, fmt16, to_bits = oracle.sqrt_f16(h), exact.BINARY16, exact.f16_bits
        val = lambda b: float(np.uint16(b).view(np.float16))
        exp_mask, man_mask = 0x7C00, 0x03FF
    else:
        got, fmt16 = oracle.sqrt_bf16(h), exact.BFLOAT16
        to_bits = lambda v: exact.f32_bits(v) >> 16
        val = _bf16_value
        exp_mask, man_mask = 0x7F80, 0x007F
    nan_out = ((got & exp_mask) == exp_mask) & ((got & man_mask) != 0)
    for b, r, is_nan in zip(h, got, nan_out):
        v = val(b)
        if math.isnan(v) or v < 0:
            assert is_nan, hex(b)
        elif v == 0 or math.isinf(v):
            assert r == b, hex(b)
        else:
            assert to_bits(exact.sqrt_rne(Fraction(v), fmt16)) == int(r), hex(b)


@pytest.mark.parametrize("fmt", ["f16", "bf16"])
def test_scalar_maps16_vs_library_and_exact_rational(fmt):
    """16-bit scale / add-scalar: against the library's own binary32 op and
    RNE narrowing (numpy float16; torch bfloat16) on every pattern, and the
    exact rational result rounded twice on a sample."""
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    if fmt == "f16":
        wide = h.view(np.float16).astype(np.float32)
        narrow = lambda f: f.astype(np.float16).view(np.uint16)
        nan = lambda u: ((u & 0x7C00) == 0x7C00) & ((u & 0x03FF) != 0)
        fns = (oracle.scale_f16, oracle.add_scalar_f16)
        fmt16, to_bits = exact.BINARY16, exact.f16_bits
        val = lambda b: float(np.uint16(b).view(np.float16))
    else:
        wide = oracle.bf16_to_f32(h)
        narrow = lambda f: torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy() \
            .view(np.uint16)
        nan = lambda u: ((u & 0x7F80) == 0x7F80) & ((u & 0x007F) != 0)
        fns = (oracle.scale_bf16, oracle.add_scalar_bf16)
        fmt16 = exact.BFLOAT16
        to_bits = lambda v: exact.f32_bits(v) >> 16
        val = _bf16_value
    for alpha in MAP_ALPHAS:
        with np.errstate(all="ignore"):
            refs = (narrow(alpha * wide), narrow(wide + alpha))
        for fn, ref in zip(fns, refs):
            got = fn(alpha, h)
            gn, rn = nan(got), nan(ref)
            assert np.array_equal(gn, rn) and np.array_equal(got[~gn], ref[~rn]), (fmt, alpha)
    g = np.random.Generator(np.random.PCG64(99 if fmt == "f16" else 100))
    sample = g.integers(0, 1 << 16, size=600, dtype=np.uint16)
    sample = sample[~nan(sample) & np.isfinite([val(b) for b in sample])]
    for alpha in MAP_ALPHAS[:3]:
        fa, sa = exact.f32_to_fraction(alpha), math.copysign(1, float(alpha))
        for fn, is_mul in ((fns[0], True), (fns[1], False)):
            for b, r in zip(sample, fn(alpha, sample)):
                v = val(b)
                sv = math.copysign(1, v)
                q = fa * Fraction(v) if is_mul else Fraction(v) + fa
                # sign of an exact zero: product of the signs / both addends negative
                neg = sa * sv < 0 if is_mul else (sa < 0 and sv < 0)
                v32 = exact.round_rne(q, exact.BINARY32, zero_sign_negative=neg)
                ref = v32 if math.isinf(v32) else exact.round_rne(
                    Fraction(v32), fmt16, zero_sign_negative=math.copysign(1, v32) < 0)
                assert to_bits(ref) == int(r), (fmt, alpha, hex(b))


def test_abs_vs_library_and_bit_identity():
    x = np.concatenate([_random_f32_bits(1 << 16, 101, False), F32_SPECIALS])
    got = oracle.abs_f32(x)
    assert np.array_equal(got.view(np.uint32), np.abs(x).view(np.uint32))   # NaN payloads too
    assert np.array_equal(got.view(np.uint32) | (x.view(np.uint32) & np.uint32(0x80000000)),
                          x.view(np.uint32))
    h = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    g16 = oracle.abs_f16(h)
    assert np.array_equal(g16, np.abs(h.view(np.float16)).view(np.uint16))
    gbf = oracle.abs_bf16(h)
    assert np.array_equal(gbf | (h & np.uint16(0x8000)), h) and not np.any(gbf & 0x8000)
