"""Every 16-bit input through the HIP path, against the oracle:

* ew_add_f16 / ew_add_bf16 on all 2^32 (a, b) bit-pattern pairs;
* ew_saxpy_f16 / ew_saxpy_bf16 on all 2^32 (x, y) pairs, for alpha = 2.5
  (the SAXPY workload's) and alpha = fl32(1/3) (inexact, so the binary32 fma
  rounds on almost every pair before the 16-bit rounding);
* ew_relu_f16 / ew_relu_bf16 on all 65,536 patterns;
* the scalar-broadcast and unary maps (scale, add-scalar with several
  alphas; sqrt; abs) on all 65,536 patterns of each 16-bit format.

Bitwise, except that a NaN matches any NaN for the arithmetic operations
(ReLU and abs pass NaNs through bitwise).  The pairs go through in four launches
of 2^30 elements (the first operand = the high half-word of the pair index,
the second = the low one), with the first operand misaligned, so the body
runs the element-aligned load path.  The oracle runs on the host, split over
the process's cores (at most 16).
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

import memory_bound_elementwise_amd as ew
import oracle
from tests.gpu_util import download, upload

pytestmark = pytest.mark.gpu

CHUNK = 1 << 30                       # pairs per launch; four launches cover 2^32
NAN16 = {"add_f16": (0x7C00, 0x03FF), "add_bf16": (0x7F80, 0x007F),
         "saxpy_f16": (0x7C00, 0x03FF), "saxpy_bf16": (0x7F80, 0x007F)}
THIRD = float(np.float32(1.0) / np.float32(3.0))


def _oracle_parallel(fn, a, b):
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    step = -(-a.size // workers)
    out = np.empty_like(a)

    def part(lo):
        out[lo:lo + step] = fn(a[lo:lo + step], b[lo:lo + step])
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(part, range(0, a.size, step)))
    return out


def _all_pairs(op, run, ref_fn):
    """run(first, second) -> the HIP result for one chunk of pairs;
    ref_fn(first, second) -> the oracle's."""
    exp, man = NAN16[op]
    low = np.tile(np.arange(1 << 16, dtype=np.uint16), CHUNK >> 16)
    for k in range((1 << 32) // CHUNK):
        print(f"[exhaustive] {op} high half-words {k * (CHUNK >> 16)}..."
              f"{(k + 1) * (CHUNK >> 16) - 1}", flush=True)
        high = np.repeat(np.arange(k * (CHUNK >> 16), (k + 1) * (CHUNK >> 16),
                                   dtype=np.uint32).astype(np.uint16), 1 << 16)
        got = run(high, low)
        torch.cuda.empty_cache()
        ref = _oracle_parallel(ref_fn, high, low)
        bad = np.flatnonzero(got != ref)
        if bad.size:                  # only NaN results may differ (in payload)
            g, r = got[bad], ref[bad]
            gn = ((g & exp) == exp) & ((g & man) != 0)
            rn = ((r & exp) == exp) & ((r & man) != 0)
            wrong = bad[~(gn & rn)]
            assert wrong.size == 0, (
                f"{op}: {wrong.size} mismatches, first pair {high[wrong[0]]:#06x}, "
                f"{low[wrong[0]]:#06x}: got {got[wrong[0]]:#06x}, want {ref[wrong[0]]:#06x}")
        del high, got, ref, bad


@pytest.mark.parametrize("op", ["add_f16", "add_bf16"])
def test_add_on_every_16bit_input_pair(op):
    fn = getattr(ew, "ew_" + op)

    def run(first, second):
        a, ka = upload(first, 1)
        b, kb = upload(second, 0)
        c, kc = upload(np.zeros(first.size, np.uint16), 3)
        fn(a, b, c)
        torch.cuda.synchronize()
        return download(c, 2)
    _all_pairs(op, run, getattr(oracle, op))


@pytest.mark.parametrize("alpha", [2.5, THIRD])
@pytest.mark.parametrize("op", ["saxpy_f16", "saxpy_bf16"])
def test_saxpy_on_every_16bit_input_pair(op, alpha):
    fn = getattr(ew, "ew_" + op)

    def run(x, y):
        xd, kx = upload(x, 1)
        yd, ky = upload(y, 0)
        fn(alpha, xd, yd)
        torch.cuda.synchronize()
        return download(yd, 2)
    _all_pairs(op, run, lambda x, y: getattr(oracle, op)(alpha, x, y))


@pytest.mark.parametrize("op", ["relu_f16", "relu_bf16"])
def test_relu_on_every_16bit_pattern(op):
    x = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    xd, kx = upload(x, 1)
    yd, ky = upload(np.zeros(x.size, np.uint16), 0)
    getattr(ew, "ew_" + op)(xd, yd)
    torch.cuda.synchronize()
    got = download(yd, 2)
    ref = getattr(oracle, op)(x)
    assert np.array_equal(got, ref), np.flatnonzero(got != ref)[:10]


MAP_ALPHAS = (2.5, THIRD, -1.0e-5, 65504.0, float(np.float32(3.0e38)))


@pytest.mark.parametrize("op", ["scale_f16", "scale_bf16", "add_scalar_f16", "add_scalar_bf16",
                                "sqrt_f16", "sqrt_bf16", "abs_f16", "abs_bf16"])
def test_maps_on_every_16bit_pattern(op):
    """Every pattern, misaligned by one element; the scalar maps under
    several alphas (inexact, tiny, at the binary16 maximum, near the
    binary32 one)."""
    x = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    scalar = op.rsplit("_", 1)[0] in ew.SCALAR_MAPS
    exp, man = (0x7C00, 0x03FF) if op.endswith("_f16") else (0x7F80, 0x007F)
    for alpha in MAP_ALPHAS if scalar else (None,):
        xd, kx = upload(x, 1)
        yd, ky = upload(np.zeros(x.size, np.uint16), 0)
        fn = getattr(ew, "ew_" + op)
        fn(alpha, xd, yd) if scalar else fn(xd, yd)
        torch.cuda.synchronize()
        got = download(yd, 2)
        ref = getattr(oracle, op)(alpha, x) if scalar else getattr(oracle, op)(x)
        if op.startswith("abs"):
            assert np.array_equal(got, ref), np.flatnonzero(got != ref)[:10]
            continue
        gn = ((got & exp) == exp) & ((got & man) != 0)
        rn = ((ref & exp) == exp) & ((ref & man) != 0)
        bad = np.flatnonzero((gn != rn) | (~gn & (got != ref)))
        assert bad.size == 0, (op, alpha, [hex(v) for v in x[bad[:5]]],
                               [hex(v) for v in got[bad[:5]]], [hex(v) for v in ref[bad[:5]]])
