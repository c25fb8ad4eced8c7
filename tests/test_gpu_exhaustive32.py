"""Every binary32 bit pattern through the HIP path, against the oracle:

* ew_relu_f32 on all 2^32 patterns, bitwise (ReLU read as IEEE maximum(x, +0):
  -0 and negatives become +0, NaNs pass through with their payload);
* ew_add_f32 with every pattern once as the first operand, paired with
  h(a) = a * 0x9E3779B1 mod 2^32 (odd multiplier, so a bijection: every
  pattern is also the second operand exactly once), bitwise except that a
  NaN matches any NaN;
* ew_saxpy_f32 (alpha = 2.5, the SAXPY workload's) with every pattern once
  as x and once as y, paired the same way, against the oracle's fmaf:
  bitwise except that a NaN matches any NaN (the 1-ulp allowance is not
  used);
* ew_sqrt_f32 on all 2^32 patterns against the correctly rounded root, and
  ew_scale_f32 / ew_add_scalar_f32 with alpha = fl32(1/3) on all 2^32
  patterns: bitwise except that a NaN matches any NaN.

Four launches of 2^30 elements each, the input misaligned by one element.
The oracle runs on the host, split over the process's cores (at most 16).
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

CHUNK = 1 << 30
MULT = np.uint32(0x9E3779B1)


def _parallel(fn, *arrays):
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    n = arrays[0].size
    step = -(-n // workers)
    out = np.empty_like(arrays[0])

    def part(lo):
        out[lo:lo + step] = fn(*(a[lo:lo + step] for a in arrays))
    with ThreadPoolExecutor(max_workers=workers) as ex:
        list(ex.map(part, range(0, n, step)))
    return out


def _chunk(k):
    print(f"[exhaustive32] patterns {k * CHUNK:#010x}..{(k + 1) * CHUNK - 1:#010x}", flush=True)
    return np.arange(k * CHUNK, (k + 1) * CHUNK, dtype=np.uint32)


def test_relu_on_every_f32_pattern():
    for k in range((1 << 32) // CHUNK):
        bits = _chunk(k)
        x = bits.view(np.float32)
        xd, kx = upload(x, 1)
        yd, ky = upload(np.zeros(CHUNK, np.float32), 0)
        ew.ew_relu_f32(xd, yd)
        torch.cuda.synchronize()
        got = download(yd, 4).view(np.uint32)
        del xd, kx, yd, ky
        torch.cuda.empty_cache()
        ref = _parallel(oracle.relu_f32, x).view(np.uint32)
        bad = np.flatnonzero(got != ref)
        assert bad.size == 0, (f"{bad.size} mismatches, first x={bits[bad[0]]:#010x}: "
                               f"got {got[bad[0]]:#010x}, want {ref[bad[0]]:#010x}")
        del bits, x, got, ref


def _both_operands(run, ref_fn):
    """run(a, b) -> the HIP result for one chunk; ref_fn(a, b) -> the oracle's."""
    for k in range((1 << 32) // CHUNK):
        a_bits = _chunk(k)
        b_bits = a_bits * MULT                      # wraps mod 2^32
        a, b = a_bits.view(np.float32), b_bits.view(np.float32)
        got = run(a, b)
        torch.cuda.empty_cache()
        ref = _parallel(ref_fn, a, b).view(np.uint32)
        bad = np.flatnonzero(got != ref)
        if bad.size:                                # NaN payloads may differ
            g, r = got[bad], ref[bad]
            both_nan = ((g & 0x7FFFFFFF) > 0x7F800000) & ((r & 0x7FFFFFFF) > 0x7F800000)
            wrong = bad[~both_nan]
            assert wrong.size == 0, (
                f"{wrong.size} mismatches, first a={a_bits[wrong[0]]:#010x} "
                f"b={b_bits[wrong[0]]:#010x}: got {got[wrong[0]]:#010x}, "
                f"want {ref[wrong[0]]:#010x}")
        del a_bits, b_bits, a, b, got, ref, bad


def test_add_with_every_f32_pattern_as_each_operand():
    def run(a, b):
        ad, ka = upload(a, 1)
        bd, kb = upload(b, 0)
        cd, kc = upload(np.zeros(a.size, np.float32), 2)
        ew.ew_add_f32(ad, bd, cd)
        torch.cuda.synchronize()
        return download(cd, 4).view(np.uint32)
    _both_operands(run, oracle.add_f32)


def test_saxpy_with_every_f32_pattern_as_x_and_as_y():
    def run(x, y):
        xd, kx = upload(x, 1)
        yd, ky = upload(y, 0)
        ew.ew_saxpy_f32(2.5, xd, yd)
        torch.cuda.synchronize()
        return download(yd, 4).view(np.uint32)
    _both_operands(run, lambda x, y: oracle.saxpy_f32(2.5, x, y))


THIRD = float(np.float32(1.0) / np.float32(3.0))


def _every_pattern_map(launch, ref_fn):
    """launch(x_view, y_view) runs the HIP map; ref_fn(x) is the oracle's."""
    for k in range((1 << 32) // CHUNK):
        bits = _chunk(k)
        x = bits.view(np.float32)
        xd, kx = upload(x, 1)
        yd, ky = upload(np.zeros(CHUNK, np.float32), 0)
        launch(xd, yd)
        torch.cuda.synchronize()
        got = download(yd, 4).view(np.uint32)
        del xd, kx, yd, ky
        torch.cuda.empty_cache()
        ref = _parallel(ref_fn, x).view(np.uint32)
        bad = np.flatnonzero(got != ref)
        if bad.size:
            g, r = got[bad], ref[bad]
            both_nan = ((g & 0x7FFFFFFF) > 0x7F800000) & ((r & 0x7FFFFFFF) > 0x7F800000)
            wrong = bad[~both_nan]
            assert wrong.size == 0, (f"{wrong.size} mismatches, first x={bits[wrong[0]]:#010x}: "
                                     f"got {got[wrong[0]]:#010x}, want {ref[wrong[0]]:#010x}")
        del bits, x, got, ref


def test_sqrt_on_every_f32_pattern():
    _every_pattern_map(ew.ew_sqrt_f32, oracle.sqrt_f32)


def test_scale_and_add_scalar_on_every_f32_pattern():
    _every_pattern_map(lambda x, y: ew.ew_scale_f32(THIRD, x, y),
                       lambda x: oracle.scale_f32(THIRD, x))
    _every_pattern_map(lambda x, y: ew.ew_add_scalar_f32(THIRD, x, y),
                       lambda x: oracle.add_scalar_f32(THIRD, x))
