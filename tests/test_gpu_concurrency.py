"""Calls from several host threads at once, each thread on its own stream,
against the oracle.

The library keeps no per-call state outside the call: the launch table is
read under a lock and the per-device properties are cached atomically, and
the ctypes binding releases the interpreter lock during a call, so the
calls really overlap on the host and on the GPU.  Four threads each run
rounds of the fp32 add (ragged n, misaligned pointers), the ReLU, the
stride-3 gather (the pass kernel, which stages through LDS) and a prepared
device-table batch, every round into buffers of its own; a fifth thread
rewrites the fp32 add's launch rows meanwhile (rows change launch shapes,
never results).  After all threads finish, every output is compared with
the oracle on every element.
"""
import os
import threading

import numpy as np
import pytest
import torch

import memory_bound_elementwise_amd as ew
import oracle
import synth
from tests.gpu_util import DEV, download, mismatches, upload

pytestmark = pytest.mark.gpu

THREADS = 4
ROUNDS = 24
KINDS = ("add_f32", "relu_f32", "gather_f32", "batch_add_f32")


def _f32(g, n):
    return (2 * g.random(n) - 1).astype(np.float32)


def _case(t, k):
    """Inputs, expected output and the call of round k of thread t."""
    g = synth.rng(7000 + 100 * t + k)
    kind = KINDS[(t + k) % len(KINDS)]
    n = int(g.integers(50_000, 300_000))
    keep = []
    if kind == "batch_add_f32":
        sizes = [int(v) for v in g.integers(0, 5000, size=40)]
        a, b = _f32(g, sum(sizes)), _f32(g, sum(sizes))
        da, ba = upload(a, off=1)
        db, bb = upload(b, off=2)
        out = torch.empty(sum(sizes) + 8, dtype=torch.float32, device=DEV)
        items, pos = [], 0
        for m in sizes:
            items.append((out[3 + pos:3 + pos + m], da[pos:pos + m], db[pos:pos + m], m))
            pos += m
        batch = ew.EwBatch("add_f32", items)
        keep += [ba, bb, batch]
        ref = oracle.add_f32(a, b)
        return kind, (lambda s: batch(stream=s)), out[3:3 + pos], ref, keep
    a = _f32(g, n)
    da, ba = upload(a, off=int(g.integers(0, 4)))
    out_base = torch.empty(n + 8, dtype=torch.float32, device=DEV)
    out = out_base[1:1 + n]
    keep += [ba, out_base]
    if kind == "add_f32":
        b = _f32(g, n)
        db, bb = upload(b, off=int(g.integers(0, 4)))
        keep.append(bb)
        return kind, (lambda s: ew.ew_add_f32(da, db, out, stream=s)), out, \
            oracle.add_f32(a, b), keep
    if kind == "relu_f32":
        return kind, (lambda s: ew.ew_relu_f32(da, out, stream=s)), out, oracle.relu_f32(a), keep
    if n % 3 == 0:                    # gcd(3, n) == 1: the pass kernel
        n -= 1
    out = out_base[1:1 + n]
    src = da[:n]
    return kind, (lambda s: ew.ew_gather_f32(src, out, 3, stream=s)), out, \
        oracle.gather_f32(a[:n], 3), keep


def test_threads_on_their_own_streams_match_the_oracle():
    print("[concurrency] 4 threads x 24 rounds, launch rows rewritten meanwhile", flush=True)
    cases = [[_case(t, k) for k in range(ROUNDS)] for t in range(THREADS)]
    torch.cuda.synchronize()
    errors = []
    start = threading.Barrier(THREADS + 1)

    def worker(t):
        try:
            s = torch.cuda.Stream(device=DEV)          # default priority
            handle = s.cuda_stream
            start.wait()
            for _, call, _, _, _ in cases[t]:
                call(handle)
            s.synchronize()
        except Exception as exc:                    # reported after the join
            errors.append(f"thread {t}: {exc!r}")

    def rewriter():
        try:
            start.wait()
            for k in range(4 * ROUNDS):
                row = (256, 8, 1) if k % 2 else (512, 2, 2)
                ew.ew_set_launch_row("add_f32", 0, *row)
                ew.ew_set_launch_row("add_f32", 1 << 22, *row)
        except Exception as exc:
            errors.append(f"rewriter: {exc!r}")

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(THREADS)]
    threads.append(threading.Thread(target=rewriter))
    try:
        for th in threads:
            th.start()
        for th in threads:
            th.join(timeout=120)
        assert not any(th.is_alive() for th in threads), "a thread did not finish"
    finally:
        ew.ew_reset_launch_config()
        if os.path.exists(ew.LAUNCH_TABLE):
            ew.ew_load_launch_table(ew.LAUNCH_TABLE)
    torch.cuda.synchronize()
    assert not errors, errors
    bad = []
    for t in range(THREADS):
        for k, (kind, _, out, ref, _) in enumerate(cases[t]):
            op = "add_f32" if kind == "batch_add_f32" else kind
            m = mismatches(op, download(out, 4), ref)
            if m.size:
                bad.append((t, k, kind, int(m.size), int(m[0])))
    assert not bad, bad[:8]
