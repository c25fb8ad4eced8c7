"""The batched entry points against the oracle, item by item: the host-array
form (ew_batch: at most EW_BATCH_MAX items per launch, here two launches) and
the device-table form (ew_batch_build + ew_batch_run: one launch for every
item).

Every batchable operation runs 100 items in one call: sizes 0 to 17, ragged
and a few tiles long, every pointer at its own element offset, all outputs in
one sentinel-filled arena whose untouched bytes must survive (guard bands);
SAXPY updates its y items in place.  Also: shared inputs across items, forced
launch rows (a grid smaller than the tile count, unroll clamped to 4), 1500
items in one table launch, and graph replay.
"""
import os

import numpy as np
import pytest
import torch

import memory_bound_elementwise_amd as ew
import synth
from tests.gpu_util import DEV, ELEM, NP_DTYPE, mismatches, upload
from tests.test_gpu_parity import (IN_PLACE, SCALAR_MAPS, SENTINEL, TWO_INPUT, UNARY_MAPS,
                                   _force_launch, _oracle, _pool)

pytestmark = pytest.mark.gpu

BATCH_OPS = ["add_f32", "add_f16", "add_bf16", "saxpy_f32", "relu_f32", "copy_f32",
             "add_relu_f32", "saxpy_relu_f32", "saxpy_f16", "saxpy_bf16", "relu_f16",
             "relu_bf16"] + list(SCALAR_MAPS + UNARY_MAPS)
GUARD = 64


def _sizes(seed, count=100, big=300_001):
    g = synth.rng(seed)
    fixed = list(range(18)) + [31, 33, 1000, 4099, 65537, big]
    rest = g.integers(0, 3000, size=count - len(fixed)).tolist()
    sizes = fixed + rest
    g.shuffle(sizes)
    return [int(v) for v in sizes]


def _run_batch(op, sizes, seed, alpha=2.5, shared_input=False, form="table"):
    """One batched call over len(sizes) items -- form "host": ew_batch;
    "table": ew_batch_build, the image copied to the device, ew_batch_run --
    returns failure strings."""
    es = ELEM[op]
    dt = NP_DTYPE[es]
    vec = 16 // es
    two = op in TWO_INPUT
    g = synth.rng(seed + 1)
    total = sum(sizes) + 32 * len(sizes) + 64
    pools = [_pool(op, total, seed + k) for k in range(2)]
    dev = [upload(p)[1] for p in pools]
    # inputs: consecutive slices of the pools at random element offsets
    in_offs, cur = [], 0
    for n in sizes:
        o = 0 if shared_input else cur + int(g.integers(0, vec))
        in_offs.append(o)
        cur = o + n + 8
    # outputs: one arena with guard bands
    out_offs, cur = [], 0
    for n in sizes:
        start = -(-(cur + GUARD) // 256) * 256 + int(g.integers(0, vec)) * es
        out_offs.append(start)
        cur = start + n * es + GUARD
    size = -(-(cur + 256) // 256) * 256
    host = np.full(size, SENTINEL, np.uint8)
    if op in IN_PLACE:                    # y is the output span itself
        for n, o, io in zip(sizes, out_offs, in_offs):
            host[o:o + n * es] = pools[1][io:io + n].view(np.uint8)
    arena = torch.from_numpy(host).to(DEV)
    base = arena.data_ptr()
    items = []
    for n, o, io in zip(sizes, out_offs, in_offs):
        in1 = dev[1].data_ptr() + io * es if (two and op not in IN_PLACE) else None
        items.append((base + o, dev[0].data_ptr() + io * es, in1, n))
    stream = torch.cuda.current_stream().cuda_stream
    if form == "host":
        ew.ew_batch(op, items, alpha=alpha, stream=stream)
    else:
        plan, image = ew.ew_batch_build(op, items)
        table = torch.frombuffer(bytearray(image), dtype=torch.uint8)[:plan.bytes].to(DEV)
        ew.ew_batch_run(plan, alpha, table, stream=stream)
    torch.cuda.synchronize()
    res = arena.cpu().numpy()
    fails, written = [], np.zeros(size, bool)
    for k, (n, o, io) in enumerate(zip(sizes, out_offs, in_offs)):
        written[o:o + n * es] = True
        got = res[o:o + n * es].view(dt)
        ins = [pools[0][io:io + n], pools[1][io:io + n]]
        ref = _oracle(op, ins, n, alpha=alpha)
        bad = mismatches(op, got, ref)
        if bad.size:
            fails.append(f"{op} item {k} n={n} out_off={o % 16} in_off={io}: {bad.size} "
                         f"mismatches, first at {bad[0]}")
    if np.any(res[~written] != SENTINEL):
        fails.append(f"{op}: bytes written outside the items' outputs")
    return fails


@pytest.mark.parametrize("form", ["host", "table"])
@pytest.mark.parametrize("op", BATCH_OPS)
def test_batch_matches_the_oracle_item_by_item(op, form):
    print(f"[batch] {op} {form}", flush=True)
    fails = _run_batch(op, _sizes(600 + BATCH_OPS.index(op)), 650, form=form)
    assert not fails, fails[:5]


@pytest.mark.parametrize("form", ["host", "table"])
def test_batch_items_may_share_an_input(form):
    print(f"[batch] shared input {form}", flush=True)
    for op in ("add_f32", "scale_bf16", "sqrt_f16"):
        fails = _run_batch(op, _sizes(670, count=60), 671, shared_input=True, form=form)
        assert not fails, fails[:5]


def test_batch_table_runs_many_items_in_one_launch():
    """1500 items (16 times what one host-array launch carries) through one
    table, with EW_LOG on in a child process: exactly one launch line."""
    print("[batch] 1500 items, one launch", flush=True)
    import subprocess
    import sys
    from tests.conftest import ROOT
    code = (
        "import sys; sys.path.insert(0, %r)\n"
        "from tests.test_gpu_batch import _run_batch, _sizes\n"
        "f = _run_batch('add_bf16', _sizes(700, count=1500, big=70_001), 701)\n"
        "print('FAILS', len(f), f[:3])\n" % ROOT)
    env = dict(os.environ, EW_LOG="1")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                       timeout=300, env=env, cwd=ROOT)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "FAILS 0 []" in r.stdout, r.stdout[-2000:]
    launches = [ln for ln in r.stderr.splitlines() if ln.startswith("[ew] add_bf16")]
    assert len(launches) == 1 and "batch table" in launches[0], launches[:3]


def test_batch_under_forced_launch_rows():
    """A grid smaller than the tile count (the grid-stride loop crosses item
    boundaries), block sizes 64..1024, and unroll 8 clamped to 4."""
    print("[batch] forced rows", flush=True)
    try:
        for op in ("add_f32", "relu_bf16", "saxpy_f16"):
            for block, bpc, unroll in ((64, 1, 1), (256, 1, 2), (1024, 1, 8), (128, 2, 4)):
                _force_launch(op, block, bpc, unroll)
                for form in ("host", "table"):
                    fails = _run_batch(op, _sizes(680, count=70, big=2_000_003), 681, form=form)
                    assert not fails, (op, block, bpc, unroll, form, fails[:3])
    finally:
        ew.ew_reset_launch_config()
        if os.path.exists(ew.LAUNCH_TABLE):
            ew.ew_load_launch_table(ew.LAUNCH_TABLE)


@pytest.mark.parametrize("form", ["host", "table"])
def test_batch_call_in_a_graph_replays_with_new_data(form):
    """A batched call captured into a graph: its items' arguments (or the
    device table) are fixed at capture, the data may change; every replay
    matches the oracle."""
    print(f"[batch] graph {form}", flush=True)
    import oracle
    m, count = 5003, 70
    a = torch.empty(m * count + 8, device=DEV)
    b = torch.empty_like(a)
    c = torch.empty_like(a)
    items = [(c[k * m + 1:(k + 1) * m + 1], a[k * m:(k + 1) * m], b[k * m + 3:(k + 1) * m + 3], m)
             for k in range(count)]
    batch = ew.EwBatch("add_f32", items, table=(form == "table"))
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        batch(stream=s)                        # warm-up outside the capture
    s.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=s):
        batch(stream=s)
    for r in range(3):
        g = synth.rng(690 + r)
        ha, hb = synth.uniform_pm1(g, a.numel()), synth.uniform_pm1(g, b.numel())
        a.copy_(torch.from_numpy(ha))
        b.copy_(torch.from_numpy(hb))
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        hc = c.cpu().numpy()
        for k in range(count):
            ref = oracle.add_f32(ha[k * m:(k + 1) * m], hb[k * m + 3:(k + 1) * m + 3])
            assert mismatches("add_f32", hc[k * m + 1:(k + 1) * m + 1], ref).size == 0, (r, k)
