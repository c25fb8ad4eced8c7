"""ew_batch_run_static -- the batched entry point that allocates nothing: its
item table lives in the library's static device array -- against the
existing entry point ew_batch_run on a caller-owned device table, through
the C ABI.  Two calls in a row on one stream (the second with a smaller
batch and another operation, so the array's contents change under the
first call's kernel unless the call orders itself after it), each output
arena compared byte for byte with the existing entry point's (guard bands
included) and every item with the oracle.
"""
import numpy as np
import pytest
import torch

import memory_bound_elementwise_amd as ew
import oracle
import synth
from tests.gpu_util import DEV

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A


def _batch(op, sizes, seed):
    """Inputs, two sentinel-filled output arenas (same layout) and the item
    lists for each arena; items at element offsets 0..3 of their slots."""
    es = 4 if op.endswith("_f32") else 2
    g = synth.rng(seed)
    offs, cur = [], 0
    for n in sizes:
        o = cur + int(g.integers(0, 4))
        offs.append(o)
        cur = o + n + 16
    total = cur + 64
    inp = synth.make_inputs(op, total, seed + 1)
    a = torch.from_numpy(inp[list(inp)[0]].view(np.int32 if es == 4 else np.int16)).to(DEV)
    b = (torch.from_numpy(inp["b"].view(np.int32)).to(DEV) if "b" in inp else None)
    arenas = [torch.full((total * es,), SENTINEL, dtype=torch.uint8, device=DEV)
              for _ in range(2)]
    lists = []
    for arena in arenas:
        items = []
        for n, o in zip(sizes, offs):
            items.append((arena.data_ptr() + o * es, a.data_ptr() + o * es,
                          b.data_ptr() + o * es if b is not None else None, n))
        lists.append(items)
    return inp, a, b, arenas, lists, offs


def _oracle_arena(op, inp, sizes, offs, nbytes, alpha):
    es = 4 if op.endswith("_f32") else 2
    out = np.full(nbytes, SENTINEL, np.uint8)
    for n, o in zip(sizes, offs):
        if op == "add_f32":
            ref = oracle.add_f32(inp["a"][o:o + n], inp["b"][o:o + n])
        else:
            ref = getattr(oracle, op)(alpha, inp["x"][o:o + n])
        out[o * es:(o + n) * es] = ref.view(np.uint8)
    return out


def test_static_table_matches_the_device_table_on_two_calls_in_a_row():
    print("[no-alloc] two calls in a row, the second smaller", flush=True)
    s = torch.cuda.current_stream()
    g = synth.rng(900)
    cases = [("add_f32", [int(v) for v in g.integers(0, 20000, size=700)] + [0, 1, 5, 17], 901,
              0.0),
             ("scale_bf16", [int(v) for v in g.integers(0, 3000, size=90)] + [3, 8], 902, 2.5)]
    runs = []
    for op, sizes, seed, alpha in cases:
        inp, a, b, arenas, lists, offs = _batch(op, sizes, seed)
        plan, image = ew.ew_batch_build(op, lists[0])
        plan_s, image_s = ew.ew_batch_build(op, lists[1])
        assert plan_s.bytes == plan.bytes and plan.bytes <= ew.BATCH_SCRATCH_BYTES
        table = torch.frombuffer(bytearray(image), dtype=torch.uint8)[:plan.bytes].to(DEV)
        runs.append((op, sizes, alpha, inp, a, b, arenas, offs, plan, table, plan_s, image_s))
    # the existing entry point, caller-owned device tables
    for op, sizes, alpha, inp, a, b, arenas, offs, plan, table, plan_s, image_s in runs:
        ew.ew_batch_run(plan, alpha, table, stream=s)
    torch.cuda.synchronize()
    # the allocation-free entry point: two calls back to back on one stream
    for op, sizes, alpha, inp, a, b, arenas, offs, plan, table, plan_s, image_s in runs:
        ew.ew_batch_run_static(plan_s, alpha, image_s, stream=s)
    torch.cuda.synchronize()
    for op, sizes, alpha, inp, a, b, arenas, offs, plan, table, plan_s, image_s in runs:
        ref_arena = arenas[0].cpu().numpy()
        got_arena = arenas[1].cpu().numpy()
        assert np.array_equal(got_arena, ref_arena), (
            op, int(np.count_nonzero(got_arena != ref_arena)))
        # the inputs hold no NaN, so the oracle's arena must match byte for byte
        want = _oracle_arena(op, inp, sizes, offs, got_arena.size, alpha)
        assert np.array_equal(got_arena, want), (op, int(np.count_nonzero(got_arena != want)))


def test_static_table_refuses_a_table_beyond_its_size():
    items = []
    base = torch.empty(1, device=DEV).data_ptr()
    for k in range(7000):            # made-up addresses: refused before any launch
        items.append((base + (1 << 30) + 3 * k * 8192, base + (1 << 31) + 3 * k * 8192,
                      base + (3 << 30) + 3 * k * 8192, 1000))
    plan, image = ew.ew_batch_build("add_f32", items)
    assert plan.bytes > ew.BATCH_SCRATCH_BYTES
    with pytest.raises(ew.EwError) as e:
        ew.ew_batch_run_static(plan, 0.0, image)
    assert e.value.status == -6
