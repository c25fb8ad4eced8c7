"""Library calls captured in a HIP graph (torch.cuda.CUDAGraph over the C ABI).

Every entry point validates and plans on the host, then makes exactly one
kernel launch on the caller's stream -- no allocation, no memset, no
synchronisation -- so a sequence of calls can be captured once and replayed.
The graph fixes the pointers, sizes and launch shapes at capture time; the
data may change between replays.  Each replay here follows eager work that
rewrites the inputs, and every replay is checked against the oracle.
"""
import pytest
import torch

import memory_bound_elementwise_amd as ew
import oracle
import synth
from tests.gpu_util import DEV, download, mismatches

pytestmark = pytest.mark.gpu


def _inputs(n, seed):
    g = synth.rng(seed)
    return synth.normal01(g, n), synth.normal01(g, n), synth.normal01(g, n)


@pytest.mark.parametrize("n", [(1 << 20) + 5, 4099])
def test_captured_chain_replays_match_the_oracle(n):
    print(f"[graph] chain n={n}", flush=True)
    alpha = 2.5
    base = torch.empty(4 * n + 64, dtype=torch.float32, device=DEV)
    # misaligned views so the captured plans carry heads and tails
    a, b, c, y = (base[k * n + 1 + k: (k + 1) * n + 1 + k] for k in range(4))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm-up outside the capture
        ew.ew_add_f32(a, b, c)
        ew.ew_relu_inplace_f32(c)
        ew.ew_saxpy_f32(alpha, c, y)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ew.ew_add_f32(a, b, c)              # c = a + b
        ew.ew_relu_inplace_f32(c)           # c = relu(c), in place
        ew.ew_saxpy_f32(alpha, c, y)        # y = alpha * c + y

    for rep in range(4):
        ha, hb, hy = _inputs(n, 700 + rep)
        # eager work between replays: new inputs, and a stale output
        a.copy_(torch.from_numpy(ha))
        b.copy_(torch.from_numpy(hb))
        y.copy_(torch.from_numpy(hy))
        c.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref_c = oracle.relu_f32(oracle.add_f32(ha, hb))
        ref_y = oracle.saxpy_f32(alpha, ref_c, hy)
        assert mismatches("relu_f32", download(c, 4), ref_c).size == 0, rep
        assert mismatches("saxpy_f32", download(y, 4), ref_y).size == 0, rep


def test_captured_launches_of_every_kind_replay_twice():
    """One graph holding a launch of each kernel family (streaming, gather,
    bias + ReLU, transposed and strided views), replayed twice with the
    inputs changed in between."""
    print("[graph] kernel families", flush=True)
    rows, cols = 96, 130
    n = rows * cols
    x = torch.empty(n + 8, device=DEV)[3:3 + n]
    bias = torch.empty(cols, device=DEV)
    outs = {k: torch.empty(n + 8, device=DEV)[1:1 + n] for k in ("gather", "bias", "t", "s2")}
    half = n // 2
    side = torch.cuda.Stream()

    def calls():
        ew.ew_gather_f32(x, outs["gather"], 3)
        ew.ew_bias_relu_f32(x, bias, outs["bias"], rows, cols)
        ew.ew_copy2d_f32(x, 1, cols, outs["t"], cols, rows)          # x as (rows, cols), transposed
        ew.ew_copy2d_f32(x, 0, 2, outs["s2"], 1, half)               # x[::2]

    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(2):
        hx, hb, _ = _inputs(n, 720 + rep)
        hb = hb[:cols].copy()
        x.copy_(torch.from_numpy(hx))
        bias.copy_(torch.from_numpy(hb))
        for t in outs.values():
            t.fill_(-1.0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        refs = {"gather": oracle.gather_f32(hx, 3),
                "bias": oracle.bias_relu_f32(hx, hb, rows, cols),
                "t": oracle.copy2d_f32(hx, 0, 1, cols, cols, rows),
                "s2": oracle.copy2d_f32(hx, 0, 0, 2, 1, half)}
        for k, ref in refs.items():
            op = {"gather": "gather_f32", "bias": "bias_relu_f32"}.get(k, "copy2d_f32")
            got = download(outs[k], 4)[:ref.size]
            assert mismatches(op, got, ref).size == 0, (rep, k)
