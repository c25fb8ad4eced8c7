"""Host-side planning: the head / body / tail split and the launch shape.

``ew_make_plan`` is pure arithmetic on pointer values, so these tests need no
GPU.  They pin the split against the pages' worked examples
(``tests/golden/worked_examples.json``) and against brute force.
"""
import json
import os

import pytest

import memory_bound_elementwise_amd as ew
from tests.conftest import ROOT

GOLDEN = json.load(open(os.path.join(ROOT, "tests", "golden", "worked_examples.json")))
BASE = 0x7F0000000000
MiB = 1 << 20
CUS = 256

ELEM = {"add_f32": 4, "add_f16": 2, "add_bf16": 2, "saxpy_f32": 4, "relu_f32": 4,
        "copy_f32": 4, "gather_f32": 4}
TWO_INPUTS = {"add_f32", "add_f16", "add_bf16", "saxpy_f32"}


@pytest.fixture(autouse=True)
def _fresh_table():
    ew.ew_reset_launch_config()
    yield
    ew.ew_reset_launch_config()
    if os.path.exists(ew.LAUNCH_TABLE):
        ew.ew_load_launch_table(ew.LAUNCH_TABLE)


def _plan(op, out, in0, in1, n, cus=CUS):
    if op == "saxpy_f32":
        in1 = out
    return ew.ew_make_plan(op, out, in0, in1 if op in TWO_INPUTS else 0, n, cus)


def test_worked_example_vector_body_plus_scalar_tail():
    """N = 10 with 4-wide vectors from an aligned base: 8 elements in the
    vector body, 2 in the scalar tail."""
    ex = GOLDEN["split_examples"][0]
    p = _plan("add_f32", BASE + 2 * MiB, BASE, BASE + MiB, ex["n"])
    assert p.vec_elems == ex["vec_elems"]
    assert p.head == 0
    assert p.vectors * p.vec_elems == ex["body_elems"]
    assert p.tail == ex["tail"]


def test_worked_example_ceil_division_of_blocks():
    """N = 1000 work items at 256 per block need 4 blocks (1024 lanes), 24 of
    them masked.  Here a work item is one 16-byte vector (4000 fp32 values),
    and a tile is block * unroll vectors."""
    ex = GOLDEN["split_examples"][1]
    ew.ew_set_launch_row("relu_f32", 0, ex["threads_per_block"], 64, 1)
    p = _plan("relu_f32", BASE + MiB, BASE, 0, 4 * ex["n"])
    assert p.vectors == ex["n"]
    assert p.tiles == ex["blocks"]
    assert p.tiles * p.block == ex["threads"]
    assert p.tiles * p.block - p.vectors == ex["masked"]
    assert p.grid == ex["blocks"]          # fewer tiles than blocks_per_cu * CUs


@pytest.mark.parametrize("op", sorted(ELEM))
def test_split_brute_force(op):
    es = ELEM[op]
    vec = 16 // es
    for n in range(0, 41):
        for ko in range(vec):
            for k0 in range(vec):
                out = BASE + 4 * MiB + ko * es
                in0 = BASE + k0 * es
                in1 = BASE + MiB + ((ko + 1) % vec) * es
                p = _plan(op, out, in0, in1, n)
                assert p.head + p.vectors * p.vec_elems + p.tail == n
                assert p.vec_elems == vec and p.elem_size == es
                if n == 0:
                    assert (p.head, p.vectors, p.tail, p.grid) == (0, 0, 0, 0)
                    continue
                assert p.head == min(((16 - out % 16) % 16) // es, n)
                assert p.tail < vec
                if p.vectors:
                    assert (out + p.head * es) % 16 == 0
                expect_co0 = 1 if op == "gather_f32" else int((in0 + p.head * es) % 16 == 0)
                assert p.in_coaligned[0] == expect_co0
                if op in ("add_f32", "add_f16", "add_bf16"):
                    assert p.in_coaligned[1] == int((in1 + p.head * es) % 16 == 0)
                assert p.grid >= 1
                assert p.tiles == -(-p.vectors // (p.block * p.unroll))


def test_misaligned_a_config_split():
    """fp32 add, n = 2^28 + 3, A one element past an aligned allocation, B and
    C aligned: no head, 2^26 vectors, a 3-element tail, A relatively
    misaligned."""
    n = (1 << 28) + 3
    a, b, c = BASE + 4, BASE + (2 << 30), BASE + (4 << 30)
    p = ew.ew_make_plan("add_f32", c, a, b, n, CUS)
    assert (p.head, p.vectors, p.tail) == (0, 1 << 26, 3)
    assert tuple(p.in_coaligned) == (0, 1)


@pytest.mark.parametrize("n,vectors", [((1 << 20), 1 << 18), ((1 << 28), 1 << 26)])
def test_grid_is_capped_by_cus_and_tiles(n, vectors):
    p = _plan("add_f32", BASE + (8 << 30), BASE, BASE + (4 << 30), n)
    assert p.vectors == vectors
    tiles = -(-vectors // (p.block * p.unroll))
    assert p.tiles == tiles
    assert p.grid == min(p.blocks_per_cu * CUS, tiles)


def test_sixteen_bit_ops_use_eight_lanes_per_vector():
    n = (1 << 28)
    p = _plan("add_f16", BASE + (8 << 30), BASE, BASE + (4 << 30), n)
    assert (p.vec_elems, p.vectors, p.tail) == (8, 1 << 25, 0)
    p = _plan("add_bf16", BASE + (8 << 30) + 6, BASE + 6, BASE + (4 << 30), n)
    assert p.head == 5 and tuple(p.in_coaligned) == (1, 0)


def test_plan_rejects_what_the_operation_rejects():
    with pytest.raises(ew.EwError):
        ew.ew_make_plan("add_f32", BASE + 4, BASE, BASE + MiB, 1024, CUS)   # overlap
    with pytest.raises(ew.EwError):
        ew.ew_make_plan("add_f32", BASE + 2, BASE, BASE + MiB, 16, CUS)     # misaligned
    with pytest.raises(ew.EwError):
        ew.ew_make_plan("nope", BASE, BASE, BASE, 16, CUS)
    with pytest.raises(ew.EwError):
        ew.ew_make_plan("add_f32", BASE + 2 * MiB, BASE, BASE + MiB, 16, 0)  # no CUs


@pytest.mark.parametrize("n,stride,reps,segment,passes", [
    (1 << 26, 2, 2, 1 << 25, 1),     # the stride-2 workload: two equal halves (spans)
    ((1 << 26) + 1, 2, 1, (1 << 26) + 1, 2),   # odd n: gcd 1, two runs
    (1024, 4, 4, 256, 1),            # gcd 4: four segments of one run
    (1200, 6, 6, 200, 1),
    (1200, 12, 12, 100, 1),          # gcd 12: twelve segments
    (1002, 2, 2, 501, 1),            # n/2 = 501 not a multiple of 4: passes, not spans
    (1024, 1026, 2, 512, 1),         # stride reduced mod n first (spans)
    (1 << 20, 3, 1, 1 << 20, 3),     # stride 3, power-of-two n: three runs
    (1 << 20, 6, 2, 1 << 19, 3),     # gcd 2: two segments of three runs
    (1000, 30, 10, 100, 3),          # gcd 10, s' = 3
    (3 << 18, 24, 24, 1 << 15, 1),   # gcd 24 = the stride
    ((1 << 20) + 1, 9, 1, (1 << 20) + 1, 9),   # stride 9, gcd 1: nine runs
    ((1 << 20) + 1, 16, 1, (1 << 20) + 1, 16),
    ((1 << 20) + 1, 32, 1, (1 << 20) + 1, 32), # the largest pass stride
    ((1 << 20) + 1, 37, 1, (1 << 20) + 1, 37),  # stride 37 > 32: tiles, 37 runs
    ((1 << 20), 40, 8, 1 << 17, 5),  # stride 40 > 32, gcd 8: tiles, 8 segments of 5 runs
    ((1 << 20), 128, 1, 1 << 20, 1),  # gcd 128 >= 32, segment 2^13: the walk over all n
    ((1 << 20), 64, 64, 1 << 14, 1),  # gcd 64, segment 2^14: the walk over one segment
    ((1 << 26), 1024, 1024, 1 << 16, 1),
    (16, 16, 1, 16, 1),              # stride == n: s = 0, gcd(0, n) = n > 8: walk
    (8, 8, 1, 8, 1),                 # s = 0, gcd 8 but n/8 = 1 is not a multiple of 4
])
def test_gather_plan_segments(n, stride, reps, segment, passes):
    p = ew.ew_make_gather_plan(BASE + (8 << 30), BASE, n, stride, CUS)
    assert (p.reps, p.segment, p.passes) == (reps, segment, passes)
    if ew.PATHS[p.path] == "gather_tiles":
        # one block of 1024 threads per tile; vectors: output groups of four
        assert p.head == 0 and p.tail == 0 and p.vectors == -(-segment // 4)
        assert (p.block, p.unroll) == (1024, 1)
        assert p.grid == min(p.tiles, p.blocks_per_cu * CUS)
    elif ew.PATHS[p.path] != "gather_passes":
        assert p.head + p.vectors * 4 + p.tail == segment
        assert p.head == 0 and p.tail == segment % 4
    else:
        # groups of four slots of the longest run
        assert p.head == 0 and p.tail == 0 and p.vectors == -(-(-(-segment // passes)) // 4)
        assert (p.block, p.unroll) == (256, 1)         # one group of 4 slots per thread
        assert p.tiles == -(-p.vectors // 256)
        assert p.grid == min(p.tiles, p.blocks_per_cu * CUS)


def _passes(n, s):
    """(first output index, residue) of each pass k = 0 .. s-1."""
    out = []
    for k in range(s):
        ik = -(-k * n // s)
        out.append((ik, s * ik - k * n))
    return out


def test_gather_pass_decomposition_matches_the_definition():
    """With g = gcd(s, n), n' = n/g and s' = s/g, the output is g copies of
    its first n' elements, and within that segment the outputs with
    floor(s'*i/n') == k form a run that reads in[s*m + g*r_k], m = 0, 1, ...,
    from residues r_k that are all different; checked against the oracle's
    output (a property of the definition, on the CPU), with the planner's
    segment count, segment length and run count."""
    import math
    import numpy as np
    import oracle
    x = np.arange(1, 1001, dtype=np.uint32).view(np.float32)
    for n in list(range(3, 120)) + [997, 1000]:
        for s in range(2, 33):
            if s >= n:
                continue
            g = math.gcd(s, n)
            n1, s1 = n // g, s // g
            p = ew.ew_make_gather_plan(BASE + (8 << 30), BASE, n, s, CUS)
            if s == 2 and g == 2 and n1 % 4 == 0:
                assert ew.PATHS[p.path] == "gather_spans"
                continue
            assert ew.PATHS[p.path] == "gather_passes"
            assert (p.reps, p.segment, p.passes) == (g, n1, s1)
            assert p.vectors == -(-(-(-n1 // s1)) // 4)
            out = oracle.gather_f32(x[:n], s).view(np.uint32)
            xs = x[:n].view(np.uint32)
            for k in range(1, g):
                assert np.array_equal(out[k * n1:(k + 1) * n1], out[:n1]), (n, s, k)
            runs = _passes(n1, s1)
            assert sorted(r for _, r in runs) == list(range(s1))
            ends = [ik for ik, _ in runs[1:]] + [n1]
            for (ik, r), end in zip(runs, ends):
                m = np.arange(end - ik)
                assert np.array_equal(out[ik:end], xs[s * m + g * r]), (n, s, ik, r)
                assert s1 * (end - ik) + r >= n1 > s1 * (end - ik - 1) + r


def test_gather_replicated_segments_match_the_definition():
    """Whenever the planner replicates, the oracle's output really consists of
    `reps` equal segments (a property of the definition, checked on the CPU)."""
    import numpy as np
    import oracle
    x = np.arange(1, 257, dtype=np.uint32).view(np.float32)
    for n in range(4, 257, 4):
        for stride in range(1, 2 * n + 3):
            p = ew.ew_make_gather_plan(BASE + (8 << 30), BASE, n, stride, CUS)
            assert p.reps * p.segment == n
            if p.reps > 1:
                out = oracle.gather_f32(x[:n], stride).view(np.uint32)
                first = out[:p.segment]
                for k in range(1, p.reps):
                    assert np.array_equal(out[k * p.segment:(k + 1) * p.segment], first)


def test_gather_plan_validation():
    with pytest.raises(ew.EwError):
        ew.ew_make_gather_plan(BASE + MiB, BASE, 16, 0, CUS)
    with pytest.raises(ew.EwError):
        ew.ew_make_gather_plan(BASE, BASE, 16, 2, CUS)
    p = ew.ew_make_gather_plan(0, 0, 0, 2, CUS)
    assert p.vectors == 0 and p.reps == 0


def test_every_plan_names_its_kernel_path():
    """ew_plan_t.path says which kernel runs: the stream kernel, the copy
    that a stride of 1 mod n becomes, the gather's walk / spans / passes, the
    view paths; ew_make_copy2d_plan reports the launch the view makes (the
    transpose's fixed 1024-thread block and its 128 x 128 tiles)."""
    P = {name: k for k, name in enumerate(ew.PATHS)}
    base, out = 1 << 40, 1 << 42
    assert ew.ew_make_plan("add_f32", out, base, base + (1 << 30), 1000, 256).path == P["stream"]
    assert ew.ew_make_plan("gather_walk_f32", out, base, 0, 1000, 256).path == P["gather_walk"]
    g = ew.ew_make_gather_plan
    assert g(out, base, 1000, 1, 256).path == P["copy"]
    assert g(out, base, 1000, 1001, 256).path == P["copy"]
    assert g(out, base, 1 << 20, 2, 256).path == P["gather_spans"]
    assert g(out, base, (1 << 20) + 1, 3, 256).path == P["gather_passes"]
    assert g(out, base, (1 << 20) + 1, 2, 256).path == P["gather_passes"]
    assert g(out, base, (1 << 20) + 1, 16, 256).path == P["gather_passes"]
    assert g(out, base, 1 << 20, 9, 256).path == P["gather_passes"]
    assert g(out, base, 1 << 20, 31, 256).path == P["gather_passes"]
    assert g(out, base, 1 << 20, 33, 256).path == P["gather_tiles"]
    assert g(out, base, 1 << 20, 18, 256).path == P["gather_passes"]   # gcd 2: two segments
    assert g(out, base, 1 << 20, 40, 256).path == P["gather_tiles"]    # > 32: tiles, 8 segments
    assert g(out, base, 1 << 20, 64, 256).path == P["gather_walk"]     # gcd 64: the walk
    c = ew.ew_make_copy2d_plan
    p = c(base, 0, 2, out, 1, 1 << 20, 256)
    assert p.path == P["gather_spans"] and p.head + 4 * p.vectors + p.tail == 1 << 20
    p = c(base, 0, 5, out, 1, 1 << 20, 256)
    assert p.path == P["gather_passes"] and p.passes == 1 and p.block == 256    # one run
    p = c(base, 0, 32, out, 1, 1 << 20, 256)
    assert p.path == P["gather_passes"] and p.passes == 1
    assert c(base, 0, 33, out, 1, 1 << 20, 256).path == P["view_generic"]
    assert c(base, 20000, 1, out, 100, 16000, 256).path == P["view_rows"]
    p = c(base, 1, 300, out, 300, 517, 256)
    assert p.path == P["view_transpose"] and p.block == 1024 and p.unroll == 1
    assert p.tiles == 3 * 5 and p.grid == min(15, 256 * p.blocks_per_cu)
    assert c(base, 7, 3, out, 100, 100, 256).path == P["view_generic"]
    # the same validation as the call itself
    with pytest.raises(ew.EwError):
        c(base, 1, 300, base + 4, 300, 517, 256)
    assert c(base, 1, 300, out, 0, 517, 256).n == 0
