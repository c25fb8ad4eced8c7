"""The tiled transposition of the strided gather (strides above 32), checked
on the CPU before any launch.

`_model` follows ew_gather_tiles_kernel step by step -- the tile grid, the
per-column run starts, every thread's loads, LDS writes, LDS reads and
stores, with the kernel's full-tile and per-element conditions (a full tile
stores every item as whole vectors unchecked, which the model asserts is
safe) -- using the
plan the library reports (path, segment, reps, runs, tiles) and the field
formulas that include/ew.h states for this path.  It asserts that every
global load and store and every LDS access stays inside its buffer, that
each output element is written exactly once, and that the result is the
definition out[i] = in[(s*i) mod n] (the oracle's gather).
"""
import math

import numpy as np
import pytest

import memory_bound_elementwise_amd as ew

BASE = 0x7F0000000000
CUS = 256
THREADS = 1024
STEPS = 4
LDS_WORDS = 256 * 68
TILE_WORDS = 16384
NO_RUN = -1


def _fields(n, s):
    """The kernel arguments of the tiled path (the formulas of include/ew.h)."""
    g = math.gcd(s, n)
    sp, seg = s // g, n // g
    rows = (n - 1) // s + 1
    narrow = s < 68
    mode = (4 if s % 4 == 0 else 1) if narrow else 2 if rows < 1024 else 3
    tile_rows = (TILE_WORDS // s) & ~3 if narrow else {2: 128, 3: 256}[mode]
    cols = s if narrow else {2: 128, 3: 64}[mode]
    tiles_m = -(-rows // tile_rows)
    tiles = tiles_m * -(-s // cols)
    return dict(g=g, sp=sp, seg=seg, inv=pow(seg % sp, -1, sp), narrow=narrow, mode=mode,
                tile_rows=tile_rows, tile_cols=cols, tiles_m=tiles_m, tiles=tiles)


def _tile_of(t, tiles_m, bands, group=16, pairs=False):
    """(row band, column band) of tile t: groups of `group` row bands, each
    group walking its column bands in turn, row band fastest; with `pairs`,
    block i of a full group (on XCD i % 8) takes row band
    2 (i % 8) + (i // 8) % 2 of column band i // 16."""
    grp, rest = divmod(t, group * bands)
    rows_in_group = min(group, tiles_m - grp * group)
    if pairs and rows_in_group == group:
        q = group // 8
        return grp * group + q * (rest % 8) + rest // 8 % q, rest // 8 // q
    return grp * group + rest % rows_in_group, rest // rows_in_group


def _xcd_run_tile(t, tiles, run=16):
    """Tile t dealt so that each of the 8 XCDs takes `run` consecutive tiles
    per window of 8 * run (the last, partial window as is)."""
    w = 8 * run
    win = t // w * w
    return win + (t - win) % 8 * run + (t - win) // 8 if win + w <= tiles else t


def test_xcd_runs_are_a_bijection():
    for tiles in list(range(1, 400)) + [1023, 1024, 1025, 4130, 65536]:
        got = sorted(_xcd_run_tile(t, tiles) for t in range(tiles))
        assert got == list(range(tiles)), tiles
    # block b of a full window lands on XCD b % 8 and its tiles there are consecutive
    for x in range(8):
        assert [_xcd_run_tile(b, 256) for b in range(x, 128, 8)] == list(range(16 * x, 16 * x + 16))


def test_tile_order_covers_every_tile_once():
    for tiles_m in range(1, 70):
        for bands in range(1, 9):
            for pairs in (False, True):
                got = {_tile_of(t, tiles_m, bands, pairs=pairs) for t in range(tiles_m * bands)}
                assert got == {(m, c) for m in range(tiles_m) for c in range(bands)}, \
                    (tiles_m, bands, pairs)
    # paired: each XCD (t % 8) holds row bands 2x, 2x + 1 of every column band,
    # the column-band neighbour of a tile two of that XCD's tiles later
    for t in range(16 * 3):
        m, c = _tile_of(t, 16, 3, pairs=True)
        assert m // 2 == t % 8 and c == t // 16
        assert c == 2 or _tile_of(t + 16, 16, 3, pairs=True) == (m, c + 1)


def _model(n, s, x):
    """Run the kernel's index arithmetic over every block; return the output."""
    f = _fields(n, s)
    g, sp, seg, inv, narrow = f["g"], f["sp"], f["seg"], f["inv"], f["narrow"]
    rows, cols = f["tile_rows"], f["tile_cols"]
    pad = narrow and s % 4 == 0          # whole rows one word apart in LDS
    pitch = (s + pad) if narrow else cols + 4
    lanes_per_row = cols // 4
    rows_per_step = THREADS // lanes_per_row
    groups = rows // 4
    assert rows % 4 == 0 and rows * cols <= TILE_WORDS
    assert narrow or rows_per_step * STEPS == rows
    out = np.zeros(n, dtype=x.dtype)
    writes = np.zeros(n, dtype=np.int64)
    tid = np.arange(THREADS)
    for t in range(f["tiles"]):
        u = _xcd_run_tile(t, f["tiles"]) if narrow or f["tiles_m"] < 16 else t
        mt, ct = _tile_of(u, f["tiles_m"], f["tiles"] // f["tiles_m"],
                          pairs=not narrow and f["tiles_m"] >= 16)
        m0 = mt * rows
        c0 = 0 if narrow else ct * cols
        run_start = np.full(128, NO_RUN, dtype=object)
        for c_t in range(cols):
            c = c0 + c_t
            if c < s and c % g == 0:
                r = c // g
                k = (sp - r) % sp * inv % sp
                assert k * seg + sp - 1 < 1 << 64
                run_start[c_t] = (k * seg + sp - 1) // sp
        lds = np.full(LDS_WORDS, -1, dtype=np.int64)        # -1: never written
        if narrow:
            base = s * m0
            quads = rows * cols // 4
            full = base + 4 * quads <= n
            for p in range(STEPS):
                q = tid + p * THREADS
                q = q[q < quads]
                idx = base + 4 * q[:, None] + np.arange(4)
                if full:
                    assert idx.max(initial=-1) < n
                    v = x[idx]
                else:
                    v = np.where(idx < n, x[np.minimum(idx, n - 1)], 0)
                w = 4 * q[:, None] + np.arange(4)          # words of the chunk
                dst = (w // s) * pitch + w % s
                assert dst.max(initial=-1) < LDS_WORDS
                lds[dst] = v
        else:
            sub, q4 = tid // lanes_per_row, (tid % lanes_per_row) * 4
            full = c0 + cols <= s and s * (m0 + rows - 1) + c0 + cols <= n
            for p in range(STEPS):
                m = p * rows_per_step + sub
                e = s * (m0 + m) + c0 + q4
                idx = e[:, None] + np.arange(4)
                if full:
                    assert idx.max() < n
                    v = x[idx]
                else:
                    ok = ((c0 + q4)[:, None] + np.arange(4) < s) & (idx < n)
                    v = np.where(ok, x[np.minimum(idx, n - 1)], 0)
                dst = (m * pitch + q4)[:, None] + np.arange(4)
                assert dst.max() < LDS_WORDS
                lds[dst] = v
        items = cols * groups
        assert items <= STEPS * THREADS
        for q in range(items):
            c, j = divmod(q, groups)
            d = run_start[c]
            if d == NO_RUN:
                continue
            src = (4 * j + np.arange(4)) * pitch + c
            assert src.max() < LDS_WORDS
            w = lds[src]
            assert (w >= 0).all() or not narrow          # read only what was loaded
            m = m0 + 4 * j
            e = s * m + c0 + c
            o = d + m
            every = e + 3 * s < n and o + 3 < seg
            # a full tile stores whole vectors with no per-element checks
            assert every or not full, (n, s, t, q)
            for rep in range(g):
                for k in range(4):
                    if every or (e + k * s < n and o + k < seg):
                        i = rep * seg + o + k
                        assert 0 <= i < n, (n, s, t, q, rep, k)
                        out[i] = w[k]
                        writes[i] += 1
    assert (writes == 1).all(), (n, s, int(writes.min()), int(writes.max()))
    return out


@pytest.mark.parametrize("n,s", [
    (4225, 33),                 # 128 rows of 33 and one element: a single narrow tile
    (20000, 33), (20011, 37), (50000, 34), (60000, 104), (65536, 80), (100003, 127),
    (70000, 44), (99999, 63), (40000, 62),
    (100001, 36), (99999, 40), (100001, 48), (100003, 64),   # whole rows one word apart in LDS
    (33000, 129), (70001, 200), (262144, 1000), (300000, 257), (200001, 1280),
    (16511, 129),               # 128 rows, the last one short by one
    (100001, 67), (100001, 68),     # the last whole-row stride, the first wide one
    (100001, 135), (100001, 136),
    (1023 * 300 - 5, 300), (1024 * 300, 301), (1024 * 300 + 7, 300),   # 1023 / 1024 rows
    (1 << 18, 2047),            # 128 rows, wide, gcd 1
    (2200000, 35),              # 135 whole-row tiles: one full window of XCD runs
    (128 * 16385 - 3, 16385),   # one row band of 129 wide tiles: XCD runs
    (300001, 69),               # 17 row bands of wide tiles: a full group in XCD pairs
])
def test_tile_model_matches_the_definition(n, s):
    p = ew.ew_make_gather_plan(BASE + (8 << 30), BASE, n, s, CUS)
    assert ew.PATHS[p.path] == "gather_tiles", (n, s)
    f = _fields(n, s)
    assert (p.reps, p.segment, p.passes, p.tiles) == (f["g"], f["seg"], f["sp"], f["tiles"])
    assert (p.block, p.unroll, p.head, p.tail) == (THREADS, 1, 0, 0)
    assert p.grid == min(f["tiles"], p.blocks_per_cu * CUS)
    assert p.vectors == -(-f["seg"] // 4)
    x = np.arange(1, n + 1, dtype=np.int64)
    want = x[(s * np.arange(n, dtype=np.int64)) % n]
    assert np.array_equal(_model(n, s, x), want)


def test_tiled_route_bounds():
    """Strides above 32 take the tiled path only with g < 32, s' >= 2 and at
    least 128 rows; otherwise the per-output walk."""
    g = ew.ew_make_gather_plan
    P = {name: k for k, name in enumerate(ew.PATHS)}
    out = BASE + (8 << 30)
    assert g(out, BASE, 1 << 20, 33, CUS).path == P["gather_tiles"]
    assert g(out, BASE, 1 << 20, 64, CUS).path == P["gather_walk"]        # g = 64
    assert g(out, BASE, 1 << 20, 96, CUS).path == P["gather_walk"]        # g = 32
    assert g(out, BASE, 1 << 20, 80, CUS).path == P["gather_tiles"]       # g = 16
    assert g(out, BASE, 4224, 33, CUS).path == P["gather_walk"]           # 128 rows need n > 127 * 33
    assert g(out, BASE, 4225, 33, CUS).path == P["gather_tiles"]
    assert g(out, BASE, (1 << 20) + 1, (1 << 20) - 1, CUS).path == P["gather_walk"]   # 2 rows
    n = (1 << 20) + 7
    assert g(out, BASE, n, (n - 1) // 127, CUS).path == P["gather_tiles"]   # 128 rows
    assert g(out, BASE, n, (n - 1) // 127 + 1, CUS).path == P["gather_walk"]  # 127 rows
    # s' * n/g must stay below 2^64 (the run starts' products): 2^40
    # elements with a stride of 2^31 + 1 (coprime with n, 2^9 rows) exceed it
    far = BASE - (1 << 43)                          # 4 TiB apart: no overlap
    assert g(far, BASE, 1 << 40, (1 << 31) + 1, CUS).path == P["gather_walk"]
    assert g(far, BASE, 1 << 40, (1 << 23) + 1, CUS).path == P["gather_tiles"]
