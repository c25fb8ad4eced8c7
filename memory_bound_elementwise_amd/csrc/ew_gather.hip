// ew_gather.hip -- the strided gather out[i] = in[(s * i) mod n] for CDNA4
// (gfx950): a per-output index walk, a pass decomposition for strides up to
// 32 (input staged through LDS, g = gcd(s, n) replicated segments), a tiled
// transposition for larger strides and a stride-2 kernel reading contiguous
// spans.

#include "ew_device.h"
#include "ew_gather_args.h"

#include <utility>

namespace ew {

// ---------------------------------------------------------------------------
// Strided gather: out[i] = in[(s * i) mod n]
// ---------------------------------------------------------------------------

// (a * b) mod n for a, b < n.  Narrow: the product fits in 64 bits.  Wide:
// double-and-add, exact for any n < 2^62 (used once per lane).
__device__ __forceinline__ uint64_t mul_mod(uint64_t a, uint64_t b, uint64_t n, int wide)
{
    if (!wide) return (a * b) % n;
    uint64_t r = 0;
    while (b) {
        if (b & 1u) r = add_mod(r, a, n);
        a = add_mod(a, a, n);
        b >>= 1;
    }
    return r;
}

template <int U>
__global__ void __launch_bounds__(1024) ew_gather_kernel(GatherArgs g)
{
    const uint32_t tid = threadIdx.x;
    const uint64_t nthr = blockDim.x;
    const uint64_t seg_bytes = g.seg * 4;

    if (blockIdx.x == 0 && tid < g.head + g.tail) {
        const uint64_t e = tid < g.head ? (uint64_t)tid : g.head + g.vectors * 4 + (tid - g.head);
        const uint32_t x = g.in[mul_mod(g.stride, e, g.n, g.wide)];
        for (uint64_t k = 0; k < g.reps; ++k) g.out[e + k * g.seg] = x;
    }

    uint64_t t = blockIdx.x;
    if (t >= g.tiles) return;
    char *out = reinterpret_cast<char *>(g.out + g.head);
    const uint64_t tile_vecs = nthr * U;
    // Input index of this lane's first element in its first tile.
    uint64_t jt = mul_mod(g.stride, g.head + 4 * (t * tile_vecs + tid), g.n, g.wide);

    for (; t < g.tiles; t += gridDim.x) {
        const uint64_t v0 = t * tile_vecs + tid;
        uint32_t r[U][4];
        uint64_t j = jt;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool live = v0 + u * nthr < g.vectors;
            uint64_t jj = j;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                r[u][k] = live ? g.in[jj] : 0u;
                jj = add_mod(jj, g.stride, g.n);
            }
            j = add_mod(j, g.step_vec, g.n);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t v = v0 + u * nthr;
            if (v < g.vectors) {
                const u32x4 x = u32x4{r[u][0], r[u][1], r[u][2], r[u][3]};
                for (uint64_t k = 0; k < g.reps; ++k) store16(out + k * seg_bytes + v * 16, x);
            }
        }
        jt = add_mod(jt, g.step_tile, g.n);
    }
}

// Small strides (2 <= s <= kMaxPasses = 32): read every input element once.
// With g = gcd(s, n), the output is g equal segments of n' = n/g elements
// (out[i + k*n'] = out[i]), and segment output i reads in[g * ((s'*i) mod
// n')] with s' = s/g coprime with n'.  So the segment is s' contiguous passes
// (k = 0 .. s'-1, the i with floor(s'*i / n') == k), pass k reading
// in[s*m + g*r_k] for m = 0, 1, ... where the residue r_k = (-k*n') mod s'
// differs from pass to pass.  Slot m of all s' passes together therefore
// reads elements g*r (r = 0 .. s'-1) of the s consecutive elements in[s*m ..
// s*m + s - 1]: S = s is the span of a slot, G = g the step within it.
//
// Each lane takes four slots (a group); a wave takes 64 groups, i.e. 1024 * S
// consecutive input bytes.  The wave reads them with S contiguous 16-byte-
// per-lane loads (1 KiB per instruction) that the memory unit writes straight
// into the wave's own part of LDS, and each lane reads back its 16 * S
// bytes; then, for each residue r, it
// writes the four values in[S*(m+q) + G*r] (q = 0..3) as one 16-byte store to
// its pass's output run at dest[r] + m, and again `reps` times one segment
// further on.  Letting each lane load its own 16 * S bytes directly instead
// (S loads 16 * S bytes apart across the lanes) ran 14 % (s = 3) to 70 %
// (s = 7) slower on MI355X.  The register permutation is fixed at compile
// time (S and G are template parameters); only the destinations are runtime
// values.  Loading into VGPRs first and writing them to LDS ran as fast for
// s <= 22, but from s = 23 on (G = 1) the compiler, short of registers,
// waited for each load before issuing the next: 2.8-2.9 TB/s against 4.8-4.9
// with the loads into LDS, which need no data registers.
//
// Each wave keeps 1 KiB * S of loads in flight, S times what a copy wave
// keeps, and on MI355X the full gather (S writes per wave) ran fastest with
// about 24-32 KiB of loads in flight per compute unit: at full occupancy
// (32 waves per CU) it lost 9 % (s = 2) to 17 % (s = 8) against the capped
// shapes.  Blocks are therefore 256 threads and each reserves enough LDS
// that at most kPassBlocksPerCu(S) blocks fit in a CU's 160 KiB: 16 waves per
// CU for s = 2, 8 for s = 3..5, 4 for s = 6..8 (the best of 4..32 waves per
// CU and blocks of 256 or 512 threads for every s), and 4 for s = 9..32,
// whose waves keep 9-32 KiB of loads in flight each.  The reservation holds
// the waves' staging slices; the rest of it is unused.  A single run (G == S:
// the strided view x[::S], out[m] = in[S*m], when reps == 1; S KiB read, 1
// KiB written per wave) ran fastest uncapped, so it reserves only its
// staging.  A wave only reads back the slice its own loads filled, so no
// block barrier is needed (one there cost up to 5 %): the wave waits for its
// loads to complete before reading, its next tile's loads are issued only
// after this tile's stores, which need every value read back, and
// wavefront-scope fences keep the compiler from moving LDS accesses across
// those points.
constexpr int kPassThreads = 256;
constexpr int kLdsBytesPerCu = 160 * 1024;

constexpr int kPassBlocksPerCu(int s) { return s == 2 ? 4 : s <= 5 ? 2 : 1; }

// 16-byte LDS slots between the starts of two consecutive 1 KiB loads of a
// wave's span: 64, or 65 for an even span.  A lane reads back its 16 * S
// bytes at slots S * lane + v; with S even that puts many lanes of a read on
// the same banks (all of them for S = 16 and 32), and one slot of padding
// after each load spreads them (odd spans are spread already).  At
// n = 2^26 + 1 the even spans ran 3-17 % below their odd neighbours before.
constexpr int kPassChunk(int s) { return s % 2 == 0 ? 65 : 64; }

// Bytes of LDS each pass block reserves: its staging (the waves' slices)
// or, with several runs if larger, just over 1/(blocks + 1) of the CU's LDS so
// that no more than kPassBlocksPerCu(S) blocks are resident on one CU.
constexpr int kPassStagingBytes(int s) { return kPassThreads / 64 * kPassChunk(s) * s * 16; }
constexpr int kPassLdsBytes(int s, int runs)
{
    return (runs == 1 || kPassStagingBytes(s) > kLdsBytesPerCu / kPassBlocksPerCu(s) - 1024)
               ? kPassStagingBytes(s)
               : kLdsBytesPerCu / kPassBlocksPerCu(s) - 1024;
}
static_assert(kPassLdsBytes(2, 2) * 5 > kLdsBytesPerCu &&
                  kPassLdsBytes(3, 3) * 3 > kLdsBytesPerCu &&
                  kPassLdsBytes(6, 2) * 2 > kLdsBytesPerCu &&
                  kPassLdsBytes(kMaxPasses, 2) * 2 > kLdsBytesPerCu &&
                  kPassLdsBytes(kMaxPasses, 2) <= kLdsBytesPerCu &&
                  kPassLdsBytes(kMaxPasses, 1) <= kLdsBytesPerCu,
              "the LDS reservation must cap the resident pass blocks per CU");

// Orders this wave's LDS accesses at a point of the program: the LDS
// performs one wave's accesses in issue order, so only the compiler needs
// holding back (no instruction is emitted).
__device__ __forceinline__ void wave_lds_order()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// The wave's S KiB input span, read with S 16-byte-per-lane loads that the
// memory unit writes straight into LDS (buffer_load_dwordx4 ... lds): load v
// puts lane i's 16 bytes, span bytes 1024 * v + 16 * i, at LDS slot
// dst + kPassChunk(S) * v + i.  No VGPR holds the data on its way, and the only per-lane operand is
// the offset 16 * i, so all S loads leave back to back at any S.  `span`
// and `dst` are the same in every lane of the wave.
template <int S>
__device__ __forceinline__ void load_span_to_lds(const char *span, u32x4 *dst, uint32_t lane)
{
    const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<char *>(span), (short)0, 1024 * S, 0x00020000);
#pragma unroll
    for (int v = 0; v < S; ++v)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            r, (__attribute__((address_space(3))) void *)(dst + kPassChunk(S) * v), 16,
            (int)(16 * lane),
            1024 * v, 0, EW_LOAD_NT ? 2 : 0);
}

// Waits until every vector memory access this wave issued has completed, so
// the LDS holds what load_span_to_lds fetched (s_waitcnt vmcnt(0); the other
// counters are left alone).
__device__ __forceinline__ void wait_lds_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

template <int S, int G>
__global__ void __launch_bounds__(kPassThreads) ew_gather_passes_kernel(GatherArgs g)
{
    static_assert(S >= 2 && S <= kMaxPasses && G >= 1 && S % G == 0,
                  "one run per residue, dest[] holds kMaxPasses");
    constexpr int kRuns = S / G;
    __shared__ u32x4 lds[kPassLdsBytes(S, kRuns) / 16];
    const uint32_t tid = threadIdx.x, lane = tid & 63u;
    const uint32_t wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // the same in every lane
    u32x4 *buf = lds + wv * kPassChunk(S) * S;   // this wave's staging slice
    const uint64_t seg = g.seg;             // replica distance (elements)
    for (uint64_t t = blockIdx.x; t < g.tiles; t += gridDim.x) {
        const uint64_t grp0 = t * kPassThreads + wv * 64;     // first group of this wave
        const uint64_t grp = grp0 + lane;
        if ((grp0 + 64) * 4 * S <= g.n) {
            // The wave's whole span is in range, so every lane's four slots
            // exist in every pass.  A path of its own, with no element-wise
            // fallback merged into its registers: the compiler then has no
            // reason to wait for one store to complete before the next.
            const uint64_t wbase = (uint64_t)S * 4 * grp0;    // its first input element
            load_span_to_lds<S>(reinterpret_cast<const char *>(g.in + wbase), buf, lane);
            wait_lds_loads();
            wave_lds_order();
            u32x4 e[S];
#pragma unroll
            for (int v = 0; v < S; ++v) {
                const uint32_t x = S * lane + v;        // slot of the unpadded span
                e[v] = buf[kPassChunk(S) == 64 ? x : x + x / 64];
            }
            wave_lds_order();       // read back before the next tile's writes
#pragma unroll
            for (int r = 0; r < kRuns; ++r) {
                u32x4 w;
#pragma unroll
                for (int q = 0; q < 4; ++q) w[q] = e[(S * q + G * r) / 4][(S * q + G * r) % 4];
                if (kRuns == 1 && g.reps == 1) {
                    // one array read, one written (the view): a device-scope
                    // store, the wave's 1 KiB as the buffer (4-byte aligned)
                    store16_device(reinterpret_cast<char *>(g.out + g.dest[0] + 4 * grp0),
                                   1024u, 16u * lane, w);
                } else {
                    // several runs or replicas written at once: plain
                    // non-temporal stores (the device-scope form ran 19 %
                    // slower for the three runs of stride 3)
                    for (uint64_t k = 0; k < g.reps; ++k) {
                        u32x4_a4 *p =
                            reinterpret_cast<u32x4_a4 *>(g.out + k * seg + g.dest[r] + 4 * grp);
                        if constexpr (EW_STORE_NT) __builtin_nontemporal_store(w, p);
                        else *p = w;
                    }
                }
            }
        } else if (grp < g.vectors) {
            // The wave at the end of the input: element by element.
            const uint64_t base = (uint64_t)S * 4 * grp;
            uint32_t e[4 * S];
#pragma unroll
            for (int k = 0; k < 4 * S; ++k) e[k] = base + k < g.n ? g.in[base + k] : 0u;
#pragma unroll
            for (int r = 0; r < kRuns; ++r) {
                for (uint64_t k = 0; k < g.reps; ++k) {
                    uint32_t *dst = g.out + k * seg + g.dest[r] + 4 * grp;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        if (base + (uint64_t)S * q + G * r < g.n) dst[q] = e[S * q + G * r];
                }
            }
        }
    }
}

// Stride 2 with two equal segments (n even, n/2 a multiple of 4): output i of
// the first segment reads in[2i] and never wraps.  Instead of four scalar
// loads per vector, each wave reads its 2 KiB input span with two contiguous
// 16-byte-per-lane loads (1 KiB per instruction) and keeps elements 0 and 2
// of each: lane l of a wave covering outputs [o, o + 256) holds the pair
// o + 2l, o + 2l + 1 from the first load and o + 128 + 2l, o + 129 + 2l from
// the second.  Neighbouring lanes 2k and 2k + 1 then swap one pair (a DPP
// lane swap, no LDS): lane 2k holds outputs o + 4k .. o + 4k + 3 and lane
// 2k + 1 outputs o + 128 + 4k .. o + 131 + 4k, and each stores them as one
// 16-byte vector at device scope -- one store instruction covers the wave's
// 1 KiB output run, once per segment.  A tile is blockDim * U vectors of 4
// outputs, so the launch shape means the same as for the general gather.
// Measured on MI355X against 8-byte pair stores: lanes loading 32 contiguous
// bytes each (two adjacent vectors) ran 1-2 % slower (each load instruction
// then touches twice the cache lines), staging the 2 KiB span through LDS
// 4 % slower, and two spans per wave 3-5 % slower.
template <int U, bool Co>
__global__ void __launch_bounds__(1024) ew_gather2_kernel(GatherArgs g)
{
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = tid >> 6;
    const bool odd = lane & 1u;
    const uint64_t nthr = blockDim.x;
    const uint64_t seg_bytes = g.seg * 4;

    if (blockIdx.x == 0 && tid < g.head + g.tail) {
        const uint64_t e = tid < g.head ? (uint64_t)tid : g.head + g.vectors * 4 + (tid - g.head);
        const uint32_t x = g.in[2 * e];
        for (uint64_t k = 0; k < g.reps; ++k) g.out[e + k * g.seg] = x;
    }

    const char *in = reinterpret_cast<const char *>(g.in);
    char *out = reinterpret_cast<char *>(g.out);
    const uint64_t body_end = g.head + g.vectors * 4;
    // this lane's output vector inside the wave's run of 256 outputs
    const uint32_t first = odd ? 128 + 4 * (lane >> 1) : 4 * (lane >> 1);
    for (uint64_t t = blockIdx.x; t < g.tiles; t += gridDim.x) {
        const uint64_t o0 = g.head + 4 * t * nthr * U;
        u32x4 x[U][2];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t o = o0 + ((uint64_t)wave * U + u) * 256;
            const uint64_t i1 = o + 2 * lane, i2 = o + 128 + 2 * lane;
            x[u][0] = i1 < body_end ? load16<Co, 4>(in + 8 * i1) : u32x4{0, 0, 0, 0};
            x[u][1] = i2 < body_end ? load16<Co, 4>(in + 8 * i2) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t o = o0 + ((uint64_t)wave * U + u) * 256;
            // even lanes pass their second pair, odd lanes their first; the
            // swap runs in every lane (full wave), the stores are guarded
            const uint32_t s0 = odd ? x[u][0].x : x[u][1].x;
            const uint32_t s1 = odd ? x[u][0].z : x[u][1].z;
            // quad_perm [1, 0, 3, 2]: each lane reads its neighbour's value
            const uint32_t r0 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s0, 0xB1, 0xF, 0xF, false);
            const uint32_t r1 = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)s1, 0xB1, 0xF, 0xF, false);
            const u32x4 v = odd ? u32x4{r0, r1, x[u][1].x, x[u][1].z}
                                : u32x4{x[u][0].x, x[u][0].z, r0, r1};
            if (o + first < body_end) {
                // one input read, one array written: device-scope stores, the
                // wave's 1 KiB run as the buffer
                for (uint64_t k = 0; k < g.reps; ++k)
                    store16_device(out + k * seg_bytes + 4 * o, 1024u, 4u * first, v);
            }
        }
    }
}

// Strides beyond the passes (s > 32; here g = gcd(s, n), s' = s/g, n' = n/g
// as above): view the input as rows of s elements, A[m][c] = in[s*m + c]
// (the last row stops at n).  Pass k of a segment reads in[s*m + g*r_k] for
// m = 0, 1, ... while that index is below n, i.e. it is column g*r_k of A,
// written to the segment's outputs from ceil(k*n'/s') on; every column
// c = g*r (r < s') is one pass, k = (-r * (n' mod s')^-1) mod s'.  The
// gather is therefore a transposition of A with the columns placed run by
// run, and a tile of A through LDS reads every input line once, where the
// per-output walk fetches a whole 128-byte line for each 4-byte element once
// s >= 32.  Tiles as in the view transpose: 1024 threads, 16-byte loads
// along A's rows, LDS rows padded by 4 words, each lane then reading four
// consecutive rows of one column and storing them as one 16-byte vector of
// that column's run (and again `reps` times one segment further on).
// Three tile shapes (the template's Mode), all of 16,384 elements:
//   1  s < 68: tile_rows = floor(16384 / s) whole rows (rounded down to a
//      multiple of 4), one contiguous chunk of the input kept in LDS with
//      pitch s;
//   4  the same when s is a multiple of 4, with the rows one word apart in
//      LDS (pitch s + 1, four 4-byte writes per loaded vector): with pitch s
//      the four-row reads down a column put 16 to 64 lanes on one bank, and
//      such strides ran at 3.2-4.1 TB/s against 4.3-4.7 padded (s = 64:
//      +45 %, 40 and 48: +40 %, 36 and 44: +12-15 %, 52 and 60: +6 %);
//   2  128 rows by 128 columns, when A has fewer than 1024 rows;
//   3  256 rows by 64 columns otherwise: each run gets 1 KiB per tile
//      instead of 512 bytes, 8-25 % faster than 128 x 128 from s = 137 to
//      4097 and equal at 65537 (1024 rows); at 128 rows half of each tile
//      would be empty (24 % slower at s = 2^19 + 1).  From s = 72 to 135 it
//      also beat whole rows (which give each run 120-228 outputs per tile)
//      by 6-30 %, 113 aside (3 % slower); at 65 and 66, where its second
//      band would hold one or two columns, whole rows were 9-11 % faster.
// Tiles go in groups of kTileBandGroup (16) row bands: within a group
// consecutive blocks take consecutive row bands of one column band, so each
// continues the runs the previous one wrote, and the group then moves to the
// next column band.  The row pieces of neighbouring bands share the lines at
// their edges (a band starts mid-line unless the stride is a multiple of 32);
// with the groups those lines are fetched while the other band's reads are
// recent, where walking every row band of one column band before the next
// fetched them twice (stride 1000, 256 x 64 tiles: 1.38 x the input read).
// 16 row bands per group ran 2-16 % faster than that order from s = 137 to
// 1281 and 2 % slower at 4097; groups of 4, 32 and 64 lost to 16 almost
// everywhere.  The dispatcher deals block b to XCD b % 8, each XCD with an L2
// of its own.  Within a full group (16 row bands) block i of the group, on
// XCD i % 8, takes row band 2 (i % 8) + (i / 8) % 2 of column band i / 16:
// each XCD works through two adjacent row bands of each column band in turn,
// so that a tile's column-band neighbour (sharing the lines at the band edge)
// runs on the same XCD two tiles later, and one row-band neighbour in two
// (continuing the same runs) shares the L2 as well.  At n = 2^26 that gained
// 1 to 5 % from s = 72 to 4097 (113: -0.3 %) over dealing the group in order
// (one row band per XCD and column band); against that order, four adjacent
// row bands in groups of 32 ran from +9 % (4097) to -6 % (2049), 16
// consecutive tiles per XCD lost 2-10 %, and a whole group per XCD
// (column-band neighbours 16 of its tiles apart) ran from +4 % (1000) to
// -28 % (2049).  Whole-row tiles have one column band (their neighbours are
// the chunks t - 1 and t + 1), and with r < 16 row bands the next column
// band, tile t + r, lands on another XCD unless r = 8; there each XCD takes
// 16 consecutive tiles instead (xcd_run_tile): +1.7 to +8.5 % from s = 33 to
// 67 and +12 to +18 % for s = 65537 to 2^19 + 1 (1 to 4 row bands).  A
// column's destination needs two 64-bit divisions: the first cols threads
// compute them once per tile into LDS.
template <int Mode> struct TileShape {                // modes 2 and 3 (1 and 4: rows vary)
    static constexpr int kRows = Mode == 2 ? 128 : 256;
    static constexpr int kCols = Mode == 2 ? 128 : 64;
    static constexpr int kPitch = kCols + 4;          // words per LDS row
    static constexpr int kLanesPerRow = kCols / 4;
};
constexpr int kTileThreads = 1024;
constexpr int kTileSteps = 4;                         // 16-byte loads / stores per thread
constexpr int kTileLdsWords = 256 * (64 + 4);         // the largest shape: 17,408 words
constexpr uint64_t kNoRun = ~(uint64_t)0;             // a column no pass reads
constexpr uint64_t kTileBandGroup = 16;               // row bands per group of tiles
constexpr int kTileRunStarts = 128;                   // the most columns a tile holds

// Tile t of `tiles`, dealt so that each XCD takes kXcdRun consecutive tiles:
// within each window of 8 * kXcdRun tiles, block b (on XCD b % 8) takes tile
// (b % 8) * kXcdRun + b / 8 of the window; the last, partial window keeps its
// order.  A bijection on [0, tiles), whatever the grid.
constexpr uint64_t kXcdRun = 16;
static_assert(kTileBandGroup % 8 == 0,
              "a full group deals each of the 8 XCDs the same number of adjacent row bands");
__device__ __forceinline__ uint64_t xcd_run_tile(uint64_t t, uint64_t tiles)
{
    constexpr uint64_t W = 8 * kXcdRun;
    const uint64_t win = t / W * W;
    return win + W <= tiles ? win + (t - win) % 8 * kXcdRun + (t - win) / 8 : t;
}
static_assert(kTileLdsWords >= (int)(kGatherTileWords + kGatherTileWords / 33) &&
                  kTileLdsWords >= TileShape<2>::kRows * TileShape<2>::kPitch &&
                  kTileLdsWords >= TileShape<3>::kRows * TileShape<3>::kPitch,
              "every tile shape fits the LDS tile");
static_assert(kGatherNarrowStrides <= (uint64_t)kTileRunStarts &&
                  TileShape<2>::kCols <= kTileRunStarts && TileShape<3>::kCols <= kTileRunStarts &&
                  kTileRunStarts <= kTileThreads && kGatherTileWords / (kGatherNarrowStrides - 1) >= 4,
              "run starts: one per column of a tile, one thread each; narrow tiles hold >= 4 rows");
static_assert(kTileSteps * kTileThreads * 4 == (int)kGatherTileWords &&
                  kTileSteps * kTileThreads / TileShape<2>::kLanesPerRow == TileShape<2>::kRows &&
                  kTileSteps * kTileThreads / TileShape<3>::kLanesPerRow == TileShape<3>::kRows,
              "four steps cover a narrow tile's words and a wide tile's rows");
static_assert(kGatherWideRows[0] == TileShape<2>::kRows &&
                  kGatherWideCols[0] == TileShape<2>::kCols &&
                  kGatherWideRows[1] == TileShape<3>::kRows &&
                  kGatherWideCols[1] == TileShape<3>::kCols,
              "the host plans the tiles the kernel moves");

template <int Mode>
__global__ void __launch_bounds__(kTileThreads) ew_gather_tiles_kernel(GatherArgs g)
{
    constexpr bool Narrow = Mode == 1 || Mode == 4;
    constexpr bool pad = Mode == 4;           // whole rows one word apart in LDS
    using W = TileShape<Narrow ? 2 : Mode>;
    __shared__ uint32_t tile[kTileLdsWords];
    __shared__ uint64_t run_start[kTileRunStarts];
    const uint32_t tid = threadIdx.x;
    const uint64_t s = g.stride, n = g.n, seg = g.seg;
    const uint32_t rows = Narrow ? g.tile_rows : (uint32_t)W::kRows;   // a multiple of 4
    const uint32_t cols = Narrow ? (uint32_t)s : (uint32_t)W::kCols;
    const uint32_t pitch = Narrow ? (uint32_t)s + (pad ? 1u : 0u) : (uint32_t)W::kPitch;
    const uint32_t groups = rows / 4;         // four-row groups per column
    for (uint64_t t = blockIdx.x; t < g.tiles; t += gridDim.x) {
        // tile u: groups of kTileBandGroup row bands, each group walking its
        // column bands in turn; with one column band or fewer than
        // kTileBandGroup row bands, 16 consecutive tiles per XCD
        const uint64_t bands = g.tiles / g.tiles_m;
        const uint64_t u = Narrow || g.tiles_m < kTileBandGroup ? xcd_run_tile(t, g.tiles) : t;
        const uint64_t grp = u / (kTileBandGroup * bands), in_grp = u % (kTileBandGroup * bands);
        const uint64_t grp_rows = g.tiles_m - grp * kTileBandGroup < kTileBandGroup
                                      ? g.tiles_m - grp * kTileBandGroup
                                      : kTileBandGroup;
        uint64_t rb = in_grp % grp_rows, cb = in_grp / grp_rows;
        if (!Narrow && g.tiles_m >= kTileBandGroup && grp_rows == kTileBandGroup) {
            // a full group: block i of it (on XCD i % 8) takes row band
            // 2 (i % 8) + (i / 8) % 2 of column band i / 16
            constexpr uint64_t q = kTileBandGroup / 8;       // row bands per XCD
            cb = in_grp / 8 / q;
            rb = q * (in_grp % 8) + in_grp / 8 % q;
        }
        const uint64_t m0 = (grp * kTileBandGroup + rb) * rows;
        const uint64_t c0 = Narrow ? 0 : cb * W::kCols;
        // the run start of each column of the tile (two 64-bit divisions),
        // computed while the tile's loads are in flight
        auto run_starts = [&]() {
            if (tid < cols) {
                const uint64_t c = c0 + tid;
                uint64_t d = kNoRun;
                if (c < s && c % g.reps == 0) {
                    const uint64_t r = c / g.reps;
                    const uint64_t k = (g.sp - r) % g.sp * g.inv % g.sp;   // < sp^2 < 2^64
                    d = (k * seg + g.sp - 1) / g.sp;                       // < sp * seg < 2^64
                }
                run_start[tid] = d;
            }
        };
        // Every row of the tile's columns exists (the same in every lane):
        // the fast path's loads are then unconditional (a lane past the
        // tile's last quad reloads an in-range one and drops it), all of
        // them in flight at once.
        const bool full = Narrow ? s * m0 + (uint64_t)rows * cols <= n
                                 : c0 + W::kCols <= s &&
                                       s * (m0 + W::kRows - 1) + c0 + W::kCols <= n;
        if constexpr (Narrow) {
            // rows m0 .. m0 + rows - 1 are the contiguous input from s * m0
            const uint64_t base = s * m0;
            const uint32_t quads = rows * cols / 4;   // <= kGatherTileWords / 4
            u32x4 v[kTileSteps];
            if (full) {
#pragma unroll
                for (int p = 0; p < kTileSteps; ++p) {
                    const uint32_t q = min(tid + p * kTileThreads, quads - 1);
                    v[p] = load16<false, 4>(reinterpret_cast<const char *>(g.in + base + 4 * q));
                }
            } else {
#pragma unroll
                for (int p = 0; p < kTileSteps; ++p) {
                    const uint64_t e = base + 4 * (uint64_t)(tid + p * kTileThreads);
#pragma unroll
                    for (int k = 0; k < 4; ++k) v[p][k] = e + k < n ? g.in[e + k] : 0u;
                }
            }
            run_starts();
            if constexpr (!pad) {
#pragma unroll
                for (int p = 0; p < kTileSteps; ++p) {
                    const uint32_t q = tid + p * kTileThreads;
                    if (q < quads) *reinterpret_cast<u32x4 *>(&tile[4 * q]) = v[p];
                }
            } else {
#pragma unroll
                for (int p = 0; p < kTileSteps; ++p) {
                    const uint32_t q = tid + p * kTileThreads;
                    if (q < quads) {
                        // words 4q .. 4q + 3 of the chunk: row 4q / s, one
                        // row further once the column reaches s
                        const uint32_t row = 4 * q / cols, col = 4 * q - row * cols;
#pragma unroll
                        for (int k = 0; k < 4; ++k) {
                            const uint32_t wrap = col + k >= cols ? 1u : 0u;
                            tile[(row + wrap) * pitch + col + k - wrap * cols] = v[p][k];
                        }
                    }
                }
            }
        } else {
            // kLanesPerRow lanes cover a row's kCols columns, kRowsPerStep
            // rows per step
            constexpr uint32_t kRowsPerStep = kTileThreads / W::kLanesPerRow;
            const uint32_t sub = tid / W::kLanesPerRow, q4 = (tid % W::kLanesPerRow) * 4;
            u32x4 v[kTileSteps];
            if (full) {
#pragma unroll
                for (int p = 0; p < kTileSteps; ++p) {
                    const uint64_t e = s * (m0 + p * kRowsPerStep + sub) + c0 + q4;
                    v[p] = load16<false, 4>(reinterpret_cast<const char *>(g.in + e));
                }
            } else {
#pragma unroll
                for (int p = 0; p < kTileSteps; ++p) {
                    const uint64_t e = s * (m0 + p * kRowsPerStep + sub) + c0 + q4;
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        v[p][k] = c0 + q4 + k < s && e + k < n ? g.in[e + k] : 0u;
                }
            }
            run_starts();
#pragma unroll
            for (int p = 0; p < kTileSteps; ++p)
                *reinterpret_cast<u32x4 *>(&tile[(p * kRowsPerStep + sub) * W::kPitch + q4]) =
                    v[p];
        }
        __syncthreads();
        // item q: column c, rows 4j .. 4j + 3 of the tile
        const uint32_t items = cols * groups;        // <= kTileSteps * kTileThreads
        if (full) {
            // Every row of every column exists: each item whose column is a
            // run stores whole vectors.  The LDS reads of all steps first,
            // then the stores, with no per-element checks (a lane past the
            // last item reads a valid one and stores nothing).
            u32x4 w[kTileSteps];
            uint64_t o[kTileSteps];
#pragma unroll
            for (int p = 0; p < kTileSteps; ++p) {
                const uint32_t q = min(tid + p * kTileThreads, items - 1);
                const uint32_t c = q / groups, j = q % groups;
#pragma unroll
                for (int k = 0; k < 4; ++k) w[p][k] = tile[(4 * j + k) * pitch + c];
                const uint64_t d = run_start[c];
                o[p] = d == kNoRun || tid + p * kTileThreads >= items ? kNoRun : d + m0 + 4 * j;
            }
#pragma unroll
            for (int p = 0; p < kTileSteps; ++p) {
                if (o[p] != kNoRun) {
                    for (uint64_t k = 0; k < g.reps; ++k) {
                        u32x4_a4 *dv = reinterpret_cast<u32x4_a4 *>(g.out + k * seg + o[p]);
                        if constexpr (EW_STORE_NT) __builtin_nontemporal_store(w[p], dv);
                        else *dv = w[p];
                    }
                }
            }
        } else
#pragma unroll 1
        for (int p = 0; p < kTileSteps; ++p) {
            const uint32_t q = tid + p * kTileThreads;
            if (q >= items) break;
            const uint32_t c = q / groups, j = q % groups;
            const uint64_t d = run_start[c];
            if (d == kNoRun) continue;
            u32x4 w;
#pragma unroll
            for (int k = 0; k < 4; ++k) w[k] = tile[(4 * j + k) * pitch + c];
            const uint64_t m = m0 + 4 * j;            // the group's first row
            const uint64_t e = s * m + c0 + c;        // its input element
            const uint64_t o = d + m;                 // its output, within a segment
            // row m + k exists iff e + k*s < n, and then o + k < seg
            const bool all = e + 3 * s < n && o + 3 < seg;
            for (uint64_t k = 0; k < g.reps; ++k) {
                uint32_t *dst = g.out + k * seg + o;
                if (all) {
                    u32x4_a4 *dv = reinterpret_cast<u32x4_a4 *>(dst);
                    if constexpr (EW_STORE_NT) __builtin_nontemporal_store(w, dv);
                    else *dv = w;
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (e + r * s < n && o + r < seg) dst[r] = w[r];
                }
            }
        }
        // the tile and run starts are rewritten only if this block has
        // another round (a block-uniform condition)
        if (t + gridDim.x < g.tiles) __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Dispatch
// ---------------------------------------------------------------------------

namespace {

// The pass kernel of span S and step G (S = 2 .. kMaxPasses, G dividing S),
// or null.
template <int S, int G>
const void *pass_ptr()
{
    if constexpr (S % G == 0) return reinterpret_cast<const void *>(&ew_gather_passes_kernel<S, G>);
    else return nullptr;
}

template <int S, int... I>
const void *pass_fn_g(int g, std::integer_sequence<int, I...>)
{
    const void *fn = nullptr;
    ((g == I + 1 ? (void)(fn = pass_ptr<S, I + 1>()) : (void)0), ...);
    return fn;
}

template <int... I>
const void *pass_fn(int s, int g, std::integer_sequence<int, I...>)
{
    const void *fn = nullptr;
    ((s == I + 2 ? (void)(fn = pass_fn_g<I + 2>(g, std::make_integer_sequence<int, I + 2>{}))
                 : (void)0),
     ...);
    return fn;
}

template <int U, bool Co>
const void *gather2_fn()
{
    return reinterpret_cast<const void *>(&ew_gather2_kernel<U, Co>);
}
}  // namespace

int gather_passes_threads() { return kPassThreads; }
int gather_tiles_threads() { return kTileThreads; }

hipError_t launch_gather(const GatherArgs &args, const Launch &l, hipStream_t s)
{
    GatherArgs a = args;
    void *kargs[] = {&a};
    const void *fn = nullptr;
    if (args.passes >= 2) {
        fn = pass_fn(args.passes, args.skip, std::make_integer_sequence<int, kMaxPasses - 1>{});
        if (!fn) return hipErrorInvalidValue;
        // A single run stored into several segments writes as many streams
        // as the runs of a full gather: cap its blocks per CU the same way,
        // with dynamic LDS on top of the staging (the view, one stream,
        // runs uncapped).
        size_t extra = 0;
        if (args.passes == args.skip && args.reps > 1) {
            const int cap = kLdsBytesPerCu / kPassBlocksPerCu(args.passes) - 1024;
            const int staging = kPassLdsBytes(args.passes, 1);
            if (cap > staging) extra = (size_t)(cap - staging);
        }
        return hipLaunchKernel(fn, dim3(l.grid), dim3(kPassThreads), kargs, extra, s);
    }
    if (args.tile_mode != 0) {
        switch (args.tile_mode) {
        case 1: fn = reinterpret_cast<const void *>(&ew_gather_tiles_kernel<1>); break;
        case 2: fn = reinterpret_cast<const void *>(&ew_gather_tiles_kernel<2>); break;
        case 3: fn = reinterpret_cast<const void *>(&ew_gather_tiles_kernel<3>); break;
        case 4: fn = reinterpret_cast<const void *>(&ew_gather_tiles_kernel<4>); break;
        default: return hipErrorInvalidValue;
        }
        return hipLaunchKernel(fn, dim3(l.grid), dim3(kTileThreads), kargs, 0, s);
    }
    if (args.stride == 2 && (args.reps == 2 || (args.reps == 1 && args.n == 2 * args.seg))) {
        // co-alignment of the input's body start: in + 8 * head
        const bool co = ((reinterpret_cast<uintptr_t>(args.in) + 8 * args.head) & 15u) == 0;
        switch (l.unroll) {
        case 1: fn = co ? gather2_fn<1, true>() : gather2_fn<1, false>(); break;
        case 2: fn = co ? gather2_fn<2, true>() : gather2_fn<2, false>(); break;
        case 4: fn = co ? gather2_fn<4, true>() : gather2_fn<4, false>(); break;
        case 8: fn = co ? gather2_fn<8, true>() : gather2_fn<8, false>(); break;
        default: return hipErrorInvalidValue;
        }
    } else {
        switch (l.unroll) {
        case 1: fn = reinterpret_cast<const void *>(&ew_gather_kernel<1>); break;
        case 2: fn = reinterpret_cast<const void *>(&ew_gather_kernel<2>); break;
        case 4: fn = reinterpret_cast<const void *>(&ew_gather_kernel<4>); break;
        case 8: fn = reinterpret_cast<const void *>(&ew_gather_kernel<8>); break;
        default: return hipErrorInvalidValue;
        }
    }
    return hipLaunchKernel(fn, dim3(l.grid), dim3(l.block), kargs, 0, s);
}
}  // namespace ew
