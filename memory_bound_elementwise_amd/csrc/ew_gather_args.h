// ew_gather_args.h -- the gather's arguments and launcher, shared by
// the host API (ew_api.cpp) and ew_gather.hip (the x[::s] views run the
// gather's kernels).  Not installed; not part of the
// C ABI.
#pragma once

#include "ew_internal.h"

namespace ew {

// The gather's index walk steps its input index (stride * i) mod n
// incrementally; the steps are reduced mod n on the host.  When
// g = gcd(stride, n) > 1 the output is g copies of one segment of n / g
// elements (out[i + k*n/g] = out[i]); then head / vectors / tail describe one
// segment and every value is stored `reps` times, `seg` elements apart, so
// each input element is fetched once instead of g times.  Strides up to
// kMaxPasses take the pass decomposition described below (one kernel
// instance per stride and gcd).
constexpr int kMaxPasses = 32;

struct GatherArgs {
    const uint32_t *in;
    uint32_t *out;
    uint64_t n;
    uint64_t stride;     // stride mod n
    uint64_t seg;        // elements per output segment (n when reps == 1)
    uint64_t reps;       // number of identical segments (1..kMaxPasses)
    uint64_t head;
    uint64_t vectors;
    uint64_t tail;
    uint64_t tiles;
    uint64_t step_vec;   // stride * 4 * blockDim            (mod n): next unrolled vector
    uint64_t step_tile;  // stride * 4 * blockDim * unroll * gridDim (mod n): next tile
    int wide;            // 1 if stride * (n - 1) can exceed 2^64 - 1
    // Pass decomposition (2 <= stride <= kMaxPasses): passes == stride (the
    // span S of a slot) and skip == g = gcd(stride, n) (the step G within
    // it), otherwise passes == 0.  The output is reps = g segments of
    // seg = n / g elements; in one segment, pass k is the run of i with
    // floor(s' * i / seg) == k (s' = stride / g); it reads in[stride * m +
    // g * r] for m = 0, 1, ... where the residue r = (-k * seg) mod s' differs
    // from pass to pass.  dest[r] is the first output index of the pass with
    // residue r, and vectors counts groups of four slots m of the longest
    // pass.  A 1-D strided view x[::s] is passes == skip == s with reps == 1:
    // one run (dest[0] = 0), n the view's input extent s * (count - 1) + 1.
    int passes;
    int skip;
    uint64_t dest[kMaxPasses];
    // Tiled transposition (larger strides, tile_mode != 0): the input viewed
    // as rows of `stride` elements, A[m][c] = in[stride * m + c]; column
    // c = g * r (g = gcd(stride, n) = reps) is one pass of a segment, its
    // rows m written to out[k * seg + dest(c) + m] for k < reps, where pass
    // k' = (-r * inv) mod sp starts at dest(c) = ceil(k' * seg / sp),
    // sp = stride / g and inv = (seg mod sp)^-1 mod sp.  tile_mode 1: one
    // tile is tile_rows whole rows (stride < kGatherNarrowStrides); 4: the
    // same, the rows one word apart in LDS (stride a multiple of 4); 2 and 3:
    // tiles of kGatherWideRows[mode - 2] rows by kGatherWideCols[mode - 2]
    // columns, tiles_m row bands by ceil(stride / columns) column bands.
    int tile_mode;
    uint32_t tile_rows;
    uint64_t sp;
    uint64_t inv;
    uint64_t tiles_m;
};

hipError_t launch_gather(const GatherArgs &args, const Launch &launch,
                         hipStream_t stream);

// Threads per block of the pass-decomposed gather (one group of four slots
// per thread, one tile per block and round).
int gather_passes_threads();

// Threads per block of the tiled transposition, and the words of LDS one
// narrow tile may fill (tile_rows * stride <= this).
int gather_tiles_threads();
constexpr uint32_t kGatherTileWords = 16384;
// Strides below this take tiles of whole rows (each run then gets at least
// 244 outputs per tile).
constexpr uint64_t kGatherNarrowStrides = 68;
// Wider strides: tiles of 128 x 128 (tile_mode 2) while A has fewer than
// kGatherTallRows rows, else 256 rows x 64 columns (tile_mode 3).
constexpr uint32_t kGatherWideRows[2] = {128, 256};
constexpr uint32_t kGatherWideCols[2] = {128, 64};
constexpr uint64_t kGatherTallRows = 1024;
// The walk replicates segments of at least this many elements for any
// g = gcd(stride, n) (below it only for g <= 8): each of a segment's
// vectors is then stored g times by one lane, so shorter segments leave too
// few lanes (n = 2^26: s = 64 422 -> 5971 GB/s, 1024 2146 -> 12495 with
// 2^14; segments of 2^10 elements ran 1.7-6.5 x slower than the unreplicated
// walk, whose repeated reads of a short segment hit in the caches).
constexpr uint64_t kGatherLongSegment = (uint64_t)1 << 14;

}  // namespace ew
