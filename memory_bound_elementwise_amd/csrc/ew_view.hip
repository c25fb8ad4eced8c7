// ew_view.hip -- strided 2-D views copied to contiguous arrays for CDNA4
// (gfx950): an output-ordered kernel walking (row, column) per lane and an
// LDS-tiled transpose for views whose rows are the input's columns.

#include "ew_device.h"
#include "ew_view_args.h"

namespace ew {

// ---------------------------------------------------------------------------
// Strided 2-D views: out[r*cols + c] = in[r*sr + c*sc], out contiguous
// ---------------------------------------------------------------------------

// Output-ordered kernel: the streaming skeleton over the contiguous output,
// each lane walking the (row, column) of its vector incrementally (one
// 64-bit division per lane, then host-precomputed steps with a carry).
// RowContig (sc == 1): a vector whose four columns lie in one row is read
// with one element-aligned 16-byte load; otherwise four 4-byte loads.
template <int U, bool RowContig>
__global__ void __launch_bounds__(1024) ew_copy2d_kernel(Copy2dArgs a)
{
    const uint32_t tid = threadIdx.x;
    const uint64_t nthr = blockDim.x;
    const uint64_t cols = a.cols;

    if (blockIdx.x == 0 && tid < a.head + a.tail) {
        const uint64_t e = tid < a.head ? (uint64_t)tid : a.head + a.vectors * 4 + (tid - a.head);
        const int64_t r = (int64_t)(e / cols), c = (int64_t)(e % cols);
        a.out[e] = a.in[r * a.sr + c * a.sc];
    }

    uint64_t t = blockIdx.x;
    if (t >= a.tiles) return;
    char *out = reinterpret_cast<char *>(a.out + a.head);
    const uint64_t tile_vecs = nthr * U;
    const uint64_t e0 = a.head + 4 * (t * tile_vecs + tid);
    uint64_t rt = e0 / cols, ct = e0 % cols;    // (row, column) of this lane's first element

    for (; t < a.tiles; t += gridDim.x) {
        const uint64_t v0 = t * tile_vecs + tid;
        u32x4 x[U];
        uint64_t r = rt, c = ct;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool live = v0 + u * nthr < a.vectors;
            if (RowContig && c + 3 < cols) {
                x[u] = live ? load16<false, 4>(reinterpret_cast<const char *>(
                                  a.in + (int64_t)r * a.sr + (int64_t)c))
                            : u32x4{0, 0, 0, 0};
            } else {
                uint64_t rr = r, cc = c;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    x[u][k] = live ? a.in[(int64_t)rr * a.sr + (int64_t)cc * a.sc] : 0u;
                    if (++cc == cols) { cc = 0; ++rr; }
                }
            }
            c += a.step_vec_c;
            r += a.step_vec_r;
            if (c >= cols) { c -= cols; ++r; }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t v = v0 + u * nthr;
            if (v < a.vectors)        // one view read, one array written: device scope
                store16_device(out + t * tile_vecs * 16, (uint32_t)(tile_vecs * 16),
                               (uint32_t)((tid + u * nthr) * 16), x[u]);
        }
        ct += a.step_tile_c;
        rt += a.step_tile_r;
        if (ct >= cols) { ct -= cols; ++rt; }
    }
}

// Transposed views (sr == 1: the input is contiguous along the output's
// rows).  Reading in output order would touch one cache line per element;
// instead each 1024-thread block moves a 128 x 128 tile through LDS: it reads
// the tile column by column (128 consecutive input elements = 512 B, 16 bytes
// per lane), writes it into LDS with 128-bit stores, and writes the output
// row by row (128 consecutive output elements, 16 bytes per lane), so both
// HBM streams are coalesced.  Rows of the LDS tile are padded to 132 words
// (67,584 B; gfx950 gives a workgroup up to 160 KB).  Consecutive blocks take
// consecutive tiles along the output's rows, so the writes of neighbouring
// blocks continue each other.  On MI355X this shape reached 96 % of the
// contiguous copy's rate, against 75 % for 64 x 64 tiles of 256 threads: each
// input and output segment is 512 B instead of 256 B.  Partial edge tiles fall
// back to 4-byte accesses with bounds checks.  Tiles are walked with a grid
// stride; one 64-bit division per tile.
constexpr int kT = 128;
constexpr int kPitch = kT + 4;
constexpr int kTThreads = 1024;
constexpr int kTLanesPerRow = kT / 4;                    // 32 lanes cover one tile row
constexpr int kTRowsPerPass = kTThreads / kTLanesPerRow;  // 32
constexpr int kTPasses = kT / kTRowsPerPass;              // 4

__global__ void __launch_bounds__(kTThreads) ew_transpose_kernel(Copy2dArgs a)
{
    __shared__ uint32_t tile[kT * kPitch];
    const uint32_t tid = threadIdx.x;
    const uint64_t tiles_c = (a.cols + kT - 1) / kT;
    const uint64_t tiles = tiles_c * ((a.rows + kT - 1) / kT);
    const uint32_t sub = tid / kTLanesPerRow;        // 0..31
    const uint32_t q4 = (tid % kTLanesPerRow) * 4;   // 0, 4, ..., 124

    for (uint64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
        const uint64_t r0 = (t / tiles_c) * kT, c0 = (t % tiles_c) * kT;
        const bool full = r0 + kT <= a.rows && c0 + kT <= a.cols;
        // Load: column c0 + c of the tile is kT consecutive input elements.
        u32x4 v[kTPasses];
#pragma unroll
        for (int p = 0; p < kTPasses; ++p) {
            const uint32_t c = p * kTRowsPerPass + sub;
            const int64_t base = (int64_t)(c0 + c) * a.sc + (int64_t)(r0 + q4);
            if (full) {
                v[p] = load16<false, 4>(reinterpret_cast<const char *>(a.in + base));
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const bool ok = c0 + c < a.cols && r0 + q4 + k < a.rows;
                    v[p][k] = ok ? a.in[base + k] : 0u;
                }
            }
        }
#pragma unroll
        for (int p = 0; p < kTPasses; ++p)
            *reinterpret_cast<u32x4 *>(&tile[(p * kTRowsPerPass + sub) * kPitch + q4]) = v[p];
        __syncthreads();
        // Store: output row r0 + r of the tile is kT consecutive elements.
#pragma unroll
        for (int p = 0; p < kTPasses; ++p) {
            const uint32_t r = p * kTRowsPerPass + sub;
            u32x4 w;
#pragma unroll
            for (int k = 0; k < 4; ++k) w[k] = tile[(q4 + k) * kPitch + r];
            uint32_t *dst = a.out + (r0 + r) * a.cols + c0 + q4;
            if (full) {
                u32x4_a4 *q = reinterpret_cast<u32x4_a4 *>(dst);
                if constexpr (EW_STORE_NT) __builtin_nontemporal_store(w, q);
                else *q = w;
            } else if (r0 + r < a.rows) {
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    if (c0 + q4 + k < a.cols) dst[k] = w[k];
            }
        }
        // the tile is rewritten only if this block has another round (a
        // block-uniform condition)
        if (t + gridDim.x < tiles) __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// Dispatch
// ---------------------------------------------------------------------------

int transpose_threads() { return kTThreads; }

hipError_t launch_copy2d(const Copy2dArgs &args, int mode, const Launch &l, hipStream_t s)
{
    Copy2dArgs a = args;
    void *kargs[] = {&a};
    const void *fn = nullptr;
    if (mode == 2) {
        fn = reinterpret_cast<const void *>(&ew_transpose_kernel);
        return hipLaunchKernel(fn, dim3(l.grid), dim3(kTThreads), kargs, 0, s);
    }
#define EW_C2D_FN(U) (mode == 1 ? reinterpret_cast<const void *>(&ew_copy2d_kernel<U, true>) \
                                : reinterpret_cast<const void *>(&ew_copy2d_kernel<U, false>))
    switch (l.unroll) {
    case 1: fn = EW_C2D_FN(1); break;
    case 2: fn = EW_C2D_FN(2); break;
    case 4: fn = EW_C2D_FN(4); break;
    case 8: fn = EW_C2D_FN(8); break;
    default: return hipErrorInvalidValue;
    }
#undef EW_C2D_FN
    return hipLaunchKernel(fn, dim3(l.grid), dim3(l.block), kargs, 0, s);
}
}  // namespace ew
