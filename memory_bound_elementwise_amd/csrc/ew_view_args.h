// ew_view_args.h -- the strided views' arguments and launcher, shared by
// the host API (ew_api.cpp) and ew_view.hip.  Not installed; not part of the
// C ABI.
#pragma once

#include "ew_internal.h"

namespace ew {

// Strided 2-D view copied to a contiguous row-major array:
// out[r*cols + c] = in[r*sr + c*sc].  head / vectors / tail split the
// contiguous output (n = rows * cols) as for the streaming kernels.
struct Copy2dArgs {
    const uint32_t *in;  // element (0, 0) of the view
    uint32_t *out;
    int64_t sr, sc;      // strides in elements
    uint64_t rows, cols;
    uint64_t head, vectors, tail, tiles;
    uint64_t step_vec_r, step_vec_c;    // (4 * blockDim) as (rows, cols) of the output
    uint64_t step_tile_r, step_tile_c;  // (4 * blockDim * unroll * gridDim) likewise
};

// Threads per block of the transpose kernel (one 128 x 128 tile per block
// and round).
int transpose_threads();

// mode 0: generic (one 4-byte load per element), 1: rows contiguous
// (sc == 1, 16-byte loads inside a row), 2: LDS-tiled transpose (sr == 1).
hipError_t launch_copy2d(const Copy2dArgs &args, int mode, const Launch &launch,
                         hipStream_t stream);

}  // namespace ew
