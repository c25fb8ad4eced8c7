// ew_internal.h -- declarations shared by the host API (ew_api.cpp) and all
// device kernels of libew: the operation numbers, the launch shape and the
// streaming kernels' arguments and launchers.  Each other kernel family
// declares its own in ew_batch_args.h, ew_gather_args.h and ew_view_args.h.
// Not installed; not part of the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ew {

enum OpId : int {
    kOpAddF32 = 0,
    kOpAddF16,
    kOpAddBF16,
    kOpSaxpyF32,
    kOpReluF32,
    kOpCopyF32,
    kOpGatherF32,
    kOpAddReluF32,
    kOpSaxpyReluF32,
    kOpBiasReluF32,
    kOpSaxpyF16,
    kOpSaxpyBF16,
    kOpReluF16,
    kOpReluBF16,
    kOpCopy2dF32,
    kOpReluInplaceF32,
    kOpScaleF32,
    kOpScaleF16,
    kOpScaleBF16,
    kOpAddScalarF32,
    kOpAddScalarF16,
    kOpAddScalarBF16,
    kOpSqrtF32,
    kOpSqrtF16,
    kOpSqrtBF16,
    kOpAbsF32,
    kOpAbsF16,
    kOpAbsBF16,
    kOpGatherWalkF32,
    kOpCount
};

// Everything a streaming kernel needs, computed on the host.  Element
// indices: [0, head) scalar head, then `vectors` 16-byte vectors starting at
// element `head`, then `tail` scalar elements.
struct StreamArgs {
    const void *in0;     // first input (x for saxpy / relu / copy)
    const void *in1;     // second input (y for saxpy), nullptr if unused
    void *out;           // output (y for saxpy)
    uint64_t head;
    uint64_t vectors;
    uint64_t tail;
    uint64_t tiles;      // ceil(vectors / (blockDim * unroll))
    float alpha;         // saxpy, scale and add-scalar only
};

// Bias + ReLU over a row-major rows x cols matrix (n = rows * cols): the
// column index of element i is i mod cols, walked incrementally per lane.
struct BiasArgs {
    const float *x;
    const float *bias;
    float *y;
    uint64_t cols;
    uint64_t head;
    uint64_t vectors;
    uint64_t tail;
    uint64_t tiles;
    uint64_t step_vec;   // (4 * blockDim) mod cols: next unrolled vector
    uint64_t step_tile;  // (4 * blockDim * unroll * gridDim) mod cols: next tile
};

struct Launch {
    int block;
    int grid;
    int unroll;
};

// Launch one streaming kernel.  co0 / co1: whether input 0 / 1 is 16-byte
// aligned at its body start.  Returns the launch status.
hipError_t launch_stream(OpId op, const StreamArgs &args, bool co0, bool co1,
                         const Launch &launch, hipStream_t stream);

// In-place ReLU on args.out (in0 == out); the body must start 64-byte
// aligned.
hipError_t launch_relu_inplace(const StreamArgs &args, const Launch &launch,
                               hipStream_t stream);

// co: x's body start is 16-byte aligned (it is read with aligned loads).
hipError_t launch_bias_relu(const BiasArgs &args, bool co, const Launch &launch,
                            hipStream_t stream);

}  // namespace ew
