// ew_internal.h -- declarations shared by the host API (ew_api.cpp) and the
// device kernels (ew_stream.hip, ew_batch.hip, ew_gather.hip, ew_view.hip)
// of libew.  Not installed; not part of the
// C ABI.
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

// A batched call: up to kBatchMax independent operand sets of one streaming
// operation in one launch.  Item k owns the global tiles [tile_end[k - 1],
// tile_end[k]) -- at least one, so that its scalar head and tail have a block.
// Each block recomputes its item's head / vectors / tail split and input
// alignment from the pointers and n, exactly as the host plans a single
// call, so an item travels as four words.  The whole struct is the kernel
// argument (3856 bytes, under the 4 KiB kernel-argument limit).
constexpr int kBatchMax = 96;
struct BatchItem {
    const void *in0;
    const void *in1;     // nullptr for one-input operations
    void *out;
    uint64_t n;
};
struct BatchArgs {
    uint64_t tiles;      // tiles of all items together
    uint32_t count;      // items in this launch, 1..kBatchMax
    float alpha;         // saxpy, scale and add-scalar only
    uint64_t tile_end[kBatchMax];
    BatchItem item[kBatchMax];
};
static_assert(sizeof(BatchArgs) <= 4096, "kernel arguments are limited to 4 KiB");

// A batched call whose item table lives in device memory (any number of
// items per launch).  Table image, 8-byte aligned: `count` BatchTableItem
// records, then one uint32_t per global tile naming the item that owns it.
// Item k owns the tiles [first_tile, first_tile + its tile count), at least
// one per item so that its scalar head and tail have a block.
struct BatchTableItem {
    const void *in0;
    const void *in1;     // nullptr for one-input operations
    void *out;
    uint64_t n;
    uint64_t first_tile;
};
static_assert(sizeof(BatchTableItem) == 40, "table record layout");
struct BatchTableArgs {
    const BatchTableItem *item;
    const uint32_t *tile_item;
    uint64_t tiles;      // tiles of all items together
    float alpha;         // saxpy, scale and add-scalar only
};

// The gather additionally walks its input index (stride * i) mod n
// incrementally; the steps are reduced mod n on the host.  When
// g = gcd(stride, n) > 1 the output is g copies of one segment of n / g
// elements (out[i + k*n/g] = out[i]); then head / vectors / tail describe one
// segment and every value is stored `reps` times, `seg` elements apart, so
// each input element is fetched once instead of g times.
// Strides up to kMaxPasses that are coprime with n take the pass
// decomposition below (one kernel instance per stride).
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

struct Launch {
    int block;
    int grid;
    int unroll;
};

// Launch one streaming kernel.  co0 / co1: whether input 0 / 1 is 16-byte
// aligned at its body start.  Returns the launch status.
hipError_t launch_stream(OpId op, const StreamArgs &args, bool co0, bool co1,
                         const Launch &launch, hipStream_t stream);

// Launch one batched streaming kernel (block and unroll from `launch`; the
// unroll must be 1, 2 or 4).
hipError_t launch_batch(OpId op, const BatchArgs &args, const Launch &launch,
                        hipStream_t stream);

// Launch one batched kernel reading its item table from device memory
// (unroll 1, 2 or 4).
hipError_t launch_batch_table(OpId op, const BatchTableArgs &args, const Launch &launch,
                              hipStream_t stream);

// Size of the library's static device array that holds a batch table for
// the entry point that allocates nothing (ew_batch_run_static).
constexpr uint64_t kBatchScratchBytes = 256 * 1024;

// Device address of that array on the current device (looked up once per
// device with hipGetSymbolAddress, then cached).
hipError_t batch_scratch(void **ptr);

hipError_t launch_gather(const GatherArgs &args, const Launch &launch,
                         hipStream_t stream);

// Threads per block of the pass-decomposed gather (one group of four slots
// per thread, one tile per block and round).
int gather_passes_threads();

// Threads per block of the transpose kernel (one 128 x 128 tile per block
// and round).
int transpose_threads();

// mode 0: generic (one 4-byte load per element), 1: rows contiguous
// (sc == 1, 16-byte loads inside a row), 2: LDS-tiled transpose (sr == 1).
hipError_t launch_copy2d(const Copy2dArgs &args, int mode, const Launch &launch,
                         hipStream_t stream);

// In-place ReLU on args.out (in0 == out); the body must start 64-byte
// aligned.
hipError_t launch_relu_inplace(const StreamArgs &args, const Launch &launch,
                               hipStream_t stream);

// co: x's body start is 16-byte aligned (it is read with aligned loads).
hipError_t launch_bias_relu(const BiasArgs &args, bool co, const Launch &launch,
                            hipStream_t stream);

}  // namespace ew
