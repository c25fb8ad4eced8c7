/*
 * ew.h -- C ABI of libew, streaming elementwise kernels for AMD Instinct
 * MI355X (gfx950).
 *
 * Plain C: no C++ or torch types.  Every operation takes device pointers, an
 * element count n and a HIP stream, validates its arguments on the host,
 * launches one kernel asynchronously on that stream (ew_batch: one per
 * EW_BATCH_MAX items; ew_batch_run: one for any number) and returns a
 * status.
 *
 * Pages cited (by title and section):
 *   [HyperAI]   HyperAI article on optimising the Elementwise operator
 *               (hyper.ai/ko/news/49090)
 *   [EwOps]     "逐元素操作算子 / Element-wise 算子优化" (517adam.github.io)
 *   [Puzzle31]  Mojo GPU Puzzles, "Puzzle 31: occupancy optimisation"
 *               (puzzles.modular.com)
 *   [PerfNotes] GPU-performance lecture notes (cyqw.cn/news/898472)
 *   [GEMM-9.3]  "9.3 project: GEMM optimisation step by step" (amittech.dev)
 *
 * Conventions shared by every operation
 * -------------------------------------
 * Memory      The caller owns every buffer (device memory, e.g. allocated by
 *             torch).  The library never allocates or frees device memory
 *             and keeps no pointer after the call returns (ew_batch and
 *             ew_batch_build alone take transient host memory for their
 *             overlap check).
 * Layout      One-dimensional, contiguous, n elements.  Pointers need only
 *             element alignment (4 bytes for fp32, 2 bytes for 16-bit data);
 *             16-byte alignment is NOT required: the library peels a scalar
 *             head so that the output's body is 16-byte aligned, streams the
 *             body with 16-byte vector accesses, and finishes a scalar tail.
 * Streams     Asynchronous on `stream` (0 = the null stream).  The library
 *             never synchronises.  A kernel fault surfaces at the caller's
 *             next synchronisation, not here.
 * n == 0      Returns EW_OK without launching anything (pointers unchecked).
 * Aliasing    An output may be exactly the same pointer as an input where the
 *             operation says so; any other overlap between an output range
 *             and an input range returns EW_ERR_OVERLAP.
 * Errors      Checked in this order, before any HIP call: null pointer or an
 *             invalid size/stride (EW_ERR_INVALID_ARG), element misalignment
 *             (EW_ERR_MISALIGNED), overlap (EW_ERR_OVERLAP).  Then: no HIP
 *             device (EW_ERR_NO_DEVICE), a failed launch (EW_ERR_HIP; the
 *             hipError_t is kept for ew_last_hip_error()).  Nothing aborts.
 * Logging     With the environment variable EW_LOG set (to anything but ""
 *             or "0") every launch prints its plan -- op, n, head, vectors,
 *             tail, grid, block, unroll and the kernel path -- as one line on
 *             stderr.  Read once per process.
 * Numerics    IEEE-754 round-to-nearest-even, subnormals preserved (no
 *             flush-to-zero).  NaN results are NaN; their payload is not part
 *             of the contract for arithmetic operations.  Copy and gather
 *             move bit patterns unchanged.
 * Threads     All functions are thread-safe.
 */
#ifndef EW_H_
#define EW_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The HIP runtime declares hipStream_t the same way; repeating an identical
 * typedef is valid C11 and C++. */
typedef struct ihipStream_t *hipStream_t;

typedef enum ew_status {
    EW_OK = 0,
    EW_ERR_INVALID_ARG = -1, /* null pointer, size overflow, zero stride, unknown op name */
    EW_ERR_MISALIGNED = -2,  /* pointer not aligned to its element size */
    EW_ERR_OVERLAP = -3,     /* output partially overlaps an input */
    EW_ERR_NO_DEVICE = -4,   /* no HIP device is usable */
    EW_ERR_HIP = -5,         /* a HIP runtime call failed; see ew_last_hip_error() */
    EW_ERR_TOO_LARGE = -6    /* a batch table larger than EW_BATCH_SCRATCH_BYTES */
} ew_status_t;

/* ------------------------------------------------------------------------ */
/* Operations                                                                */
/* ------------------------------------------------------------------------ */

/* c[i] = a[i] + b[i] in binary32, i < n.
 * [HyperAI] "Version 1: FP32 baseline" and "Version 2: FP32x4 vectorisation";
 * [EwOps] section 二, template code and optimisation points 2-3 (grid-stride
 * loop, float4 body with a scalar tail).
 * a, b: inputs (device, 4-byte aligned).  c: output (device, 4-byte aligned);
 * c may equal a or b exactly. */
ew_status_t ew_add_f32(const float *a, const float *b, float *c, size_t n,
                       hipStream_t stream);

/* c[i] = rne16(widen(a[i]) + widen(b[i])) on binary16 data passed as raw
 * uint16_t bit patterns: each pair is widened exactly to binary32, added
 * once, and the sum rounded to binary16, nearest-even.  This equals the
 * correctly rounded binary16 sum.
 * [HyperAI] "Version 3: FP16 baseline" (half add per element) and
 * "Version 6: FP16x8 pack" (eight halves per 128-bit access).
 * Pointers 2-byte aligned; c may equal a or b exactly. */
ew_status_t ew_add_f16(const uint16_t *a, const uint16_t *b, uint16_t *c,
                       size_t n, hipStream_t stream);

/* The same as ew_add_f16 for bfloat16 bit patterns: widen, add in binary32,
 * round to bfloat16 nearest-even.  (The pages treat binary16; bfloat16 takes
 * the same rule.)  Pointers 2-byte aligned; c may equal a or b exactly. */
ew_status_t ew_add_bf16(const uint16_t *a, const uint16_t *b, uint16_t *c,
                        size_t n, hipStream_t stream);

/* In place: y[i] = fma(alpha, x[i], y[i]), one rounding per element.
 * [Puzzle31] overview: single-precision alpha times x plus y.
 * x: input, y: input and output (both 4-byte aligned); x may equal y
 * exactly. */
ew_status_t ew_saxpy_f32(float alpha, const float *x, float *y, size_t n,
                         hipStream_t stream);

/* y[i] = maximum(x[i], +0) in the IEEE 754-2019 sense: x > 0 gives x, a NaN
 * gives a NaN, everything else (negative, -0, -inf) gives +0.
 * [PerfNotes] section 5.2, ReLU as a memory-bound example.
 * x: input, y: output (4-byte aligned); y may equal x exactly. */
ew_status_t ew_relu_f32(const float *x, float *y, size_t n, hipStream_t stream);

/* x[i] = maximum(x[i], +0) in place, with the result of ew_relu_f32, but
 * storing only what changes: an element that is already >= 0 (or a NaN)
 * costs a read and no write ([PerfNotes] section 5.2, the ReLU intensity
 * example, its second case).  Stores are decided per aligned 64-byte span:
 * a span holding at least one element to clear is written whole, any other
 * span is left untouched (a partial span is never written: on MI355X that
 * costs more than writing it whole).  The body is aligned to 64 bytes by a
 * scalar head of up to 15 elements.  x: 4-byte aligned.  Errors as for
 * ew_relu_f32.  On data whose every element is already >= 0 it moves half
 * the bytes of ew_relu_f32(x, x).  When to prefer ew_relu_f32(x, x): data
 * with mixed signs.  On normal(0, 1) data almost every 64-byte span holds a
 * negative element, so nearly every span is written and the call moves the
 * same bytes as ew_relu_f32(x, x) (measured on MI355X: 1.33 x the bytes it
 * must move, and a few per cent slower than ew_relu_f32(x, x)). */
ew_status_t ew_relu_inplace_f32(float *x, size_t n, hipStream_t stream);

/* out[i] = in[i], bit patterns unchanged (NaN payloads included).
 * [PerfNotes] section 3.2, the coalesced copy kernel.
 * out == in is allowed and launches nothing. */
ew_status_t ew_copy_f32(const float *in, float *out, size_t n,
                        hipStream_t stream);

/* out[i] = in[(stride * i) mod n], bit patterns unchanged; the index product
 * is reduced exactly for every stride (no 32- or 64-bit wrap-around).
 * [PerfNotes] section 3.2, the non-coalesced copy kernel reads in[idx*2 % n].
 * Reads are strided; writes are contiguous.  stride 0 -> EW_ERR_INVALID_ARG.
 * in and out must not overlap at all. */
ew_status_t ew_gather_f32(const float *in, float *out, size_t n, size_t stride,
                          hipStream_t stream);

/* The same result as ew_gather_f32 -- out[i] = in[(stride * i) mod n], bits
 * unchanged -- computed the way the non-coalesced copy kernel of [PerfNotes]
 * section 3.2 computes it: every output element loads its own input element
 * (4-byte loads, index stepped per lane), whatever the stride, with none of
 * ew_gather_f32's reuse (no replicated segments, no pass decomposition, no
 * tiled transposition, no contiguous-span path).  For stride 2 on even n it reads the input twice
 * (outputs i and i + n/2 read the same element).  It is the baseline against
 * which the cost of strided reads is measured ([PerfNotes] 3.3).  Arguments,
 * errors and launch rows ("gather_walk_f32") as for ew_gather_f32; stride 1
 * also walks (no redirection to the copy). */
ew_status_t ew_gather_walk_f32(const float *in, float *out, size_t n, size_t stride,
                               hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Strided views                                                            */
/* ------------------------------------------------------------------------ */

/* A strided 2-D view copied to a contiguous row-major array, bit patterns
 * unchanged: out[r*cols + c] = in[r*stride_r + c*stride_c] for r < rows,
 * c < cols.  Strides are in elements and signed (zero and negative strides
 * are allowed); `in` points at element (0, 0) of the view.  A 1-D strided
 * view (PyTorch x[::s]) is rows = 1, stride_c = s; a submatrix has
 * stride_c = 1; a transposed view has stride_r = 1.
 * [PerfNotes] 3.4 (non-contiguous tensors show up as strides) and 3.1-3.2
 * (coalesced versus strided reads).
 * Paths: rows == 1 with stride_c == 2 reads contiguous 16-byte spans and
 * keeps the even elements; rows == 1 with 3 <= stride_c <= 32 reads the
 * view's span contiguously (staged through LDS) and keeps one element in
 * stride_c; stride_c == 1 reads whole 16-byte row segments;
 * stride_r == 1 moves 128 x 128 tiles through LDS so that both reads and
 * writes are coalesced; otherwise one 4-byte load per element.  out is written with 16-byte
 * stores after a scalar head.
 * Errors: rows or cols 0 -> EW_OK; null pointers, rows*cols overflow, or a
 * view reaching outside the address space -> EW_ERR_INVALID_ARG; in or out
 * not 4-byte aligned -> EW_ERR_MISALIGNED; any overlap between out and the
 * span of elements the view touches -> EW_ERR_OVERLAP. */
ew_status_t ew_copy2d_f32(const float *in, int64_t stride_r, int64_t stride_c,
                          float *out, size_t rows, size_t cols, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* SAXPY and ReLU on 16-bit data                                             */
/* ------------------------------------------------------------------------ */
/* The operator template of [EwOps] section 二 (only the middle operation
 * changes) applied to the 16-bit formats of [HyperAI] Stage 2.  Data are raw
 * uint16_t bit patterns, pointers 2-byte aligned, 8 lanes per 16-byte vector. */

/* In place: y[i] = rne16(fma(alpha, widen(x[i]), widen(y[i]))): x and y are
 * widened exactly, one binary32 fused multiply-add with the binary32 alpha,
 * then one round-to-nearest-even to binary16.  x may equal y. */
ew_status_t ew_saxpy_f16(float alpha, const uint16_t *x, uint16_t *y, size_t n,
                         hipStream_t stream);

/* The same for bfloat16. */
ew_status_t ew_saxpy_bf16(float alpha, const uint16_t *x, uint16_t *y, size_t n,
                          hipStream_t stream);

/* y[i] = maximum(x[i], +0) on binary16 / bfloat16: x's bits when x > 0 or x
 * is a NaN, else +0 (no rounding).  y may equal x. */
ew_status_t ew_relu_f16(const uint16_t *x, uint16_t *y, size_t n, hipStream_t stream);
ew_status_t ew_relu_bf16(const uint16_t *x, uint16_t *y, size_t n, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Scalar-broadcast and unary maps, in every format                          */
/* ------------------------------------------------------------------------ */
/* More instances of [EwOps] section 二's template (index, bounds check and
 * store fixed; only the middle operation replaced): y[i] = f(x[i]), one
 * input stream and one output stream, 8 bytes per fp32 element and 4 per
 * 16-bit element.  fp32: f is one binary32 operation rounded to nearest-
 * even.  _f16 / _bf16: x is widened exactly to binary32, f is applied in
 * binary32 (with the binary32 alpha), and the result is rounded once to the
 * 16-bit format, nearest-even -- the rule of the 16-bit add ([HyperAI]
 * Stage 2).  Data are raw bit patterns for the 16-bit formats; pointers
 * need element alignment.  y may equal x (in place); any other overlap is
 * EW_ERR_OVERLAP.  NaN results are NaN (payload not part of the contract)
 * except for abs, which moves bits. */

/* Scalar broadcast, multiply: y[i] = alpha * x[i]. */
ew_status_t ew_scale_f32(float alpha, const float *x, float *y, size_t n, hipStream_t stream);
ew_status_t ew_scale_f16(float alpha, const uint16_t *x, uint16_t *y, size_t n,
                         hipStream_t stream);
ew_status_t ew_scale_bf16(float alpha, const uint16_t *x, uint16_t *y, size_t n,
                          hipStream_t stream);

/* Scalar broadcast, add: y[i] = x[i] + alpha. */
ew_status_t ew_add_scalar_f32(float alpha, const float *x, float *y, size_t n,
                              hipStream_t stream);
ew_status_t ew_add_scalar_f16(float alpha, const uint16_t *x, uint16_t *y, size_t n,
                              hipStream_t stream);
ew_status_t ew_add_scalar_bf16(float alpha, const uint16_t *x, uint16_t *y, size_t n,
                               hipStream_t stream);

/* Unary: y[i] = sqrt(x[i]), correctly rounded in binary32 (sqrt(-0) = -0,
 * negative inputs give NaN); the 16-bit forms round that binary32 root to
 * the 16-bit format, which equals the correctly rounded 16-bit root. */
ew_status_t ew_sqrt_f32(const float *x, float *y, size_t n, hipStream_t stream);
ew_status_t ew_sqrt_f16(const uint16_t *x, uint16_t *y, size_t n, hipStream_t stream);
ew_status_t ew_sqrt_bf16(const uint16_t *x, uint16_t *y, size_t n, hipStream_t stream);

/* Unary: y[i] = |x[i]|, the sign bit cleared and every other bit (NaN
 * payloads included) unchanged. */
ew_status_t ew_abs_f32(const float *x, float *y, size_t n, hipStream_t stream);
ew_status_t ew_abs_f16(const uint16_t *x, uint16_t *y, size_t n, hipStream_t stream);
ew_status_t ew_abs_bf16(const uint16_t *x, uint16_t *y, size_t n, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Batched calls: many small arrays, one launch                              */
/* ------------------------------------------------------------------------ */
/* [HyperAI] Stage 3: at the smallest size every kernel version takes the
 * same few microseconds -- the launch, not the memory.  Many small arrays
 * each cost that floor through the single-array entry points; a batched call
 * runs up to EW_BATCH_MAX of them per kernel launch. */

#define EW_BATCH_MAX 96

/* One operand set: the pointers of the single call, in ew_make_plan's
 * order.  out = c (add), y (saxpy, in place), y (ReLU, maps), out (copy).
 * in0 = a (add) or x.  in1 = b (add); ignored for the one-input operations
 * and for SAXPY, whose second input is out itself. */
typedef struct ew_batch_item {
    void *out;
    const void *in0;
    const void *in1;
    size_t n;
} ew_batch_item_t;

/* Runs count independent instances of one streaming operation -- any of
 * "add_f32", "add_f16", "add_bf16", "saxpy_f32", "relu_f32", "copy_f32",
 * "add_relu_f32", "saxpy_relu_f32", "saxpy_f16", "saxpy_bf16", "relu_f16",
 * "relu_bf16" and the scale / add_scalar / sqrt / abs maps -- each with the
 * result its single call would give, in ceil(items / EW_BATCH_MAX) kernel
 * launches on `stream` (items with n == 0 are skipped).  alpha is used by
 * the SAXPY, scale and add-scalar operations and ignored otherwise.  items:
 * a host array, read during the call only.
 * Errors: an unknown or non-batchable op name, items == NULL with count >
 * 0, or host memory for the overlap check (about 72 bytes per item) not
 * available -> EW_ERR_INVALID_ARG; each item is validated like its single call
 * (first failing item's status); an item's output range intersecting any
 * range of another item -> EW_ERR_OVERLAP (the items run concurrently; reads
 * of shared inputs are fine).  count == 0 or all n == 0 -> EW_OK, no launch.
 * The launch shape is the table's row of the operation for the total element
 * count (unroll at most 4). */
ew_status_t ew_batch(const char *op, float alpha, const ew_batch_item_t *items,
                     size_t count, hipStream_t stream);

/* Batched calls with the item table in device memory: one kernel launch for
 * any number of items.  The library builds the table image on the host
 * (ew_batch_build, into memory the caller provides), the caller places it in
 * device memory (any copy; it may be reused for every call on the same
 * items), and ew_batch_run launches one kernel that reads it.  This is the
 * form to use for many items and for repeated calls on the same arrays; it
 * also suits graph capture (ew_batch_run makes no copy and allocates
 * nothing).
 *
 * ew_batch_plan_t describes a built table; fill it only through
 * ew_batch_build.  The launch shape is the table's row of the operation for
 * the total element count (unroll at most 4); the grid is min(blocks_per_cu
 * * CU count, tiles). */
typedef struct ew_batch_plan {
    int32_t op;             /* operation (library-internal number) */
    int32_t block;          /* threads per block */
    int32_t unroll;         /* 16-byte vectors per lane per tile */
    int32_t blocks_per_cu;  /* grid cap per compute unit */
    uint64_t items;         /* records in the table: the items with n > 0 */
    uint64_t tiles;         /* tiles of all items together (one block each) */
    uint64_t bytes;         /* size of the table image, a multiple of 8 */
    uint64_t total_n;       /* elements of all items together */
} ew_batch_plan_t;

/* Validates items exactly as ew_batch does (same operations, same errors)
 * and fills *plan.  With table == NULL it only sizes the image (plan->bytes)
 * and returns EW_OK; otherwise it writes the image -- plan->items records of
 * 40 bytes (in0, in1, out, n, first tile), then one 32-bit item index per
 * tile, zero padded to plan->bytes -- into `table` (host memory, 8-byte
 * aligned, table_bytes >= plan->bytes; EW_ERR_INVALID_ARG if smaller,
 * EW_ERR_MISALIGNED if not 8-byte aligned).  No device is needed.  The
 * image holds the items' device pointers: it stays valid while those
 * buffers do. */
ew_status_t ew_batch_build(const char *op, const ew_batch_item_t *items, size_t count,
                           void *table, size_t table_bytes, ew_batch_plan_t *plan);

/* Runs a built table in one kernel launch on `stream`: the result of
 * ew_batch on the same items and alpha.  table: device memory (8-byte
 * aligned) holding exactly the plan->bytes bytes that ew_batch_build wrote
 * for this plan; the kernel trusts its pointers as every entry point trusts
 * its buffers, so a table that was changed or built for other buffers is
 * undefined behaviour.  The plan's fields are checked for consistency
 * (EW_ERR_INVALID_ARG).  plan->tiles == 0 (no item with n > 0) -> EW_OK, no
 * launch.  Calls on different streams may share one table (it is only
 * read). */
ew_status_t ew_batch_run(const ew_batch_plan_t *plan, float alpha, const void *table,
                         hipStream_t stream);

/* For callers that cannot allocate device memory (no hipMalloc of their own
 * for the table: code that must not allocate, allocation-free serving
 * loops): ew_batch_run with the table image taken from host memory and
 * placed by the library in a static device array of EW_BATCH_SCRATCH_BYTES
 * that it holds on each GPU it runs on until the process ends.  The call
 * allocates nothing.  It waits for `stream` (earlier work may still read
 * the array), copies the plan->bytes bytes of table_host (the image
 * ew_batch_build wrote, in host memory) into the array on the current
 * device, waits for the copy, and launches the kernel asynchronously;
 * table_host may be reused when the call returns.  Because it waits, it
 * cannot be captured into a graph (ew_batch_run with a caller-owned device
 * table can).  Every call on one GPU shares that GPU's array, which keeps
 * the last call's table: calls that overlap on one GPU -- on different
 * streams, or from several threads -- race; calls on one stream do not.
 * plan->bytes > EW_BATCH_SCRATCH_BYTES -> EW_ERR_TOO_LARGE (use
 * ew_batch_run); other errors as for ew_batch_run. */
#define EW_BATCH_SCRATCH_BYTES (256 * 1024)
ew_status_t ew_batch_run_static(const ew_batch_plan_t *plan, float alpha, const void *table_host,
                                hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Fused chains: one pass over memory instead of two                         */
/* ------------------------------------------------------------------------ */
/* An epilogue fused into the producing kernel saves a full pass through HBM
 * ([GEMM-9.3] "what comes next": bias and ReLU inside the same kernel;
 * [PerfNotes] 5.3: fusion raises the arithmetic intensity of memory-bound
 * work).  Each result is rounded exactly as the unfused sequence would round
 * it, so the fused and unfused paths agree bit for bit. */

/* c[i] = maximum(a[i] + b[i], +0): the binary32 sum, then the ReLU of
 * ew_relu_f32.  12 bytes per element, where ew_add_f32 followed by
 * ew_relu_f32 moves 20.  Pointers 4-byte aligned; c may equal a or b. */
ew_status_t ew_add_relu_f32(const float *a, const float *b, float *c, size_t n,
                            hipStream_t stream);

/* In place: y[i] = maximum(fma(alpha, x[i], y[i]), +0).  x may equal y. */
ew_status_t ew_saxpy_relu_f32(float alpha, const float *x, float *y, size_t n,
                              hipStream_t stream);

/* y[r*cols + c] = maximum(x[r*cols + c] + bias[c], +0) for a row-major
 * rows x cols matrix: the bias row is broadcast down the rows (a bias-and-
 * activation epilogue).  x, y: rows*cols elements (y may equal x); bias: cols
 * elements, must not overlap y.  rows or cols 0 -> EW_OK.  Errors as for the
 * other operations; the bias pointer is checked after x and y. */
ew_status_t ew_bias_relu_f32(const float *x, const float *bias, float *y,
                             size_t rows, size_t cols, hipStream_t stream);

/* ------------------------------------------------------------------------ */
/* Status, launch configuration and planning                                */
/* ------------------------------------------------------------------------ */

/* Static string for a status code (never NULL). */
const char *ew_status_string(ew_status_t status);

/* The hipError_t behind the most recent EW_ERR_HIP on the calling thread
 * (0 if none). */
int ew_last_hip_error(void);

/* Library ABI version (incremented on any incompatible change). */
int ew_abi_version(void);

/* Launch configuration, per operation name ("add_f32", "add_f16",
 * "add_bf16", "saxpy_f32", "relu_f32", "copy_f32", "gather_f32",
 * "gather_walk_f32", "add_relu_f32", "saxpy_relu_f32", "bias_relu_f32",
 * "saxpy_f16", "saxpy_bf16", "relu_f16", "relu_bf16", "copy2d_f32",
 * "relu_inplace_f32", "scale_f32", "scale_f16", "scale_bf16",
 * "add_scalar_f32", "add_scalar_f16", "add_scalar_bf16", "sqrt_f32",
 * "sqrt_f16", "sqrt_bf16", "abs_f32", "abs_f16", "abs_bf16").
 * A launch is `grid` blocks of `block` threads; each block walks tiles of
 * block * unroll 16-byte vectors with a grid stride, and the grid is
 * min(blocks_per_cu * CU count, number of tiles) ([EwOps] section 二,
 * optimisation point 2: a grid sized to the processor count times a small
 * factor).  block: a multiple of 64 in [64, 1024]; blocks_per_cu in
 * [1, 1024]; unroll in {1, 2, 4, 8}.  Out of range or unknown op ->
 * EW_ERR_INVALID_ARG.
 *
 * The table holds, per operation, rows for size classes (see
 * ew_set_launch_row); the compiled-in rows were tuned on MI355X. */

/* One launch configuration for every size of `op`: replaces all of op's
 * rows with one row applying to every n. */
ew_status_t ew_set_launch_config(const char *op, int block, int blocks_per_cu, int unroll);

/* The launch the next call of `op` with n elements would make on the
 * current device, for pointers 16-byte aligned (as device allocations are):
 * threads per block, grid (0 when n == 0: no launch) and unroll.  For the
 * gather this is the index walk's grid (ew_gather_walk_f32, or
 * ew_gather_f32 at a stride that takes the walk); ew_make_gather_plan gives
 * the grid for a given stride.  Needs a device: EW_ERR_NO_DEVICE without
 * one. */
ew_status_t ew_get_launch_config(const char *op, size_t n, int *block, int *grid, int *unroll);

/* Size classes: a row applies to every n >= min_n up to the next row's
 * min_n; setting a row with an existing min_n replaces it (at most 16 rows
 * per operation, else EW_ERR_INVALID_ARG). */
ew_status_t ew_set_launch_row(const char *op, size_t min_n, int block, int blocks_per_cu,
                              int unroll);

/* The row that applies to n (no device needed). */
ew_status_t ew_get_launch_row(const char *op, size_t n, int *block, int *blocks_per_cu,
                              int *unroll);

/* Restore the compiled-in table (tuned on MI355X). */
void ew_reset_launch_config(void);

/* Read rows "op min_n block blocks_per_cu unroll" (one per line, '#'
 * comments) from a text file and apply them with ew_set_launch_row.
 * EW_ERR_INVALID_ARG on an unreadable file or a malformed row (rows before
 * it stay applied). */
ew_status_t ew_load_launch_table(const char *path);

/* The host-side plan of one call: how the n elements split into a scalar
 * head, a body of 16-byte vectors and a scalar tail, and how the body is
 * launched.  Pure arithmetic on the pointer values -- nothing is touched and
 * no device is needed (pass cu_count explicitly).
 *   head       elements before the output reaches 16-byte alignment
 *              ((16 - out mod 16) mod 16) / element size, capped at n
 *              (64-byte alignment, 64 in place of 16, for relu_inplace_f32)
 *   vectors    16-byte vectors in the body, floor((n - head) / vec_elems)
 *   tail       n - head - vectors * vec_elems  (< vec_elems)
 *   in_coaligned[k]  1 if input k's body start is 16-byte aligned too
 *              (then it is read with aligned 16-byte loads; otherwise with
 *              4- or 2-byte aligned 16-byte loads); unused inputs report 1
 *   tiles      ceil(vectors / (block * unroll))
 *   grid       min(blocks_per_cu * cu_count, tiles), at least 1 when n > 0
 *   segment, reps, passes   n, 1 and 1, except for the gather
 *              (ew_make_gather_plan)
 *   path       the kernel path (ew_path_t): EW_PATH_STREAM, or
 *              EW_PATH_GATHER_WALK for "gather_walk_f32"
 * Validation is the same as the operation's (in1 is ignored for one-input
 * ops; for saxpy in0 = x and out = y). */
/* Which kernel path a plan launches. */
typedef enum ew_path {
    EW_PATH_STREAM = 0,          /* the streaming kernel: head / 16-byte body / tail */
    EW_PATH_COPY = 1,            /* a gather with stride 1 mod n: the contiguous copy */
    EW_PATH_GATHER_WALK = 2,     /* per-output index walk (reps equal segments) */
    EW_PATH_GATHER_SPANS = 3,    /* stride 2: contiguous 16-byte loads, even elements kept */
    EW_PATH_GATHER_PASSES = 4,   /* stride 2..32: spans staged through LDS, runs written */
    EW_PATH_VIEW_ROWS = 5,       /* strided view, rows contiguous */
    EW_PATH_VIEW_TRANSPOSE = 6,  /* strided view, 128 x 128 tiles through LDS */
    EW_PATH_VIEW_GENERIC = 7,    /* strided view, one 4-byte load per element */
    EW_PATH_GATHER_TILES = 8     /* stride > 32: rows of `stride` elements transposed
                                    through LDS, each column written as a run */
} ew_path_t;

typedef struct ew_plan {
    size_t n;
    size_t head;
    size_t vectors;
    size_t tail;
    size_t tiles;
    int vec_elems;
    int elem_size;
    int in_coaligned[2];
    int block;
    int blocks_per_cu;
    int unroll;
    int grid;
    size_t segment;
    int reps;
    int passes;
    int path;               /* an ew_path_t */
} ew_plan_t;

ew_status_t ew_make_plan(const char *op, const void *out, const void *in0,
                         const void *in1, size_t n, int cu_count,
                         ew_plan_t *plan);

/* The gather's plan.  Let s = stride mod n and g = gcd(s, n): output
 * elements i and i + n/g read the same input element, so the output
 * consists of reps = g equal segments of segment = n/g elements, and the
 * kernels compute one segment and store each value g times, so that each
 * input line is fetched once rather than g times.
 * s == 1 (or n == 1): the contiguous copy (path EW_PATH_COPY, the copy's
 * plan).  s == 2 with g == 2 and n/2 a multiple of 4: a kernel that reads the
 * input with contiguous 16-byte loads (EW_PATH_GATHER_SPANS; head / vectors
 * / tail describe one segment).
 * Otherwise 2 <= s <= 32 (EW_PATH_GATHER_PASSES): with s' = s/g, a segment
 * splits into passes = s' contiguous runs: run k holds the i with
 * floor(s'*i / segment) == k and reads every s-th input element from an
 * offset g*r that differs per run (0 <= r < s'), so slot m of all runs reads
 * from the s consecutive elements s*m .. s*m + s - 1.  The kernel reads the
 * input once, contiguously (staged through LDS), and writes the runs;
 * vectors = groups of four slots of the longest run (ceil(segment / s')),
 * head = tail = 0, block = 256 and unroll = 1 whatever the table says (its
 * blocks_per_cu still caps the grid; the kernel's own LDS reservation limits
 * how many of its blocks share a compute unit).
 * Otherwise, for s > 32 with s' = s/g >= 2, g < 32, at least 128 rows
 * (ceil(n / s) >= 128), s' < 2^32 and s' * (n/g) < 2^64
 * (EW_PATH_GATHER_TILES): the input viewed as rows of s elements,
 * A[m][c] = in[s*m + c], is transposed through LDS: column g*r of A is one
 * run of a segment (passes = s', clamped to INT_MAX; the run of column g*r
 * is the k-th with k = (-r * (n/g)^-1) mod s'), written from output
 * ceil(k * segment / s') on.  block = 1024, unroll = 1, one block per tile
 * (tiles: for s < 68 bands of floor(16384 / s) rounded down to a multiple
 * of 4 whole rows, kept one word apart in LDS when s is a multiple of 4,
 * else 128 x 128 tiles while A has fewer than 1024 rows and
 * 256 rows x 64 columns from there on), the grid capped at the table's
 * blocks_per_cu per compute unit, vectors = ceil(segment / 4),
 * head = tail = 0.
 * Otherwise (s == 0, or a large stride outside those bounds) the per-output
 * index walk (EW_PATH_GATHER_WALK), on one segment when n/g is a multiple of
 * 4 and 2 <= g <= 8 or n/g >= 2^14 (else segment = n and reps = 1);
 * passes = 1.
 * Same validation as ew_gather_f32. */
ew_status_t ew_make_gather_plan(const void *out, const void *in, size_t n,
                                size_t stride, int cu_count, ew_plan_t *plan);

/* The plan of ew_copy2d_f32 with these arguments: its path (x[::2] ->
 * EW_PATH_GATHER_SPANS, x[::s] with s = 3..32 -> EW_PATH_GATHER_PASSES with
 * passes = 1 (one run), stride_c == 1 -> EW_PATH_VIEW_ROWS, stride_r == 1 ->
 * EW_PATH_VIEW_TRANSPOSE, else EW_PATH_VIEW_GENERIC) and the launch it makes
 * (block, grid, unroll as launched; a kernel with a fixed block shape reports
 * that shape; tiles counts 128 x 128 tiles for the transpose).  No device is
 * needed.  Same validation as ew_copy2d_f32. */
ew_status_t ew_make_copy2d_plan(const void *in, int64_t stride_r, int64_t stride_c,
                                const void *out, size_t rows, size_t cols, int cu_count,
                                ew_plan_t *plan);

#ifdef __cplusplus
}
#endif

#endif /* EW_H_ */
