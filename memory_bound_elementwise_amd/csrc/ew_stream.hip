// ew_stream.hip -- the streaming skeleton for CDNA4 (gfx950) and the kernels
// built directly on it: ew_stream_kernel (every one-pass operation and the
// fused add + ReLU / SAXPY + ReLU chains), ew_bias_relu_kernel (a broadcast
// bias row) and ew_relu_inplace_kernel (ReLU storing only what changes).
//
// One skeleton serves every operation; only the per-element operator changes
// ([EwOps] section 二, template code: index, bounds check and operator form a
// fixed frame around a replaceable middle).  The skeleton:
//
//   * a scalar head (elements before the output is 16-byte aligned) and a
//     scalar tail (fewer than one vector at the end), handled by the first
//     lanes of block 0;
//   * a body of 16-byte vectors (4 fp32 or 8 fp16/bf16 lanes), each wave
//     instruction moving 64 lanes x 16 B = 1 KiB of contiguous memory with
//     global_load_dwordx4 / global_store_dwordx4 ([HyperAI] "Version 2" and
//     "Version 6": one 128-bit access per lane instead of four 32-bit ones);
//   * tiles of blockDim * U vectors, walked with a grid stride by a grid of a
//     few blocks per compute unit ([EwOps] optimisation point 2), with all U
//     loads of a tile issued before the first store so that enough bytes are
//     in flight to cover HBM latency ([EwOps] point 2 on overlapping
//     requests; [PerfNotes] section 2.2, hide latency rather than reduce it);
//   * non-temporal stores: nothing written is read again by this kernel
//     (single-input streams store at device scope as well, see
//     store16_device).
//
// No matrix cores: nothing is contracted.  The streaming kernels use no LDS
// either (every byte is used once); LDS only reorders data where the access
// order of the input and the output differ -- the transpose's tiles and the
// pass-decomposed gather's staging.  Inputs whose body start is not 16-byte
// aligned relative to the output are read with element-aligned 16-byte loads
// (the hardware splits them across cache lines); the streaming kernels'
// output is always aligned.

#include "ew_device.h"

namespace ew {

// ---------------------------------------------------------------------------
// The streaming skeleton
// ---------------------------------------------------------------------------

template <class Op, int U, bool Co0, bool Co1>
__global__ void __launch_bounds__(1024) ew_stream_kernel(StreamArgs args)
{
    using E = typename Op::Elem;
    constexpr uint64_t kElem = sizeof(E);
    constexpr uint64_t kVec = 16 / kElem;
    constexpr bool kTwo = Op::kInputs == 2;
    const uint32_t tid = threadIdx.x;
    const uint64_t nthr = blockDim.x;

    // Scalar head and tail: at most 2 * (kVec - 1) elements, one per lane.
    if (blockIdx.x == 0 && tid < args.head + args.tail) {
        const uint64_t e = tid < args.head
                               ? (uint64_t)tid
                               : args.head + args.vectors * kVec + (tid - args.head);
        const E a = static_cast<const E *>(args.in0)[e];
        const E b = kTwo ? static_cast<const E *>(args.in1)[e] : E(0);
        static_cast<E *>(args.out)[e] = Op::one(a, b, args.alpha);
    }

    const char *in0 = static_cast<const char *>(args.in0) + args.head * kElem;
    const char *in1 = kTwo ? static_cast<const char *>(args.in1) + args.head * kElem : nullptr;
    char *out = static_cast<char *>(args.out) + args.head * kElem;
    const uint64_t tile_vecs = nthr * U;
    const float alpha = args.alpha;

    for (uint64_t t = blockIdx.x; t < args.tiles; t += gridDim.x) {
        const uint64_t v0 = t * tile_vecs + tid;
        if (v0 + (U - 1) * nthr < args.vectors) {
            // Whole tile for this lane: issue every load, then every store.
            u32x4 x[U], y[U];
#pragma unroll
            for (int u = 0; u < U; ++u) x[u] = load16<Co0, kElem>(in0 + (v0 + u * nthr) * 16);
            if constexpr (kTwo) {
#pragma unroll
                for (int u = 0; u < U; ++u) y[u] = load16<Co1, kElem>(in1 + (v0 + u * nthr) * 16);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const u32x4 b = kTwo ? y[u] : u32x4{0, 0, 0, 0};
                if constexpr (kTwo)
                    store16(out + (v0 + u * nthr) * 16, Op::vec(x[u], b, alpha));
                else
                    store16_device(out + t * tile_vecs * 16, (uint32_t)(tile_vecs * 16),
                                   (uint32_t)((tid + u * nthr) * 16), Op::vec(x[u], b, alpha));
            }
        } else {
            // Last, partial tile.
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint64_t v = v0 + u * nthr;
                if (v < args.vectors) {
                    const u32x4 a = load16<Co0, kElem>(in0 + v * 16);
                    const u32x4 b = kTwo ? load16<Co1, kElem>(in1 + v * 16) : u32x4{0, 0, 0, 0};
                    if constexpr (kTwo)
                        store16(out + v * 16, Op::vec(a, b, alpha));
                    else
                        store16_device(out + t * tile_vecs * 16, (uint32_t)(tile_vecs * 16),
                                       (uint32_t)((tid + u * nthr) * 16), Op::vec(a, b, alpha));
                }
            }
        }
    }
}
// ---------------------------------------------------------------------------
// Bias + ReLU: y[i] = maximum(x[i] + bias[i mod cols], +0)
// ---------------------------------------------------------------------------

// The streaming skeleton with a broadcast second operand: x and y stream
// through 16-byte vectors; each lane walks the column of its vector's first
// element incrementally (one 64-bit remainder per lane, then
// compare-and-subtract steps precomputed on the host).  VecBias: cols is a
// multiple of 4 and the body starts at a row start's alignment (head == 0),
// so a vector's four columns are contiguous and never wrap; the bias is then
// read as one 16-byte load.  Otherwise four 4-byte loads.  Bias loads use
// the default cache policy: the bias row is reused by every row.
template <int U, bool Co, bool VecBias>
__global__ void __launch_bounds__(1024) ew_bias_relu_kernel(BiasArgs a)
{
    const uint32_t tid = threadIdx.x;
    const uint64_t nthr = blockDim.x;
    const uint64_t cols = a.cols;

    if (blockIdx.x == 0 && tid < a.head + a.tail) {
        const uint64_t e = tid < a.head ? (uint64_t)tid : a.head + a.vectors * 4 + (tid - a.head);
        a.y[e] = OpReluF32::relu(a.x[e] + a.bias[e % cols]);
    }

    uint64_t t = blockIdx.x;
    if (t >= a.tiles) return;
    const char *x = reinterpret_cast<const char *>(a.x + a.head);
    char *y = reinterpret_cast<char *>(a.y + a.head);
    const uint64_t tile_vecs = nthr * U;
    uint64_t ct = (a.head + 4 * (t * tile_vecs + tid)) % cols;   // column of the first element

    for (; t < a.tiles; t += gridDim.x) {
        const uint64_t v0 = t * tile_vecs + tid;
        u32x4 xv[U];
        f32x4 bv[U];
        uint64_t c = ct;
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const bool live = v0 + u * nthr < a.vectors;
            xv[u] = live ? load16<Co, 4>(x + (v0 + u * nthr) * 16) : u32x4{0, 0, 0, 0};
            if constexpr (VecBias) {
                bv[u] = live ? __builtin_bit_cast(
                                   f32x4, *reinterpret_cast<const u32x4_a4 *>(a.bias + c))
                             : f32x4{0, 0, 0, 0};
            } else {
                uint64_t cc = c;
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    bv[u][k] = live ? a.bias[cc] : 0.0f;
                    cc = cc + 1 == cols ? 0 : cc + 1;
                }
            }
            c = add_mod(c, a.step_vec, cols);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t v = v0 + u * nthr;
            if (v < a.vectors) {
                f32x4 s = __builtin_bit_cast(f32x4, xv[u]) + bv[u], r;
#pragma unroll
                for (int k = 0; k < 4; ++k) r[k] = OpReluF32::relu(s[k]);
                // one array read (and the small bias row), one written
                store16_device(y + t * tile_vecs * 16, (uint32_t)(tile_vecs * 16),
                               (uint32_t)((tid + u * nthr) * 16), __builtin_bit_cast(u32x4, r));
            }
        }
        ct = add_mod(ct, a.step_tile, cols);
    }
}
// ---------------------------------------------------------------------------
// In-place ReLU that stores only what changes
// ---------------------------------------------------------------------------

// Width, in lanes of 16 bytes, of one store decision: the lanes of a group
// store together when any element in the group changes, and not at all
// otherwise.  4 lanes = one aligned 64-byte span (the body starts 64-byte
// aligned), so a span is either written whole or left untouched.  On MI355X
// narrower decisions lose: a 16-byte or 4-byte store that covers part of a
// 64-byte span ran 1.2x and 3x slower than writing every element, while
// whole 64-byte spans cost nothing extra and skip more than 128-byte lines.
#ifndef EW_RELU_INPLACE_GROUP
#define EW_RELU_INPLACE_GROUP 4
#endif

// ReLU changes x exactly when its sign bit is set and it is not a NaN
// (negative numbers, -inf and -0 become +0; NaNs pass through unchanged).
__device__ __forceinline__ bool relu_changes(uint32_t u)
{
    return u >= 0x80000000u && u <= 0xff800000u;
}

// x = maximum(x, +0) in place, writing only where the result differs from
// what is already stored ([PerfNotes] 5.2, scenario B: an element that is
// already >= 0 costs a read and no write).  The host aligns the body to 64
// bytes (head of up to 15 elements); head and tail are scalar, stored only
// when the element changes.
template <int U>
__global__ void __launch_bounds__(1024) ew_relu_inplace_kernel(StreamArgs args)
{
    constexpr int G = EW_RELU_INPLACE_GROUP;
    static_assert(G == 0 || G == 1 || G == 2 || G == 4 || G == 8, "group of 0-8 lanes");
    const uint32_t tid = threadIdx.x;
    const uint64_t nthr = blockDim.x;
    uint32_t *x = static_cast<uint32_t *>(args.out);

    if (blockIdx.x == 0 && tid < args.head + args.tail) {
        const uint64_t e = tid < args.head ? (uint64_t)tid
                                           : args.head + args.vectors * 4 + (tid - args.head);
        if (relu_changes(x[e])) x[e] = 0u;
    }

    char *body = reinterpret_cast<char *>(x + args.head);
    const uint64_t tile_vecs = nthr * U;
    const uint32_t lane = __lane_id();

    // Store vector v of tile t (already loaded as w) if its group needs it.
    auto finish = [&](uint64_t t, uint64_t v, u32x4 w) {
        bool ch[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) ch[k] = relu_changes(w[k]);
        if constexpr (G == 0) {
            // element granularity: one 4-byte store per changed element
            uint32_t *q = reinterpret_cast<uint32_t *>(body + v * 16);
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (ch[k]) __builtin_nontemporal_store(0u, q + k);
        } else {
            bool any = ch[0] || ch[1] || ch[2] || ch[3];
            if constexpr (G > 1) {
                const uint64_t m = __ballot(any);
                any = ((m >> (lane & ~(uint32_t)(G - 1))) & ((1ull << G) - 1)) != 0;
            }
            if (any) {
                u32x4 r;
#pragma unroll
                for (int k = 0; k < 4; ++k) r[k] = ch[k] ? 0u : w[k];
                // one array read, (part of) it written: a device-scope store
                store16_device(body + t * tile_vecs * 16, (uint32_t)(tile_vecs * 16),
                               (uint32_t)((v - t * tile_vecs) * 16), r);
            }
        }
    };

    for (uint64_t t = blockIdx.x; t < args.tiles; t += gridDim.x) {
        const uint64_t v0 = t * tile_vecs + tid;
        if (v0 + (U - 1) * nthr < args.vectors) {
            u32x4 w[U];
#pragma unroll
            for (int u = 0; u < U; ++u) w[u] = load16<true, 4>(body + (v0 + u * nthr) * 16);
#pragma unroll
            for (int u = 0; u < U; ++u) finish(t, v0 + u * nthr, w[u]);
        } else {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint64_t v = v0 + u * nthr;
                if (v < args.vectors) finish(t, v, load16<true, 4>(body + v * 16));
            }
        }
    }
}
// ---------------------------------------------------------------------------
// Dispatch
// ---------------------------------------------------------------------------

namespace {

template <class Op, int U, bool Co0, bool Co1>
hipError_t launch_typed(const StreamArgs &args, const Launch &l, hipStream_t s)
{
    StreamArgs a = args;
    void *kargs[] = {&a};
    return hipLaunchKernel(reinterpret_cast<const void *>(&ew_stream_kernel<Op, U, Co0, Co1>),
                           dim3(l.grid), dim3(l.block), kargs, 0, s);
}

template <class Op, int U>
hipError_t launch_aligned(const StreamArgs &args, bool co0, bool co1, const Launch &l,
                          hipStream_t s)
{
    if constexpr (Op::kInputs == 2) {
        if (co0 && co1) return launch_typed<Op, U, true, true>(args, l, s);
        if (co0) return launch_typed<Op, U, true, false>(args, l, s);
        if (co1) return launch_typed<Op, U, false, true>(args, l, s);
        return launch_typed<Op, U, false, false>(args, l, s);
    } else {
        (void)co1;
        if (co0) return launch_typed<Op, U, true, true>(args, l, s);
        return launch_typed<Op, U, false, true>(args, l, s);
    }
}

template <class Op>
hipError_t launch_op(const StreamArgs &args, bool co0, bool co1, const Launch &l, hipStream_t s)
{
    switch (l.unroll) {
    case 1: return launch_aligned<Op, 1>(args, co0, co1, l, s);
    case 2: return launch_aligned<Op, 2>(args, co0, co1, l, s);
    case 4: return launch_aligned<Op, 4>(args, co0, co1, l, s);
    case 8: return launch_aligned<Op, 8>(args, co0, co1, l, s);
    default: return hipErrorInvalidValue;
    }
}
}  // namespace

hipError_t launch_stream(OpId op, const StreamArgs &args, bool co0, bool co1,
                         const Launch &launch, hipStream_t stream)
{
    switch (op) {
    case kOpAddF32: return launch_op<OpAddF32>(args, co0, co1, launch, stream);
    case kOpAddF16: return launch_op<OpAddF16>(args, co0, co1, launch, stream);
    case kOpAddBF16: return launch_op<OpAddBF16>(args, co0, co1, launch, stream);
    case kOpSaxpyF32: return launch_op<OpSaxpyF32>(args, co0, co1, launch, stream);
    case kOpReluF32: return launch_op<OpReluF32>(args, co0, co1, launch, stream);
    case kOpCopyF32: return launch_op<OpCopyF32>(args, co0, co1, launch, stream);
    case kOpAddReluF32: return launch_op<OpAddReluF32>(args, co0, co1, launch, stream);
    case kOpSaxpyReluF32: return launch_op<OpSaxpyReluF32>(args, co0, co1, launch, stream);
    case kOpSaxpyF16: return launch_op<OpSaxpyF16>(args, co0, co1, launch, stream);
    case kOpSaxpyBF16: return launch_op<OpSaxpyBF16>(args, co0, co1, launch, stream);
    case kOpReluF16: return launch_op<OpReluF16>(args, co0, co1, launch, stream);
    case kOpReluBF16: return launch_op<OpReluBF16>(args, co0, co1, launch, stream);
    case kOpScaleF32: return launch_op<OpScaleF32>(args, co0, co1, launch, stream);
    case kOpScaleF16: return launch_op<OpScaleF16>(args, co0, co1, launch, stream);
    case kOpScaleBF16: return launch_op<OpScaleBF16>(args, co0, co1, launch, stream);
    case kOpAddScalarF32: return launch_op<OpAddScalarF32>(args, co0, co1, launch, stream);
    case kOpAddScalarF16: return launch_op<OpAddScalarF16>(args, co0, co1, launch, stream);
    case kOpAddScalarBF16: return launch_op<OpAddScalarBF16>(args, co0, co1, launch, stream);
    case kOpSqrtF32: return launch_op<OpSqrtF32>(args, co0, co1, launch, stream);
    case kOpSqrtF16: return launch_op<OpSqrtF16>(args, co0, co1, launch, stream);
    case kOpSqrtBF16: return launch_op<OpSqrtBF16>(args, co0, co1, launch, stream);
    case kOpAbsF32: return launch_op<OpAbsF32>(args, co0, co1, launch, stream);
    // binary16 and bfloat16 share the sign bit's position: one kernel
    case kOpAbsF16:
    case kOpAbsBF16: return launch_op<OpAbs16>(args, co0, co1, launch, stream);
    default: return hipErrorInvalidValue;
    }
}
hipError_t launch_bias_relu(const BiasArgs &args, bool co, const Launch &l, hipStream_t s)
{
    BiasArgs a = args;
    void *kargs[] = {&a};
    const void *fn = nullptr;
    const bool vb = args.cols % 4 == 0 && args.head == 0;
#define EW_BIAS_FN(U)                                                                      \
    (vb ? (co ? reinterpret_cast<const void *>(&ew_bias_relu_kernel<U, true, true>)         \
              : reinterpret_cast<const void *>(&ew_bias_relu_kernel<U, false, true>))       \
        : (co ? reinterpret_cast<const void *>(&ew_bias_relu_kernel<U, true, false>)        \
              : reinterpret_cast<const void *>(&ew_bias_relu_kernel<U, false, false>)))
    switch (l.unroll) {
    case 1: fn = EW_BIAS_FN(1); break;
    case 2: fn = EW_BIAS_FN(2); break;
    case 4: fn = EW_BIAS_FN(4); break;
    case 8: fn = EW_BIAS_FN(8); break;
    default: return hipErrorInvalidValue;
    }
#undef EW_BIAS_FN
    return hipLaunchKernel(fn, dim3(l.grid), dim3(l.block), kargs, 0, s);
}
hipError_t launch_relu_inplace(const StreamArgs &args, const Launch &l, hipStream_t s)
{
    StreamArgs a = args;
    void *kargs[] = {&a};
    const void *fn = nullptr;
    switch (l.unroll) {
    case 1: fn = reinterpret_cast<const void *>(&ew_relu_inplace_kernel<1>); break;
    case 2: fn = reinterpret_cast<const void *>(&ew_relu_inplace_kernel<2>); break;
    case 4: fn = reinterpret_cast<const void *>(&ew_relu_inplace_kernel<4>); break;
    case 8: fn = reinterpret_cast<const void *>(&ew_relu_inplace_kernel<8>); break;
    default: return hipErrorInvalidValue;
    }
    return hipLaunchKernel(fn, dim3(l.grid), dim3(l.block), kargs, 0, s);
}
}  // namespace ew
