// ew_kernels.hip -- streaming elementwise kernels for CDNA4 (gfx950).
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
//
// Kernels in this file: ew_stream_kernel (every one-pass operation and the
// fused chains), ew_gather_kernel / ew_gather_passes_kernel /
// ew_gather2_kernel (the strided gather), ew_bias_relu_kernel,
// ew_copy2d_kernel and ew_transpose_kernel (strided views), and
// ew_relu_inplace_kernel.
//
// Numerics: IEEE binary32 arithmetic in round-to-nearest-even with
// subnormals preserved (the code object's float denorm modes are "preserve";
// this file must not be built with fast-math or FTZ flags).

#include "ew_internal.h"

#include <stdint.h>

// Cache policy of the 16-byte body accesses: non-temporal ("streaming")
// loads and stores.  Every byte is touched once, so nothing is worth keeping
// in L2 or the Infinity Cache; on MI355X the nt forms measured 5-8% faster
// than the default policy for these kernels.
#ifndef EW_LOAD_NT
#define EW_LOAD_NT 1
#endif
#ifndef EW_STORE_NT
#define EW_STORE_NT 1
#endif

namespace ew {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_a4 __attribute__((ext_vector_type(4), aligned(4)));
typedef uint32_t u32x4_a2 __attribute__((ext_vector_type(4), aligned(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// ---------------------------------------------------------------------------
// 16-byte accesses
// ---------------------------------------------------------------------------

// Load the 16 bytes at p.  Co: p is 16-byte aligned.  Otherwise p is only
// element aligned (4 or 2 bytes) and the load must not assume more.
template <bool Co, int ElemSize>
__device__ __forceinline__ u32x4 load16(const char *p)
{
    if constexpr (Co) {
        const u32x4 *q = reinterpret_cast<const u32x4 *>(p);
        if constexpr (EW_LOAD_NT) return __builtin_nontemporal_load(q);
        else return *q;
    } else if constexpr (ElemSize >= 4) {
        const u32x4_a4 *q = reinterpret_cast<const u32x4_a4 *>(p);
        if constexpr (EW_LOAD_NT) return __builtin_nontemporal_load(q);
        else return *q;
    } else {
        const u32x4_a2 *q = reinterpret_cast<const u32x4_a2 *>(p);
        if constexpr (EW_LOAD_NT) return __builtin_nontemporal_load(q);
        else return *q;
    }
}

__device__ __forceinline__ void store16(char *p, u32x4 v)
{
    u32x4 *q = reinterpret_cast<u32x4 *>(p);
    if constexpr (EW_STORE_NT) __builtin_nontemporal_store(v, q);
    else *q = v;
}

// A non-temporal 16-byte store at device scope (the sc1 bit as well as nt).
// On MI355X a stream that reads one array and writes one (copy, ReLU) ran
// about 3 % faster with these stores, at 128-256-thread blocks, than with
// plain non-temporal ones; streams that read two arrays per one written (the
// adds, SAXPY) ran 1-2 % slower with them, so they keep store16.  No builtin
// sets sc1 on a global store, so this is a raw buffer store (cache-policy
// bits 0x12 = sc1 | nt) through a descriptor whose base is the caller's tile
// start (uniform across the block) and whose range is tile_bytes; the
// compiler emits it, so it also handles the instruction's hazards (a
// hand-written store in inline assembly got no wait state before the next
// write of its data registers and stored stale data).
__device__ __forceinline__ void store16_device(char *tile, uint32_t tile_bytes, uint32_t off,
                                               u32x4 v)
{
    const __amdgpu_buffer_rsrc_t r =
        __builtin_amdgcn_make_buffer_rsrc(tile, (short)0, (int)tile_bytes, 0x00020000);
    __builtin_amdgcn_raw_buffer_store_b128(v, r, (int)off, 0, 0x12);
}

// ---------------------------------------------------------------------------
// Per-element operators.  `vec` works on one 16-byte vector, `one` on one
// element; both see raw bit patterns so that the skeleton is type-agnostic.
// ---------------------------------------------------------------------------

// c = a + b, binary32.
struct OpAddF32 {
    using Elem = uint32_t;
    static constexpr int kInputs = 2;
    __device__ static u32x4 vec(u32x4 a, u32x4 b, float)
    {
        f32x4 r = __builtin_bit_cast(f32x4, a) + __builtin_bit_cast(f32x4, b);
        return __builtin_bit_cast(u32x4, r);
    }
    __device__ static Elem one(Elem a, Elem b, float)
    {
        return __builtin_bit_cast(Elem, __builtin_bit_cast(float, a) + __builtin_bit_cast(float, b));
    }
};

// c = rne16(widen(a) + widen(b)).  The compiler may lower this to a native
// binary16 add: the binary32 detour rounds twice, and 24 >= 2*11 + 2 makes
// that double rounding innocuous, so both give the correctly rounded sum.
struct OpAddF16 {
    using Elem = uint16_t;
    static constexpr int kInputs = 2;
    __device__ static u32x4 vec(u32x4 a, u32x4 b, float)
    {
        f32x8 s = __builtin_convertvector(__builtin_bit_cast(f16x8, a), f32x8) +
                  __builtin_convertvector(__builtin_bit_cast(f16x8, b), f32x8);
        return __builtin_bit_cast(u32x4, __builtin_convertvector(s, f16x8));
    }
    __device__ static Elem one(Elem a, Elem b, float)
    {
        float s = (float)__builtin_bit_cast(_Float16, a) + (float)__builtin_bit_cast(_Float16, b);
        return __builtin_bit_cast(Elem, (_Float16)s);
    }
};

// c = rnebf(widen(a) + widen(b)); the narrowing is gfx950's hardware
// round-to-nearest-even binary32 -> bfloat16 conversion.
struct OpAddBF16 {
    using Elem = uint16_t;
    static constexpr int kInputs = 2;
    __device__ static u32x4 vec(u32x4 a, u32x4 b, float)
    {
        f32x8 s = __builtin_convertvector(__builtin_bit_cast(bf16x8, a), f32x8) +
                  __builtin_convertvector(__builtin_bit_cast(bf16x8, b), f32x8);
        return __builtin_bit_cast(u32x4, __builtin_convertvector(s, bf16x8));
    }
    __device__ static Elem one(Elem a, Elem b, float)
    {
        float s = (float)__builtin_bit_cast(__bf16, a) + (float)__builtin_bit_cast(__bf16, b);
        return __builtin_bit_cast(Elem, (__bf16)s);
    }
};

// y = fma(alpha, x, y): an explicit fused multiply-add, one rounding, never
// left to floating-point contraction.  Input 0 is x, input 1 is y.
struct OpSaxpyF32 {
    using Elem = uint32_t;
    static constexpr int kInputs = 2;
    __device__ static u32x4 vec(u32x4 x, u32x4 y, float alpha)
    {
        f32x4 xf = __builtin_bit_cast(f32x4, x), yf = __builtin_bit_cast(f32x4, y), r;
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = __builtin_fmaf(alpha, xf[j], yf[j]);
        return __builtin_bit_cast(u32x4, r);
    }
    __device__ static Elem one(Elem x, Elem y, float alpha)
    {
        return __builtin_bit_cast(Elem, __builtin_fmaf(alpha, __builtin_bit_cast(float, x),
                                                       __builtin_bit_cast(float, y)));
    }
};

// y = maximum(x, +0): keep x when x > 0 or x is NaN, else +0.  Written as a
// compare and select rather than the hardware max, whose NaN rule returns the
// other operand.
struct OpReluF32 {
    using Elem = uint32_t;
    static constexpr int kInputs = 1;
    __device__ static float relu(float v) { return (v > 0.0f || v != v) ? v : 0.0f; }
    __device__ static u32x4 vec(u32x4 x, u32x4, float)
    {
        f32x4 xf = __builtin_bit_cast(f32x4, x), r;
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = relu(xf[j]);
        return __builtin_bit_cast(u32x4, r);
    }
    __device__ static Elem one(Elem x, Elem, float)
    {
        return __builtin_bit_cast(Elem, relu(__builtin_bit_cast(float, x)));
    }
};

// c = maximum(a + b, +0): the add and the ReLU fused into one pass over
// memory (12 bytes per element instead of 12 + 8 for two kernels).
struct OpAddReluF32 {
    using Elem = uint32_t;
    static constexpr int kInputs = 2;
    __device__ static u32x4 vec(u32x4 a, u32x4 b, float)
    {
        f32x4 s = __builtin_bit_cast(f32x4, a) + __builtin_bit_cast(f32x4, b), r;
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = OpReluF32::relu(s[j]);
        return __builtin_bit_cast(u32x4, r);
    }
    __device__ static Elem one(Elem a, Elem b, float)
    {
        return __builtin_bit_cast(
            Elem, OpReluF32::relu(__builtin_bit_cast(float, a) + __builtin_bit_cast(float, b)));
    }
};

// y = maximum(fma(alpha, x, y), +0), in place.
struct OpSaxpyReluF32 {
    using Elem = uint32_t;
    static constexpr int kInputs = 2;
    __device__ static u32x4 vec(u32x4 x, u32x4 y, float alpha)
    {
        f32x4 xf = __builtin_bit_cast(f32x4, x), yf = __builtin_bit_cast(f32x4, y), r;
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = OpReluF32::relu(__builtin_fmaf(alpha, xf[j], yf[j]));
        return __builtin_bit_cast(u32x4, r);
    }
    __device__ static Elem one(Elem x, Elem y, float alpha)
    {
        return __builtin_bit_cast(Elem, OpReluF32::relu(__builtin_fmaf(
                                            alpha, __builtin_bit_cast(float, x),
                                            __builtin_bit_cast(float, y))));
    }
};

// SAXPY on 16-bit data: widen x and y exactly, one binary32 fused
// multiply-add with the binary32 alpha, round to the 16-bit format RNE.
// The binary32 result is pinned in a register before the narrowing: left
// alone, the compiler fuses fma + narrow into v_fma_mixlo_f16, which rounds
// the exact product-sum once, straight to binary16 -- a different result
// whenever the binary32 rounding step changes the binary16 tie decision.
template <typename H>
struct OpSaxpy16 {
    using Elem = uint16_t;
    static constexpr int kInputs = 2;
    typedef H h8 __attribute__((ext_vector_type(8)));
    __device__ static float fma32(float alpha, float x, float y)
    {
        float r = __builtin_fmaf(alpha, x, y);
        asm("" : "+v"(r));
        return r;
    }
    __device__ static u32x4 vec(u32x4 x, u32x4 y, float alpha)
    {
        const f32x8 xf = __builtin_convertvector(__builtin_bit_cast(h8, x), f32x8);
        const f32x8 yf = __builtin_convertvector(__builtin_bit_cast(h8, y), f32x8);
        f32x8 r;
#pragma unroll
        for (int j = 0; j < 8; ++j) r[j] = fma32(alpha, xf[j], yf[j]);
        return __builtin_bit_cast(u32x4, __builtin_convertvector(r, h8));
    }
    __device__ static Elem one(Elem x, Elem y, float alpha)
    {
        const float r = fma32(alpha, (float)__builtin_bit_cast(H, x), (float)__builtin_bit_cast(H, y));
        return __builtin_bit_cast(Elem, (H)r);
    }
};
using OpSaxpyF16 = OpSaxpy16<_Float16>;
using OpSaxpyBF16 = OpSaxpy16<__bf16>;

// ReLU on 16-bit data: keep x's bits when x > 0 or x is NaN, else +0.  The
// comparison is made on the exactly widened value; no rounding happens.
template <typename H>
struct OpRelu16 {
    using Elem = uint16_t;
    static constexpr int kInputs = 1;
    typedef H h8 __attribute__((ext_vector_type(8)));
    typedef uint16_t u16x8 __attribute__((ext_vector_type(8)));
    __device__ static u32x4 vec(u32x4 x, u32x4, float)
    {
        const f32x8 xf = __builtin_convertvector(__builtin_bit_cast(h8, x), f32x8);
        const u16x8 xb = __builtin_bit_cast(u16x8, x);
        u16x8 r;
#pragma unroll
        for (int j = 0; j < 8; ++j) r[j] = (xf[j] > 0.0f || xf[j] != xf[j]) ? xb[j] : (uint16_t)0;
        return __builtin_bit_cast(u32x4, r);
    }
    __device__ static Elem one(Elem x, Elem, float)
    {
        const float v = (float)__builtin_bit_cast(H, x);
        return (v > 0.0f || v != v) ? x : (Elem)0;
    }
};
using OpReluF16 = OpRelu16<_Float16>;
using OpReluBF16 = OpRelu16<__bf16>;

// Scalar-broadcast and unary maps y = f(x): the template's middle operation
// replaced and nothing else ([EwOps] section 二, template code).  Each f is
// one IEEE binary32 operation rounded to nearest-even: alpha * x, x + alpha,
// or the square root (HIP's sqrtf is correctly rounded unless fast-math
// relaxes it; this file is never built so).
struct FnScale {
    __device__ static float f(float v, float alpha) { return alpha * v; }
};
struct FnAddScalar {
    __device__ static float f(float v, float alpha) { return v + alpha; }
};
struct FnSqrt {
    __device__ static float f(float v, float) { return __builtin_sqrtf(v); }
};

// The square root of a widened binary16 value, which is never subnormal in
// binary32, so the hardware root needs no input scaling.  v_sqrt_f32 is
// within one ulp; of it and its two neighbours the correctly rounded root is
// selected by the sign of the exact residuals x - n * s (one fma each): the
// lower neighbour is taken when x <= n_lo * s, the upper when x > n_hi * s.
// Zeros, infinities and NaNs come out of v_sqrt_f32 already right and the
// residual tests leave them (their neighbours give NaN or a zero residual).
// About half the vector work of the general binary32 sequence, which for
// widened data refines a reciprocal root; only the binary16 map uses it.
struct FnSqrtWidenedF16 {
    __device__ static float f(float v, float)
    {
        const float s = __builtin_amdgcn_sqrtf(v);
        const uint32_t si = __builtin_bit_cast(uint32_t, s);
        const float lo = __builtin_bit_cast(float, si - 1u);
        const float hi = __builtin_bit_cast(float, si + 1u);
        float r = s;
        if (__builtin_fmaf(-lo, s, v) <= 0.0f) r = lo;
        if (__builtin_fmaf(-hi, s, v) > 0.0f) r = hi;
        return r;
    }
};

// The square root of a widened bfloat16 value, to be rounded to bfloat16.
// Every positive bfloat16 root lies at least 32 binary32 ulps from a
// bfloat16 rounding boundary, so any binary32 root within a few ulps -- the
// hardware's is within one -- rounds to the same bfloat16 as the exact root;
// no refinement is needed.  Inputs below 2^-96 (bfloat16 subnormals are
// binary32 subnormals, which the hardware root is not specified for) are
// scaled by 2^32 first and the root by 2^-16 after, both exactly.
struct FnSqrtWidenedBF16 {
    __device__ static float f(float v, float)
    {
        const bool tiny = v < 0x1p-96f;
        const float s = __builtin_amdgcn_sqrtf(tiny ? v * 0x1p32f : v);
        return tiny ? s * 0x1p-16f : s;
    }
};

template <class Fn>
struct OpMapF32 {
    using Elem = uint32_t;
    static constexpr int kInputs = 1;
    __device__ static u32x4 vec(u32x4 x, u32x4, float alpha)
    {
        f32x4 xf = __builtin_bit_cast(f32x4, x), r;
#pragma unroll
        for (int j = 0; j < 4; ++j) r[j] = Fn::f(xf[j], alpha);
        return __builtin_bit_cast(u32x4, r);
    }
    __device__ static Elem one(Elem x, Elem, float alpha)
    {
        return __builtin_bit_cast(Elem, Fn::f(__builtin_bit_cast(float, x), alpha));
    }
};
using OpScaleF32 = OpMapF32<FnScale>;
using OpAddScalarF32 = OpMapF32<FnAddScalar>;
using OpSqrtF32 = OpMapF32<FnSqrt>;

// The same maps on 16-bit data: widen x exactly, apply f in binary32, round
// the result once to the 16-bit format (RNE).  The binary32 result is pinned
// in a register before the narrowing, as in OpSaxpy16, so that the compiler
// neither fuses the multiply or add with the narrowing into one mixed-
// precision instruction nor narrows a square root of a widened value into a
// native 16-bit one: either would round straight from the exact value.
template <typename H, class Fn>
struct OpMap16 {
    using Elem = uint16_t;
    static constexpr int kInputs = 1;
    typedef H h8 __attribute__((ext_vector_type(8)));
    __device__ static float f32(float v, float alpha)
    {
        float r = Fn::f(v, alpha);
        asm("" : "+v"(r));
        return r;
    }
    __device__ static u32x4 vec(u32x4 x, u32x4, float alpha)
    {
        const f32x8 xf = __builtin_convertvector(__builtin_bit_cast(h8, x), f32x8);
        f32x8 r;
#pragma unroll
        for (int j = 0; j < 8; ++j) r[j] = f32(xf[j], alpha);
        return __builtin_bit_cast(u32x4, __builtin_convertvector(r, h8));
    }
    __device__ static Elem one(Elem x, Elem, float alpha)
    {
        return __builtin_bit_cast(Elem, (H)f32((float)__builtin_bit_cast(H, x), alpha));
    }
};
using OpScaleF16 = OpMap16<_Float16, FnScale>;
using OpScaleBF16 = OpMap16<__bf16, FnScale>;
using OpAddScalarF16 = OpMap16<_Float16, FnAddScalar>;
using OpAddScalarBF16 = OpMap16<__bf16, FnAddScalar>;
using OpSqrtF16 = OpMap16<_Float16, FnSqrtWidenedF16>;
using OpSqrtBF16 = OpMap16<__bf16, FnSqrtWidenedBF16>;

// |x|: the sign bit cleared, every other bit kept (IEEE abs is a sign-bit
// operation, so NaN payloads pass unchanged).  E is the element's width.
template <typename E>
struct OpAbs {
    using Elem = E;
    static constexpr int kInputs = 1;
    static constexpr uint32_t kMask = sizeof(E) == 4 ? 0x7fffffffu : 0x7fff7fffu;
    __device__ static u32x4 vec(u32x4 x, u32x4, float) { return x & kMask; }
    __device__ static Elem one(Elem x, Elem, float) { return (Elem)(x & (Elem)kMask); }
};
using OpAbsF32 = OpAbs<uint32_t>;
using OpAbs16 = OpAbs<uint16_t>;

// out = in, bits unchanged.
struct OpCopyF32 {
    using Elem = uint32_t;
    static constexpr int kInputs = 1;
    __device__ static u32x4 vec(u32x4 x, u32x4, float) { return x; }
    __device__ static Elem one(Elem x, Elem, float) { return x; }
};

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
// Batched streaming: independent operand sets of one operation, one launch
// ---------------------------------------------------------------------------

// One tile of one batch item: the body of ew_stream_kernel for local tile lt.
template <class Op, int U, bool Co0, bool Co1>
__device__ __forceinline__ void batch_tile(const char *in0, const char *in1, char *out,
                                           uint64_t vectors, uint64_t lt, uint32_t tid,
                                           uint64_t nthr, float alpha)
{
    using E = typename Op::Elem;
    constexpr uint64_t kElem = sizeof(E);
    constexpr bool kTwo = Op::kInputs == 2;
    const uint64_t tile_vecs = nthr * U;
    const uint64_t v0 = lt * tile_vecs + tid;
    char *tile = out + lt * tile_vecs * 16;
    const uint32_t tile_bytes = (uint32_t)(tile_vecs * 16);
    if (v0 + (U - 1) * nthr < vectors) {
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
                store16_device(tile, tile_bytes, (uint32_t)((tid + u * nthr) * 16),
                               Op::vec(x[u], b, alpha));
        }
    } else {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint64_t v = v0 + u * nthr;
            if (v < vectors) {
                const u32x4 a = load16<Co0, kElem>(in0 + v * 16);
                const u32x4 b = kTwo ? load16<Co1, kElem>(in1 + v * 16) : u32x4{0, 0, 0, 0};
                if constexpr (kTwo)
                    store16(out + v * 16, Op::vec(a, b, alpha));
                else
                    store16_device(tile, tile_bytes, (uint32_t)((tid + u * nthr) * 16),
                                   Op::vec(a, b, alpha));
            }
        }
    }
}

// Many small arrays cost one launch each through the single-array entry
// points, and below about 2^21 elements the launch, not HBM, sets the time
// ([HyperAI] Stage 3: the smallest size runs at the same few microseconds in
// every version).  Here the tiles of all items are numbered consecutively and
// walked with a grid stride; a block finds the item that owns its tile by a
// binary search over tile_end (block-uniform, kernel-argument loads),
// recomputes the item's head / body / tail split and input alignment (scalar
// arithmetic on its pointers and n, the same as the host's plan of a single
// call), does the scalar head and tail if the tile is the item's first, and
// streams the tile's vectors with the item's own alignment path.
template <class Op, int U>
__global__ void __launch_bounds__(1024) ew_batch_kernel(BatchArgs args)
{
    using E = typename Op::Elem;
    constexpr uint64_t kVec = 16 / sizeof(E);
    constexpr bool kTwo = Op::kInputs == 2;
    const uint32_t tid = threadIdx.x;
    const uint64_t nthr = blockDim.x;
    for (uint64_t t = blockIdx.x; t < args.tiles; t += gridDim.x) {
        uint32_t lo = 0, hi = args.count - 1;
        while (lo < hi) {
            const uint32_t mid = (lo + hi) / 2;
            if (args.tile_end[mid] > t) hi = mid;
            else lo = mid + 1;
        }
        const BatchItem &it = args.item[lo];
        const uint64_t lt = t - (lo ? args.tile_end[lo - 1] : 0);
        // the single call's split: the head aligns the output to 16 bytes
        const uint64_t n = it.n;
        uint64_t head = ((16u - (reinterpret_cast<uintptr_t>(it.out) & 15u)) & 15u) / sizeof(E);
        if (head > n) head = n;
        const uint64_t vectors = (n - head) / kVec;
        const uint64_t tail = n - head - vectors * kVec;
        if (lt == 0 && tid < head + tail) {
            const uint64_t e = tid < head ? (uint64_t)tid : head + vectors * kVec + (tid - head);
            const E a = static_cast<const E *>(it.in0)[e];
            const E b = kTwo ? static_cast<const E *>(it.in1)[e] : E(0);
            static_cast<E *>(it.out)[e] = Op::one(a, b, args.alpha);
        }
        const char *in0 = static_cast<const char *>(it.in0) + head * sizeof(E);
        const char *in1 = kTwo ? static_cast<const char *>(it.in1) + head * sizeof(E) : nullptr;
        char *out = static_cast<char *>(it.out) + head * sizeof(E);
        const bool co0 = (reinterpret_cast<uintptr_t>(in0) & 15u) == 0;
        const bool co1 = !kTwo || (reinterpret_cast<uintptr_t>(in1) & 15u) == 0;
        const float al = args.alpha;
        if constexpr (kTwo) {
            if (co0 && co1) batch_tile<Op, U, true, true>(in0, in1, out, vectors, lt, tid, nthr, al);
            else if (co0) batch_tile<Op, U, true, false>(in0, in1, out, vectors, lt, tid, nthr, al);
            else if (co1) batch_tile<Op, U, false, true>(in0, in1, out, vectors, lt, tid, nthr, al);
            else batch_tile<Op, U, false, false>(in0, in1, out, vectors, lt, tid, nthr, al);
        } else {
            if (co0) batch_tile<Op, U, true, true>(in0, in1, out, vectors, lt, tid, nthr, al);
            else batch_tile<Op, U, false, true>(in0, in1, out, vectors, lt, tid, nthr, al);
        }
    }
}

// ---------------------------------------------------------------------------
// Strided gather: out[i] = in[(s * i) mod n]
// ---------------------------------------------------------------------------

// (a + b) mod n for a, b < n < 2^62.
__device__ __forceinline__ uint64_t add_mod(uint64_t a, uint64_t b, uint64_t n)
{
    const uint64_t r = a + b;
    return r >= n ? r - n : r;
}

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

// Small strides coprime with n (2 <= s <= 8, gcd(s, n) == 1): read every
// input element once.  Output index i reads in[s*i - k*n] where
// k = floor(s*i / n), so the output is s contiguous passes (k = 0 .. s-1),
// pass k reading every s-th input element from a residue r_k = (-k*n) mod s,
// and the s residues are all different.  Slot m of all s passes together
// therefore reads the s consecutive elements in[s*m .. s*m + s - 1].
//
// Each lane takes four slots (a group); a wave takes 64 groups, i.e. 1024 * s
// consecutive input bytes.  The wave reads them with s contiguous 16-byte-
// per-lane loads (1 KiB per instruction), parks them in its own part of LDS,
// and each lane reads back its 16 * s bytes; then, for each residue r, it
// writes the four values in[s*(m+q) + r] (q = 0..3) as one 16-byte store to
// its pass's output run at dest[r] + m.  Letting each lane load its own 16 * s
// bytes directly instead (s loads 16 * s bytes apart across the lanes) ran
// 14 % (s = 3) to 70 % (s = 7) slower on MI355X.  The register permutation is
// fixed at compile time (S is a template parameter); only the destinations
// are runtime values.
//
// Each wave keeps 1 KiB * S of loads in flight, S times what a copy wave
// keeps, and on MI355X the full gather (S writes per wave) ran fastest with
// about 24-32 KiB of loads in flight per compute unit: at full occupancy
// (32 waves per CU) it lost 9 % (s = 2) to 17 % (s = 8) against the capped
// shapes.  Blocks are therefore 256 threads and each reserves enough LDS
// that at most kPassBlocksPerCu(S) blocks fit in a CU's 160 KiB: 16 waves per
// CU for s = 2, 8 for s = 3..5, 4 for s = 6..8 (the best of 4..32 waves per
// CU and blocks of 256 or 512 threads for every s).  The reservation holds
// the waves' staging slices; the rest of it is unused.  The view (FirstOnly:
// S KiB read, 1 KiB written per wave) ran fastest uncapped, so it reserves
// only its staging.  A wave only reads back the slice it wrote itself, so no
// block barrier is needed: the LDS performs one wave's accesses in issue
// order, and wavefront-scope fences keep the compiler from moving them (a
// block barrier there cost up to 5 %).
// FirstOnly keeps only the residue-0 pass: that is the strided view
// x[::S] (out[m] = in[S*m]), read as contiguous spans of which 1/S is kept.
constexpr int kPassThreads = 256;
constexpr int kLdsBytesPerCu = 160 * 1024;

constexpr int kPassBlocksPerCu(int s) { return s == 2 ? 4 : s <= 5 ? 2 : 1; }

// Bytes of LDS each pass block reserves: its staging (16 * S bytes per lane)
// or, for the full gather if larger, just over 1/(blocks + 1) of the CU's LDS
// so that no more than kPassBlocksPerCu(S) blocks are resident on one CU.
constexpr int kPassLdsBytes(int s, bool first_only)
{
    return (first_only || kPassThreads * 16 * s > kLdsBytesPerCu / kPassBlocksPerCu(s) - 1024)
               ? kPassThreads * 16 * s
               : kLdsBytesPerCu / kPassBlocksPerCu(s) - 1024;
}
static_assert(kPassLdsBytes(2, false) * 5 > kLdsBytesPerCu &&
                  kPassLdsBytes(3, false) * 3 > kLdsBytesPerCu &&
                  kPassLdsBytes(6, false) * 2 > kLdsBytesPerCu &&
                  kPassLdsBytes(8, false) <= kLdsBytesPerCu,
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

template <int S, bool FirstOnly>
__global__ void __launch_bounds__(kPassThreads) ew_gather_passes_kernel(GatherArgs g)
{
    __shared__ u32x4 lds[kPassLdsBytes(S, FirstOnly) / 16];
    const uint32_t tid = threadIdx.x, lane = tid & 63u, wv = tid >> 6;
    u32x4 *buf = lds + wv * 64 * S;         // this wave's staging slice
    constexpr int kRuns = FirstOnly ? 1 : S;
    for (uint64_t t = blockIdx.x; t < g.tiles; t += gridDim.x) {
        const uint64_t grp0 = t * kPassThreads + wv * 64;     // first group of this wave
        const uint64_t grp = grp0 + lane;
        if ((grp0 + 64) * 4 * S <= g.n) {
            // The wave's whole span is in range, so every lane's four slots
            // exist in every pass.  A path of its own, with no element-wise
            // fallback merged into its registers: the compiler then has no
            // reason to wait for one store to complete before the next.
            const uint64_t wbase = (uint64_t)S * 4 * grp0;    // its first input element
#pragma unroll
            for (int v = 0; v < S; ++v)
                buf[64 * v + lane] = load16<false, 4>(
                    reinterpret_cast<const char *>(g.in + wbase + 4 * (64 * v + lane)));
            wave_lds_order();
            u32x4 e[S];
#pragma unroll
            for (int v = 0; v < S; ++v) e[v] = buf[S * lane + v];
            wave_lds_order();       // read back before the next tile's writes
#pragma unroll
            for (int r = 0; r < kRuns; ++r) {
                u32x4 w;
#pragma unroll
                for (int q = 0; q < 4; ++q) w[q] = e[(S * q + r) / 4][(S * q + r) % 4];
                u32x4_a4 *p = reinterpret_cast<u32x4_a4 *>(g.out + g.dest[r] + 4 * grp);
                if constexpr (EW_STORE_NT) __builtin_nontemporal_store(w, p);
                else *p = w;
            }
        } else if (grp < g.vectors) {
            // The wave at the end of the input: element by element.
            const uint64_t base = (uint64_t)S * 4 * grp;
            uint32_t e[4 * S];
#pragma unroll
            for (int k = 0; k < 4 * S; ++k) e[k] = base + k < g.n ? g.in[base + k] : 0u;
#pragma unroll
            for (int r = 0; r < kRuns; ++r) {
                uint32_t *dst = g.out + g.dest[r] + 4 * grp;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    if (base + (uint64_t)S * q + r < g.n) dst[q] = e[S * q + r];
            }
        }
    }
}

// Stride 2 with two equal segments (n even, n/2 a multiple of 4): output i of
// the first segment reads in[2i] and never wraps.  Instead of four scalar
// loads per vector, each wave reads its 2 KiB input span with two contiguous
// 16-byte-per-lane loads (1 KiB per instruction) and keeps elements 0 and 2
// of each: lane l of a wave covering outputs [o, o + 256) produces outputs
// o + 2l, o + 2l + 1 from the first load and o + 128 + 2l, o + 129 + 2l from
// the second, stored as 8-byte pairs (512 contiguous bytes per instruction),
// once per segment.  A tile is blockDim * U vectors of 4 outputs, so the
// launch shape means the same as for the general gather.
template <int U, bool Co>
__global__ void __launch_bounds__(1024) ew_gather2_kernel(GatherArgs g)
{
    typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
    const uint32_t tid = threadIdx.x;
    const uint32_t lane = tid & 63u;
    const uint32_t wave = tid >> 6;
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
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint64_t i = o + 128 * h + 2 * lane;
                if (i < body_end) {
                    const u32x2 pair = u32x2{x[u][h].x, x[u][h].z};
                    for (uint64_t k = 0; k < g.reps; ++k) {
                        u32x2 *q = reinterpret_cast<u32x2 *>(out + k * seg_bytes + 4 * i);
                        if constexpr (EW_STORE_NT) __builtin_nontemporal_store(pair, q);
                        else *q = pair;
                    }
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

template <class Op>
hipError_t launch_batch_op(const BatchArgs &args, const Launch &l, hipStream_t s)
{
    BatchArgs a = args;
    void *kargs[] = {&a};
    const void *fn = nullptr;
    switch (l.unroll) {
    case 1: fn = reinterpret_cast<const void *>(&ew_batch_kernel<Op, 1>); break;
    case 2: fn = reinterpret_cast<const void *>(&ew_batch_kernel<Op, 2>); break;
    case 4: fn = reinterpret_cast<const void *>(&ew_batch_kernel<Op, 4>); break;
    default: return hipErrorInvalidValue;
    }
    return hipLaunchKernel(fn, dim3(l.grid), dim3(l.block), kargs, 0, s);
}

}  // namespace

hipError_t launch_batch(OpId op, const BatchArgs &args, const Launch &l, hipStream_t s)
{
    switch (op) {
    case kOpAddF32: return launch_batch_op<OpAddF32>(args, l, s);
    case kOpAddF16: return launch_batch_op<OpAddF16>(args, l, s);
    case kOpAddBF16: return launch_batch_op<OpAddBF16>(args, l, s);
    case kOpSaxpyF32: return launch_batch_op<OpSaxpyF32>(args, l, s);
    case kOpReluF32: return launch_batch_op<OpReluF32>(args, l, s);
    case kOpCopyF32: return launch_batch_op<OpCopyF32>(args, l, s);
    case kOpAddReluF32: return launch_batch_op<OpAddReluF32>(args, l, s);
    case kOpSaxpyReluF32: return launch_batch_op<OpSaxpyReluF32>(args, l, s);
    case kOpSaxpyF16: return launch_batch_op<OpSaxpyF16>(args, l, s);
    case kOpSaxpyBF16: return launch_batch_op<OpSaxpyBF16>(args, l, s);
    case kOpReluF16: return launch_batch_op<OpReluF16>(args, l, s);
    case kOpReluBF16: return launch_batch_op<OpReluBF16>(args, l, s);
    case kOpScaleF32: return launch_batch_op<OpScaleF32>(args, l, s);
    case kOpScaleF16: return launch_batch_op<OpScaleF16>(args, l, s);
    case kOpScaleBF16: return launch_batch_op<OpScaleBF16>(args, l, s);
    case kOpAddScalarF32: return launch_batch_op<OpAddScalarF32>(args, l, s);
    case kOpAddScalarF16: return launch_batch_op<OpAddScalarF16>(args, l, s);
    case kOpAddScalarBF16: return launch_batch_op<OpAddScalarBF16>(args, l, s);
    case kOpSqrtF32: return launch_batch_op<OpSqrtF32>(args, l, s);
    case kOpSqrtF16: return launch_batch_op<OpSqrtF16>(args, l, s);
    case kOpSqrtBF16: return launch_batch_op<OpSqrtBF16>(args, l, s);
    case kOpAbsF32: return launch_batch_op<OpAbsF32>(args, l, s);
    case kOpAbsF16:
    case kOpAbsBF16: return launch_batch_op<OpAbs16>(args, l, s);
    default: return hipErrorInvalidValue;
    }
}

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

namespace {

template <int U, bool Co>
const void *gather2_fn()
{
    return reinterpret_cast<const void *>(&ew_gather2_kernel<U, Co>);
}

}  // namespace

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

int gather_passes_threads() { return kPassThreads; }

hipError_t launch_gather(const GatherArgs &args, const Launch &l, hipStream_t s)
{
    GatherArgs a = args;
    void *kargs[] = {&a};
    const void *fn = nullptr;
    if (args.passes >= 2) {
#define EW_PASS_FN(S) (args.first_only                                                        \
                           ? reinterpret_cast<const void *>(&ew_gather_passes_kernel<S, true>)   \
                           : reinterpret_cast<const void *>(&ew_gather_passes_kernel<S, false>))
        switch (args.passes) {
        case 2: fn = EW_PASS_FN(2); break;
        case 3: fn = EW_PASS_FN(3); break;
        case 4: fn = EW_PASS_FN(4); break;
        case 5: fn = EW_PASS_FN(5); break;
        case 6: fn = EW_PASS_FN(6); break;
        case 7: fn = EW_PASS_FN(7); break;
        case 8: fn = EW_PASS_FN(8); break;
        default: return hipErrorInvalidValue;
        }
#undef EW_PASS_FN
        return hipLaunchKernel(fn, dim3(l.grid), dim3(kPassThreads), kargs, 0, s);
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
