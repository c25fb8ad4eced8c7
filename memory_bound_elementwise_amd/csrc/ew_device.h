// ew_device.h -- device-side building blocks shared by every kernel family
// of libew (gfx950): 16-byte vector types, the 16-byte load and store forms
// and their cache policies, and the per-element operators of the streaming
// skeleton.  Not installed; not part of the C ABI.
//
// Numerics: IEEE binary32 arithmetic in round-to-nearest-even with
// subnormals preserved (the code object's float denorm modes are "preserve";
// no source that includes this header may be built with fast-math or FTZ
// flags).
#pragma once

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

// (a + b) mod n for a, b < n < 2^62.
__device__ __forceinline__ uint64_t add_mod(uint64_t a, uint64_t b, uint64_t n)
{
    const uint64_t r = a + b;
    return r >= n ? r - n : r;
}

}  // namespace ew
