/*
 * oracle.c -- plain scalar CPU definition of every elementwise operation the
 * library computes.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check and
 * the bench's CPU-baseline leg call it; the product path never does.
 *
 * It shares no source, header, macro, table or helper with the HIP library.
 * Every function is a plain `for (i = 0; i < n; ++i)` loop over size_t, built
 * with -O2 -fno-fast-math -ffp-contract=off on x86-64 SSE (no x87 excess
 * precision), so each C expression below is exactly one IEEE-754 binary32
 * operation rounded to nearest-even with subnormals kept.
 *
 * Pages cited (by title and section):
 *   [HyperAI]   HyperAI article "optimising the Elementwise operator"
 *               (hyper.ai/ko/news/49090)
 *   [EwOps]     "逐元素操作算子 / Element-wise 算子优化" (517adam.github.io)
 *   [Puzzle31]  Mojo GPU Puzzles, "Puzzle 31: occupancy optimisation"
 *               (puzzles.modular.com)
 *   [PerfNotes] GPU-performance lecture notes (cyqw.cn/news/898472)
 *   [GEMM-9.3]  "9.3 project: GEMM optimisation step by step" (amittech.dev)
 *
 * Parity status: every function here is pinned by tests against library
 * routines (numpy, torch CPU, the x86 F16C instructions), exact rational arithmetic,
 * closed forms and brute force.  None is "parity unpinned".
 */
#include <stddef.h>
#include <stdint.h>
#include <string.h>
#include <math.h>
#include <xmmintrin.h>

/* ------------------------------------------------------------------------ */
/* Floating-point environment                                               */
/* ------------------------------------------------------------------------ */

/* Returns 1 when SSE arithmetic is IEEE default: flush-to-zero (MXCSR bit 15)
 * and denormals-are-zero (bit 6) clear, rounding control (bits 13-14) at
 * round-to-nearest-even.  A fast-math library loaded into the process can set
 * FTZ/DAZ globally, which would silently change every subnormal result. */
int oracle_fpenv_ok(void)
{
    unsigned int csr = _mm_getcsr();
    int ftz = (csr >> 15) & 1u;
    int daz = (csr >> 6) & 1u;
    int rc = (csr >> 13) & 3u;
    return (!ftz && !daz && rc == 0) ? 1 : 0;
}

static uint32_t f32_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_f32(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* Round the unsigned integer x right by s bits to nearest, ties to even.
 * This is the IEEE-754 roundTiesToEven rule applied to a fixed-point value:
 * the kept part q is incremented when the dropped part exceeds one half, or
 * equals exactly one half and q is odd. */
static uint32_t rne_shift_right(uint32_t x, unsigned s)
{
    if (s == 0) return x;
    if (s >= 32) {
        /* Everything is dropped; the dropped part is below one half unless
         * s == 32 and the top bit is set (not reachable by the callers). */
        return 0;
    }
    uint32_t q = x >> s;
    uint32_t rem = x & ((1u << s) - 1u);
    uint32_t half = 1u << (s - 1);
    if (rem > half || (rem == half && (q & 1u))) q += 1u;
    return q;
}

/* ------------------------------------------------------------------------ */
/* binary16 <-> binary32, from the IEEE-754 interchange-format definition    */
/* ------------------------------------------------------------------------ */
/* binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits.  Normal numbers
 * span [2^-14, 65504]; subnormals are multiples of 2^-24.                   */

/* Exact widening of a binary16 bit pattern to binary32 (every binary16 value
 * is representable in binary32). */
float oracle_f16_to_f32(uint16_t h)
{
    uint32_t sign = ((uint32_t)h & 0x8000u) << 16;
    uint32_t e = ((uint32_t)h >> 10) & 0x1fu;
    uint32_t m = (uint32_t)h & 0x3ffu;
    uint32_t out;
    if (e == 0x1fu) {
        /* infinity, or NaN: the payload moves to the top of the binary32
         * fraction, and a signalling NaN comes out quiet (IEEE 754
         * convertFormat delivers a quiet NaN for a signalling input). */
        out = sign | 0x7f800000u | (m << 13);
        if (m != 0) out |= 0x00400000u;
    } else if (e != 0) {
        out = sign | ((e - 15u + 127u) << 23) | (m << 13);
    } else if (m == 0) {
        out = sign; /* signed zero */
    } else {
        /* subnormal m * 2^-24: normalise so the leading one becomes implicit */
        int shift = 0;
        while ((m & 0x400u) == 0) { m <<= 1; ++shift; }
        m &= 0x3ffu;
        /* value = 1.m * 2^(-14 - shift) */
        out = sign | ((uint32_t)(127 - 14 - shift) << 23) | (m << 13);
    }
    return bits_f32(out);
}

/* binary32 -> binary16, round to nearest, ties to even.
 * NaN becomes a quiet NaN with the same sign (top payload bits kept);
 * magnitudes >= 65520 (the midpoint between 65504 and 2^16, which ties to the
 * even neighbour 2^16) become infinity; the normal range drops 13 fraction
 * bits with RNE; below 2^-14 the result is a multiple of 2^-24, rounded RNE. */
uint16_t oracle_f32_to_f16(float f)
{
    uint32_t u = f32_bits(f);
    uint32_t sign = (u >> 16) & 0x8000u;
    uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) {
        return (uint16_t)(sign | 0x7c00u | 0x0200u | ((a >> 13) & 0x3ffu));
    }
    if (a >= 0x477ff000u) {                      /* >= 65520, or infinity */
        return (uint16_t)(sign | 0x7c00u);
    }
    uint32_t E = a >> 23;                        /* biased binary32 exponent */
    if (E >= 113u) {                             /* a >= 2^-14: normal */
        /* Re-bias the exponent (127 -> 15) in place, then drop 13 bits.
         * A carry out of the fraction correctly bumps the exponent. */
        uint32_t r = a - ((127u - 15u) << 23);
        return (uint16_t)(sign | rne_shift_right(r, 13));
    }
    if (E == 0) {
        /* binary32 zero or subnormal (< 2^-126): far below 2^-25 */
        return (uint16_t)sign;
    }
    /* 2^-126 <= a < 2^-14: value = m24 * 2^(E-150); in units of 2^-24 that
     * is m24 * 2^(E-126), i.e. a right shift by 126-E >= 14 bits. */
    uint32_t m24 = (a & 0x7fffffu) | 0x800000u;
    uint32_t q = rne_shift_right(m24, 126u - E);
    return (uint16_t)(sign | q);                /* q == 0x400 is 2^-14: fine */
}

/* ------------------------------------------------------------------------ */
/* bfloat16 <-> binary32                                                      */
/* ------------------------------------------------------------------------ */
/* bfloat16 is the top half of a binary32: 1 sign, 8 exponent, 7 fraction.   */

float oracle_bf16_to_f32(uint16_t b) { return bits_f32((uint32_t)b << 16); }

/* binary32 -> bfloat16, round to nearest, ties to even; NaN stays a quiet NaN
 * with its sign.  Rounding a finite value past the largest bfloat16 carries
 * into the exponent field and yields infinity, as IEEE rounding requires. */
uint16_t oracle_f32_to_bf16(float f)
{
    uint32_t u = f32_bits(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) {
        return (uint16_t)((u >> 16) | 0x0040u);
    }
    uint32_t sign = u & 0x80000000u;
    uint32_t mag = rne_shift_right(u & 0x7fffffffu, 16);
    return (uint16_t)((sign >> 16) | mag);
}

/* ------------------------------------------------------------------------ */
/* The operations                                                           */
/* ------------------------------------------------------------------------ */

/* C = A + B in binary32.  [HyperAI] "Version 1: FP32 baseline" and
 * [EwOps] "二、优化方向 / template code": c[i] = a[i] + b[i] per element. */
void oracle_add_f32(const float *a, const float *b, float *c, size_t n)
{
    for (size_t i = 0; i < n; ++i) c[i] = a[i] + b[i];
}

/* C = A + B on binary16 data: widen both operands exactly, add once in
 * binary32, round the sum to binary16 RNE.  [HyperAI] "Version 3: FP16
 * baseline" (half-precision add per element) and "Version 6: FP16x8 pack"
 * (same sum, eight lanes at a time). */
void oracle_add_f16(const uint16_t *a, const uint16_t *b, uint16_t *c, size_t n)
{
    for (size_t i = 0; i < n; ++i) {
        float s = oracle_f16_to_f32(a[i]) + oracle_f16_to_f32(b[i]);
        c[i] = oracle_f32_to_f16(s);
    }
}

/* C = A + B on bfloat16 data: widen, add once in binary32, round RNE.
 * (The pages name bfloat16 only as a matrix-unit input type; the rule here
 * is the same fp32-then-RNE rule as for binary16.) */
void oracle_add_bf16(const uint16_t *a, const uint16_t *b, uint16_t *c, size_t n)
{
    for (size_t i = 0; i < n; ++i) {
        float s = oracle_bf16_to_f32(a[i]) + oracle_bf16_to_f32(b[i]);
        c[i] = oracle_f32_to_bf16(s);
    }
}

/* SAXPY in place, y[i] <- alpha*x[i] + y[i], with one rounding (fused
 * multiply-add; C99 fmaf is correctly rounded).  [Puzzle31] "Overview":
 * single-precision alpha times x plus y, alpha = 2.5, 32M elements. */
void oracle_saxpy_f32(float alpha, const float *x, float *y, size_t n)
{
    for (size_t i = 0; i < n; ++i) y[i] = fmaf(alpha, x[i], y[i]);
}

/* ReLU y[i] = max(x[i], 0) in the IEEE 754-2019 `maximum` sense: a positive
 * x is returned unchanged, a NaN propagates, everything else (negative
 * values, -0, -inf) gives +0.  [PerfNotes] section 5.2, ReLU example. */
void oracle_relu_f32(const float *x, float *y, size_t n)
{
    for (size_t i = 0; i < n; ++i) {
        float v = x[i];
        if (v > 0.0f)      y[i] = v;
        else if (v != v)   y[i] = v;
        else               y[i] = 0.0f;
    }
}

/* ReLU of one binary32 value in the IEEE maximum(v, +0) sense (see above). */
static float relu1(float v)
{
    if (v > 0.0f) return v;
    if (v != v) return v;
    return 0.0f;
}

/* Fused add and ReLU: c[i] = maximum(a[i] + b[i], +0), the sum rounded once
 * to binary32 before the maximum.  An epilogue that saves the second pass
 * over memory ([GEMM-9.3] "what comes next": fuse bias and ReLU into the
 * producing kernel; [PerfNotes] 5.3: fusion raises the intensity of
 * memory-bound operations). */
void oracle_add_relu_f32(const float *a, const float *b, float *c, size_t n)
{
    for (size_t i = 0; i < n; ++i) c[i] = relu1(a[i] + b[i]);
}

/* Fused SAXPY and ReLU in place: y[i] = maximum(fmaf(alpha, x[i], y[i]), +0). */
void oracle_saxpy_relu_f32(float alpha, const float *x, float *y, size_t n)
{
    for (size_t i = 0; i < n; ++i) y[i] = relu1(fmaf(alpha, x[i], y[i]));
}

/* Bias and ReLU over a row-major rows x cols matrix: the bias vector is
 * broadcast along rows, y[r*cols + c] = maximum(x[r*cols + c] + bias[c], +0). */
void oracle_bias_relu_f32(const float *x, const float *bias, float *y, size_t rows, size_t cols)
{
    for (size_t r = 0; r < rows; ++r)
        for (size_t c = 0; c < cols; ++c)
            y[r * cols + c] = relu1(x[r * cols + c] + bias[c]);
}

/* SAXPY in place on binary16 / bfloat16 data: widen x and y exactly, one
 * fused multiply-add in binary32 with a binary32 alpha, round the result to
 * the 16-bit format nearest-even (the same rule as the 16-bit add). */
void oracle_saxpy_f16(float alpha, const uint16_t *x, uint16_t *y, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        y[i] = oracle_f32_to_f16(fmaf(alpha, oracle_f16_to_f32(x[i]), oracle_f16_to_f32(y[i])));
}

void oracle_saxpy_bf16(float alpha, const uint16_t *x, uint16_t *y, size_t n)
{
    for (size_t i = 0; i < n; ++i)
        y[i] = oracle_f32_to_bf16(fmaf(alpha, oracle_bf16_to_f32(x[i]), oracle_bf16_to_f32(y[i])));
}

/* ReLU on binary16 / bfloat16 data: IEEE maximum(x, +0) is x itself (a
 * positive value or a NaN, bits unchanged) or +0; no rounding is involved. */
void oracle_relu_f16(const uint16_t *x, uint16_t *y, size_t n)
{
    for (size_t i = 0; i < n; ++i) {
        float v = oracle_f16_to_f32(x[i]);
        y[i] = (v > 0.0f || v != v) ? x[i] : (uint16_t)0;
    }
}

void oracle_relu_bf16(const uint16_t *x, uint16_t *y, size_t n)
{
    for (size_t i = 0; i < n; ++i) {
        float v = oracle_bf16_to_f32(x[i]);
        y[i] = (v > 0.0f || v != v) ? x[i] : (uint16_t)0;
    }
}

/* Scalar-broadcast and unary maps, y[i] = f(x[i]): [EwOps] section 二 (the
 * template code whose middle operation is the only part that changes).
 * binary32: f is a single binary32 operation, rounded to nearest-even --
 * alpha * x, x + alpha, or sqrtf (IEEE 754 requires the square root to be
 * correctly rounded, and C99 sqrtf is that operation).  |x| clears the sign
 * bit and keeps every other bit. */
void oracle_scale_f32(float alpha, const float *x, float *y, size_t n)
{
    for (size_t i = 0; i < n; ++i) y[i] = alpha * x[i];
}

void oracle_add_scalar_f32(float alpha, const float *x, float *y, size_t n)
{
    for (size_t i = 0; i < n; ++i) y[i] = x[i] + alpha;
}

void oracle_sqrt_f32(const float *x, float *y, size_t n)
{
    for (size_t i = 0; i < n; ++i) y[i] = sqrtf(x[i]);
}

void oracle_abs_f32(const float *x, float *y, size_t n)
{
    const uint32_t *s = (const uint32_t *)x;
    uint32_t *d = (uint32_t *)y;
    for (size_t i = 0; i < n; ++i) d[i] = s[i] & 0x7fffffffu;
}

/* The same maps on 16-bit data: widen x exactly, apply f once in binary32
 * (with the binary32 alpha), round the result to the 16-bit format
 * nearest-even -- the rule of the 16-bit add.  |x| clears bit 15. */
void oracle_scale_f16(float alpha, const uint16_t *x, uint16_t *y, size_t n)
{
    for (size_t i = 0; i < n; ++i) y[i] = oracle_f32_to_f16(alpha * oracle_f16_to_f32(x[i]));
}

void oracle_scale_bf16(float alpha, const uint16_t *x, uint16_t *y, size_t n)
{
    for (size_t i = 0; i < n; ++i) y[i] = oracle_f32_to_bf16(alpha * oracle_bf16_to_f32(x[i]));
}

void oracle_add_scalar_f16(float alpha, const uint16_t *x, uint16_t *y, size_t n)
{
    for (size_t i = 0; i < n; ++i) y[i] = oracle_f32_to_f16(oracle_f16_to_f32(x[i]) + alpha);
}

void oracle_add_scalar_bf16(float alpha, const uint16_t *x, uint16_t *y, size_t n)
{
    for (size_t i = 0; i < n; ++i) y[i] = oracle_f32_to_bf16(oracle_bf16_to_f32(x[i]) + alpha);
}

void oracle_sqrt_f16(const uint16_t *x, uint16_t *y, size_t n)
{
    for (size_t i = 0; i < n; ++i) y[i] = oracle_f32_to_f16(sqrtf(oracle_f16_to_f32(x[i])));
}

void oracle_sqrt_bf16(const uint16_t *x, uint16_t *y, size_t n)
{
    for (size_t i = 0; i < n; ++i) y[i] = oracle_f32_to_bf16(sqrtf(oracle_bf16_to_f32(x[i])));
}

void oracle_abs_16(const uint16_t *x, uint16_t *y, size_t n)
{
    for (size_t i = 0; i < n; ++i) y[i] = (uint16_t)(x[i] & 0x7fffu);
}

/* Strided view copied to a contiguous row-major array, bit patterns
 * unchanged: out[r*cols + c] = in[r*stride_r + c*stride_c], strides in
 * elements and signed (a transposed view has stride_r = 1; x[::2] is the
 * rows = 1, stride_c = 2 case).  [PerfNotes] 3.4: non-contiguous access in
 * PyTorch appears as a stride; 3.1-3.2: coalesced versus strided reads. */
void oracle_copy2d_f32(const float *in, int64_t stride_r, int64_t stride_c, float *out,
                       size_t rows, size_t cols)
{
    const uint32_t *s = (const uint32_t *)in;
    uint32_t *d = (uint32_t *)out;
    for (size_t r = 0; r < rows; ++r)
        for (size_t c = 0; c < cols; ++c)
            d[r * cols + c] = s[(int64_t)r * stride_r + (int64_t)c * stride_c];
}

/* Contiguous copy out[i] = in[i], moved as bit patterns so NaN payloads and
 * signalling NaNs survive.  [PerfNotes] section 3.2, coalesced copy kernel. */
void oracle_copy_f32(const float *in, float *out, size_t n)
{
    const uint32_t *s = (const uint32_t *)in;
    uint32_t *d = (uint32_t *)out;
    for (size_t i = 0; i < n; ++i) d[i] = s[i];
}

/* Strided gather out[i] = in[(stride*i) mod n], moved as bit patterns.  The
 * index product is formed in 128-bit arithmetic so it is exact for every
 * stride and n.  [PerfNotes] section 3.2, non-coalesced copy kernel, whose
 * index is idx*2 % n (multiply, then remainder). */
void oracle_gather_f32(const float *in, float *out, size_t n, size_t stride)
{
    const uint32_t *s = (const uint32_t *)in;
    uint32_t *d = (uint32_t *)out;
    for (size_t i = 0; i < n; ++i) {
        unsigned __int128 p = (unsigned __int128)stride * (unsigned __int128)i;
        size_t j = (size_t)(p % (unsigned __int128)n);
        d[i] = s[j];
    }
}

/* The input index the gather reads for output i: (stride * i) mod n, exact
 * for every 64-bit stride and i (one element of oracle_gather_f32, for
 * checking sampled outputs of arrays too large to gather on the host). */
size_t oracle_gather_index(size_t n, size_t stride, size_t i)
{
    unsigned __int128 p = (unsigned __int128)stride * (unsigned __int128)i;
    return (size_t)(p % (unsigned __int128)n);
}

/* ------------------------------------------------------------------------ */
/* Helpers for the tests                                                     */
/* ------------------------------------------------------------------------ */

/* Element-wise conversions over arrays (used to pin the scalar conversions
 * exhaustively against library routines). */
void oracle_f32_to_f16_array(const float *x, uint16_t *y, size_t n)
{
    for (size_t i = 0; i < n; ++i) y[i] = oracle_f32_to_f16(x[i]);
}
void oracle_f16_to_f32_array(const uint16_t *x, float *y, size_t n)
{
    for (size_t i = 0; i < n; ++i) y[i] = oracle_f16_to_f32(x[i]);
}
void oracle_f32_to_bf16_array(const float *x, uint16_t *y, size_t n)
{
    for (size_t i = 0; i < n; ++i) y[i] = oracle_f32_to_bf16(x[i]);
}
void oracle_bf16_to_f32_array(const uint16_t *x, float *y, size_t n)
{
    for (size_t i = 0; i < n; ++i) y[i] = oracle_bf16_to_f32(x[i]);
}

/* Convert every binary32 bit pattern in [start, start+count) to binary16 and
 * bfloat16, so the exhaustive pins do not need a 16 GiB input array. */
void oracle_f32_range_to_f16(uint32_t start, uint32_t count, uint16_t *y)
{
    for (uint32_t k = 0; k < count; ++k) y[k] = oracle_f32_to_f16(bits_f32(start + k));
}
void oracle_f32_range_to_bf16(uint32_t start, uint32_t count, uint16_t *y)
{
    for (uint32_t k = 0; k < count; ++k) y[k] = oracle_f32_to_bf16(bits_f32(start + k));
}

/* Distance in units in the last place between two binary32 values: map each
 * bit pattern to a monotone integer (negatives mirrored, both zeros -> 0) and
 * take |ord(a) - ord(b)|.  Meaningless for NaN inputs. */
static int64_t f32_ord(float f)
{
    uint32_t u = f32_bits(f);
    if (u & 0x80000000u) return -(int64_t)(u & 0x7fffffffu);
    return (int64_t)u;
}
uint64_t oracle_ulp_distance_f32(float a, float b)
{
    int64_t d = f32_ord(a) - f32_ord(b);
    return (uint64_t)(d < 0 ? -d : d);
}

int oracle_abi_version(void) { return 2; }
