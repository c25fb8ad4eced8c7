/*
 * f16c_ref.c -- reference binary32 <-> binary16 conversions computed by the
 * x86 F16C instructions (VCVTPS2PH with an explicit round-to-nearest-even
 * immediate, VCVTPH2PS).  Test-only: it pins the oracle's own conversions,
 * which are written from the IEEE-754 definition, against the hardware.
 */
#include <immintrin.h>
#include <stdint.h>
#include <stddef.h>

/* Convert every binary32 bit pattern in [start, start+count) to binary16. */
void pin_f16c_range(uint32_t start, uint32_t count, uint16_t *out)
{
    const __m256i lane = _mm256_setr_epi32(0, 1, 2, 3, 4, 5, 6, 7);
    uint32_t k = 0;
    for (; k + 8 <= count; k += 8) {
        __m256i v = _mm256_add_epi32(_mm256_set1_epi32((int)(start + k)), lane);
        __m128i h = _mm256_cvtps_ph(_mm256_castsi256_ps(v),
                                    _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC);
        _mm_storeu_si128((__m128i *)(out + k), h);
    }
    for (; k < count; ++k) {
        uint32_t u = start + k;
        float f;
        __builtin_memcpy(&f, &u, 4);
        out[k] = _cvtss_sh(f, _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC);
    }
}

/* Widen n binary16 bit patterns to binary32. */
void pin_f16c_widen(const uint16_t *in, float *out, size_t n)
{
    size_t k = 0;
    for (; k + 8 <= n; k += 8) {
        __m128i h = _mm_loadu_si128((const __m128i *)(in + k));
        _mm256_storeu_ps(out + k, _mm256_cvtph_ps(h));
    }
    for (; k < n; ++k) out[k] = _cvtsh_ss(in[k]);
}

/* Compare a binary32 -> binary16 conversion `fn` with VCVTPS2PH (RNE) on the
 * bit patterns [start, start + count).  Non-NaN inputs must match bitwise;
 * NaN inputs must give a binary16 NaN with the input's sign.  Returns the
 * number of patterns that fail. */
uint64_t pin_f16c_count_mismatches(uint16_t (*fn)(float), uint64_t start, uint64_t count)
{
    uint64_t bad = 0;
    uint16_t ref[8];
    for (uint64_t k = 0; k < count; k += 8) {
        const uint32_t base = (uint32_t)(start + k);
        __m256i v = _mm256_add_epi32(_mm256_set1_epi32((int)base),
                                     _mm256_setr_epi32(0, 1, 2, 3, 4, 5, 6, 7));
        _mm_storeu_si128((__m128i *)ref,
                         _mm256_cvtps_ph(_mm256_castsi256_ps(v),
                                         _MM_FROUND_TO_NEAREST_INT | _MM_FROUND_NO_EXC));
        const int lanes = (count - k) < 8 ? (int)(count - k) : 8;
        for (int j = 0; j < lanes; ++j) {
            const uint32_t u = base + (uint32_t)j;
            float f;
            __builtin_memcpy(&f, &u, 4);
            const uint16_t got = fn(f);
            if ((u & 0x7fffffffu) > 0x7f800000u) {
                const int is_nan = (got & 0x7c00u) == 0x7c00u && (got & 0x03ffu) != 0;
                if (!is_nan || (got >> 15) != (u >> 31)) ++bad;
            } else if (got != ref[j]) {
                ++bad;
            }
        }
    }
    return bad;
}
