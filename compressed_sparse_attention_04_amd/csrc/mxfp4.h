// mxfp4.h -- MXFP4 (OCP microscaling, e2m1 elements + E8M0 scale per 32
// values) encoder used for the indexer keys and, inside the indexer kernel,
// for the indexer queries (studioglobal.ai answer, FP4/FP8 mixed precision:
// MXFP4 packs two values per byte; every page: the indexer runs at FP4).
//
// Scale exponent e = floor(log2 max|x|) - 2, clamped to [-127, 127]
// (-127 for an all-zero run).  Element code: nearest of the e2m1 magnitudes
// {0, .5, 1, 1.5, 2, 3, 4, 6} to |x| * 2^-e, ties to the even code,
// saturating at 6; bit 3 = sign bit of x.  |x| * 2^-e is formed in fp32:
// 2^-e is a normal fp32 for every e the rule produces (-127 <= e <= 125),
// so the product is exact whenever it is >= 2^-126, and a smaller product
// (possible only for elements far below the block maximum) has code 0
// however it rounds.  The thresholds are exact fp32 constants.
#pragma once
#include "common.h"

namespace csa {

// e2m1 code of y = |x| * 2^-e (0 <= y < 8); a tie goes to the even code
__device__ __forceinline__ uint32_t e2m1_code(float y) {
    return (uint32_t)(y > 0.25f) + (uint32_t)(y >= 0.75f) + (uint32_t)(y > 1.25f) +
           (uint32_t)(y >= 1.75f) + (uint32_t)(y > 2.5f) + (uint32_t)(y >= 3.5f) +
           (uint32_t)(y > 5.0f);
}

// 2^-e as fp32 (normal for -127 <= e <= 126)
__device__ __forceinline__ float pow2_neg(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }

// sign | code of one value under scale exponent e
__device__ __forceinline__ uint32_t mxfp4_code(float x, float p2e) {
    const uint32_t bits = __float_as_uint(x);
    return e2m1_code(__uint_as_float(bits & 0x7fffffffu) * p2e) | ((bits >> 28) & 8u);
}

__device__ __forceinline__ int mxfp4_exponent(uint32_t amax_bits) {
    if (amax_bits == 0) return -127;
    int ef = (int)(amax_bits >> 23);
    if (ef == 0) return -127;                  // subnormal: floor(log2) - 2 < -127
    int e = ef - 127 - 2;
    return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Encode 32 fp32 values: 16 bytes of packed codes (element i = nibble i,
// low nibble first) and the biased scale byte.
__device__ __forceinline__ void mxfp4_encode32(const float (&v)[32], uint32_t (&packed)[4],
                                               uint32_t& scale_byte) {
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        uint32_t a = __float_as_uint(v[i]) & 0x7fffffffu;
        amax = a > amax ? a : amax;
    }
    int e = mxfp4_exponent(amax);
    scale_byte = (uint32_t)(e + 127);
#pragma unroll
    for (int w = 0; w < 4; ++w) packed[w] = 0;
    const float p2e = pow2_neg(e);
#pragma unroll
    for (int i = 0; i < 32; ++i) packed[i / 8] |= mxfp4_code(v[i], p2e) << (4 * (i % 8));
}

}  // namespace csa
