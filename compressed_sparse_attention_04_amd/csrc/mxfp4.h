// mxfp4.h -- MXFP4 (OCP microscaling, e2m1 elements + E8M0 scale per 32
// values) encoder used for the indexer keys and, inside the indexer kernel,
// for the indexer queries (studioglobal.ai answer, FP4/FP8 mixed precision:
// MXFP4 packs two values per byte; every page: the indexer runs at FP4).
//
// Scale exponent e = floor(log2 max|x|) - 2, clamped to [-127, 127]
// (-127 for an all-zero run).  Element code: nearest of the e2m1 magnitudes
// {0, .5, 1, 1.5, 2, 3, 4, 6} to |x| * 2^-e, ties to the even code,
// saturating at 6; bit 3 = sign bit of x.  The comparison runs in fp64 on a
// value rebuilt from the fp32 bit fields, so it is exact for every finite
// input including fp32 subnormals.
#pragma once
#include "common.h"

namespace csa {

__device__ __forceinline__ double pow2_f64(int k) {
    return __longlong_as_double((long long)(k + 1023) << 52);
}

// |x| * 2^-e for a non-negative fp32 bit pattern a, exactly, in fp64
__device__ __forceinline__ double scaled_mag(uint32_t a, int e) {
    uint32_t ef = a >> 23, mant = a & 0x7fffffu;
    if (ef == 0) return (double)mant * pow2_f64(-149 - e);
    return (double)(mant | 0x800000u) * pow2_f64((int)ef - 150 - e);
}

__device__ __forceinline__ uint32_t e2m1_code(double y) {
    // boundaries between neighbouring magnitudes; equality goes to the even code
    uint32_t c;
    if (y <= 0.25) c = 0;
    else if (y < 0.75) c = 1;
    else if (y <= 1.25) c = 2;
    else if (y < 1.75) c = 3;
    else if (y <= 2.5) c = 4;
    else if (y < 3.5) c = 5;
    else if (y <= 5.0) c = 6;
    else c = 7;
    return c;
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
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        uint32_t bits = __float_as_uint(v[i]);
        uint32_t code = e2m1_code(scaled_mag(bits & 0x7fffffffu, e)) | ((bits >> 28) & 8u);
        packed[i / 8] |= code << (4 * (i % 8));
    }
}

}  // namespace csa
