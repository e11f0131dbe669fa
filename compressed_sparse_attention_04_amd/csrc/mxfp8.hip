// mxfp8.hip -- MXFP8 (E4M3) encoding of rows for the compressed KV cache
// (ai-papers.net article, hybrid attention section: most KV entries are
// stored in FP8; the block format is the OCP Microscaling one also used for
// the FP4 indexer keys).  One thread per run of 32 values: the run's scale is
// 2^e with e = floor(log2 max|x|) - 8 (8 = largest E4M3 exponent), clamped
// to [-127, 127] (an all-zero run takes -127), stored as e + 127; every
// x * 2^-e is rounded to the nearest E4M3 value, ties to even, saturating at
// 448.  Inputs must be finite.
#include "internal.h"
#include "common.h"

namespace csa {

// E4M3 code of y (|y| may exceed 448: saturates).  With a = min(|y|, 448)
// and E = max(floor(log2 a), -6), the code is 8 (E + 6) + rne(a * 2^(3-E)):
// the rounded significand q is in [8, 16] for E > -6 (q = 16 carries into
// the next exponent), and for E = -6 it is the subnormal step count 0 .. 8.
__device__ __forceinline__ uint32_t e4m3_code(float y) {
    const float a = fminf(fabsf(y), 448.f);
    int E = (int)((__float_as_uint(a) >> 23) & 0xff) - 127;   // zero / subnormal: < -6
    E = E < -6 ? -6 : E;
    const float q = rintf(ldexpf(a, 3 - E));                  // exact scaling, then RNE
    const uint32_t code = (uint32_t)(8 * (E + 6)) + (uint32_t)q;
    return code | (__float_as_uint(y) >> 31 << 7);
}

template <typename T>
__global__ void __launch_bounds__(256)
k_quant_mxfp8(const T* __restrict__ x, uint8_t* __restrict__ codes,
              uint8_t* __restrict__ scales, int64_t nblocks) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= nblocks) return;
    float v[32];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        float t[8];
        Elem<T>::load8(x + g * 32 + p * 8, t);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[p * 8 + i] = t[i];
    }
    float amax = 0.f;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
    // floor(log2 amax) from the exponent field; a subnormal or zero maximum
    // gives at most -127 - 8, clamped to -127
    int e = (int)((__float_as_uint(amax) >> 23) & 0xff) - 127 - 8;
    e = e < -127 ? -127 : e;
    uint32_t w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t b = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) b |= e4m3_code(ldexpf(v[4 * j + i], -e)) << (8 * i);
        w[j] = b;
    }
    u32x4* out = reinterpret_cast<u32x4*>(codes + g * 32);
    out[0] = u32x4{w[0], w[1], w[2], w[3]};
    out[1] = u32x4{w[4], w[5], w[6], w[7]};
    scales[g] = (uint8_t)(e + 127);
}

hipError_t launch_quant_mxfp8(int dt, const void* x, uint8_t* codes, uint8_t* scales,
                              int64_t rows, int d, hipStream_t st) {
    const int64_t nb = rows * (d / 32);
    if (nb == 0) return hipSuccess;
    const dim3 grid((unsigned)((nb + 255) / 256));
    if (dt == 0)
        hipLaunchKernelGGL(k_quant_mxfp8<float>, grid, dim3(256), 0, st, (const float*)x, codes,
                           scales, nb);
    else
        hipLaunchKernelGGL(k_quant_mxfp8<uint16_t>, grid, dim3(256), 0, st, (const uint16_t*)x,
                           codes, scales, nb);
    return hipGetLastError();
}

}  // namespace csa
