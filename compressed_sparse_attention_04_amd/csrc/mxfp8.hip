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
#include "e4m3.h"

namespace csa {

// One thread per run of 32 values.  ROW = false: the run has its own scale,
// one byte per run (MXFP8).  ROW = true: the ROWN = d / 32 consecutive
// threads of a row (lanes of one wave, ROWN a power of two dividing 64)
// share the row's maximum, so the whole row takes one scale, written once as
// a 32-bit word holding the bits of the fp32 power of two 2^e (the byte
// e + 127 in bits 23..30; zero for a zero row).
template <typename T, int ROWN, bool ROW>
__global__ void __launch_bounds__(256)
k_quant_mxfp8(const T* __restrict__ x, uint8_t* __restrict__ codes,
              void* __restrict__ scales, int64_t nblocks) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    // nblocks is a multiple of ROWN: a row's threads are all present or all gone
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
#pragma unroll
    for (int o = 1; o < ROWN; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, WAVE));
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
    if constexpr (ROW) {
        if (g % ROWN == 0) static_cast<uint32_t*>(scales)[g / ROWN] = (uint32_t)(e + 127) << 23;
    } else {
        static_cast<uint8_t*>(scales)[g] = (uint8_t)(e + 127);
    }
}

hipError_t launch_quant_mxfp8(int dt, const void* x, uint8_t* codes, uint8_t* scales,
                              int64_t rows, int d, hipStream_t st) {
    const int64_t nb = rows * (d / 32);
    if (nb == 0) return hipSuccess;
    const dim3 grid((unsigned)((nb + 255) / 256));
    if (dt == 0)
        hipLaunchKernelGGL((k_quant_mxfp8<float, 1, false>), grid, dim3(256), 0, st,
                           (const float*)x, codes, (void*)scales, nb);
    else
        hipLaunchKernelGGL((k_quant_mxfp8<uint16_t, 1, false>), grid, dim3(256), 0, st,
                           (const uint16_t*)x, codes, (void*)scales, nb);
    return hipGetLastError();
}

template <int ROWN>
static void launch_rows(int dt, const void* x, uint8_t* codes, uint32_t* scales, int64_t nb,
                        hipStream_t st) {
    const dim3 grid((unsigned)((nb + 255) / 256));
    if (dt == 0)
        hipLaunchKernelGGL((k_quant_mxfp8<float, ROWN, true>), grid, dim3(256), 0, st,
                           (const float*)x, codes, (void*)scales, nb);
    else
        hipLaunchKernelGGL((k_quant_mxfp8<uint16_t, ROWN, true>), grid, dim3(256), 0, st,
                           (const uint16_t*)x, codes, (void*)scales, nb);
}

hipError_t launch_quant_fp8_rows(int dt, const void* x, uint8_t* codes, uint32_t* scales,
                                 int64_t rows, int d, hipStream_t st) {
    const int64_t nb = rows * (d / 32);
    if (nb == 0) return hipSuccess;
    switch (d / 32) {
        case 1: launch_rows<1>(dt, x, codes, scales, nb, st); break;
        case 2: launch_rows<2>(dt, x, codes, scales, nb, st); break;
        case 4: launch_rows<4>(dt, x, codes, scales, nb, st); break;
        case 8: launch_rows<8>(dt, x, codes, scales, nb, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace csa
