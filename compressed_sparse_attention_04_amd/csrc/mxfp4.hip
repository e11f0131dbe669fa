// mxfp4.hip -- MXFP4 encoding of rows (one thread per 32-value run).
#include "internal.h"
#include "mxfp4.h"

namespace csa {

template <typename T>
__global__ void __launch_bounds__(256)
k_quant_mxfp4(const T* __restrict__ x, int64_t x_rs, int nbr, uint8_t* __restrict__ codes,
              uint8_t* __restrict__ scales, int64_t nblocks) {
    int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= nblocks) return;
    // run g is run g % nbr of row g / nbr (rows x_rs elements apart)
    const T* src = x + (g / nbr) * x_rs + (g % nbr) * 32;
    float v[32];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        float t[8];
        Elem<T>::load8(src + p * 8, t);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[p * 8 + i] = t[i];
    }
    uint32_t packed[4], sb;
    mxfp4_encode32(v, packed, sb);
    u32x4 pk = {packed[0], packed[1], packed[2], packed[3]};
    *reinterpret_cast<u32x4*>(codes + g * 16) = pk;
    scales[g] = (uint8_t)sb;
}

hipError_t launch_quant_mxfp4(int dt, const void* x, int64_t x_rs, uint8_t* codes,
                              uint8_t* scales, int64_t rows, int d, hipStream_t st) {
    int64_t nb = rows * (d / 32);
    if (nb == 0) return hipSuccess;
    dim3 grid((unsigned)((nb + 255) / 256));
    if (dt == 0)
        hipLaunchKernelGGL(k_quant_mxfp4<float>, grid, dim3(256), 0, st, (const float*)x, x_rs,
                           d / 32, codes, scales, nb);
    else
        hipLaunchKernelGGL(k_quant_mxfp4<uint16_t>, grid, dim3(256), 0, st,
                           (const uint16_t*)x, x_rs, d / 32, codes, scales, nb);
    return hipGetLastError();
}

}  // namespace csa
