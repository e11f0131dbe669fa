// compress.hip -- softmax-gated pooling of m adjacent KV rows into one
// compressed entry (jiwasawa.github.io post, CSA token-level compression;
// studioglobal.ai answer, CSA bullet: softmax-gated pooling; the same pooling
// with m' = 128 feeds HCA).
//
//   out[b][j][c] = sum_{i<m} softmax_i(z[b][m*j+i][g(c)]) * x[b][m*j+i][c]
//
// HBM-bound streaming op: every thread owns 8 consecutive channels (one
// 16-byte bf16 / 32-byte fp32 vector), so a wave reads whole rows with
// coalesced vector loads.  The softmax runs online in fp32 (running max,
// rescaled denominator and accumulator), so x and z are read exactly once.
#include "common.h"
#include "internal.h"

namespace csa {

struct OnlineSoftmax8 {
    float mx[8], den[8], acc[8];
    __device__ __forceinline__ void init() {
#pragma unroll
        for (int c = 0; c < 8; ++c) { mx[c] = -INFINITY; den[c] = 0.f; acc[c] = 0.f; }
    }
    // fold in one token: logits z, values x
    __device__ __forceinline__ void add(const float (&z)[8], const float (&x)[8]) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float nm = fmaxf(mx[c], z[c]);
            float a = __expf(mx[c] - nm);      // 0 on the first token
            float e = __expf(z[c] - nm);
            den[c] = den[c] * a + e;
            acc[c] = acc[c] * a + e * x[c];
            mx[c] = nm;
        }
    }
    // merge another partial state
    __device__ __forceinline__ void merge(const float* omx, const float* oden, const float* oacc) {
#pragma unroll
        for (int c = 0; c < 8; ++c) {
            float nm = fmaxf(mx[c], omx[c]);
            if (nm == -INFINITY) continue;
            float a = __expf(mx[c] - nm), b = __expf(omx[c] - nm);
            den[c] = den[c] * a + oden[c] * b;
            acc[c] = acc[c] * a + oacc[c] * b;
            mx[c] = nm;
        }
    }
};

template <typename T>
__device__ __forceinline__ void load_gate8(const T* gate, int64_t row, int C, int gc, int c8,
                                           float (&z)[8]) {
    if (gc == 1) {
        float v = Elem<T>::load1(gate + row);
#pragma unroll
        for (int c = 0; c < 8; ++c) z[c] = v;
    } else {
        Elem<T>::load8(gate + row * (int64_t)C + c8 * 8, z);
    }
}

// Small m: one thread per (output row, 8-channel group).
template <typename T>
__global__ void __launch_bounds__(256)
k_compress_small(const T* __restrict__ x, const T* __restrict__ gate, T* __restrict__ out,
                 int64_t B, int64_t T_, int C, int m, int gc, int64_t nout) {
    const int groups = C / 8;
    int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t total = B * nout * groups;
    if (gid >= total) return;
    int c8 = (int)(gid % groups);
    int64_t bj = gid / groups;
    int64_t b = bj / nout, j = bj % nout;
    OnlineSoftmax8 s;
    s.init();
    int64_t row0 = b * T_ + j * m;
    for (int i = 0; i < m; ++i) {
        float xv[8], z[8];
        Elem<T>::load8(x + (row0 + i) * (int64_t)C + c8 * 8, xv);
        load_gate8(gate, row0 + i, C, gc, c8, z);
        s.add(z, xv);
    }
    float o[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] = s.acc[c] / s.den[c];
    Elem<T>::store8(out + bj * (int64_t)C + c8 * 8, o);
}

// Large m: one 256-thread block per output row; the m rows are split over
// R = 256 / (C/8) row groups whose partial softmax states merge in LDS.
template <typename T>
__global__ void __launch_bounds__(256)
k_compress_large(const T* __restrict__ x, const T* __restrict__ gate, T* __restrict__ out,
                 int64_t B, int64_t T_, int C, int m, int gc, int64_t nout) {
    __shared__ float smx[256 * 8], sden[256 * 8], sacc[256 * 8];
    const int groups = C / 8;
    const int R = 256 / groups;
    const int tid = threadIdx.x;
    const int c8 = tid % groups, rg = tid / groups;
    int64_t bj = blockIdx.x;
    int64_t b = bj / nout, j = bj % nout;
    OnlineSoftmax8 s;
    s.init();
    int64_t row0 = b * T_ + j * m;
    if (rg < R) {
        for (int i = rg; i < m; i += R) {
            float xv[8], z[8];
            Elem<T>::load8(x + (row0 + i) * (int64_t)C + c8 * 8, xv);
            load_gate8(gate, row0 + i, C, gc, c8, z);
            s.add(z, xv);
        }
    }
#pragma unroll
    for (int c = 0; c < 8; ++c) {
        smx[tid * 8 + c] = s.mx[c];
        sden[tid * 8 + c] = s.den[c];
        sacc[tid * 8 + c] = s.acc[c];
    }
    __syncthreads();
    if (rg == 0) {
        for (int r = 1; r < R; ++r) {
            int o = (r * groups + c8) * 8;
            s.merge(smx + o, sden + o, sacc + o);
        }
        float ov[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) ov[c] = s.acc[c] / s.den[c];
        Elem<T>::store8(out + bj * (int64_t)C + c8 * 8, ov);
    }
}

template <typename T>
static hipError_t launch_compress_t(const void* x, const void* gate, void* out, int64_t B,
                                    int64_t T_, int C, int m, int gc, hipStream_t st) {
    int64_t nout = T_ / m;
    if (B * nout == 0) return hipSuccess;
    if (m <= 16) {
        int64_t total = B * nout * (C / 8);
        int64_t blocks = (total + 255) / 256;
        hipLaunchKernelGGL(k_compress_small<T>, dim3((unsigned)blocks), dim3(256), 0, st,
                           (const T*)x, (const T*)gate, (T*)out, B, T_, C, m, gc, nout);
    } else {
        hipLaunchKernelGGL(k_compress_large<T>, dim3((unsigned)(B * nout)), dim3(256), 0, st,
                           (const T*)x, (const T*)gate, (T*)out, B, T_, C, m, gc, nout);
    }
    return hipGetLastError();
}

hipError_t launch_compress(int dt, const void* x, const void* gate, void* out, int64_t B,
                           int64_t T_, int C, int m, int gc, hipStream_t st) {
    if (dt == 0) return launch_compress_t<float>(x, gate, out, B, T_, C, m, gc, st);
    return launch_compress_t<uint16_t>(x, gate, out, B, T_, C, m, gc, st);
}

}  // namespace csa
