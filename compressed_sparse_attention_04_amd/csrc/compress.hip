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

// gate logits of one row (grow: the row's first element) for 8 channels
// from c8: the row's single logit (gc = 1) or 8 per-channel logits
template <typename T>
__device__ __forceinline__ void load_gate8(const T* grow, int gc, int c8, float (&z)[8]) {
    if (gc == 1) {
        float v = Elem<T>::load1(grow);
#pragma unroll
        for (int c = 0; c < 8; ++c) z[c] = v;
    } else {
        Elem<T>::load8(grow + c8 * 8, z);
    }
}

// Strided inputs and output of one pooling call
template <typename T>
struct PoolIO {
    const T* x;
    const T* gate;
    T* out;
    RowStrides xs, gs, os;
};

// Small m: one thread per (output row, 8-channel group).
template <typename T>
__global__ void __launch_bounds__(256)
k_compress_small(PoolIO<T> io, int64_t B, int64_t T_, int C, int m, int gc, int64_t nout) {
    const int groups = C / 8;
    int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    int64_t total = B * nout * groups;
    if (gid >= total) return;
    int c8 = (int)(gid % groups);
    int64_t bj = gid / groups;
    int64_t b = bj / nout, j = bj % nout;
    OnlineSoftmax8 s;
    s.init();
    const T* xr = io.x + b * io.xs.ss + j * m * io.xs.rs + c8 * 8;
    const T* gr = io.gate + b * io.gs.ss + j * m * io.gs.rs;
    for (int i = 0; i < m; ++i) {
        float xv[8], z[8];
        Elem<T>::load8(xr + i * io.xs.rs, xv);
        load_gate8(gr + i * io.gs.rs, gc, c8, z);
        s.add(z, xv);
    }
    float o[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) o[c] = s.acc[c] / s.den[c];
    Elem<T>::store8(io.out + b * io.os.ss + j * io.os.rs + c8 * 8, o);
}

// Large m: one 256-thread block per output row; the m rows are split over
// R = 256 / (C/8) row groups whose partial softmax states merge in LDS.
template <typename T>
__global__ void __launch_bounds__(256)
k_compress_large(PoolIO<T> io, int64_t B, int64_t T_, int C, int m, int gc, int64_t nout) {
    __shared__ float smx[256 * 8], sden[256 * 8], sacc[256 * 8];
    const int groups = C / 8;
    const int R = 256 / groups;
    const int tid = threadIdx.x;
    const int c8 = tid % groups, rg = tid / groups;
    int64_t bj = blockIdx.x;
    int64_t b = bj / nout, j = bj % nout;
    OnlineSoftmax8 s;
    s.init();
    const T* xr = io.x + b * io.xs.ss + j * m * io.xs.rs + c8 * 8;
    const T* gr = io.gate + b * io.gs.ss + j * m * io.gs.rs;
    if (rg < R) {
        for (int i = rg; i < m; i += R) {
            float xv[8], z[8];
            Elem<T>::load8(xr + i * io.xs.rs, xv);
            load_gate8(gr + i * io.gs.rs, gc, c8, z);
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
        Elem<T>::store8(io.out + b * io.os.ss + j * io.os.rs + c8 * 8, ov);
    }
}

// ---- one decode step of cache upkeep -------------------------------------
// The token at position t joins the window rows and the gate logits of its
// block; when it completes a block of m, the block is pooled into its
// compressed entry with the same arithmetic as k_compress_small (m <= 16)
// or k_compress_large (row groups rg, rg + R, ... merged in order), so
// entries come out identical to a pooling of the whole sequence.  The block
// rows are read where they were before this call (the move to the front
// writes other rows), so no thread reads what another one writes.

template <typename T>
__device__ __forceinline__ void copy8(T* dst, const T* src) {
    constexpr int N = 8 * sizeof(T) / 16;                 // 16-byte chunks
#pragma unroll
    for (int i = 0; i < N; ++i)
        reinterpret_cast<u32x4*>(dst)[i] = reinterpret_cast<const u32x4*>(src)[i];
}

struct AppendArgs {
    int64_t B, wcap, nc_cap;
    int C, m, gc, W;
    int64_t row_new;      // window row of the new token (after the move)
    int64_t move_from;    // rows move_from .. move_from + W - 2 move to the front, or -1
    int64_t row_blk;      // window row, before the move, of the block's first token
    int slot;             // t mod m
    int64_t entry;        // compressed entry the token completes, or -1
};

template <typename T>
struct AppendSide {       // one of K, V: new row and gates, window, gate slots, cache
    const T* x_new;
    const T* g_new;
    T* win;
    T* gblk;
    T* out;
};

// block row i (0 .. m - 1) of sequence b, 8 channels from c8: the token
// itself from its inputs, the others from the window and gate slots
template <typename T>
__device__ __forceinline__ void block_row(const AppendSide<T>& sd, const AppendArgs& a,
                                          int64_t b, int c8, int i, float (&xv)[8],
                                          float (&z)[8]) {
    if (i == a.m - 1) {
        Elem<T>::load8(sd.x_new + b * a.C + c8 * 8, xv);
        load_gate8(sd.g_new + b * a.gc, a.gc, c8, z);
    } else {
        Elem<T>::load8(sd.win + (b * a.wcap + a.row_blk + i) * a.C + c8 * 8, xv);
        load_gate8(sd.gblk + (b * a.m + i) * a.gc, a.gc, c8, z);
    }
}

// move (rows r = r0, r0 + rs, ...), new row and gate slot for (b, c8)
template <typename T>
__device__ __forceinline__ void append_rows(const AppendSide<T>& sd, const AppendArgs& a,
                                            int64_t b, int c8, int r0, int rs) {
    T* wrow = sd.win + b * a.wcap * a.C + c8 * 8;
    if (a.move_from >= 0)
        for (int r = r0; r < a.W - 1; r += rs)
            copy8(wrow + (int64_t)r * a.C, wrow + (a.move_from + r) * a.C);
    if (r0 == 0) {
        copy8(wrow + a.row_new * a.C, sd.x_new + b * a.C + c8 * 8);
        T* grow = sd.gblk + (b * a.m + a.slot) * (int64_t)a.gc;
        if (a.gc == a.C) copy8(grow + c8 * 8, sd.g_new + b * a.gc + c8 * 8);
        else if (c8 == 0) *grow = sd.g_new[b];
    }
}

// m <= 16: one thread per (sequence, 8 channels), the block's rows in order
template <typename T>
__global__ void __launch_bounds__(256)
k_append_small(AppendSide<T> sk, AppendSide<T> sv, AppendArgs a, int shared) {
    const int groups = a.C / 8;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (gid >= a.B * groups) return;
    const int64_t b = gid / groups;
    const int c8 = (int)(gid % groups);
    for (int side = 0; side < (shared ? 1 : 2); ++side) {
        const AppendSide<T>& sd = side == 0 ? sk : sv;
        append_rows(sd, a, b, c8, 0, 1);
        if (a.entry < 0) continue;
        OnlineSoftmax8 s;
        s.init();
        for (int i = 0; i < a.m; ++i) {
            float xv[8], z[8];
            block_row(sd, a, b, c8, i, xv, z);
            s.add(z, xv);
        }
        float o[8];
#pragma unroll
        for (int c = 0; c < 8; ++c) o[c] = s.acc[c] / s.den[c];
        Elem<T>::store8(sd.out + (b * a.nc_cap + a.entry) * a.C + c8 * 8, o);
    }
}

// m > 16: one 256-thread block per sequence, R = 256 / (C/8) row groups
// whose partial states merge in LDS, as in k_compress_large
template <typename T>
__global__ void __launch_bounds__(256)
k_append_large(AppendSide<T> sk, AppendSide<T> sv, AppendArgs a, int shared) {
    __shared__ float smx[256 * 8], sden[256 * 8], sacc[256 * 8];
    const int groups = a.C / 8;
    const int R = 256 / groups;
    const int tid = threadIdx.x;
    const int c8 = tid % groups, rg = tid / groups;
    const int64_t b = blockIdx.x;
    for (int side = 0; side < (shared ? 1 : 2); ++side) {
        const AppendSide<T>& sd = side == 0 ? sk : sv;
        if (rg < R) append_rows(sd, a, b, c8, rg, R);
        if (a.entry < 0) continue;
        OnlineSoftmax8 s;
        s.init();
        if (rg < R) {
            for (int i = rg; i < a.m; i += R) {
                float xv[8], z[8];
                block_row(sd, a, b, c8, i, xv, z);
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
                const int o = (r * groups + c8) * 8;
                s.merge(smx + o, sden + o, sacc + o);
            }
            float ov[8];
#pragma unroll
            for (int c = 0; c < 8; ++c) ov[c] = s.acc[c] / s.den[c];
            Elem<T>::store8(sd.out + (b * a.nc_cap + a.entry) * a.C + c8 * 8, ov);
        }
        __syncthreads();                      // the LDS states are reused
    }
}

template <typename T>
static void launch_append_t(const AppendArgs& a, const void* k_new, const void* v_new,
                            const void* gk_new, const void* gv_new, void* rk, void* rv,
                            void* gk_blk, void* gv_blk, void* ck, void* cv, int shared,
                            hipStream_t st) {
    const AppendSide<T> sk{(const T*)k_new, (const T*)gk_new, (T*)rk, (T*)gk_blk, (T*)ck};
    const AppendSide<T> sv{(const T*)v_new, (const T*)gv_new, (T*)rv, (T*)gv_blk, (T*)cv};
    if (a.m <= 16) {
        const int64_t threads = a.B * (a.C / 8);
        hipLaunchKernelGGL(k_append_small<T>, dim3((unsigned)((threads + 255) / 256)), dim3(256),
                           0, st, sk, sv, a, shared);
    } else {
        hipLaunchKernelGGL(k_append_large<T>, dim3((unsigned)a.B), dim3(256), 0, st, sk, sv, a,
                           shared);
    }
}

hipError_t launch_append(int dt, int64_t B, int64_t C, int64_t m, int64_t W, int64_t t,
                         int64_t win_pos0, int64_t wcap, int64_t gc, int64_t nc_cap,
                         const void* k_new, const void* v_new, const void* gk_new,
                         const void* gv_new, void* rk, void* rv, void* gk_blk, void* gv_blk,
                         void* ck, void* cv, int64_t* new_win_pos0, hipStream_t st) {
    AppendArgs a;
    a.B = B;
    a.wcap = wcap;
    a.nc_cap = nc_cap;
    a.C = (int)C;
    a.m = (int)m;
    a.gc = (int)gc;
    a.W = (int)W;
    a.row_blk = t - (m - 1) - win_pos0;           // before the move
    a.move_from = -1;
    if (t - win_pos0 == wcap) {                   // full: keep the newest W - 1 rows
        a.move_from = wcap - (W - 1);
        win_pos0 = t - (W - 1);
    }
    a.row_new = t - win_pos0;
    a.slot = (int)(t % m);
    a.entry = (t + 1) % m == 0 ? (t + 1) / m - 1 : -1;
    *new_win_pos0 = win_pos0;
    const int shared = ck == cv && rk == rv;
    if (dt == 0)
        launch_append_t<float>(a, k_new, v_new, gk_new, gv_new, rk, rv, gk_blk, gv_blk, ck, cv,
                               shared, st);
    else
        launch_append_t<uint16_t>(a, k_new, v_new, gk_new, gv_new, rk, rv, gk_blk, gv_blk, ck,
                                  cv, shared, st);
    return hipGetLastError();
}

template <typename T>
static hipError_t launch_compress_t(const PoolIO<T>& io, int64_t B, int64_t T_, int C, int m,
                                    int gc, hipStream_t st) {
    int64_t nout = T_ / m;
    if (B * nout == 0) return hipSuccess;
    if (m <= 16) {
        int64_t total = B * nout * (C / 8);
        int64_t blocks = (total + 255) / 256;
        hipLaunchKernelGGL(k_compress_small<T>, dim3((unsigned)blocks), dim3(256), 0, st, io, B,
                           T_, C, m, gc, nout);
    } else {
        hipLaunchKernelGGL(k_compress_large<T>, dim3((unsigned)(B * nout)), dim3(256), 0, st, io,
                           B, T_, C, m, gc, nout);
    }
    return hipGetLastError();
}

hipError_t launch_compress(int dt, const void* x, RowStrides xs, const void* gate, RowStrides gs,
                           void* out, RowStrides os, int64_t B, int64_t T_, int C, int m, int gc,
                           hipStream_t st) {
    if (dt == 0)
        return launch_compress_t<float>({(const float*)x, (const float*)gate, (float*)out, xs, gs,
                                         os}, B, T_, C, m, gc, st);
    return launch_compress_t<uint16_t>({(const uint16_t*)x, (const uint16_t*)gate, (uint16_t*)out,
                                        xs, gs, os}, B, T_, C, m, gc, st);
}

}  // namespace csa
