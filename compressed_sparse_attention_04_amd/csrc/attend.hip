// attend.hip -- shared-KV multi-query attention over compressed entries
// joined with the raw sliding window (jiwasawa.github.io post: CSA "Shared
// Key-Value MQA" over the selected entries, HCA dense attention over every
// compressed entry, and the SWA branch over the newest tokens;
// studioglobal.ai answer: the 128-token window branch is always present).
//
// For the query at position t the key list is
//   [ selected (CSA) or all (HCA) compressed candidates | raw tokens w0..t ]
// and one softmax runs over it.  All H query heads share the one K/V head,
// so the H heads are the M dimension of the bf16 MFMAs and every K/V row is
// fetched once per query token for all heads.
//
// bf16 kernel, per block: one query token (all H = 32 * NW heads, one wave
// per 32 heads) and one split of its key list.  Per tile of 32 keys:
//   S^T = K * Q^T      (V_MFMA_F32_32X32X16_BF16, K rows from LDS, Q^T held
//                       in registers) -> every lane owns one head's column
//   online softmax in fp32 (exp2 domain), rows = keys, so the running max
//   and sum are per lane plus one cross-half exchange
//   O^T += V^T * P^T   (P^T straight from the S^T registers as bf16; V^T
//                       read from an LDS tile stored transposed, with its
//                       key order permuted to match P^T's register order)
// With more than one split the unnormalised (acc, max, sum) go to the
// workspace and k_attend_combine merges them (log-sum-exp).
#include "common.h"
#include "internal.h"

namespace csa {

constexpr int KT = 32;           // keys per tile

struct KeyList {
    int64_t t, w0, nsel, nwin, len;
};

__device__ __forceinline__ KeyList key_list(int64_t t, int64_t m, int64_t W, int k,
                                            bool sparse) {
    KeyList L;
    L.t = t;
    L.w0 = t - W + 1 < 0 ? 0 : t - W + 1;
    int64_t nc = n_candidates(t, m, W);
    L.nsel = sparse ? (nc < k ? nc : (int64_t)k) : nc;
    L.nwin = t - L.w0 + 1;
    L.len = L.nsel + L.nwin;
    return L;
}

// Row of key-list entry s: compressed row (>= 0 in ck/cv), raw row encoded
// as -(r+2) in rk/rv, or -1 for an entry that contributes nothing.
__device__ __forceinline__ int64_t list_row(const KeyList& L, int64_t s, const int32_t* sel,
                                            int64_t nc_t, int64_t raw_pos0) {
    if (s < L.nsel) {
        int64_t j = sel ? (int64_t)sel[s] : s;
        return (j >= 0 && j < nc_t) ? j : -1;
    }
    return -((L.w0 + (s - L.nsel) - raw_pos0) + 2);
}

template <int D, int NW>
__global__ void __launch_bounds__(NW * 64)
k_attend_bf16(const uint16_t* __restrict__ q, const uint16_t* __restrict__ ck,
              const uint16_t* __restrict__ cv, const int32_t* __restrict__ topk,
              const uint16_t* __restrict__ rk, const uint16_t* __restrict__ rv,
              uint16_t* __restrict__ o, float* __restrict__ part, int64_t Tq, int64_t Nc,
              int64_t m, int64_t W, int k, int64_t q_pos0, float scale_log2, int64_t raw_pos0,
              int64_t raw_len, int splits) {
    constexpr int NT = NW * 64;
    constexpr int H = NW * 32;
    constexpr int KPAD = D + 8;            // K row stride (bf16)
    constexpr int VPAD = KT + 8;           // V^T row stride (bf16)
    __shared__ __attribute__((aligned(16))) uint16_t sK[KT * KPAD];
    __shared__ __attribute__((aligned(16))) uint16_t sVt[D * VPAD];
    __shared__ int sValid[KT];

    const int64_t i = blockIdx.x;
    const int split = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
    const int col = lane & 31, kb = lane >> 5;
    const int64_t t = q_pos0 + i;
    const bool sparse = topk != nullptr;
    const KeyList L = key_list(t, m, W, k, sparse);
    const int64_t nc_t = n_candidates(t, m, W);
    const int32_t* sel = sparse ? topk + (b * Tq + i) * k : nullptr;

    // this split's range of the key list, in whole tiles
    const int64_t ntile = (L.len + KT - 1) / KT;
    const int64_t tps = (ntile + splits - 1) / splits;
    const int64_t s_begin = split * tps * KT;
    const int64_t s_end = min(L.len, s_begin + tps * KT);

    // Q^T operand: head hq, d = 16*kk + 8*kb + 0..7
    const int hq = wave * 32 + col;
    bf16x8 qop[D / 16];
    {
        const uint16_t* qp = q + ((b * Tq + i) * H + hq) * D + 8 * kb;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            qop[kk] = *reinterpret_cast<const bf16x8*>(qp + 16 * kk);
    }
    f32x16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
    float m_run = -INFINITY, l_run = 0.f;

    const uint16_t* ckb = ck + b * Nc * D;
    const uint16_t* cvb = cv + b * Nc * D;
    const uint16_t* rkb = rk + b * raw_len * D;
    const uint16_t* rvb = rv + b * raw_len * D;

    for (int64_t s0 = s_begin; s0 < s_end; s0 += KT) {
        __syncthreads();
        // cooperative load: KT keys x D/8 16-byte pieces of K and of V
        constexpr int PIECES = KT * (D / 8);
#pragma unroll
        for (int c = tid; c < PIECES; c += NT) {
            const int kk = c / (D / 8), p = c % (D / 8);
            const int64_t s = s0 + kk;
            int64_t row = s < s_end ? list_row(L, s, sel, nc_t, raw_pos0) : -1;
            u32x4 kv = {0u, 0u, 0u, 0u}, vv = {0u, 0u, 0u, 0u};
            if (row >= 0) {
                kv = *reinterpret_cast<const u32x4*>(ckb + row * D + p * 8);
                vv = *reinterpret_cast<const u32x4*>(cvb + row * D + p * 8);
            } else if (row <= -2) {
                const int64_t r = -row - 2;
                kv = *reinterpret_cast<const u32x4*>(rkb + r * D + p * 8);
                vv = *reinterpret_cast<const u32x4*>(rvb + r * D + p * 8);
            }
            *reinterpret_cast<u32x4*>(sK + kk * KPAD + p * 8) = kv;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                sVt[(p * 8 + 2 * e) * VPAD + kk] = (uint16_t)(vv[e] & 0xffffu);
                sVt[(p * 8 + 2 * e + 1) * VPAD + kk] = (uint16_t)(vv[e] >> 16);
            }
            if (p == 0) sValid[kk] = row != -1;
        }
        __syncthreads();

        // S^T = K Q^T : rows = keys (8*(r/4) + 4*kb + r%4), column = head
        f32x16 st = {};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
            bf16x8 a = *reinterpret_cast<const bf16x8*>(sK + col * KPAD + 16 * kk + 8 * kb);
            st = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[kk], st, 0, 0, 0);
        }
        float tmax = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = 8 * (r / 4) + 4 * kb + (r % 4);
            float v = sValid[key] ? st[r] * scale_log2 : -INFINITY;
            st[r] = v;
            tmax = fmaxf(tmax, v);
        }
        tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
        const float m_new = fmaxf(m_run, tmax);
        const float m_use = m_new == -INFINITY ? 0.f : m_new;
        const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
        m_run = m_new;
        float psum = 0.f;
        uint32_t pb[8];
#pragma unroll
        for (int r = 0; r < 16; r += 2) {
            float p0 = __builtin_amdgcn_exp2f(st[r] - m_use);
            float p1 = __builtin_amdgcn_exp2f(st[r + 1] - m_use);
            psum += p0 + p1;
            pb[r / 2] = f32_to_bf16_bits(p0) | (f32_to_bf16_bits(p1) << 16);
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;

        // O^T += V^T P^T, two k-steps of 16 keys; k-slot s of lane half kb
        // in step u is key 16u + 8*(s/4) + 4*kb + s%4 (the S^T register order)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
            bf16x8 pop;
            {
                u32x4 w = {pb[4 * u], pb[4 * u + 1], pb[4 * u + 2], pb[4 * u + 3]};
                pop = *reinterpret_cast<bf16x8*>(&w);
            }
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                const uint16_t* vr = sVt + (32 * dt + col) * VPAD + 16 * u + 4 * kb;
                u32x2 lo = *reinterpret_cast<const u32x2*>(vr);
                u32x2 hi = *reinterpret_cast<const u32x2*>(vr + 8);
                u32x4 w = {lo[0], lo[1], hi[0], hi[1]};
                bf16x8 a = *reinterpret_cast<bf16x8*>(&w);
                acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pop, acc[dt], 0, 0, 0);
            }
        }
    }
    const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
    if (splits == 1) {
        const float inv = 1.f / l_tot;
        uint16_t* op = o + ((b * Tq + i) * H + hq) * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * dt + 8 * g + 4 * kb;
                u32x2 w;
                w[0] = f32_to_bf16_bits(acc[dt][4 * g] * inv) |
                       (f32_to_bf16_bits(acc[dt][4 * g + 1] * inv) << 16);
                w[1] = f32_to_bf16_bits(acc[dt][4 * g + 2] * inv) |
                       (f32_to_bf16_bits(acc[dt][4 * g + 3] * inv) << 16);
                *reinterpret_cast<u32x2*>(op + d) = w;
            }
    } else {
        // partial record per (query, split, head): D accumulators, max, sum
        float* pr = part + (((b * Tq + i) * splits + split) * H + hq) * (D + 2);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int d = 32 * dt + 8 * g + 4 * kb;
                f32x4 w = {acc[dt][4 * g], acc[dt][4 * g + 1], acc[dt][4 * g + 2],
                           acc[dt][4 * g + 3]};
                *reinterpret_cast<f32x4*>(pr + d) = w;
            }
        if (kb == 0) {
            pr[D] = m_run;
            pr[D + 1] = l_tot;
        }
    }
}

// Log-sum-exp merge of the split partials; one thread per (head, 8 dims).
template <typename TO>
__global__ void __launch_bounds__(256)
k_attend_combine(const float* __restrict__ part, TO* __restrict__ o, int64_t Tq, int H, int D,
                 int splits) {
    const int64_t i = blockIdx.x, b = blockIdx.y;
    const int groups = D / 8;
    for (int w = threadIdx.x; w < H * groups; w += blockDim.x) {
        const int h = w / groups, d0 = (w % groups) * 8;
        const float* base = part + ((b * Tq + i) * splits * H + h) * (int64_t)(D + 2);
        const int64_t sstride = (int64_t)H * (D + 2);
        float M = -INFINITY;
        for (int s = 0; s < splits; ++s) M = fmaxf(M, base[s * sstride + D]);
        float Lsum = 0.f, a[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (M != -INFINITY) {
            for (int s = 0; s < splits; ++s) {
                const float* pr = base + s * sstride;
                float ms = pr[D];
                if (ms == -INFINITY) continue;
                float wgt = __builtin_amdgcn_exp2f(ms - M);
                Lsum += pr[D + 1] * wgt;
#pragma unroll
                for (int e = 0; e < 8; ++e) a[e] += pr[d0 + e] * wgt;
            }
        }
        const float inv = 1.f / Lsum;
#pragma unroll
        for (int e = 0; e < 8; ++e) a[e] *= inv;
        Elem<TO>::store8(o + ((b * Tq + i) * H + h) * (int64_t)D + d0, a);
    }
}

// fp32 kernel: one wave per (query, head) at a time, keys in sequence, the
// D dims spread over the lanes; fp32 arithmetic with accurate expf.
__global__ void __launch_bounds__(256)
k_attend_f32(const float* __restrict__ q, const float* __restrict__ ck,
             const float* __restrict__ cv, const int32_t* __restrict__ topk,
             const float* __restrict__ rk, const float* __restrict__ rv, float* __restrict__ o,
             int64_t Tq, int H, int D, int64_t Nc, int64_t m, int64_t W, int k, int64_t q_pos0,
             float scale, int64_t raw_pos0, int64_t raw_len) {
    const int64_t i = blockIdx.x, b = blockIdx.y;
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
    const int64_t t = q_pos0 + i;
    const bool sparse = topk != nullptr;
    const KeyList L = key_list(t, m, W, k, sparse);
    const int64_t nc_t = n_candidates(t, m, W);
    const int32_t* sel = sparse ? topk + (b * Tq + i) * k : nullptr;
    constexpr int DPL = 4;                 // dims per lane (D <= 256)
    for (int h = wave; h < H; h += blockDim.x / 64) {
        const float* qh = q + ((b * Tq + i) * H + h) * (int64_t)D;
        float qv[DPL], acc[DPL];
#pragma unroll
        for (int e = 0; e < DPL; ++e) {
            const int d = lane + 64 * e;
            qv[e] = d < D ? qh[d] : 0.f;
            acc[e] = 0.f;
        }
        float mx = -INFINITY, den = 0.f;
        for (int64_t s = 0; s < L.len; ++s) {
            int64_t row = list_row(L, s, sel, nc_t, raw_pos0);
            if (row == -1) continue;
            const float* kr = row >= 0 ? ck + (b * Nc + row) * (int64_t)D
                                       : rk + (b * raw_len + (-row - 2)) * (int64_t)D;
            const float* vr = row >= 0 ? cv + (b * Nc + row) * (int64_t)D
                                       : rv + (b * raw_len + (-row - 2)) * (int64_t)D;
            float dot = 0.f;
#pragma unroll
            for (int e = 0; e < DPL; ++e) {
                const int d = lane + 64 * e;
                if (d < D) dot += qv[e] * kr[d];
            }
#pragma unroll
            for (int off = 32; off > 0; off >>= 1) dot += __shfl_xor(dot, off, 64);
            const float lg = dot * scale;
            const float nm = fmaxf(mx, lg);
            const float a = expf(mx - nm), p = expf(lg - nm);
            den = den * a + p;
#pragma unroll
            for (int e = 0; e < DPL; ++e) {
                const int d = lane + 64 * e;
                acc[e] = acc[e] * a + (d < D ? p * vr[d] : 0.f);
            }
            mx = nm;
        }
        float* oh = o + ((b * Tq + i) * H + h) * (int64_t)D;
#pragma unroll
        for (int e = 0; e < DPL; ++e) {
            const int d = lane + 64 * e;
            if (d < D) oh[d] = acc[e] / den;
        }
    }
}

AttendPlan plan_attend(int dt, int64_t B, int64_t Tq, int64_t H, int64_t D, int64_t max_keys) {
    AttendPlan p{};
    p.splits = 1;
    if (dt == 1) {
        const int64_t rows = B * Tq;
        const int64_t tiles = (max_keys + KT - 1) / KT;
        if (rows < 1024 && tiles > 2) {
            int64_t want = (1024 + rows - 1) / rows;          // ~4 blocks per CU
            int64_t cap = (tiles + 1) / 2;                     // >= 2 tiles per split
            p.splits = (int)min(min(want, cap), (int64_t)64);
            if (p.splits < 1) p.splits = 1;
        }
    }
    p.ws_bytes = p.splits > 1 ? (size_t)(B * Tq * p.splits * H * (D + 2)) * sizeof(float) : 0;
    return p;
}

template <int D, int NW>
static void launch_bf16(const AttendPlan& p, int64_t B, int64_t Tq, int64_t Nc, int64_t m,
                        int64_t W, int k, int64_t q_pos0, float scale, const void* q,
                        const void* ck, const void* cv, const int32_t* topk, const void* rk,
                        const void* rv, int64_t raw_pos0, int64_t raw_len, void* o, void* ws,
                        hipStream_t st) {
    const float scale_log2 = scale * 1.4426950408889634f;
    hipLaunchKernelGGL((k_attend_bf16<D, NW>), dim3((unsigned)Tq, (unsigned)p.splits, (unsigned)B),
                       dim3(NW * 64), 0, st, (const uint16_t*)q, (const uint16_t*)ck,
                       (const uint16_t*)cv, topk, (const uint16_t*)rk, (const uint16_t*)rv,
                       (uint16_t*)o, (float*)ws, Tq, Nc, m, W, k, q_pos0, scale_log2, raw_pos0,
                       raw_len, p.splits);
    if (p.splits > 1)
        hipLaunchKernelGGL(k_attend_combine<uint16_t>, dim3((unsigned)Tq, (unsigned)B),
                           dim3(256), 0, st, (const float*)ws, (uint16_t*)o, Tq, NW * 32, D,
                           p.splits);
}

hipError_t launch_attend(int dt, const AttendPlan& p, int64_t B, int64_t Tq, int64_t H,
                         int64_t D, int64_t Nc, int64_t m, int64_t W, int64_t k,
                         int64_t q_pos0, float scale, const void* q, const void* ck,
                         const void* cv, const int32_t* topk, const void* rk, const void* rv,
                         int64_t raw_pos0, int64_t raw_len, void* o, void* ws, hipStream_t st) {
    if (B == 0 || Tq == 0) return hipSuccess;
    if (dt == 0) {
        hipLaunchKernelGGL(k_attend_f32, dim3((unsigned)Tq, (unsigned)B), dim3(256), 0, st,
                           (const float*)q, (const float*)ck, (const float*)cv, topk,
                           (const float*)rk, (const float*)rv, (float*)o, Tq, (int)H, (int)D,
                           Nc, m, W, (int)k, q_pos0, scale, raw_pos0, raw_len);
        return hipGetLastError();
    }
    const int nw = (int)(H / 32);
#define CSA_ATT_CASE(DD, NN)                                                                  \
    launch_bf16<DD, NN>(p, B, Tq, Nc, m, W, (int)k, q_pos0, scale, q, ck, cv, topk, rk, rv,   \
                        raw_pos0, raw_len, o, ws, st)
    if (D == 128) {
        switch (nw) {
            case 1: CSA_ATT_CASE(128, 1); break;
            case 2: CSA_ATT_CASE(128, 2); break;
            case 4: CSA_ATT_CASE(128, 4); break;
            case 8: CSA_ATT_CASE(128, 8); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (nw) {
            case 1: CSA_ATT_CASE(64, 1); break;
            case 2: CSA_ATT_CASE(64, 2); break;
            case 4: CSA_ATT_CASE(64, 4); break;
            case 8: CSA_ATT_CASE(64, 8); break;
            default: return hipErrorInvalidValue;
        }
    }
#undef CSA_ATT_CASE
    return hipGetLastError();
}

}  // namespace csa
