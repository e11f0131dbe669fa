// index_decode.hip -- Lightning Indexer for a few query rows over a long
// compressed context (decode): jiwasawa.github.io post, CSA indexer bullet
// (score every compressed entry, keep the top k); ai-papers.net, hybrid
// attention section (the FP4 indexer scans the already 4x shorter sequence).
//
// The FP4 key stream dominates (34 bytes per candidate at dI = 64), so the
// work is spread over many blocks that each read one chunk of keys once:
//   k_dscore : scores of <= 8 query rows against one chunk (scaled FP4
//              MFMA), written as fp32 to the workspace, plus the level-1
//              threshold histogram of each row (LDS, then global atomics);
//   k_dselect: one block per query row narrows the threshold from the
//              histogram, collects from the stored scores and emits the
//              kept indices in ascending order (same exact rule as the
//              streaming kernel: score desc, index asc).
#include "internal.h"
#include "mxfp4.h"
#include "wave_select.h"

namespace csa {

constexpr int DS_NT = 256;
constexpr int DS_QT = 8;
constexpr int DS_CH = 2048;            // candidates per scoring block
constexpr int DL_NT = 1024;
constexpr int DL_CAP = 1024;           // collected keys per row
constexpr int DL_MAXW = 8192;          // bitmap words -> 262144 candidates

// score rows are padded to whole 16-byte vectors
__host__ __device__ __forceinline__ int64_t score_stride(int64_t nc) { return (nc + 3) & ~(int64_t)3; }

__global__ void k_zero_u32(uint32_t* p, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

template <typename T, int HI>
__global__ void __launch_bounds__(DS_NT)
k_dscore(const T* __restrict__ q_idx, const uint8_t* __restrict__ kc,
         const uint8_t* __restrict__ ks, uint32_t* __restrict__ scores,
         uint32_t* __restrict__ ghist, int64_t Tq, int dI, int64_t Nc, int64_t m, int64_t W,
         int64_t q_pos0, int64_t ncap) {
    __shared__ uint32_t hist[DS_QT][SEL_NB];
    constexpr int NU = 16 / HI;
    const int64_t c0 = (int64_t)blockIdx.x * DS_CH;
    const int64_t b = blockIdx.y;
    const int qv = (int)Tq;                          // Tq <= DS_QT on this path
    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
    const int row = lane & 31, kb = lane >> 5;
    const int64_t nc_max = n_candidates(q_pos0 + qv - 1, m, W);
    const int nkeys = (int)min((int64_t)DS_CH, nc_max - c0);
    if (nkeys <= 0) return;
    for (int i = tid; i < DS_QT * SEL_NB; i += DS_NT) (&hist[0][0])[i] = 0u;

    i32x8 aop = {0, 0, 0, 0, 0, 0, 0, 0};
    int sa = 127;
    {
        const int qi = row / HI, h = row % HI;
        if (qi < qv && kb * 32 < dI) {
            const T* src = q_idx + (((b * Tq + qi) * HI + h) * dI + kb * 32);
            float v[32];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
                float t8[8];
                Elem<T>::load8(src + p * 8, t8);
#pragma unroll
                for (int i = 0; i < 8; ++i) v[p * 8 + i] = t8[i];
            }
            uint32_t pk[4], sb;
            mxfp4_encode32(v, pk, sb);
            aop[0] = (int)pk[0]; aop[1] = (int)pk[1]; aop[2] = (int)pk[2]; aop[3] = (int)pk[3];
            sa = (int)sb;
        }
    }
    const int kbq = kb * 4 / HI;
    int qslot[NU];
    int64_t ncq[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int g = (u * HI) / 4, i = (u * HI) % 4;
        qslot[u] = (8 * g + i) / HI + kbq;
        ncq[u] = qslot[u] < qv ? n_candidates(q_pos0 + qslot[u], m, W) : 0;
    }
    __syncthreads();

    const int kbytes = dI / 2, kscales = dI / 32;
    const uint8_t* kcb = kc + b * Nc * kbytes;
    const uint8_t* ksb = ks + b * Nc * kscales;
    constexpr int UNR = 4;                           // tiles in flight per wave
    const int ntiles = (nkeys + 31) / 32;
    for (int t0 = wave * UNR; t0 < ntiles; t0 += (DS_NT / WAVE) * UNR) {
        i32x8 bop[UNR];
        int sbk[UNR];
#pragma unroll
        for (int x = 0; x < UNR; ++x) {
            const int jj = (t0 + x) * 32 + row;
            bop[x] = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
            sbk[x] = 127;
            if (jj < nkeys && kb < kscales) {
                const int64_t j = c0 + jj;
                u32x4 w = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4*>(kcb + j * kbytes + kb * 16));
                bop[x][0] = (int)w[0]; bop[x][1] = (int)w[1];
                bop[x][2] = (int)w[2]; bop[x][3] = (int)w[3];
                sbk[x] = ksb[j * kscales + kb];
            }
        }
#pragma unroll
        for (int x = 0; x < UNR; ++x) {
            const int jj = (t0 + x) * 32 + row;
            const int64_t j = c0 + jj;
            f32x16 acc = {};
            acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop, bop[x], acc, 4, 4, 0, sa, 0,
                                                                   sbk[x]);
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int q = qslot[u];
                if (q >= qv || jj >= nkeys) continue;
                float s = 0.f;
#pragma unroll
                for (int hh = 0; hh < HI; ++hh) s += fmaxf(acc[u * HI + hh], 0.f);
                const uint32_t key = s == 0.f ? 0u : __float_as_uint(s);
                scores[((b * Tq + q) * ncap) + j] = key;
                if (j < ncq[u]) atomicAdd(&hist[q][lvl1_bin(key)], 1u);
            }
        }
    }
    __syncthreads();
    for (int i = tid; i < qv * SEL_NB; i += DS_NT) {
        const uint32_t c = (&hist[0][0])[i];
        if (c) atomicAdd(&ghist[(b * Tq) * SEL_NB + i], c);
    }
}

// Visit the nc stored keys of one row, 16-byte vectors, four in flight per
// thread, calling fn(key, candidate index).
template <typename F>
__device__ __forceinline__ void scan_scores(const uint32_t* __restrict__ sc, int nc, F&& fn) {
    const int nv = nc / 4;
    const u32x4* v4 = reinterpret_cast<const u32x4*>(sc);
    constexpr int U = 4;
    for (int v0 = threadIdx.x; v0 < nv; v0 += DL_NT * U) {
        u32x4 w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + u * DL_NT;
            w[u] = v < nv ? __builtin_nontemporal_load(v4 + v) : u32x4{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int v = v0 + u * DL_NT;
            if (v < nv) {
#pragma unroll
                for (int e = 0; e < 4; ++e) fn(w[u][e], 4 * v + e);
            }
        }
    }
    for (int j = 4 * nv + (int)threadIdx.x; j < nc; j += DL_NT) fn(sc[j], j);
}

struct DselSmem {
    uint32_t sel[DL_MAXW];
    uint32_t eq[DL_MAXW];
    uint32_t hist[SEL_NB];
    u32x2 cb[DL_CAP];
    uint32_t lo, hi;
    int shift, above, in, mode, cnt, eqmode;
};

__global__ void __launch_bounds__(DL_NT)
k_dselect(const uint32_t* __restrict__ scores, const uint32_t* __restrict__ ghist,
          int32_t* __restrict__ topk, int64_t Tq, int64_t m, int64_t W, int k, int64_t q_pos0,
          int64_t ncap) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    DselSmem& S = *reinterpret_cast<DselSmem*>(smem_raw);
    const int64_t q = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
    const int nc = (int)n_candidates(q_pos0 + q, m, W);
    const int nw = (nc + 31) / 32;
    const int need = min(nc, k);
    const uint32_t* sc = scores + (b * Tq + q) * ncap;
    int32_t* out = topk + (b * Tq + q) * k;

    for (int w = tid; w < nw; w += DL_NT) {
        uint32_t full = 0u;
        if (nc <= k) {
            const int lo_b = w * 32;
            full = lo_b + 32 <= nc ? 0xFFFFFFFFu : ((1u << (nc - lo_b)) - 1u);
        }
        S.sel[w] = full;
        S.eq[w] = 0u;
    }
    if (nc > k) {
        // level 1 from the scoring blocks' histogram
        if (wave == 0) {
            int gt, in;
            for (int i = lane; i < SEL_NB; i += WAVE) S.hist[i] = ghist[(b * Tq + q) * SEL_NB + i];
            __builtin_amdgcn_wave_barrier();
            const int d = wave_hist_find(S.hist, need, &gt, &in);
            if (lane == 0) {
                uint32_t lo, hi;
                lvl1_range(d, &lo, &hi);
                S.lo = lo;
                S.hi = hi;
                S.above = gt;
                S.in = in;
            }
        }
        __syncthreads();
        // refine while the threshold range holds too many keys
#pragma unroll 1
        for (int it = 0; it < 6; ++it) {
            const uint32_t lo = S.lo, hi = S.hi;
            if (S.in <= DL_CAP || hi - lo == 1u) break;
            const int sh = range_shift(lo, hi);
            __syncthreads();
            for (int i = tid; i < SEL_NB; i += DL_NT) S.hist[i] = 0u;
            __syncthreads();
            scan_scores(sc, nc, [&](uint32_t key, int j) {
                if (key >= lo && key < hi) atomicAdd(&S.hist[(key - lo) >> sh], 1u);
            });
            __syncthreads();
            if (wave == 0) {
                int gt, in;
                const int d = wave_hist_find(S.hist, need - S.above, &gt, &in);
                if (lane == 0) {
                    S.lo = lo + ((uint32_t)d << sh);
                    uint64_t top = (uint64_t)lo + ((uint64_t)(d + 1) << sh);
                    S.hi = top < (uint64_t)hi ? (uint32_t)top : hi;
                    S.above += gt;
                    S.in = in;
                }
            }
            __syncthreads();
        }
        // collect
        const uint32_t lo = S.lo, hi = S.hi;
        const bool eqmode = S.in > DL_CAP;             // single-valued range with many ties
        if (tid == 0) S.cnt = 0;
        __syncthreads();
        scan_scores(sc, nc, [&](uint32_t key, int j) {
            if (key >= hi) {
                atomicOr(&S.sel[j >> 5], 1u << (j & 31));
            } else if (key >= lo) {
                if (eqmode) {
                    atomicOr(&S.eq[j >> 5], 1u << (j & 31));
                } else {
                    const int pos = atomicAdd(&S.cnt, 1);
                    if (pos < DL_CAP) {
                        u32x2 e = {key, (uint32_t)j};
                        S.cb[pos] = e;
                    }
                }
            }
        });
        __syncthreads();
        if (wave == 0) {
            const int need_in = need - S.above;
            int need_eq = need_in;
            if (!eqmode) {
                const int n = min(S.cnt, DL_CAP);
                constexpr int EPT = DL_CAP / WAVE;
                uint32_t key[EPT];
                bool valid[EPT];
#pragma unroll
                for (int e = 0; e < EPT; ++e) {
                    const int p = lane * EPT + e;
                    valid[e] = p < n;
                    key[e] = valid[e] ? S.cb[p][0] : 0u;
                }
                uint32_t T;
                wave_radix_threshold<EPT>(key, valid, need_in, S.hist, &T, &need_eq);
#pragma unroll
                for (int e = 0; e < EPT; ++e) {
                    if (!valid[e]) continue;
                    const uint32_t j = S.cb[lane * EPT + e][1];
                    if (key[e] > T) atomicOr(&S.sel[j >> 5], 1u << (j & 31));
                    else if (key[e] == T) atomicOr(&S.eq[j >> 5], 1u << (j & 31));
                }
                __builtin_amdgcn_wave_barrier();
            }
            wave_merge_first_bits(S.sel, S.eq, nw, need_eq);
        }
    }
    __syncthreads();
    if (wave == 0) wave_emit_bitmap(S.sel, nw, out, k);
}

size_t dselect_smem_bytes() { return sizeof(DselSmem); }
int decode_max_candidates() { return DL_MAXW * 32; }
int decode_max_rows() { return DS_QT; }

size_t decode_ws_bytes(int64_t B, int64_t Tq, int64_t ncap) {
    return (size_t)(B * Tq) * (size_t)(score_stride(ncap) + SEL_NB) * sizeof(uint32_t);
}

template <typename T, int HI>
static void launch_dscore(int64_t B, int64_t Tq, int dI, int64_t Nc, int64_t m, int64_t W,
                          int64_t q_pos0, const void* q_idx, const uint8_t* kc, const uint8_t* ks,
                          uint32_t* scores, uint32_t* ghist, int64_t ncap, hipStream_t st) {
    dim3 grid((unsigned)((ncap + DS_CH - 1) / DS_CH), (unsigned)B);
    hipLaunchKernelGGL((k_dscore<T, HI>), grid, dim3(DS_NT), 0, st, (const T*)q_idx, kc, ks,
                       scores, ghist, Tq, dI, Nc, m, W, q_pos0, ncap);
}

hipError_t launch_index_decode(int dt, int64_t B, int64_t Tq, int HI, int dI, int64_t Nc,
                               int64_t m, int64_t W, int k, int64_t q_pos0, const void* q_idx,
                               const uint8_t* kc, const uint8_t* ks, int32_t* topk, void* ws,
                               hipStream_t st) {
    if (B == 0 || Tq == 0) return hipSuccess;
    const int64_t ncap = score_stride(n_candidates(q_pos0 + Tq - 1, m, W));
    uint32_t* ghist = reinterpret_cast<uint32_t*>(ws);
    uint32_t* scores = ghist + B * Tq * SEL_NB;
    const int64_t nh = B * Tq * SEL_NB;
    hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)((nh + 255) / 256)), dim3(256), 0, st, ghist, nh);
    if (ncap > 0) {
#define CSA_DS_CASE(TT, HH) \
    launch_dscore<TT, HH>(B, Tq, dI, Nc, m, W, q_pos0, q_idx, kc, ks, scores, ghist, ncap, st)
        if (dt == 0) {
            if (HI == 1) CSA_DS_CASE(float, 1);
            else if (HI == 2) CSA_DS_CASE(float, 2);
            else CSA_DS_CASE(float, 4);
        } else {
            if (HI == 1) CSA_DS_CASE(uint16_t, 1);
            else if (HI == 2) CSA_DS_CASE(uint16_t, 2);
            else CSA_DS_CASE(uint16_t, 4);
        }
#undef CSA_DS_CASE
    }
    const size_t lds = sizeof(DselSmem);
    hipFuncSetAttribute((const void*)k_dselect, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(k_dselect, dim3((unsigned)Tq, (unsigned)B), dim3(DL_NT), lds, st, scores,
                       ghist, topk, Tq, m, W, k, q_pos0, ncap);
    return hipGetLastError();
}

}  // namespace csa
