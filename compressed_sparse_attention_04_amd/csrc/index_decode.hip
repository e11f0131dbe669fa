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
//   k_dcollect: blocks over (chunk of 4096 stored scores, row) find the
//              threshold range from the row's histogram, write the chunk's
//              bitmap words of the surely kept keys (above the range) and
//              put the keys inside the range in the chunk's own slots of the
//              row's buffer (no global atomics: same-address device atomics
//              from every chunk would serialise);
//   k_dfinal : one block per row resolves the range exactly from the buffer
//              (or, when the range holds too many keys, narrows it further
//              by scanning the stored scores) and emits the kept indices in
//              ascending order (score desc, index asc, as everywhere).
#include "internal.h"
#include "mxfp4.h"
#include "wave_select.h"
#include "fp4_tiles.h"

namespace csa {

constexpr int DS_NT = 256;
constexpr int DS_QT = 8;
constexpr int DS_CH = 4096;            // candidates per scoring block
constexpr int DL_NT = 1024;
constexpr int DL_CAP = 1024;           // collected keys per row
constexpr int DL_MAXW = 8192;          // bitmap words -> 262144 candidates
constexpr int DC_CH_ = 4096;           // stored scores per collecting block
constexpr int DC_NB = DL_MAXW * 32 / DC_CH_;   // collecting blocks per row (64)
constexpr int DC_SLOTS = DL_CAP / DC_NB;       // buffer slots per collecting block (16)

// score rows are padded to whole 16-byte vectors
__host__ __device__ __forceinline__ int64_t score_stride(int64_t nc) { return (nc + 3) & ~(int64_t)3; }

__global__ void k_zero_u32(uint32_t* p, int64_t n) {
    int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

// Workspace of the decode path (rows = B * Tq; u32 words, counts padded to
// multiples of 4): hist [rows][1024] | cnt [rows][DC_NB] (keys in range per
// collecting block) | thr [rows][4] | bitmap [rows][DL_MAXW] | buffer
// [rows][DC_NB][DC_SLOTS] (key, index) | scores [rows][stride].  Only hist
// starts at zero.
struct DecodeWs {
    uint32_t* hist;
    uint32_t* cnt;
    u32x4* thr;        // [rows] level-1 range: lo, hi, count above, count inside
    uint32_t* bmp;
    u32x2* cb;
    uint32_t* scores;
};

__host__ __device__ __forceinline__ int64_t pad4(int64_t n) { return (n + 3) & ~(int64_t)3; }

__host__ __device__ __forceinline__ DecodeWs decode_ws(void* ws, int64_t B, int64_t rows) {
    DecodeWs w;
    uint32_t* p = reinterpret_cast<uint32_t*>(ws);
    w.hist = p;
    p += rows * SEL_NB;
    w.cnt = p;
    p += rows * DC_NB;
    w.thr = reinterpret_cast<u32x4*>(p);
    p += rows * 4;
    w.bmp = p;
    p += rows * DL_MAXW;
    w.cb = reinterpret_cast<u32x2*>(p);
    p += rows * DL_CAP * 2;
    w.scores = p;
    return w;
}

// Threshold range of a row at level 1 from its histogram (one wave).
__device__ __forceinline__ void lvl1_threshold(const uint32_t* hist, int need, uint32_t* lo,
                                               uint32_t* hi, int* above, int* in) {
    int gt, cnt_in;
    const int d = wave_hist_find(hist, need, &gt, &cnt_in);
    lvl1_range(d, lo, hi);
    *above = gt;
    *in = cnt_in;
}

template <typename T, int HI>
__global__ void __launch_bounds__(DS_NT)
k_dscore(const T* __restrict__ q_idx, const uint8_t* __restrict__ kc,
         const uint8_t* __restrict__ ks, DecodeWs ws, int64_t Tq, int dI, int64_t Nc, int64_t m,
         int64_t W, int k, int64_t q_pos0, int64_t ncap) {
    extern __shared__ uint32_t hist_raw[];           // [Tq][SEL_NB]
    uint32_t (*hist)[SEL_NB] = reinterpret_cast<uint32_t (*)[SEL_NB]>(hist_raw);
    constexpr int NU = 16 / HI;
    const int64_t c0 = (int64_t)blockIdx.x * DS_CH;
    const int64_t b = blockIdx.y;
    const int qv = (int)Tq;                          // Tq <= DS_QT on this path
    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
    const int row = lane & 31, kb = lane >> 5;
    const int64_t nc_max = n_candidates(q_pos0 + qv - 1, m, W);
    const int nkeys = (int)min((int64_t)DS_CH, nc_max - c0);   // >= 1: grid covers nc_max
    uint32_t* scores = ws.scores;
    for (int i = tid; i < qv * SEL_NB; i += DS_NT) hist_raw[i] = 0u;

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
    const TileSrc ts{kc + (b * Nc + c0) * kbytes, ks + (b * Nc + c0) * kscales, kbytes, kscales,
                     nkeys, row, kb};
    stream_tiles<DS_NT, 4, true>(ts, (nkeys + 31) / 32, 1, aop, sa,
                                 [&](const f32x16& acc, int jt) {
        const int jj = jt + row;
        const int64_t j = c0 + jj;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int q = qslot[u];
            if (q >= qv || jj >= nkeys) continue;
            const uint32_t key = score_key<HI>(acc, u);
            scores[((b * Tq + q) * ncap) + j] = key;
            if (j < ncq[u]) atomicAdd(&hist[q][lvl1_bin(key)], 1u);
        }
    });
    __syncthreads();
    for (int i = tid; i < qv * SEL_NB; i += DS_NT) {
        const uint32_t c = hist_raw[i];
        if (c) atomicAdd(&ws.hist[(b * Tq) * SEL_NB + i], c);
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

constexpr int DC_NT = 256;
constexpr int DC_CH = DC_CH_;

__global__ void __launch_bounds__(DC_NT)
k_dcollect(DecodeWs ws, int64_t Tq, int64_t m, int64_t W, int k, int64_t q_pos0,
           int64_t stride) {
    __shared__ uint32_t words[DC_CH / 32];
    const int64_t c0 = (int64_t)blockIdx.x * DC_CH;
    const int64_t q = blockIdx.y, b = blockIdx.z;
    const int64_t rowi = b * Tq + q;
    const int nc = (int)n_candidates(q_pos0 + q, m, W);
    if (nc <= k || c0 >= nc) return;                 // the final kernel needs nothing here
    const int tid = threadIdx.x;
    const int n = (int)min((int64_t)DC_CH, (int64_t)nc - c0);
    const uint32_t* sc = ws.scores + rowi * stride + c0;
    const int nv = n / 4;
    // this block's scores are in flight while wave 0 finds the range
    constexpr int VPT = DC_CH / 4 / DC_NT;
    u32x4 vals[VPT];
#pragma unroll
    for (int x = 0; x < VPT; ++x) {
        const int v = tid + x * DC_NT;
        vals[x] = v < nv ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(sc) + v)
                         : u32x4{0u, 0u, 0u, 0u};
    }
    __shared__ u32x4 s_thr;
    if (tid < WAVE) {
        uint32_t lo, hi;
        int above, in;
        lvl1_threshold(ws.hist + rowi * SEL_NB, k, &lo, &hi, &above, &in);
        const u32x4 t = {lo, hi, (uint32_t)above, (uint32_t)in};
        if (tid == 0) {
            s_thr = t;
            if (blockIdx.x == 0) ws.thr[rowi] = t;   // for the final kernel
        }
    }
    __shared__ uint32_t s_cnt;
    for (int w = tid; w < DC_CH / 32; w += DC_NT) words[w] = 0u;
    if (tid == 0) s_cnt = 0u;
    __syncthreads();
    const uint32_t lo = s_thr[0], hi = s_thr[1];
    const bool collect = s_thr[3] <= (uint32_t)DL_CAP;
    uint32_t* cnt = &s_cnt;
    u32x2* cb = ws.cb + rowi * DL_CAP + blockIdx.x * DC_SLOTS;
#pragma unroll
    for (int x = 0; x < VPT; ++x) {
        const int v = tid + x * DC_NT;
        if (v >= nv) break;
        const u32x4 w = vals[x];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int j = 4 * v + e;
            const uint32_t key = w[e];
            if (key >= hi) {
                atomicOr(&words[j >> 5], 1u << (j & 31));
            } else if (key >= lo && collect) {
                const uint32_t pos = atomicAdd(cnt, 1u);
                if (pos < (uint32_t)DC_SLOTS) cb[pos] = u32x2{key, (uint32_t)(c0 + j)};
            }
        }
    }
    for (int j = 4 * nv + tid; j < n; j += DC_NT) {
        const uint32_t key = sc[j];
        if (key >= hi) {
            atomicOr(&words[j >> 5], 1u << (j & 31));
        } else if (key >= lo && collect) {
            const uint32_t pos = atomicAdd(cnt, 1u);
            if (pos < (uint32_t)DC_SLOTS) cb[pos] = u32x2{key, (uint32_t)(c0 + j)};
        }
    }
    __syncthreads();
    for (int w = tid; w < (n + 31) / 32; w += DC_NT) ws.bmp[rowi * DL_MAXW + c0 / 32 + w] = words[w];
    // more than DC_SLOTS keys here reads as an overflow in the final kernel
    if (tid == 0) ws.cnt[rowi * DC_NB + blockIdx.x] = s_cnt;
}

struct DselSmem {
    uint32_t sel[DL_MAXW];
    uint32_t eq[DL_MAXW];
    uint32_t hist[SEL_NB];
    u32x2 cb[DL_CAP];
    uint32_t lo, hi;
    int shift, above, in, mode, cnt, eqmode, need_eq;
    int scratch[DL_NT / WAVE + 1];
    int boff[DC_NB];                // first buffer position of each collecting block
};

__global__ void __launch_bounds__(DL_NT)
k_dfinal(DecodeWs ws, int32_t* __restrict__ topk, int64_t Tq, int64_t m, int64_t W, int k,
         int64_t q_pos0, int64_t stride) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    DselSmem& S = *reinterpret_cast<DselSmem*>(smem_raw);
    const int64_t q = blockIdx.x, b = blockIdx.y;
    const int64_t rowi = b * Tq + q;
    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
    const int nc = (int)n_candidates(q_pos0 + q, m, W);
    const int nw = (nc + 31) / 32;
    const int need = min(nc, k);
    const uint32_t* sc = ws.scores + rowi * stride;
    int32_t* out = topk + rowi * k;

    if (nc <= k) {                                  // every candidate is kept
        for (int s2 = tid; s2 < k; s2 += DL_NT) out[s2] = s2 < nc ? s2 : -1;
        return;
    }
    // every global read of this block is issued up front: the bitmap words of
    // the keys above the range (8 per thread), one buffer slot and its
    // block's count per thread, the threshold range
    static_assert(DL_MAXW == 8 * DL_NT && DC_NB * DC_SLOTS == DL_NT, "one pass of loads");
    const int nblk = (nc + DC_CH_ - 1) / DC_CH_;
    const u32x4* bw = reinterpret_cast<const u32x4*>(ws.bmp + rowi * DL_MAXW) + 2 * tid;
    const bool wlive = 8 * tid < nw;
    const u32x4 w0 = wlive ? bw[0] : u32x4{0u, 0u, 0u, 0u};
    const u32x4 w1 = wlive ? bw[1] : u32x4{0u, 0u, 0u, 0u};
    const int sblk = tid / DC_SLOTS, sidx = tid % DC_SLOTS;
    const bool slive = sblk < nblk;
    const uint32_t scnt = slive ? ws.cnt[rowi * DC_NB + sblk] : 0u;
    // (read whether or not it holds a key, so it does not wait for the count)
    const u32x2 slot = slive ? ws.cb[rowi * DL_CAP + tid] : u32x2{0u, 0u};
    const uint32_t c = lane < nblk ? ws.cnt[rowi * DC_NB + lane] : 0u;   // (wave 0)
    const u32x4 thr = ws.thr[rowi];
    // (words past nw are never read: every bitmap pass stops at nw)
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        S.sel[8 * tid + x] = w0[x];
        S.sel[8 * tid + 4 + x] = w1[x];
        S.eq[8 * tid + x] = 0u;
        S.eq[8 * tid + 4 + x] = 0u;
    }
    if (wave == 0) {
        // per collecting block: keys in range (more than DC_SLOTS: overflow)
        const bool over = __ballot(c > (uint32_t)DC_SLOTS) != 0ull;
        const int incl = wave_incl_scan((int)c);
        const int total = __shfl(incl, WAVE - 1, WAVE);
        S.boff[lane] = incl - (int)c;
        if (lane == 0) {
            S.lo = thr[0];
            S.hi = thr[1];
            S.above = (int)thr[2];
            S.in = (int)thr[3];
            S.cnt = S.in <= DL_CAP && !over ? total : -1;
        }
    }
    __syncthreads();
    if (S.cnt >= 0) {
        // the collecting blocks gathered the range's keys into their slots
        if (slive && sidx < (int)scnt) S.cb[S.boff[sblk] + sidx] = slot;
        __syncthreads();
    } else {
        // too many keys in the level-1 range: narrow it over the stored scores
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
        // collect the narrowed range (keys above it are kept for sure)
        const uint32_t lo = S.lo, hi = S.hi;
        const bool eqmode = S.in > DL_CAP;         // single-valued range with many ties
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
                    if (pos < DL_CAP) S.cb[pos] = u32x2{key, (uint32_t)j};
                }
            }
        });
        __syncthreads();
        if (eqmode && tid == 0) S.cnt = -1;
        __syncthreads();
    }
    if (wave == 0) {
        const int need_in = need - S.above;
        int need_eq = need_in;
        if (S.cnt >= 0) {
            const int n = min(S.cnt, DL_CAP);
            constexpr int EPT = DL_CAP / WAVE;
            uint32_t key[EPT];
            bool valid[EPT];
#pragma unroll
            for (int e = 0; e < EPT; ++e) {
                const int p = e * WAVE + lane;          // lane-contiguous: no bank conflicts
                valid[e] = p < n;
                key[e] = valid[e] ? S.cb[p][0] : 0u;
            }
            uint32_t thr;
            wave_radix_threshold<EPT>(key, valid, need_in, S.hist, &thr, &need_eq);
#pragma unroll
            for (int e = 0; e < EPT; ++e) {
                if (!valid[e]) continue;
                const uint32_t j = S.cb[e * WAVE + lane][1];
                if (key[e] > thr) atomicOr(&S.sel[j >> 5], 1u << (j & 31));
                else if (key[e] == thr) atomicOr(&S.eq[j >> 5], 1u << (j & 31));
            }
            __builtin_amdgcn_wave_barrier();
        }
        if (lane == 0) S.need_eq = need_eq;
    }
    __syncthreads();
    block_merge_emit8<DL_NT>(S.sel, S.eq, nw, S.need_eq, out, k, S.scratch);
}

size_t dselect_smem_bytes() { return sizeof(DselSmem); }
int decode_max_candidates() { return DL_MAXW * 32; }
int decode_max_rows() { return DS_QT; }

size_t decode_ws_bytes(int64_t B, int64_t Tq, int64_t ncap) {
    const int64_t rows = B * Tq;
    const int64_t words = rows * SEL_NB + rows * DC_NB + rows * 4 + rows * DL_MAXW +
                          rows * DL_CAP * 2 + rows * score_stride(ncap);
    return (size_t)words * sizeof(uint32_t);
}

template <typename T, int HI>
static void launch_dscore(int64_t B, int64_t Tq, int dI, int64_t Nc, int64_t m, int64_t W, int k,
                          int64_t q_pos0, const void* q_idx, const uint8_t* kc, const uint8_t* ks,
                          const DecodeWs& w, int64_t ncand, int64_t stride, hipStream_t st) {
    dim3 grid((unsigned)((ncand + DS_CH - 1) / DS_CH), (unsigned)B);
    hipLaunchKernelGGL((k_dscore<T, HI>), grid, dim3(DS_NT), Tq * SEL_NB * sizeof(uint32_t), st,
                       (const T*)q_idx, kc, ks, w, Tq, dI, Nc, m, W, k, q_pos0, stride);
}

hipError_t launch_index_decode(int dt, int64_t B, int64_t Tq, int HI, int dI, int64_t Nc,
                               int64_t m, int64_t W, int k, int64_t q_pos0, const void* q_idx,
                               const uint8_t* kc, const uint8_t* ks, int32_t* topk, void* ws,
                               hipStream_t st) {
    if (B == 0 || Tq == 0) return hipSuccess;
    const int64_t ncand = n_candidates(q_pos0 + Tq - 1, m, W);
    const int64_t stride = score_stride(ncand);
    const int64_t rows = B * Tq;
    DecodeWs w = decode_ws(ws, B, rows);
    if (ncand > 0) {
        // histograms start at zero
        const int64_t nz = rows * SEL_NB;
        hipLaunchKernelGGL(k_zero_u32, dim3((unsigned)((nz + 255) / 256)), dim3(256), 0, st,
                           w.hist, nz);
#define CSA_DS_CASE(TT, HH) \
    launch_dscore<TT, HH>(B, Tq, dI, Nc, m, W, k, q_pos0, q_idx, kc, ks, w, ncand, stride, st)
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
        hipLaunchKernelGGL(k_dcollect, dim3((unsigned)((ncand + DC_CH - 1) / DC_CH), (unsigned)Tq,
                                             (unsigned)B),
                           dim3(DC_NT), 0, st, w, Tq, m, W, k, q_pos0, stride);
    }
    const size_t lds = sizeof(DselSmem);
    hipFuncSetAttribute((const void*)k_dfinal, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    hipLaunchKernelGGL(k_dfinal, dim3((unsigned)Tq, (unsigned)B), dim3(DL_NT), lds, st, w, topk, Tq,
                       m, W, k, q_pos0, stride);
    return hipGetLastError();
}

}  // namespace csa
