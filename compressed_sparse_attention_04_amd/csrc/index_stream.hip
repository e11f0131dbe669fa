// index_stream.hip -- Lightning Indexer with streaming exact top-k, for
// query tiles whose candidates fit one block (jiwasawa.github.io post, CSA
// indexer bullet: per query token, score every compressed entry and keep the
// top k; studioglobal.ai answer: FP4 indexer, k = 512).
//
//   I(t, j) = sum_{h < HI} max(0, qhat[t][h] . khat[j])
//
// One block owns 8 query rows and streams their candidates in tiles of 32
// keys; every pass recomputes the FP4 scores on the scaled MFMA (cheaper
// than keeping 8 x 32K fp32 scores anywhere).  Key order: fp32 bits of the
// score, larger first, ties to the lower candidate index.
//
// Rows with enough candidates take the sampled path:
//   1. a level-1 histogram (1/64-octave bins) of every 8th key tile;
//   2. from the sample's rank statistics, a key range [lo, hi) that holds
//      the k-th key with a margin of 3 sigma + 4 sample ranks each side;
//   3. one pass over all keys: keys >= hi go to the kept bitmap, keys in
//      [lo, hi) to the wave's own segment of a buffer (ballot compaction,
//      no shared counter);
//   4. if the counts prove that the k-th key lies in the buffer (kept < k
//      <= kept + buffered, no overflow), an exact radix threshold over the
//      buffer finishes the row.
// Other rows, and any row whose check fails, run the exact multi-pass
// search: histogram passes narrow the range of the k-th key until it holds
// at most 256 keys (or one key value), then a collecting pass.  Either way
// ties at the threshold are resolved by candidate order and the kept set is
// read out of the bitmap in ascending order.
#include "internal.h"
#include "mxfp4.h"
#include "wave_select.h"
#include "fp4_tiles.h"

namespace csa {

constexpr int ST_NT = 512;             // 8 waves: one per query row at the decisions
constexpr int ST_QT = 8;               // query rows per block
constexpr int ST_CAP = 256;            // collected keys per row (multi-pass search)
constexpr int ST_SEG = 96;             // buffered keys per row and wave (sampled path)
constexpr int ST_BUF = ST_SEG * (ST_NT / WAVE);
constexpr int ST_MAXW = 1024;          // bitmap words per row -> 32768 candidates
constexpr int ST_SAMPLE = 8;           // one key tile in ST_SAMPLE is sampled
constexpr int ST_SAMPLE_MIN = 2048;    // candidates a row needs for the sampled path
// key tiles per wave and batch (two batches and two tiles' scores are live)
template <int HI> constexpr int st_unr() { return 4; }

enum : int { M_DONE = 0, M_HIST1 = 1, M_HIST = 2, M_COLLECT = 3, M_SAMPLED = 4 };

struct StreamSmem {
    uint32_t sel[ST_QT][ST_MAXW];      // kept candidates
    uint32_t hist[ST_QT][SEL_NB];      // histograms; radix scratch
    uint32_t eq[ST_QT][ST_MAXW];       // candidates equal to the threshold key
    u32x2 buf[ST_QT][ST_BUF];          // (key, index): one segment per wave (sampled
                                       // path); the first ST_CAP: multi-pass buffer
    int segcnt[ST_QT][ST_NT / WAVE];
    u32x4 aq[64];                      // MFMA A operand of lane kb*32 + row
    uint32_t as[64];                   // and its scale byte
    uint32_t lo[ST_QT], hi[ST_QT];
    int shift[ST_QT], mode[ST_QT], above[ST_QT], need[ST_QT], cnt[ST_QT], eqmode[ST_QT];
    int nc[ST_QT];
    int any_active, any_sampled;
};

template <typename T, int HI>
__global__ void __launch_bounds__(ST_NT)
k_index_stream(const T* __restrict__ q_idx, RowStrides qs, const uint8_t* __restrict__ kc,
               const uint8_t* __restrict__ ks, int32_t* __restrict__ topk, int64_t Tq, int dI,
               int64_t Nc, int64_t m, int64_t W, int k, int64_t q_pos0) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    StreamSmem& S = *reinterpret_cast<StreamSmem*>(smem_raw);
    constexpr int NU = 16 / HI;                     // query slots per lane in an MFMA tile

    // the longest row groups (latest queries, most candidates) go first, so
    // the kernel's last blocks are its shortest
    const int64_t q0 = (int64_t)(gridDim.x - 1 - blockIdx.x) * ST_QT;
    const int64_t b = blockIdx.y;
    const int qv = (int)min((int64_t)ST_QT, Tq - q0);
    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
    const int row = lane & 31, kb = lane >> 5;
    const int nc_max = (int)n_candidates(q_pos0 + q0 + qv - 1, m, W);
    const int nw = (nc_max + 31) / 32;

    // ---- per-query setup
    if (tid < ST_QT) {
        const int nc = tid < qv ? (int)n_candidates(q_pos0 + q0 + tid, m, W) : 0;
        for (int w = 0; w < ST_NT / WAVE; ++w) S.segcnt[tid][w] = 0;
        const int need = min(nc, k);
        S.nc[tid] = nc;
        S.need[tid] = need;
        S.above[tid] = 0;
        S.cnt[tid] = 0;
        S.eqmode[tid] = 0;
        S.lo[tid] = 0u;
        S.hi[tid] = KEY_END;
        S.shift[tid] = 0;
        // all candidates kept when there are at most k of them
        S.mode[tid] = (need == 0 || nc <= k) ? M_DONE
                      : nc >= ST_SAMPLE_MIN ? M_SAMPLED : M_HIST1;
    }
    // ---- MXFP4 of the query rows, once per block: 8 threads per 32-value
    // block (lane kb*32 + row of the MFMA A operand: query row / HI, head
    // row % HI, dims kb*32..), 4 values each, staged in LDS
    static_assert(ST_NT == 64 * 8, "one 32-value block per 8 threads");
    {
        const int bl = tid >> 3, part = tid & 7;
        const int brow = bl & 31, bkb = bl >> 5;
        const int qi = brow / HI, h = brow % HI;
        float v[4] = {0.f, 0.f, 0.f, 0.f};
        if (qi < qv && bkb * 32 < dI)
            Elem<T>::load4(q_idx + b * qs.ss + (q0 + qi) * qs.rs + h * dI + bkb * 32 + part * 4,
                           v);
        uint32_t amax = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) amax = max(amax, __float_as_uint(v[i]) & 0x7fffffffu);
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) amax = max(amax, (uint32_t)__shfl_xor((int)amax, o, WAVE));
        const int e = mxfp4_exponent(amax);
        const float p2e = pow2_neg(e);
        uint32_t c = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) c |= mxfp4_code(v[i], p2e) << (4 * i);
        const uint32_t c2 = (uint32_t)__shfl_xor((int)c, 1, WAVE);
        if (!(part & 1)) S.aq[bl][part >> 1] = c | (c2 << 16);
        if (part == 0) S.as[bl] = (uint32_t)(e + 127);
    }
    __syncthreads();
    for (int q = 0; q < ST_QT; ++q) {
        const int nc = S.nc[q];
        for (int w = tid; w < nw; w += ST_NT) {
            // queries with nc <= k keep every candidate
            uint32_t full = 0u;
            if (nc <= k) {
                const int lo_b = w * 32;
                full = lo_b + 32 <= nc ? 0xFFFFFFFFu
                                       : (lo_b >= nc ? 0u : ((1u << (nc - lo_b)) - 1u));
            }
            S.sel[q][w] = full;
            S.eq[q][w] = 0u;
        }
    }
    const u32x4 aw = S.aq[kb * 32 + row];
    const i32x8 aop = {(int)aw[0], (int)aw[1], (int)aw[2], (int)aw[3], 0, 0, 0, 0};
    const int sa = (int)S.as[kb * 32 + row];
    // the queries this lane's MFMA output rows belong to
    const int kbq = kb * 4 / HI;
    int qslot[NU];
    int ncq[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int g = (u * HI) / 4, i = (u * HI) % 4;
        const int qi = (8 * g + i) / HI + kbq;
        qslot[u] = qi;
        ncq[u] = (qi < qv) ? S.nc[qi] : 0;
    }
    __syncthreads();

    const int ntiles = (nc_max + 31) / 32;
    const TileSrc ts{kc + b * Nc * (dI / 2), ks + b * Nc * (dI / 32), dI / 2, dI / 32, nc_max,
                     row, kb};

    // ================= sampled path
    if (tid == 0) {
        int a = 0;
        for (int q = 0; q < ST_QT; ++q) a |= S.mode[q] == M_SAMPLED;
        S.any_sampled = a;
    }
    for (int i = tid; i < ST_QT * SEL_NB; i += ST_NT) (&S.hist[0][0])[i] = 0u;
    __syncthreads();
    if (S.any_sampled) {
        bool act[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) act[u] = qslot[u] < qv && S.mode[qslot[u]] == M_SAMPLED;
        // 1. level-1 histogram of the sampled tiles
        stream_tiles<ST_NT, st_unr<HI>()>(ts, (ntiles + ST_SAMPLE - 1) / ST_SAMPLE, ST_SAMPLE, aop, sa,
                     [&](const f32x16& acc, int j0) {
            const int j = j0 + row;
            uint32_t key[NU];
            tile_keys<HI>(acc, key);
#pragma unroll
            for (int u = 0; u < NU; ++u)
                if (act[u] && j < ncq[u])
                    atomicAdd(&S.hist[qslot[u]][lvl1_bin(key[u])], 1u);
        });
        __syncthreads();
        // 2. key range of the k-th key, per sampled row (wave q)
        for (int q = wave; q < ST_QT; q += ST_NT / WAVE) {
            if (S.mode[q] != M_SAMPLED) continue;
            const int nc = S.nc[q], need = S.need[q];
            const int ns = (nc / (32 * ST_SAMPLE)) * 32 + min(32, nc % (32 * ST_SAMPLE));
            const float f = (float)ns / (float)nc;
            const float rt = (float)need * f;
            const float margin = 3.f * sqrtf(rt * (1.f - f)) + 4.f;
            const int need_hi = (int)floorf(rt - margin);
            const int need_lo = (int)ceilf(rt + margin);
            uint32_t khi = KEY_END, klo = 0u;
            int gt, in;
            if (need_hi >= 1) {
                const int d = wave_hist_find(&S.hist[q][0], need_hi, &gt, &in);
                uint32_t l0, h0;
                lvl1_range(d, &l0, &h0);
                khi = h0;
            }
            if (need_lo <= ns) {
                const int d = wave_hist_find(&S.hist[q][0], need_lo, &gt, &in);
                uint32_t l0, h0;
                lvl1_range(d, &l0, &h0);
                klo = l0;
            }
            if (lane == 0) {
                S.lo[q] = klo;
                S.hi[q] = khi;
                S.cnt[q] = 0;
            }
        }
        __syncthreads();
        // 3. one pass over every key
        uint32_t lo[NU], hi[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int q = qslot[u] < ST_QT ? qslot[u] : 0;
            lo[u] = S.lo[q];
            hi[u] = S.hi[q];
        }
        int wc0[NU], wc1[NU];           // this wave's segment counts, half-waves 0 / 1
#pragma unroll
        for (int u = 0; u < NU; ++u) wc0[u] = wc1[u] = 0;
        stream_tiles<ST_NT, st_unr<HI>()>(ts, ntiles, 1, aop, sa, [&](const f32x16& acc, int j0) {
            const int j = j0 + row;
            uint32_t keys[NU];
            tile_keys<HI>(acc, keys);
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const bool ok = act[u] && j < ncq[u];
                const uint32_t key = keys[u];
                const bool above = ok && key >= hi[u];
                const bool in = ok && !above && key >= lo[u];
                const int q = qslot[u] < ST_QT ? qslot[u] : 0;
                // the 32 lanes of a half-wave hold the tile's 32 keys of
                // one query, and each bitmap word is written by one tile
                // only (sel starts at zero for sampled rows)
                const uint64_t bab = __ballot(above);
                if (row == 0 && act[u]) S.sel[q][j0 >> 5] = kb ? (uint32_t)(bab >> 32) : (uint32_t)bab;
                const uint64_t bin = __ballot(in);
                if (bin != 0ull) {
                    const uint32_t h0 = (uint32_t)bin, h1 = (uint32_t)(bin >> 32);
                    if (in) {
                        const uint32_t mine = kb ? h1 : h0;
                        const int pos = (kb ? wc1[u] : wc0[u]) +
                                        __popc(mine & ((1u << row) - 1u));
                        if (pos < ST_SEG)
                            S.buf[q][wave * ST_SEG + pos] = u32x2{key, (uint32_t)j};
                    }
                    wc0[u] += __popc(h0);
                    wc1[u] += __popc(h1);
                }
            }
        });
#pragma unroll
        for (int u = 0; u < NU; ++u)
            if (row == 0 && act[u]) S.segcnt[qslot[u]][wave] = kb ? wc1[u] : wc0[u];
        __syncthreads();
        // 4. check the counts and finish the row, or hand it to the search
        for (int q = wave; q < ST_QT; q += ST_NT / WAVE) {
            if (S.mode[q] != M_SAMPLED) continue;
            const int qnw = (S.nc[q] + 31) / 32;
            int c = 0;
            for (int w = lane; w < qnw; w += WAVE) c += __popc(S.sel[q][w]);
            const int kept = wave_sum(c);
            int nin = 0, over = 0;
            for (int w = 0; w < ST_NT / WAVE; ++w) {
                nin += S.segcnt[q][w];
                over |= S.segcnt[q][w] > ST_SEG;
            }
            const int need = S.need[q];
            if (kept < need && kept + nin >= need && !over) {
                constexpr int EPT = ST_BUF / WAVE;
                uint32_t key[EPT];
                bool valid[EPT];
#pragma unroll
                for (int e = 0; e < EPT; ++e) {
                    const int p = lane * EPT + e;
                    valid[e] = p % ST_SEG < S.segcnt[q][p / ST_SEG];
                    key[e] = valid[e] ? S.buf[q][p][0] : 0u;
                }
                uint32_t thr;
                int need_eq;
                wave_radix_threshold<EPT>(key, valid, need - kept, &S.hist[q][0], &thr, &need_eq);
#pragma unroll
                for (int e = 0; e < EPT; ++e) {
                    if (!valid[e]) continue;
                    const uint32_t j = S.buf[q][lane * EPT + e][1];
                    if (key[e] > thr) atomicOr(&S.sel[q][j >> 5], 1u << (j & 31));
                    else if (key[e] == thr) atomicOr(&S.eq[q][j >> 5], 1u << (j & 31));
                }
                __builtin_amdgcn_wave_barrier();
                wave_merge_first_bits(&S.sel[q][0], &S.eq[q][0], qnw, need_eq);
                if (lane == 0) S.mode[q] = M_DONE;
            } else {
                for (int w = lane; w < qnw; w += WAVE) S.sel[q][w] = 0u;
                if (lane == 0) {
                    S.mode[q] = M_HIST1;
                    S.lo[q] = 0u;
                    S.hi[q] = KEY_END;
                    S.cnt[q] = 0;
                }
            }
        }
        __syncthreads();
    }

    // ================= exact multi-pass search for the remaining rows: every
    // row still searching starts at level 1 here, so EXACT_PASSES passes
    // (level 1, the narrowing passes, the collection) finish every row
#pragma unroll 1
    for (int pass = 0; pass < EXACT_PASSES; ++pass) {
        // per-slot state of this pass (registers)
        int md[NU], sh[NU];
        uint32_t lo[NU], hi[NU];
        bool eqm[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            const int q = qslot[u] < ST_QT ? qslot[u] : 0;
            md[u] = qslot[u] < qv ? S.mode[q] : M_DONE;
            sh[u] = S.shift[q];
            lo[u] = S.lo[q];
            hi[u] = S.hi[q];
            eqm[u] = S.eqmode[q] != 0;
        }
        if (tid == 0) {
            int a = 0;
            for (int q = 0; q < ST_QT; ++q) a |= S.mode[q] != M_DONE;
            S.any_active = a;
        }
        for (int i = tid; i < ST_QT * SEL_NB; i += ST_NT) (&S.hist[0][0])[i] = 0u;
        __syncthreads();
        if (!S.any_active) break;

        stream_tiles<ST_NT, st_unr<HI>()>(ts, ntiles, 1, aop, sa, [&](const f32x16& acc, int j0) {
            const int j = j0 + row;
            uint32_t keys[NU];
            tile_keys<HI>(acc, keys);
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                if (md[u] == M_DONE || j >= ncq[u]) continue;
                const uint32_t key = keys[u];
                const int q = qslot[u];
                if (md[u] == M_HIST1) {
                    atomicAdd(&S.hist[q][lvl1_bin(key)], 1u);
                } else if (md[u] == M_HIST) {
                    if (key >= lo[u] && key < hi[u])
                        atomicAdd(&S.hist[q][(key - lo[u]) >> sh[u]], 1u);
                } else {                                  // collect
                    if (key >= hi[u]) {
                        atomicOr(&S.sel[q][j >> 5], 1u << (j & 31));
                    } else if (key >= lo[u]) {
                        if (eqm[u]) {
                            atomicOr(&S.eq[q][j >> 5], 1u << (j & 31));
                        } else {
                            int pos = atomicAdd(&S.cnt[q], 1);
                            if (pos < ST_CAP) S.buf[q][pos] = u32x2{key, (uint32_t)j};
                        }
                    }
                }
            }
        });
        __syncthreads();

        // ---- per-query decisions: wave w handles query w
        for (int q = wave; q < ST_QT; q += ST_NT / WAVE) {
            const int mode = S.mode[q];
            if (mode == M_HIST1 || mode == M_HIST) {
                const int rem = S.need[q] - S.above[q];
                int gt, in;
                const int d = wave_hist_find(&S.hist[q][0], rem, &gt, &in);
                uint32_t nlo, nhi;
                if (mode == M_HIST1) {
                    lvl1_range(d, &nlo, &nhi);
                } else {
                    nlo = S.lo[q] + ((uint32_t)d << S.shift[q]);
                    uint64_t top = (uint64_t)S.lo[q] + ((uint64_t)(d + 1) << S.shift[q]);
                    nhi = top < (uint64_t)S.hi[q] ? (uint32_t)top : S.hi[q];
                }
                if (lane == 0) {
                    S.above[q] += gt;
                    S.lo[q] = nlo;
                    S.hi[q] = nhi;
                    const bool single = nhi - nlo == 1u;
                    if (in <= ST_CAP || single) {
                        S.mode[q] = M_COLLECT;
                        S.eqmode[q] = single && in > ST_CAP;
                        S.cnt[q] = 0;
                    } else {
                        S.mode[q] = M_HIST;
                        S.shift[q] = range_shift(nlo, nhi);
                    }
                }
            } else if (mode == M_COLLECT) {
                const int need_in = S.need[q] - S.above[q];
                int need_eq;
                if (S.eqmode[q]) {
                    need_eq = need_in;
                } else {
                    // exact threshold among the collected keys
                    const int n = min(S.cnt[q], ST_CAP);
                    constexpr int EPT = ST_CAP / WAVE;
                    uint32_t key[EPT];
                    bool valid[EPT];
#pragma unroll
                    for (int e = 0; e < EPT; ++e) {
                        const int p = lane * EPT + e;
                        valid[e] = p < n;
                        key[e] = valid[e] ? S.buf[q][p][0] : 0u;
                    }
                    uint32_t thr;
                    wave_radix_threshold<EPT>(key, valid, need_in, &S.hist[q][0], &thr, &need_eq);
#pragma unroll
                    for (int e = 0; e < EPT; ++e) {
                        if (!valid[e]) continue;
                        const uint32_t j = S.buf[q][lane * EPT + e][1];
                        if (key[e] > thr) atomicOr(&S.sel[q][j >> 5], 1u << (j & 31));
                        else if (key[e] == thr) atomicOr(&S.eq[q][j >> 5], 1u << (j & 31));
                    }
                    __builtin_amdgcn_wave_barrier();
                }
                wave_merge_first_bits(&S.sel[q][0], &S.eq[q][0], nw, need_eq);
                if (lane == 0) S.mode[q] = M_DONE;
            }
        }
        __syncthreads();
    }

    // ---- read out: wave w writes query w
    for (int q = wave; q < qv; q += ST_NT / WAVE) {
        const int nc = S.nc[q];
        wave_emit_bitmap(&S.sel[q][0], (nc + 31) / 32, topk + (b * Tq + q0 + q) * k, k);
    }
}

size_t stream_smem_bytes() { return sizeof(StreamSmem); }
int stream_max_candidates() { return ST_MAXW * 32; }

template <typename T, int HI>
static hipError_t launch_stream_t(int64_t B, int64_t Tq, int dI, int64_t Nc, int64_t m,
                                  int64_t W, int k, int64_t q_pos0, const void* q_idx,
                                  RowStrides qs, const uint8_t* kc, const uint8_t* ks,
                                  int32_t* topk, hipStream_t st) {
    auto kern = k_index_stream<T, HI>;
    const size_t lds = sizeof(StreamSmem);
    hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    dim3 grid((unsigned)((Tq + ST_QT - 1) / ST_QT), (unsigned)B);
    hipLaunchKernelGGL(kern, grid, dim3(ST_NT), lds, st, (const T*)q_idx, qs, kc, ks, topk, Tq,
                       dI, Nc, m, W, k, q_pos0);
    return hipGetLastError();
}

hipError_t launch_index_stream(int dt, int64_t B, int64_t Tq, int HI, int dI, int64_t Nc,
                               int64_t m, int64_t W, int k, int64_t q_pos0, const void* q_idx,
                               RowStrides qs, const uint8_t* kc, const uint8_t* ks,
                               int32_t* topk, hipStream_t st) {
    if (B == 0 || Tq == 0) return hipSuccess;
#define CSA_ST_CASE(TT, HH) \
    return launch_stream_t<TT, HH>(B, Tq, dI, Nc, m, W, k, q_pos0, q_idx, qs, kc, ks, topk, st)
    if (dt == 0) {
        if (HI == 1) CSA_ST_CASE(float, 1);
        if (HI == 2) CSA_ST_CASE(float, 2);
        CSA_ST_CASE(float, 4);
    }
    if (HI == 1) CSA_ST_CASE(uint16_t, 1);
    if (HI == 2) CSA_ST_CASE(uint16_t, 2);
    CSA_ST_CASE(uint16_t, 4);
#undef CSA_ST_CASE
}

}  // namespace csa
