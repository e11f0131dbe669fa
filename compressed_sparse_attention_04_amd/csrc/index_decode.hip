// index_decode.hip -- Lightning Indexer for a few query rows over a long
// compressed context (decode): jiwasawa.github.io post, CSA indexer bullet
// (score every compressed entry, keep the top k); ai-papers.net, hybrid
// attention section (the FP4 indexer scans the already 4x shorter sequence).
//
// The FP4 key stream dominates (34 bytes per candidate at dI = 64), so it is
// read once, by many blocks, and no score goes back to HBM:
//   k_dscan : a block per (chunk of ch candidates, sequence) scores the
//             chunk for every row of the sequence (scaled FP4 MFMA) into
//             LDS, with each row's level-1 histogram.  Each row keeps a
//             threshold-closed list: every key >= tau, where tau is 0 (the
//             whole chunk fits the list's cap slots) or the upper edge of
//             the level-1 bin at which the list would overflow.  The list
//             (key, index) in ascending index order and (count, tau) go to
//             the workspace.
//   k_dmerge : a block per row selects the exact top k of the union U of
//             the row's lists.  That is the row's top k whenever every chunk
//             that left keys out has tau <= the k-th key of U: a key left
//             out is then below k keys of U, so it is not among the top k.
//             Otherwise (heavy ties, scores clustered in one chunk) the
//             block finds the top k exactly over all candidates, rescoring
//             the keys pass by pass (level-1 histogram, narrowed ranges,
//             collection).
// The order is the one used everywhere: score desc, index asc; the output
// lists the kept indices in ascending order, -1 padded.
#include "internal.h"
#include "mxfp4.h"
#include "select.h"
#include "wave_select.h"
#include "fp4_tiles.h"

namespace csa {

constexpr int DS_NT = 256;             // threads of a scanning block
constexpr int DS_UNR = 4;              // key tiles per load batch of a scanning wave
constexpr int DS_QT = 8;               // rows (queries x sequence) per sequence at most
constexpr int DS_KEYS = 8192;          // LDS key words of a scanning block (all its rows)
constexpr int DM_NT = 512;             // threads of a merging block
constexpr int DM_UCAP = 8192;          // union capacity (chunks x cap)
constexpr int DM_MAXW = 8192;          // bitmap words of the exact path -> 262144 candidates
constexpr int DM_CAP = 1024;           // collected keys of the exact path

// Chunk geometry of a launch: ch candidates per chunk (at most 4096; the
// rows' keys fill at most DS_KEYS words of LDS), nchunks chunks over the
// longest row, cap list slots per (row, chunk): a power of two near four
// times the expected share of the top k (k ch / ncand), at least 32, with
// nchunks * cap <= DM_UCAP.
struct DecodeGeom {
    int ch, nchunks, cap, ept;
};

__host__ __device__ __forceinline__ DecodeGeom decode_geom(int64_t Tq, int64_t ncand, int k) {
    DecodeGeom g;
    g.ch = Tq <= 2 ? 4096 : Tq <= 4 ? 2048 : 1024;
    g.nchunks = (int)((ncand + g.ch - 1) / g.ch);
    const int64_t want = 4 * (int64_t)k * g.ch / (ncand > 0 ? ncand : 1);
    int cap = 32;
    while (cap < want) cap *= 2;
    int lim = 1;                                     // largest power of two <= DM_UCAP / nchunks
    while (2 * lim * (g.nchunks > 0 ? g.nchunks : 1) <= DM_UCAP) lim *= 2;
    cap = cap < lim ? cap : lim;
    g.cap = cap < g.ch ? cap : g.ch;
    const int u = g.nchunks * g.cap;
    g.ept = u <= 4 * DM_NT ? 4 : u <= 8 * DM_NT ? 8 : u <= 16 * DM_NT ? 16 : 32;
    return g;
}

// Workspace: lists [rows][nchunks][cap] (key, index) | meta [rows][nchunks]
// (count, tau).  Nothing needs to start at any value.
__host__ __device__ __forceinline__ u32x2* ws_lists(void* ws) {
    return reinterpret_cast<u32x2*>(ws);
}
__host__ __device__ __forceinline__ u32x2* ws_meta(void* ws, int64_t rows, const DecodeGeom& g) {
    return reinterpret_cast<u32x2*>(ws) + rows * g.nchunks * g.cap;
}

// MXFP4 A operand of the lane's (query, head) row of an MFMA: rows
// (qi, h) = (row / HI, row % HI), 32-value block kb of its dI values
// (dI = 32 leaves block 1 zero); query qi of the tile is row q0 + qi.
template <typename T, int HI>
__device__ __forceinline__ void encode_q(const T* q_idx, RowStrides qs, int64_t b, int64_t q0,
                                         int qv, int dI, i32x8& aop, int& sa) {
    const int lane = threadIdx.x % WAVE, row = lane & 31, kb = lane >> 5;
    aop = i32x8{0, 0, 0, 0, 0, 0, 0, 0};
    sa = 127;
    const int qi = row / HI, h = row % HI;
    if (qi < qv && kb * 32 < dI) {
        const T* src = q_idx + b * qs.ss + (q0 + qi) * qs.rs + h * dI + kb * 32;
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

template <typename T, int HI, bool ONE>
__global__ void __launch_bounds__(DS_NT)
k_dscan(const T* __restrict__ q_idx, RowStrides qs, const uint8_t* __restrict__ kc,
        const uint8_t* __restrict__ ks, void* ws, int64_t Tq, int dI, int64_t Nc, int64_t m,
        int64_t W, int64_t q_pos0, DecodeGeom g) {
    extern __shared__ uint32_t smem[];               // keys [Tq][ch] | hist [Tq][SEL_NB]
    constexpr int NU = 16 / HI;
    constexpr int NWV = DS_NT / WAVE;
    const int ch = g.ch, cap = g.cap;
    const int cx = blockIdx.x;
    const int64_t c0 = (int64_t)cx * ch;
    const int64_t b = blockIdx.y;
    const int qv = (int)Tq;                          // Tq <= DS_QT on this path
    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
    const int row = lane & 31, kb = lane >> 5;
    uint32_t* keys = smem;
    uint32_t* hist = smem + qv * ch;
    __shared__ uint32_t s_tau[DS_QT];
    __shared__ int s_nv[DS_QT];
    __shared__ int s_wcnt[DS_QT][NWV];
    const int64_t nc_max = n_candidates(q_pos0 + qv - 1, m, W);
    const int nkeys = (int)min((int64_t)ch, nc_max - c0);   // >= 1: the grid covers nc_max
    // the first key batch of every wave is in flight during the set-up below
    const int kbytes = dI / 2, kscales = dI / 32;
    const TileSrc ts{kc + (b * Nc + c0) * kbytes, ks + (b * Nc + c0) * kscales, kbytes, kscales,
                     nkeys, row, kb};
    const int ntiles = (nkeys + 31) / 32;
    u32x4 kwA[DS_UNR];
    int ksA[DS_UNR];
    load_first<DS_NT, DS_UNR, true>(ts, ntiles, 1, kwA, ksA);
    for (int i = tid; i < qv * SEL_NB; i += DS_NT) hist[i] = 0u;

    i32x8 aop;
    int sa;
    encode_q<T, HI>(q_idx, qs, b, 0, qv, dI, aop, sa);
    // lane slot u of a tile holds the scores of query qslot[u]; slots from
    // nlive on hold no query of this launch
    const int nlive = live_slots<HI>(qv);
    const int kbq = kb * 4 / HI;
    int qslot[NU], nvq[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        const int gg = (u * HI) / 4, i = (u * HI) % 4;
        qslot[u] = (8 * gg + i) / HI + kbq;
        const int64_t nq = qslot[u] < qv ? n_candidates(q_pos0 + qslot[u], m, W) - c0 : 0;
        nvq[u] = (int)max((int64_t)0, min((int64_t)nkeys, nq));
    }
    __syncthreads();

    if constexpr (ONE) {
        // one query row (Tq = 1): tiles in pairs, 64 keys per pass (the ReLU head sum
        // in the order of score_key); nv0 for every lane (nvq holds it on
        // lanes 0-31 only)
        const int nv0 = (int)max((int64_t)0, min((int64_t)nkeys, n_candidates(q_pos0, m, W) - c0));
        stream_tile_pairs<DS_NT, DS_UNR, HI, true>(ts, ntiles, aop, sa, kwA, ksA,
                                                   [&](const float (&sc)[HI], int jj, bool ok) {
            float sum = __int_as_float(max(__float_as_int(sc[0]), 0));
#pragma unroll
            for (int hh = 1; hh < HI; ++hh) sum += __int_as_float(max(__float_as_int(sc[hh]), 0));
            const uint32_t key = __float_as_uint(sum);
            if (ok && jj < nkeys) {
                keys[jj] = key;
                if (jj < nv0) atomicAdd(&hist[lvl1_bin(key)], 1u);
            }
        });
    } else {
        stream_tiles_from<DS_NT, DS_UNR, true>(ts, ntiles, 1, aop, sa, kwA, ksA,
                                               [&](const f32x16& acc, int jt) {
            const int jj = jt + row;
            uint32_t key[NU];
            tile_keys<HI>(acc, key, nlive);
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                const int q = qslot[u];
                if (u >= nlive || q >= qv || jj >= nkeys) continue;
                keys[q * ch + jj] = key[u];
                if (jj < nvq[u]) atomicAdd(&hist[q * SEL_NB + lvl1_bin(key[u])], 1u);
            }
        });
    }
    __syncthreads();

    u32x2* meta = ws_meta(ws, Tq * gridDim.y, g);
    // per row: the list threshold (one wave per row)
    for (int q = wave; q < qv; q += NWV) {
        const int nv = (int)max((int64_t)0, min((int64_t)nkeys,
                                                n_candidates(q_pos0 + q, m, W) - c0));
        uint32_t tau = 0u;
        int cnt = nv;
        if (nv > cap) {
            int gt, in;
            const int d = wave_hist_find(hist + q * SEL_NB, cap + 1, &gt, &in);
            uint32_t lo, hi;
            lvl1_range(d, &lo, &hi);
            tau = hi;                                // bins above d: gt <= cap keys
            cnt = gt;
        }
        if (lane == 0) {
            s_tau[q] = tau;
            s_nv[q] = nv;
            meta[(b * Tq + q) * g.nchunks + cx] = u32x2{(uint32_t)cnt, tau};
        }
    }
    __syncthreads();
    // per row: the keys >= tau in index order -> the list (each wave takes a
    // contiguous quarter of the chunk; counts first, then positions)
    const int span = ch / NWV;                       // a multiple of WAVE
    const int j0 = wave * span;
    for (int q = 0; q < qv; ++q) {
        const uint32_t tau = s_tau[q];
        const int j1 = min(j0 + span, s_nv[q]);
        int c = 0;
        for (int jb = j0; jb < j1; jb += WAVE) {
            const int j = jb + lane;
            const bool take = j < j1 && keys[q * ch + j] >= tau;
            c += __popcll(__ballot(take));
        }
        if (lane == 0) s_wcnt[q][wave] = c;
    }
    __syncthreads();
    u32x2* lists = ws_lists(ws);
    for (int q = 0; q < qv; ++q) {
        const uint32_t tau = s_tau[q];
        const int j1 = min(j0 + span, s_nv[q]);
        int pos = 0;
        for (int w = 0; w < wave; ++w) pos += s_wcnt[q][w];
        u32x2* dst = lists + ((b * Tq + q) * g.nchunks + cx) * (int64_t)cap;
        for (int jb = j0; jb < j1; jb += WAVE) {
            const int j = jb + lane;
            const uint32_t key = j < j1 ? keys[q * ch + j] : 0u;
            const bool take = j < j1 && key >= tau;
            const uint64_t bal = __ballot(take);
            if (take) dst[pos + __popcll(bal & ((1ull << lane) - 1ull))] =
                u32x2{key, (uint32_t)(c0 + j)};
            pos += __popcll(bal);
        }
    }
}

// ---- the exact path of a merging block -------------------------------------
// The key of the need-th largest among n <= DM_NT / 2 keys cb[0..n-1][0]
// (LDS, any order) and how many keys equal to it are kept, from each key's
// exact rank: threads 2p and 2p + 1 count the keys above and equal to key p
// over the two halves of the list (16-byte broadcast reads, two keys each)
// and add their counts.  The value T with gt < need <= gt + eq is the
// need-th largest, and need - gt keys equal to it are kept; every thread
// holding a key equal to T writes the same T and need - gt.  The block
// synchronises before the results are read.  1 <= need <= n.
__device__ __forceinline__ void bin_rank_threshold(const u32x2* cb, int n, int need,
                                                   uint32_t* T_out, int* need_eq_out) {
    const int tid = threadIdx.x, p = tid >> 1, h = tid & 1;
    const uint32_t x = p < n ? cb[p][0] : 0u;
    const int npair = (n + 1) / 2, mid = (npair + 1) / 2;
    const int j0 = h ? mid : 0, j1 = h ? npair : mid;
    int gt = 0, eq = 0;
    // four pair reads in flight per round (indices clamped into the half,
    // the surplus masked)
    for (int jp = j0; jp < j1; jp += 4) {
        u32x4 w[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            w[u] = *reinterpret_cast<const u32x4*>(cb + 2 * min(jp + u, j1 - 1));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const bool v0 = jp + u < j1;
            const bool v1 = v0 && 2 * (jp + u) + 1 < n;  // entry n (odd n): not a key
            gt += (int)(v0 && w[u][0] > x) + (int)(v1 && w[u][2] > x);
            eq += (int)(v0 && w[u][0] == x) + (int)(v1 && w[u][2] == x);
        }
    }
    gt += __shfl_xor(gt, 1, WAVE);
    eq += __shfl_xor(eq, 1, WAVE);
    if (h == 0 && p < n && gt < need && need <= gt + eq) {
        *T_out = x;
        *need_eq_out = need - gt;
    }
}

struct DmSmem {
    SelectSmem sel_sm;
    uint32_t cnt[DM_UCAP / 32];      // list counts per chunk (nchunks <= DM_UCAP / 32)
    __attribute__((aligned(16))) uint32_t sel[DM_MAXW];
    __attribute__((aligned(16))) uint32_t eq[DM_MAXW];
    uint32_t hist[SEL_NB];
    __attribute__((aligned(16))) u32x2 cb[DM_CAP];
    uint32_t lo, hi, tau_thr;
    int above, in, ccnt, need_eq;
    int w_total[DM_NT / WAVE], w_ul[DM_NT / WAVE];
    uint32_t w_tau[DM_NT / WAVE];
    int scratch[DM_NT / WAVE + 1];
};

// Exact top `need` of the row's nc candidates by rescoring the keys
// (scan(fn) calls fn(key, j) once for every candidate j < nc, spread over the
// block).  Level 1 fixes a range of 2^17 keys (2^30 for bin 0, < 2^32 for
// bin 1023); each narrowing pass splits it into SEL_NB parts, so
// NARROW_PASSES passes always end with <= DM_CAP keys in range or a single
// key value.
template <typename Scan>
__device__ __forceinline__ void exact_select(Scan&& scan, int nc, int need, int32_t* out, int k,
                                             DmSmem& S) {
    static_assert(DM_MAXW % (8 * DM_NT) == 0, "merge-emit takes whole segments of 8 words per thread");
    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
    const int nw = (nc + 31) / 32;
    for (int i = tid; i < SEL_NB; i += DM_NT) S.hist[i] = 0u;
    __syncthreads();
    scan([&](uint32_t key, int j) { atomicAdd(&S.hist[lvl1_bin(key)], 1u); });
    __syncthreads();
    if (wave == 0) {
        int gt, in;
        const int d = wave_hist_find(S.hist, need, &gt, &in);
        uint32_t lo, hi;
        lvl1_range(d, &lo, &hi);
        if (lane == 0) {
            S.lo = lo;
            S.hi = hi;
            S.above = gt;
            S.in = in;
        }
    }
    __syncthreads();
#pragma unroll 1
    for (int it = 0; it < NARROW_PASSES; ++it) {
        const uint32_t lo = S.lo, hi = S.hi;
        if (S.in <= DM_CAP || hi - lo == 1u) break;
        const int sh = range_shift(lo, hi);
        __syncthreads();
        for (int i = tid; i < SEL_NB; i += DM_NT) S.hist[i] = 0u;
        __syncthreads();
        scan([&](uint32_t key, int j) {
            if (key >= lo && key < hi) atomicAdd(&S.hist[(key - lo) >> sh], 1u);
        });
        __syncthreads();
        if (wave == 0) {
            int gt, in;
            const int d = wave_hist_find(S.hist, need - S.above, &gt, &in);
            if (lane == 0) {
                S.lo = lo + ((uint32_t)d << sh);
                const uint64_t top = (uint64_t)lo + ((uint64_t)(d + 1) << sh);
                S.hi = top < (uint64_t)hi ? (uint32_t)top : hi;
                S.above += gt;
                S.in = in;
            }
        }
        __syncthreads();
    }
    // collect: keys above the range are kept; keys inside go to the buffer,
    // or, for a single-valued range with many ties, to the tie bitmap
    const uint32_t lo = S.lo, hi = S.hi;
    const bool eqmode = S.in > DM_CAP;
    for (int w = tid; w < DM_MAXW; w += DM_NT) {
        S.sel[w] = 0u;
        S.eq[w] = 0u;
    }
    if (tid == 0) S.ccnt = 0;
    __syncthreads();
    scan([&](uint32_t key, int j) {
        if (key >= hi) {
            atomicOr(&S.sel[j >> 5], 1u << (j & 31));
        } else if (key >= lo) {
            if (eqmode) {
                atomicOr(&S.eq[j >> 5], 1u << (j & 31));
            } else {
                const int pos = atomicAdd(&S.ccnt, 1);
                if (pos < DM_CAP) S.cb[pos] = u32x2{key, (uint32_t)j};
            }
        }
    });
    __syncthreads();
    if (wave == 0) {
        const int need_in = need - S.above;
        int need_eq = need_in;
        if (!eqmode) {
            const int n = min(S.ccnt, DM_CAP);
            constexpr int EPT = DM_CAP / WAVE;
            uint32_t key[EPT];
            bool valid[EPT];
#pragma unroll
            for (int e = 0; e < EPT; ++e) {
                const int p = e * WAVE + lane;
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
    block_merge_emit8<DM_NT>(S.sel, S.eq, nw, S.need_eq, out, k, S.scratch);
}

template <typename T, int HI, int EPT>
__global__ void __launch_bounds__(DM_NT)
k_dmerge(const T* __restrict__ q_idx, RowStrides qs, const uint8_t* __restrict__ kc,
         const uint8_t* __restrict__ ks, void* ws, int32_t* __restrict__ topk, int64_t Tq,
         int dI, int64_t Nc, int64_t m, int64_t W, int k, int64_t q_pos0, DecodeGeom g) {
    extern __shared__ __attribute__((aligned(16))) unsigned char smem_raw[];
    DmSmem& S = *reinterpret_cast<DmSmem*>(smem_raw);
    const int64_t q = blockIdx.x, b = blockIdx.y;
    const int64_t bq = b * Tq + q;
    const int tid = threadIdx.x;
    const int nc = (int)n_candidates(q_pos0 + q, m, W);
    const int need = min(nc, k);
    int32_t* out = topk + bq * k;
    if (nc <= k) {                                  // every candidate is kept
        for (int s = tid; s < k; s += DM_NT) out[s] = s < nc ? s : -1;
        return;
    }
    const int cap = g.cap, ch = g.ch;
    const int nchk = (nc + ch - 1) / ch;            // chunks holding this row's candidates
    const u32x2* meta = ws_meta(ws, Tq * gridDim.y, g) + bq * g.nchunks;
    const u32x2* lists = ws_lists(ws) + bq * g.nchunks * (int64_t)cap;
    // the union, EPT list slots per thread in (chunk, slot) order, i.e. in
    // ascending candidate index; keys + 1 (0: an empty slot)
    u32x2 ent[EPT];
#pragma unroll
    for (int e = 0; e < EPT; e += 2) {
        const int p = tid * EPT + e;
        const u32x4 v = p < nchk * cap ? *reinterpret_cast<const u32x4*>(lists + p)
                                       : u32x4{0u, 0u, 0u, 0u};
        ent[e] = u32x2{v[0], v[1]};
        ent[e + 1] = u32x2{v[2], v[3]};
    }
    // the chunks' (count, tau), loaded with the union (nchk <= DM_NT: at most
    // DM_UCAP / 32 chunks).  The union's size, the largest tau of a chunk
    // that left keys out and whether any did: wave reductions, one word
    // per wave in LDS (single-address LDS atomics from every thread cost
    // more than the rest of the merge)
    const u32x2 mt0 = tid < nchk ? meta[tid] : u32x2{0u, 0u};
    int w_tot = 0, w_ul = 0;
    uint32_t w_tau = 0u;
    for (int c = tid; c < nchk; c += DM_NT) {
        const u32x2 mt = c == tid ? mt0 : meta[c];
        S.cnt[c] = mt[0];
        const int nv = min(ch, nc - c * ch);
        w_tot += (int)mt[0];
        if ((int)mt[0] < nv) {                       // the chunk left keys out
            w_tau = max(w_tau, mt[1]);
            w_ul = 1;
        }
    }
    {
        const int wave = tid / WAVE;
        w_tot = wave_sum(w_tot);
        w_tau = wave_max_u32_sw(w_tau);
        const bool ul = __ballot(w_ul != 0) != 0;
        if (tid % WAVE == 0) {
            S.w_total[wave] = w_tot;
            S.w_tau[wave] = w_tau;
            S.w_ul[wave] = ul ? 1 : 0;
        }
    }
    __syncthreads();
    int total = 0, unlisted = 0;
    uint32_t tau_need = 0u;
#pragma unroll
    for (int w = 0; w < DM_NT / WAVE; ++w) {
        total += S.w_total[w];
        tau_need = max(tau_need, S.w_tau[w]);
        unlisted |= S.w_ul[w];
    }
    uint32_t key[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int p = tid * EPT + e;
        const int c = p / cap, s = p - c * cap;
        key[e] = c < nchk && s < (int)S.cnt[c] ? ent[e][0] + 1u : 0u;
    }
    // The k-th key of the union: its level-1 bin d from a histogram of the
    // union, then the keys of bin d (few, as a rule) resolved exactly by one
    // wave; a bin with more keys than the buffer takes the block-wide radix
    // search.  The selection is key > thr, or key == thr among the first
    // need_eq such keys in union order (= ascending candidate index).
    bool exact_needed = total < need;
    if (!exact_needed) {
        for (int i = tid; i < SEL_NB; i += DM_NT) S.hist[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < EPT; ++e)
            if (key[e]) atomicAdd(&S.hist[lvl1_bin(key[e] - 1u)], 1u);
        __syncthreads();
        if (tid < WAVE) {
            int gt, in;
            const int d = wave_hist_find(S.hist, need, &gt, &in);
            uint32_t lo, hi;
            lvl1_range(d, &lo, &hi);
            if (tid == 0) {
                S.lo = lo;
                S.hi = hi;
                S.above = gt;
                S.in = in;
            }
        }
        __syncthreads();
        uint32_t thr1;                               // threshold in key + 1 form
        int need_eq;
        if (S.in <= DM_CAP) {
            // the bin's keys, at offsets from a block prefix sum of the
            // threads' counts (a returning atomic on one LDS word costs a
            // round trip per slot and wave)
            const uint32_t lo = S.lo, hi = S.hi;
            uint32_t inb = 0u;
            int cnt = 0;
#pragma unroll
            for (int e = 0; e < EPT; ++e) {
                const uint32_t v = key[e] - 1u;
                if (key[e] && v >= lo && v < hi) {
                    inb |= 1u << e;
                    ++cnt;
                }
            }
            const int incl = wave_incl_scan(cnt);
            if (tid % WAVE == WAVE - 1) S.w_total[tid / WAVE] = incl;
            __syncthreads();
            int pos = incl - cnt;
            for (int w = 0; w < tid / WAVE; ++w) pos += S.w_total[w];
#pragma unroll
            for (int e = 0; e < EPT; ++e)
                if (inb & (1u << e)) S.cb[pos++] = u32x2{key[e] - 1u, 0u};
            __syncthreads();
            if (S.in <= DM_NT / 2) {
                // few keys in the bin (the rule): their exact ranks
                bin_rank_threshold(S.cb, S.in, need - S.above, &S.tau_thr, &S.need_eq);
            } else if (tid < WAVE) {
                constexpr int CE = DM_CAP / WAVE;
                uint32_t ck[CE];
                bool valid[CE];
#pragma unroll
                for (int e = 0; e < CE; ++e) {
                    const int p = e * WAVE + tid;
                    valid[e] = p < S.in;
                    ck[e] = valid[e] ? S.cb[p][0] : 0u;
                }
                uint32_t t;
                int ne;
                wave_radix_threshold<CE>(ck, valid, need - S.above, S.sel, &t, &ne);
                if (tid == 0) {
                    S.tau_thr = t;
                    S.need_eq = ne;
                }
            }
            __syncthreads();
            thr1 = S.tau_thr + 1u;
            need_eq = S.need_eq;
        } else {
            block_topk_threshold<DM_NT, EPT>(key, need, S.sel_sm, &thr1, &need_eq);
        }
        // thr1 - 1 is the k-th key of the union; every left-out key is < tau
        exact_needed = unlisted && thr1 - 1u < tau_need;
        if (!exact_needed) {
            int base, total;
            const uint32_t flags = block_select_flags<DM_NT, EPT>(key, thr1, need_eq, S.sel_sm,
                                                                 &base, &total);
#pragma unroll
            for (int e = 0; e < EPT; ++e)
                if (flags & (1u << e)) out[base++] = (int32_t)ent[e][1];
            for (int s = total + tid; s < k; s += DM_NT) out[s] = -1;
            return;
        }
    }
    // exact path: rescore every candidate of the row, pass by pass
    i32x8 aop;
    int sa;
    encode_q<T, HI>(q_idx, qs, b, q, 1, dI, aop, sa);
    const int lane = tid % WAVE, row = lane & 31, kb = lane >> 5;
    const int kbytes = dI / 2, kscales = dI / 32;
    const TileSrc ts{kc + b * Nc * kbytes, ks + b * Nc * kscales, kbytes, kscales, nc, row, kb};
    auto scan = [&](auto&& fn) {
        stream_tiles<DM_NT, 2>(ts, (nc + 31) / 32, 1, aop, sa, [&](const f32x16& acc, int jt) {
            // the row's HI head scores sit in slots 0..HI-1 of lanes 0-31
            const int j = jt + row;
            uint32_t key[1];
            tile_keys<HI>(acc, key);
            if (kb == 0 && j < nc) fn(key[0], j);
        });
    };
    __syncthreads();
    exact_select(scan, nc, need, out, k, S);
}

int decode_max_candidates() { return DM_MAXW * 32; }
int decode_max_rows() { return DS_QT; }

size_t decode_ws_bytes(int64_t B, int64_t Tq, int64_t ncap, int k) {
    const DecodeGeom g = decode_geom(Tq, ncap, k);
    const int64_t rows = B * Tq;
    return (size_t)(rows * g.nchunks * g.cap + rows * g.nchunks) * sizeof(u32x2);
}

template <typename T, int HI>
static void launch_decode_t(int64_t B, int64_t Tq, int dI, int64_t Nc, int64_t m, int64_t W,
                            int k, int64_t q_pos0, const void* q_idx, RowStrides qs,
                            const uint8_t* kc, const uint8_t* ks, int32_t* topk, void* ws,
                            const DecodeGeom& g, hipStream_t st) {
    const size_t lds_scan = (size_t)Tq * (g.ch + SEL_NB) * sizeof(uint32_t);
    if (Tq == 1)
        hipLaunchKernelGGL((k_dscan<T, HI, true>), dim3((unsigned)g.nchunks, (unsigned)B),
                           dim3(DS_NT), lds_scan, st, (const T*)q_idx, qs, kc, ks, ws, Tq, dI, Nc,
                           m, W, q_pos0, g);
    else
        hipLaunchKernelGGL((k_dscan<T, HI, false>), dim3((unsigned)g.nchunks, (unsigned)B),
                           dim3(DS_NT), lds_scan, st, (const T*)q_idx, qs, kc, ks, ws, Tq, dI, Nc,
                           m, W, q_pos0, g);
    const size_t lds = sizeof(DmSmem);
#define CSA_DM_CASE(E)                                                                       \
    do {                                                                                     \
        auto kern = k_dmerge<T, HI, E>;                                                      \
        hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize, \
                            (int)lds);                                                       \
        hipLaunchKernelGGL(kern, dim3((unsigned)Tq, (unsigned)B), dim3(DM_NT), lds, st,      \
                           (const T*)q_idx, qs, kc, ks, ws, topk, Tq, dI, Nc, m, W, k, q_pos0, \
                           g);                                                               \
    } while (0)
    if (g.ept == 4) CSA_DM_CASE(4);
    else if (g.ept == 8) CSA_DM_CASE(8);
    else if (g.ept == 16) CSA_DM_CASE(16);
    else CSA_DM_CASE(32);
#undef CSA_DM_CASE
}

hipError_t launch_index_decode(int dt, int64_t B, int64_t Tq, int HI, int dI, int64_t Nc,
                               int64_t m, int64_t W, int k, int64_t q_pos0, const void* q_idx,
                               RowStrides qs, const uint8_t* kc, const uint8_t* ks,
                               int32_t* topk, void* ws, hipStream_t st) {
    if (B == 0 || Tq == 0) return hipSuccess;
    const int64_t ncand = n_candidates(q_pos0 + Tq - 1, m, W);
    const DecodeGeom g = decode_geom(Tq, ncand, k);
#define CSA_DS_CASE(TT, HH) \
    launch_decode_t<TT, HH>(B, Tq, dI, Nc, m, W, k, q_pos0, q_idx, qs, kc, ks, topk, ws, g, st)
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
    return hipGetLastError();
}

}  // namespace csa
