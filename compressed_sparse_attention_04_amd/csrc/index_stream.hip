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
// Each row owns an 8 KB region of LDS, reused phase by phase (so two blocks
// share a CU and four waves share a SIMD).  Rows with enough candidates take
// the sampled path:
//   1. a level-1 histogram (1/64-octave bins) of every 8th key tile;
//   2. from the sample's rank statistics, a lower key bound lo that the k-th
//      key clears with a margin of 3 sigma + 4 sample ranks;
//   3. one pass over all keys: every key >= lo goes, with its candidate
//      index, to the wave's own segment of the row region (ballot
//      compaction, no shared counter);
//   4. if the segments hold at least k keys and none overflowed, the k-th
//      key is among them: its exact value, decided bit by bit with wave
//      ballots over the collected keys, finishes the row.
// Other rows, and any row whose check fails, run the exact multi-pass
// search: histogram passes narrow the range of the k-th key until it holds
// at most 256 keys (or one key value), then a collecting pass.  Either way
// ties at the threshold are resolved by candidate order and the kept set is
// read out of a candidate bitmap in ascending order.
#include <type_traits>
#include "internal.h"
#include "mxfp4.h"
#include "wave_select.h"
#include "fp4_tiles.h"

namespace csa {

constexpr int ST_NT = 512;             // 8 waves: one per query row at the decisions
constexpr int ST_NWV = ST_NT / WAVE;
constexpr int ST_QT = 8;               // query rows per block
constexpr int ST_MAXW = 1024;          // bitmap words per row -> 32768 candidates
constexpr int ST_RW = 2 * ST_MAXW;     // 32-bit words of a row's region
// sampled path: keys [ST_NWV][ST_SEG] from word 0, their candidate indices
// (16 bits) [ST_NWV][ST_SEG] from word ST_JOFF
constexpr int ST_SEG = 170;            // collected keys per row and wave
constexpr int ST_BUF = ST_SEG * ST_NWV;
constexpr int ST_JOFF = ST_BUF;
static_assert(ST_JOFF + (ST_BUF + 1) / 2 <= ST_RW, "sampled buffers fit the row region");
// multi-pass search: histogram at word 0; collection: kept bitmap at word 0,
// (key, index) pairs at word ST_MAXW, then the tie bitmap there; the read-out
// stages the kept indices there too
constexpr int ST_CAP = 256;            // collected keys per row (multi-pass search)
constexpr int ST_SAMPLE = 8;           // one key tile in ST_SAMPLE is sampled
constexpr int ST_SAMPLE_MIN = 2048;    // candidates a row needs for the sampled path
constexpr int ST_SAMPLE_MAXK = 768;    // and at most this many kept ones
constexpr int ST_UNR = 2;              // key tiles per wave and batch
// registers per lane of the sampled finish (a segment of up to 8 x that many
// collected keys)
constexpr int ST_FIN_EPT0 = 12, ST_FIN_EPT1 = 16, ST_FIN_EPT2 = (ST_SEG + 7) / 8;

enum : int { M_DONE = 0, M_HIST1 = 1, M_HIST = 2, M_COLLECT = 3, M_SAMPLED = 4 };

struct StreamSmem {
    uint32_t reg[ST_QT][ST_RW];        // one region per query row
    u32x4 aq[64];                      // MFMA A operand of lane kb*32 + row
    uint32_t as[64];                   // and its scale byte
    int segcnt[ST_QT][ST_NWV];
    uint32_t lo[ST_QT], hi[ST_QT];
    int shift[ST_QT], mode[ST_QT], above[ST_QT], need[ST_QT], cnt[ST_QT], eqmode[ST_QT];
    int nc[ST_QT];
    int any_active, any_sampled;
};

template <typename T, int HI>
__global__ void __launch_bounds__(ST_NT) __attribute__((amdgpu_waves_per_eu(4)))
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

    // ---- per-query setup
    if (tid < ST_QT) {
        const int nc = tid < qv ? (int)n_candidates(q_pos0 + q0 + tid, m, W) : 0;
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
        S.mode[tid] = (need == 0 || nc <= k)                          ? M_DONE
                      : (nc >= ST_SAMPLE_MIN && need <= ST_SAMPLE_MAXK) ? M_SAMPLED
                                                                        : M_HIST1;
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
        amax = max(amax, swizzle_xor<1>(amax));
        amax = max(amax, swizzle_xor<2>(amax));
        amax = max(amax, swizzle_xor<4>(amax));
        const int e = mxfp4_exponent(amax);
        const float p2e = pow2_neg(e);
        uint32_t c = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) c |= mxfp4_code(v[i], p2e) << (4 * i);
        const uint32_t c2 = swizzle_xor<1>(c);
        if (!(part & 1)) S.aq[bl][part >> 1] = c | (c2 << 16);
        if (part == 0) S.as[bl] = (uint32_t)(e + 127);
    }
    __syncthreads();
    // row regions: the kept bitmap of rows that keep every candidate, a zero
    // level-1 histogram for the others
    for (int q = 0; q < ST_QT; ++q) {
        const int nc = S.nc[q];
        const bool all = S.mode[q] == M_DONE;
        for (int w = tid; w < ST_MAXW; w += ST_NT) {
            uint32_t v = 0u;
            if (all) {
                const int lo_b = w * 32;
                v = lo_b + 32 <= nc ? 0xFFFFFFFFu : (lo_b >= nc ? 0u : ((1u << (nc - lo_b)) - 1u));
            }
            S.reg[q][w] = v;
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
    if (tid == 0) {
        int a = 0;
        for (int q = 0; q < ST_QT; ++q) a |= S.mode[q] == M_SAMPLED;
        S.any_sampled = a;
    }
    __syncthreads();

    const int ntiles = (nc_max + 31) / 32;
    const TileSrc ts{kc + b * Nc * (dI / 2), ks + b * Nc * (dI / 32), dI / 2, dI / 32, nc_max,
                     row, kb};

    // ================= sampled path
    if (S.any_sampled) {
        bool act[NU];
#pragma unroll
        for (int u = 0; u < NU; ++u) act[u] = qslot[u] < qv && S.mode[qslot[u]] == M_SAMPLED;
        // 1. level-1 histogram of the sampled tiles
        stream_tiles<ST_NT, ST_UNR>(ts, (ntiles + ST_SAMPLE - 1) / ST_SAMPLE, ST_SAMPLE, aop, sa,
                                    [&](const f32x16& acc, int j0) {
            const int j = j0 + row;
            uint32_t key[NU];
            tile_keys<HI>(acc, key);
#pragma unroll
            for (int u = 0; u < NU; ++u)
                if (act[u] && j < ncq[u]) atomicAdd(&S.reg[qslot[u]][lvl1_bin(key[u])], 1u);
        });
        __syncthreads();
        // 2. lower key bound of the k-th key, per sampled row (wave q)
        for (int q = wave; q < ST_QT; q += ST_NWV) {
            if (S.mode[q] != M_SAMPLED) continue;
            const int nc = S.nc[q], need = S.need[q];
            const int ns = (nc / (32 * ST_SAMPLE)) * 32 + min(32, nc % (32 * ST_SAMPLE));
            const float f = (float)ns / (float)nc;
            const float rt = (float)need * f;
            const float margin = 3.f * sqrtf(rt * (1.f - f)) + 4.f;
            const int need_lo = (int)ceilf(rt + margin);
            uint32_t klo = 0u;
            if (need_lo <= ns) {
                int gt, in;
                const int d = wave_hist_find(&S.reg[q][0], need_lo, &gt, &in);
                uint32_t h0;
                lvl1_range(d, &klo, &h0);
            }
            if (lane == 0) S.lo[q] = klo;
        }
        __syncthreads();
        // 3. one pass over every key: the keys >= lo, with their indices, go
        // to this wave's segment of their row's region
        // (a slot of no sampled row gets the bound KEY_END, which no key
        // reaches)
        uint32_t lo[NU];
        int cnt[NU];                    // lanes of half-wave kb count the keys of its row
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            lo[u] = act[u] ? S.lo[qslot[u]] : KEY_END;
            cnt[u] = 0;
        }
        // tiles below every row's candidate count need no per-lane bound
        int nc_min = S.nc[0];
        for (int q = 1; q < qv; ++q) nc_min = min(nc_min, S.nc[q]);
        nc_min = __builtin_amdgcn_readfirstlane(nc_min);
        auto collect = [&](const f32x16& acc, int j0, auto bounded) {
            const int j = j0 + row;
            uint32_t keys[NU];
            tile_keys<HI>(acc, keys);
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                // the 32 lanes of a half-wave hold the tile's 32 keys of one
                // query row; the two halves serve different rows
                bool hit = keys[u] >= lo[u];
                if constexpr (decltype(bounded)::value) hit = hit && j < ncq[u];
                const uint64_t bal = __ballot(hit);
                if (bal != 0ull) {
                    const uint32_t mine = kb ? (uint32_t)(bal >> 32) : (uint32_t)bal;
                    if (hit) {
                        const int pos = cnt[u] + __popc(mine & ((1u << row) - 1u));
                        if (pos < ST_SEG) {
                            uint32_t* r = &S.reg[qslot[u]][0];
                            r[wave * ST_SEG + pos] = keys[u];
                            reinterpret_cast<uint16_t*>(r + ST_JOFF)[wave * ST_SEG + pos] =
                                (uint16_t)j;
                        }
                    }
                    cnt[u] += __popc(mine);
                }
            }
        };
        stream_tiles<ST_NT, ST_UNR>(ts, ntiles, 1, aop, sa, [&](const f32x16& acc, int j0) {
            // j0 is the same on every lane: a scalar branch
            if (__builtin_amdgcn_readfirstlane(j0) + 32 <= nc_min)
                collect(acc, j0, std::false_type{});
            else collect(acc, j0, std::true_type{});
        });
#pragma unroll
        for (int u = 0; u < NU; ++u)
            if (row == 0 && act[u]) S.segcnt[qslot[u]][wave] = cnt[u];
        __syncthreads();
        // 4. check the counts and finish the row, or hand it to the search
        for (int q = wave; q < ST_QT; q += ST_NWV) {
            if (S.mode[q] != M_SAMPLED) continue;
            const int qnw = (S.nc[q] + 31) / 32;
            uint32_t* r = &S.reg[q][0];
            int nin = 0, over = 0;
            for (int w = 0; w < ST_NWV; ++w) {
                nin += S.segcnt[q][w];
                over |= S.segcnt[q][w] > ST_SEG;
            }
            const int need = S.need[q];
            if (nin >= need && !over) {
                // every key >= lo is collected and the k-th key is one of
                // them.  Lane l takes entries l / 8 + 8 e of segment l % 8,
                // so EPT registers cover segments of up to 8 EPT entries:
                // the smallest of three register counts that holds the
                // fullest segment is used.
                const int mycnt = S.segcnt[q][lane % ST_NWV];
                int maxc = 0;
                for (int w = 0; w < ST_NWV; ++w) maxc = max(maxc, S.segcnt[q][w]);
                const int rbase = (lane % ST_NWV) * ST_SEG + lane / ST_NWV;
                auto finish = [&](auto ept) {
                    constexpr int EPT = decltype(ept)::value;
                    uint32_t key[EPT], jj[EPT];
                    bool valid[EPT];
#pragma unroll
                    for (int e = 0; e < EPT; ++e) {
                        const int pos = 8 * e + lane / ST_NWV;
                        const int p = rbase + 8 * e;
                        valid[e] = pos < mycnt;
                        key[e] = valid[e] ? r[p] : 0u;
                        jj[e] = valid[e] ? reinterpret_cast<const uint16_t*>(r + ST_JOFF)[p] : 0u;
                    }
                    __builtin_amdgcn_wave_barrier();
                    uint32_t thr;
                    int need_eq;
                    wave_ballot_threshold<EPT>(key, valid, need, &thr, &need_eq);
                    // the region now holds the kept bitmap and the tie bitmap
                    for (int w = lane; w < qnw; w += WAVE) {
                        r[w] = 0u;
                        r[ST_MAXW + w] = 0u;
                    }
                    __builtin_amdgcn_wave_barrier();
#pragma unroll
                    for (int e = 0; e < EPT; ++e) {
                        if (!valid[e]) continue;
                        const uint32_t bit = 1u << (jj[e] & 31);
                        if (key[e] > thr) atomicOr(&r[jj[e] >> 5], bit);
                        else if (key[e] == thr) atomicOr(&r[ST_MAXW + (jj[e] >> 5)], bit);
                    }
                    __builtin_amdgcn_wave_barrier();
                    wave_merge_first_bits(r, r + ST_MAXW, qnw, need_eq);
                };
                static_assert(8 * ST_FIN_EPT2 >= ST_SEG, "the widest finish covers a segment");
                if (maxc <= 8 * ST_FIN_EPT0) finish(std::integral_constant<int, ST_FIN_EPT0>{});
                else if (maxc <= 8 * ST_FIN_EPT1) finish(std::integral_constant<int, ST_FIN_EPT1>{});
                else finish(std::integral_constant<int, ST_FIN_EPT2>{});
                if (lane == 0) S.mode[q] = M_DONE;
            } else {
                for (int w = lane; w < ST_MAXW; w += WAVE) r[w] = 0u;
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
    // (level 1, the narrowing passes, the collection) finish every row.  A
    // row's histogram is zero whenever it enters a histogram pass; its kept
    // bitmap (and, for a single key value, tie bitmap) is zero when it
    // enters the collection.  (Entered only by blocks with such rows: its
    // per-row state does not fit the registers next to the tile stream.)
    if (tid == 0) {
        int a = 0;
        for (int q = 0; q < ST_QT; ++q) a |= S.mode[q] != M_DONE;
        S.any_active = a;
    }
    __syncthreads();
    if (S.any_active) {
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
        __syncthreads();
        if (!S.any_active) break;

        stream_tiles<ST_NT, ST_UNR>(ts, ntiles, 1, aop, sa, [&](const f32x16& acc, int j0) {
            const int j = j0 + row;
            uint32_t keys[NU];
            tile_keys<HI>(acc, keys);
#pragma unroll
            for (int u = 0; u < NU; ++u) {
                if (md[u] == M_DONE || j >= ncq[u]) continue;
                const uint32_t key = keys[u];
                uint32_t* r = &S.reg[qslot[u]][0];
                if (md[u] == M_HIST1) {
                    atomicAdd(&r[lvl1_bin(key)], 1u);
                } else if (md[u] == M_HIST) {
                    if (key >= lo[u] && key < hi[u]) atomicAdd(&r[(key - lo[u]) >> sh[u]], 1u);
                } else {                                  // collect
                    if (key >= hi[u]) {
                        atomicOr(&r[j >> 5], 1u << (j & 31));
                    } else if (key >= lo[u]) {
                        if (eqm[u]) {
                            atomicOr(&r[ST_MAXW + (j >> 5)], 1u << (j & 31));
                        } else {
                            const int pos = atomicAdd(&S.cnt[qslot[u]], 1);
                            if (pos < ST_CAP)
                                reinterpret_cast<u32x2*>(r + ST_MAXW)[pos] = u32x2{key, (uint32_t)j};
                        }
                    }
                }
            }
        });
        __syncthreads();

        // ---- per-query decisions: wave w handles query w
        for (int q = wave; q < ST_QT; q += ST_NWV) {
            const int mode = S.mode[q];
            const int qnw = (S.nc[q] + 31) / 32;
            uint32_t* r = &S.reg[q][0];
            if (mode == M_HIST1 || mode == M_HIST) {
                const int rem = S.need[q] - S.above[q];
                int gt, in;
                const int d = wave_hist_find(r, rem, &gt, &in);
                uint32_t nlo, nhi;
                if (mode == M_HIST1) {
                    lvl1_range(d, &nlo, &nhi);
                } else {
                    nlo = S.lo[q] + ((uint32_t)d << S.shift[q]);
                    uint64_t top = (uint64_t)S.lo[q] + ((uint64_t)(d + 1) << S.shift[q]);
                    nhi = top < (uint64_t)S.hi[q] ? (uint32_t)top : S.hi[q];
                }
                const bool single = nhi - nlo == 1u;
                const bool collect = in <= ST_CAP || single;
                const bool eq = single && in > ST_CAP;
                __builtin_amdgcn_wave_barrier();
                // the next pass's zero histogram, or zero bitmaps for the collection
                for (int w = lane; w < ST_MAXW; w += WAVE) r[w] = 0u;
                if (eq)
                    for (int w = lane; w < ST_MAXW; w += WAVE) r[ST_MAXW + w] = 0u;
                if (lane == 0) {
                    S.above[q] += gt;
                    S.lo[q] = nlo;
                    S.hi[q] = nhi;
                    if (collect) {
                        S.mode[q] = M_COLLECT;
                        S.eqmode[q] = eq;
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
                    uint32_t key[EPT], jj[EPT];
                    bool valid[EPT];
#pragma unroll
                    for (int e = 0; e < EPT; ++e) {
                        const int p = e * WAVE + lane;
                        valid[e] = p < n;
                        const u32x2 v = valid[e] ? reinterpret_cast<const u32x2*>(r + ST_MAXW)[p]
                                                 : u32x2{0u, 0u};
                        key[e] = v[0];
                        jj[e] = v[1];
                    }
                    __builtin_amdgcn_wave_barrier();
                    uint32_t thr;
                    wave_ballot_threshold<EPT>(key, valid, need_in, &thr, &need_eq);
                    for (int w = lane; w < qnw; w += WAVE) r[ST_MAXW + w] = 0u;
                    __builtin_amdgcn_wave_barrier();
#pragma unroll
                    for (int e = 0; e < EPT; ++e) {
                        if (!valid[e]) continue;
                        const uint32_t bit = 1u << (jj[e] & 31);
                        if (key[e] > thr) atomicOr(&r[jj[e] >> 5], bit);
                        else if (key[e] == thr) atomicOr(&r[ST_MAXW + (jj[e] >> 5)], bit);
                    }
                    __builtin_amdgcn_wave_barrier();
                }
                wave_merge_first_bits(r, r + ST_MAXW, qnw, need_eq);
                if (lane == 0) S.mode[q] = M_DONE;
            }
        }
        __syncthreads();
    }
    }

    // ---- read out: wave w writes query w (through the free half of its
    // region when k fits there)
    for (int q = wave; q < qv; q += ST_NWV) {
        const int nc = S.nc[q];
        int32_t* out = topk + (b * Tq + q0 + q) * k;
        if (k <= ST_MAXW)
            wave_emit_bitmap_staged(&S.reg[q][0], (nc + 31) / 32,
                                    reinterpret_cast<int32_t*>(&S.reg[q][ST_MAXW]), out, k);
        else
            wave_emit_bitmap(&S.reg[q][0], (nc + 31) / 32, out, k);
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
