// attend.hip -- shared-KV multi-query attention over compressed entries
// joined with the raw sliding window (jiwasawa.github.io post: CSA "Shared
// Key-Value MQA" over the selected entries, HCA dense attention over every
// compressed entry, and the SWA branch over the newest tokens;
// studioglobal.ai answer: the 128-token window branch is always present).
//
// For the query at position t the key list is
//   [ kept (CSA) or all (HCA) compressed candidates | raw tokens w0..t ]
// and one softmax runs over it.  All H query heads share the one K/V head,
// so the H heads are a dimension of the bf16 MFMAs and every K/V row is
// fetched once per query token for all heads.
//
// bf16 kernel, per block: one query token (all H = 32 * NW heads, one wave
// per 32 heads) and one split of its key list, in tiles of 32 keys that
// never mix the two sources.  K and V rows are copied straight into LDS
// (global_load_lds) three tiles ahead of use.  Per tile and wave:
//   S^T = K Q^T          (8 x V_MFMA_F32_32X32X16_BF16, K rows from LDS,
//                         Q^T in registers) -> each lane owns one head
//   online softmax in fp32 (exp2 domain) with lazy rescaling
//   O^T += V^T P^T       (P^T straight from the S^T registers as bf16; V^T
//                         by transposing LDS reads, ds_read_b64_tr_b16)
// With more than one split each split's normalised output (bf16) and its
// (max, sum) go to the workspace and k_attend_combine merges them
// (log-sum-exp weights).
#include "common.h"
#include "internal.h"
#include "attend_common.h"

namespace csa {

constexpr int ATT_KT = 32;       // keys per tile of the bf16 kernel
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

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

// Key rows of one tile are copied straight from global memory into LDS
// (global_load_lds, 16 bytes per lane, lane-contiguous).  A row of D bf16 is
// CH = D/8 chunks of 16 bytes; chunk c of tile row r sits in slot
// c ^ f(r) (row_swz below) so that the rows read together by one operand
// load hit different LDS banks.
template <int D>
struct TileGeom {
    static constexpr int KT = 32;                   // keys per tile
    static constexpr int NST = 4;                   // LDS stages (3 tiles in flight)
    static constexpr int CH = D / 8;                // 16-byte chunks per row
    static constexpr int ROWB = D * 2;              // bytes per row
    static constexpr int RPI = 64 / CH;             // rows per wave-wide copy
    static constexpr int NINS = KT / RPI;           // wave-wide copies per tile and tensor
    static constexpr int BYTES = KT * ROWB;         // bytes per tile and tensor
};

// Swizzle of row r, chunk c -> slot c ^ f(r).  With 64 banks of 4 bytes, a
// 16-lane pass of a K operand read (16 rows, one 16-byte chunk each) and a
// 32-lane pass of a transposing V read (4 consecutive rows x 4 chunks)
// touch every bank once:
//   D = 128 (16 slots): f(r) = 4 (r mod 4) + (r / 4 mod 4), a bijection of
//     r mod 16 whose four values on rows 4m .. 4m + 3 lie in distinct
//     4-slot groups;
//   D = 64 (8 slots, a row covers half the banks): f(r) maps bits 1, 2, 3
//     of r to bits 2, 0, 1; the odd rows use the other half of the banks.
template <int D>
__device__ __forceinline__ int row_swz(int r) {
    if constexpr (TileGeom<D>::CH == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | (((r >> 3) & 1) << 1) | ((r >> 2) & 1);
}
template <int D>
__device__ __forceinline__ int slot_of(int r, int c) { return c ^ row_swz<D>(r); }

// Issue the copies of wave `wave` (of the NW that share a tile) of the K
// and V rows of tile tau.  The key list
// of a query is cut into ct tiles of compressed rows (row ssel[s] for CSA,
// row s for HCA; s < nval) followed by the tiles of its raw window (nwin
// rows from raw_first), so every tile reads from one source.  Rows past the
// end of a part repeat a row that exists and are masked by the caller.
// All offsets fit 32 bits (validated on the host).
// SHARED: one vector serves as key and value (the same rows passed as K and
// V), so only the K rows are copied and the V operands are read from them.
// Rows of one sequence's four K/V sources: base addresses and row strides in
// bytes (a source's rows lie within 2 GiB of its base; checked on the host).
struct KvRows {
    const char *ck, *cv, *rk, *rv;
    uint32_t ck_rb, cv_rb, rk_rb, rv_rb;
};

template <int NW, int D, bool SHARED>
__device__ __forceinline__ void issue_tile(int wave, int tau, int ct, int nval, int nwin,
                                           int raw_first,
                                           bool sparse, const CSA_LDS int32_t* ssel,
                                           const KvRows& kv, CSA_LDS uint8_t* sk,
                                           CSA_LDS uint8_t* sv) {
    using G = TileGeom<D>;
    const int lane = threadIdx.x % 64;
    const bool comp = tau < ct;
    const int base = comp ? ATT_KT * tau : ATT_KT * (tau - ct);
    const char* kb = comp ? kv.ck : kv.rk;
    const char* vb = comp ? kv.cv : kv.rv;
    const uint32_t krb = comp ? kv.ck_rb : kv.rk_rb;
    const uint32_t vrb = comp ? kv.cv_rb : kv.rv_rb;
#pragma unroll
    for (int ins = wave; ins < G::NINS; ins += NW) {
        const int r = ins * G::RPI + lane / G::CH;
        const int cb = slot_of<D>(r, lane % G::CH) * 16;   // slot <-> chunk: involution
        int row;
        if (comp) row = sparse ? ssel[base + r] : min(base + r, nval - 1);
        else row = raw_first + min(base + r, nwin - 1);
        __builtin_amdgcn_global_load_lds(kb + ((uint32_t)row * krb + (uint32_t)cb),
                                         (CSA_LDS void*)(sk + ins * G::RPI * G::ROWB), 16, 0, 0);
        if constexpr (!SHARED)
            __builtin_amdgcn_global_load_lds(vb + ((uint32_t)row * vrb + (uint32_t)cb),
                                             (CSA_LDS void*)(sv + ins * G::RPI * G::ROWB), 16, 0,
                                             0);
    }
}

// Pointers and strides of one attention call (element strides; Q and O rows
// are query tokens holding [H][D], K/V rows are entries or raw tokens)
template <typename TQ, typename TKV>
struct AttnArgs {
    const TQ* q;
    const TKV *ck, *cv;
    const TQ *rk, *rv;
    TQ* o;
    RowStrides qs, cks, cvs, rks, rvs, os;
};

// Per-wave attention engine.  An engine owns HPW heads of the block's
// query token: their Q^T operand, running softmax state and accumulators,
// the work of one 32-key tile (K and V in LDS; the first nvalid keys
// contribute), and the final store.  Scores stay in the exp2 domain
// (scale_log2 = softmax scale * log2 e).
//
// Lazy rescaling: the reference maximum of a head moves only
// when one of its scores exceeds it by more than a factor 2^8 in
// probability, so p stays <= 256; sum and accumulators share the
// reference, so the quotient is unchanged.  (tmax - m_run) is NaN while
// both are -inf: no move.  The row sum adds the same bf16-rounded p that
// the PV product takes.

// 32 heads per wave, V_MFMA_F32_32X32X16_BF16:
//   S^T = K Q^T: lane l holds head l%32, keys 8*(r/4) + 4*(l/32) + r%4
//   O^T += V^T P^T: P^T straight from the S^T registers; V^T by
//   transposing LDS reads (lane (16g + 4j + a) points at
//   V[key 16u + 8h + 4kb + j][32dt + 16(g%2) + 4a])
template <int D>
struct Heads32 {
    static constexpr int HPW = 32;
    f32x16 acc[D / 32];
    bf16x8 qop[D / 16];
    float m_run, mb, l_run;

    // qh: the query token's [H][D] rows, from this wave's first head
    __device__ __forceinline__ void init(const uint16_t* qh) {
        const int lane = threadIdx.x % 64, col = lane & 31, kb = lane >> 5;
        const uint16_t* qp = qh + col * D + 8 * kb;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) qop[kk] = *reinterpret_cast<const bf16x8*>(qp + 16 * kk);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[dt][r] = 0.f;
        m_run = -INFINITY;
        mb = 0.f;
        l_run = 0.f;
    }

    // state carried between the phases of a tile
    f32x16 sacc;                  // S^T of the current tile
    uint32_t pb[8];               // its probabilities as packed bf16 (P^T operand)
    bf16x8 vop[2][D / 32];        // its V^T operands

    // K operands kk in [K0, K1) of a tile (row col, 8 dims per lane and K step)
    template <int K0 = 0, int K1 = D / 16>
    __device__ __forceinline__ void read_k(const CSA_LDS uint8_t* K, bf16x8 (&kop)[D / 16]) const {
        using G = TileGeom<D>;
        const int lane = threadIdx.x % 64, col = lane & 31, kb = lane >> 5;
#pragma unroll
        for (int kk = K0; kk < K1; ++kk)
            kop[kk] = *reinterpret_cast<const CSA_LDS bf16x8*>(
                K + col * G::ROWB + slot_of<D>(col, 2 * kk + kb) * 16);
    }

    // S^T = K Q^T
    __device__ __forceinline__ void qk(const bf16x8 (&kop)[D / 16]) {
        f32x16 s = {};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[kk], qop[kk], s, 0, 0, 0);
        sacc = s;
    }

    // V^T operands of a tile (keys 16u .. 16u + 15 for u in [U0, U1)) by
    // transposing reads
    template <int U0 = 0, int U1 = 2>
    __device__ __forceinline__ void read_v(const CSA_LDS uint8_t* V) {
        using G = TileGeom<D>;
        const int lane = threadIdx.x % 64;
        const int g = lane >> 4, wj = (lane >> 2) & 3, wa = lane & 3;
#pragma unroll
        for (int u = U0; u < U1; ++u)
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt) {
                const int d = 32 * dt + 16 * (g & 1) + 4 * wa;
                const int key0 = 16 * u + 4 * (g >> 1) + wj;
                const int key1 = key0 + 8;
                const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((CSA_LDS bf16x4*)(
                    V + key0 * G::ROWB + slot_of<D>(key0, d / 8) * 16 + (d % 8) * 2));
                const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((CSA_LDS bf16x4*)(
                    V + key1 * G::ROWB + slot_of<D>(key1, d / 8) * 16 + (d % 8) * 2));
                vop[u][dt] = bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
    }

    // online softmax of S^T (the first nvalid keys count): state update
    // (mask, maximum, rescaling), then probabilities into pb and row sums
    __device__ __forceinline__ void softmax(int nvalid, float scale_log2) {
        softmax_max(nvalid, scale_log2);
        softmax_exp(scale_log2);
    }
    __device__ __forceinline__ void softmax_max(int nvalid, float scale_log2) {
        const int lane = threadIdx.x % 64, kb = lane >> 5;
        if (nvalid < ATT_KT) {                     // wave-uniform
            // key 8 (r/4) + 4 kb + r%4 is masked when 8 (r/4) + r%4 >= lim
            const int lim = nvalid - 4 * kb;
#pragma unroll
            for (int r = 0; r < 16; ++r)
                if (8 * (r / 4) + (r % 4) >= lim) sacc[r] = -INFINITY;
        }
        float t = -INFINITY;
#pragma unroll
        for (int r = 0; r < 16; ++r) t = fmaxf(t, sacc[r]);
        const float tmax = max_halves(t);
        const bool grow = (tmax - m_run) * scale_log2 > 8.f;
        if (__ballot(grow)) {
            float alpha = 1.f;
            if (grow) {
                alpha = __builtin_amdgcn_exp2f((m_run - tmax) * scale_log2);   // 0 from -inf
                m_run = tmax;
                mb = -tmax * scale_log2;
            }
            l_run *= alpha;
#pragma unroll
            for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[dt][r] *= alpha;
        }
    }
    __device__ __forceinline__ void softmax_exp(float scale_log2) {
#pragma unroll
        for (int r = 0; r < 16; r += 2)
            pb[r / 2] = pack_bf16x2(__builtin_amdgcn_exp2f(fmaf(sacc[r], scale_log2, mb)),
                                    __builtin_amdgcn_exp2f(fmaf(sacc[r + 1], scale_log2, mb)));
        const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
        float psum = l_run;
#pragma unroll
        for (int x = 0; x < 8; ++x)
            psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, pb[x]), ones, psum,
                                                   false);
        l_run = psum;
    }

    // O^T += V^T P^T over keys 16u .. 16u + 15 of the tile
    __device__ __forceinline__ void pv_half(int u) {
        const u32x4 w = {pb[4 * u], pb[4 * u + 1], pb[4 * u + 2], pb[4 * u + 3]};
        const bf16x8 pop = __builtin_bit_cast(bf16x8, w);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
            acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[u][dt], pop, acc[dt], 0, 0, 0);
    }
    __device__ __forceinline__ void pv() {
        pv_half(0);
        pv_half(1);
    }

    // one whole tile: every K operand read is issued before the QK chain,
    // the V^T operands (independent of P) are read while the softmax runs
    __device__ __forceinline__ void tile(const CSA_LDS uint8_t* K, const CSA_LDS uint8_t* V,
                                         int nvalid, float scale_log2) {
        tile(K, V, nvalid, scale_log2, [] {});
    }
    // the same with mid() (the copies of a later tile) issued right after the
    // QK chain: the copy queue fills while the matrix cores run, instead of
    // every wave of the block queueing its copies at the barrier
    template <class F>
    __device__ __forceinline__ void tile(const CSA_LDS uint8_t* K, const CSA_LDS uint8_t* V,
                                         int nvalid, float scale_log2, F&& mid) {
        bf16x8 kop[D / 16];
        read_k(K, kop);
        __builtin_amdgcn_sched_barrier(0);
        qk(kop);
        __builtin_amdgcn_sched_barrier(0);
        mid();
        __builtin_amdgcn_sched_barrier(0);
        read_v<0, 1>(V);
        softmax_max(nvalid, scale_log2);
        read_v<1, 2>(V);
        softmax_exp(scale_log2);
        pv();
    }

    // oh: output rows [HPW][D] of this wave's heads (splits == 1), else the
    // split's partial record: po [HPW][D] bf16, the split's own normalised
    // output (zero for a split without keys), and pml [HPW][2] fp32, its
    // maximum in the exp2 domain and its sum
    __device__ __forceinline__ void store(uint16_t* oh, uint16_t* po, float* pml,
                                          float scale_log2) {
        const int lane = threadIdx.x % 64, col = lane & 31, kb = lane >> 5;
        const float l_tot = sum_halves(l_run);
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        uint16_t* op = (oh ? oh : po) + col * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                const int d = 32 * dt + 8 * gg + 4 * kb;
                const float a0 = acc[dt][4 * gg] * inv, a1 = acc[dt][4 * gg + 1] * inv;
                const float a2 = acc[dt][4 * gg + 2] * inv, a3 = acc[dt][4 * gg + 3] * inv;
                u32x2 w;
                w[0] = pack_bf16x2(a0, a1);
                w[1] = pack_bf16x2(a2, a3);
                *reinterpret_cast<u32x2*>(op + d) = w;
            }
        if (!oh && kb == 0) {
            pml[2 * col] = m_run == -INFINITY ? -INFINITY : m_run * scale_log2;
            pml[2 * col + 1] = l_tot;
        }
    }
};

template <int NW, int D, class E, bool SHARED>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
k_attend_bf16(AttnArgs<uint16_t, uint16_t> A, const int32_t* __restrict__ topk,
              float* __restrict__ part, int64_t Tq, int64_t Nc, int64_t m, int64_t W, int k,
              int64_t q_pos0, float scale_log2, int64_t raw_pos0, int64_t raw_len, int splits) {
    using G = TileGeom<D>;
    constexpr int NT = NW * 64;
    constexpr int H = NW * E::HPW;
    constexpr int KT = G::KT;
    constexpr int PER = (SHARED ? 1 : 2) * ((G::NINS + NW - 1) / NW);   // copies per wave per tile
    // the stages live in distinct arrays, so the compiler can tell which
    // stage an LDS read touches and never waits on another stage's copies
    __shared__ __attribute__((aligned(16))) uint8_t sK0[G::BYTES], sV0[G::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t sK1[G::BYTES], sV1[G::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t sK2[G::BYTES], sV2[G::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t sK3[G::BYTES], sV3[G::BYTES];
    __shared__ int32_t sSel[2048];                  // this query's kept indices (CSA)
    __shared__ int sCnt[NW];

    const int i = (int)blockIdx.x;
    const int split = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
    const int64_t t = q_pos0 + i;
    const bool sparse = topk != nullptr;
    const int nc_t = (int)n_candidates(t, m, W);
    const int64_t w0 = t - W + 1 < 0 ? 0 : t - W + 1;
    const int nwin = (int)(t - w0 + 1), raw_first = (int)(w0 - raw_pos0);

    // compressed part of the key list: CSA keeps the valid selected indices
    // (0 <= j < n_cand), in order, padded with row 0 to whole tiles
    int nval = nc_t;
    if (sparse) {
        const int nsel = min(k, nc_t);
        const int32_t* sel = topk + (b * Tq + i) * k;
        nval = 0;
        int jn = tid < nsel ? sel[tid] : -1;
        for (int x0 = 0; x0 < nsel; x0 += NT) {
            const int j = jn;
            jn = x0 + NT + tid < nsel ? sel[x0 + NT + tid] : -1;
            const bool ok = j >= 0 && j < nc_t;
            const uint64_t bal = __ballot(ok);
            if (lane == 0) sCnt[wave] = __popcll(bal);
            __syncthreads();
            int before = nval, total = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const int c = sCnt[w];
                before += w < wave ? c : 0;
                total += c;
            }
            if (ok) sSel[before + __popcll(bal & ((1ull << lane) - 1ull))] = j;
            nval += total;
            __syncthreads();
        }
        for (int x = nval + tid; x < ((nval + KT - 1) & ~(KT - 1)); x += NT) sSel[x] = 0;
        __syncthreads();
    }
    const CSA_LDS int32_t* ssel = (const CSA_LDS int32_t*)sSel;

    // this split's range of tiles
    const int ct = (nval + KT - 1) / KT;
    const int ntile = ct + (nwin + KT - 1) / KT;
    // the ntile tiles dealt evenly over the splits (they differ by at most one
    // tile, so the blocks of a decode launch finish together)
    const int tau0 = (int)((int64_t)split * ntile / splits);
    const int tau1 = (int)((int64_t)(split + 1) * ntile / splits);

    const KvRows kv{reinterpret_cast<const char*>(A.ck + b * A.cks.ss),
                    reinterpret_cast<const char*>(A.cv + b * A.cvs.ss),
                    reinterpret_cast<const char*>(A.rk + b * A.rks.ss),
                    reinterpret_cast<const char*>(A.rv + b * A.rvs.ss),
                    (uint32_t)(A.cks.rs * 2), (uint32_t)(A.cvs.rs * 2), (uint32_t)(A.rks.rs * 2),
                    (uint32_t)(A.rvs.rs * 2)};

    E eng;
    eng.init(A.q + b * A.qs.ss + i * A.qs.rs + wave * E::HPW * D);

    auto issue = [&](int tau, uint8_t* sk, uint8_t* sv) {
        if (tau < tau1)
            issue_tile<NW, D, SHARED>(wave, tau, ct, nval, nwin, raw_first, sparse, ssel, kv,
                                      (CSA_LDS uint8_t*)sk, (CSA_LDS uint8_t*)sv);
    };
    // one tile: wait for its copies, barrier (the stage written next is then
    // free on every wave), compute, with the copies three tiles ahead issued
    // once the QK chain is on the matrix cores
    auto step = [&](int tau, uint8_t* ck_, uint8_t* cv_, uint8_t* nk_, uint8_t* nv_) {
        const int after = min(G::NST - 2, tau1 - tau - 1);
        if (after >= 2) CSA_WAIT_VM(2 * PER);
        else if (after == 1) CSA_WAIT_VM(PER);
        else CSA_WAIT_VM(0);
        lds_barrier();
        const int nvalid = tau < ct ? nval - KT * tau : nwin - KT * (tau - ct);
        eng.tile((const CSA_LDS uint8_t*)ck_, (const CSA_LDS uint8_t*)(SHARED ? ck_ : cv_), nvalid,
                 scale_log2, [&] { issue(tau + G::NST - 1, nk_, nv_); });
    };

    issue(tau0, sK0, sV0);
    issue(tau0 + 1, sK1, sV1);
    issue(tau0 + 2, sK2, sV2);
    for (int tau = tau0; tau < tau1; tau += 4) {
        step(tau, sK0, sV0, sK3, sV3);
        if (tau + 1 >= tau1) break;
        step(tau + 1, sK1, sV1, sK0, sV0);
        if (tau + 2 >= tau1) break;
        step(tau + 2, sK2, sV2, sK1, sV1);
        if (tau + 3 >= tau1) break;
        step(tau + 3, sK3, sV3, sK2, sV2);
    }
    if (splits == 1) {
        eng.store(A.o + b * A.os.ss + i * A.os.rs + wave * E::HPW * D, nullptr, nullptr,
                  scale_log2);
    } else {
        const int64_t rec = ((b * Tq + i) * splits + split) * H + wave * E::HPW;
        const int64_t nrec = (int64_t)gridDim.x * gridDim.y * gridDim.z * H;
        uint16_t* po = reinterpret_cast<uint16_t*>(part);
        eng.store(nullptr, po + rec * D, reinterpret_cast<float*>(po + nrec * D) + rec * 2,
                  scale_log2);
    }
}

// ---- compressed entries stored as MXFP8 -------------------------------------
// (ai-papers.net article, hybrid attention section: most KV entries are kept
// in FP8.)  Compressed K/V rows arrive as E4M3 codes [Nc][128] with one
// power-of-two scale byte per 32 values [Nc][4]; the raw window stays bf16.
// Per block and tile of 32 compressed rows the codes and scales are copied
// into an LDS staging slot (global_load_lds, half the bytes of bf16 rows),
// three tiles ahead; one tile ahead, the block converts the staged tile into
// the swizzled bf16 layout of the engine above (each value times its scale
// is exact in bf16), so the MFMA work and its numerics are those of the
// bf16 kernel.  Window tiles are copied straight into the bf16 buffer one
// tile ahead.
//
// Staging slot (D = 128): K codes [32][128] | V codes [32][128] | K scales
// [32][4] | V scales [32][4].  A wave-wide copy moves 8 code rows (64 lanes
// x 16 bytes); one more copy moves both tensors' scale rows (lanes 0-31 K,
// 32-63 V, 4 bytes each).  Copies are dealt to the waves round-robin.
struct Mx8Geom {
    static constexpr int D = 128;
    static constexpr int CODE_B = ATT_KT * D;             // 4096 bytes per tensor
    static constexpr int SC_OFF = 2 * CODE_B;             // scales after the codes
    static constexpr int BYTES = SC_OFF + 2 * ATT_KT * 4; // 8448
    static constexpr int NCOPY_CODES = CODE_B / 1024;     // 4 per tensor
};

// copies of this wave for one compressed tile
template <int NW, bool SHARED>
__device__ __forceinline__ int mx8_comp_copies(int wave) {
    constexpr int n = (SHARED ? 1 : 2) * Mx8Geom::NCOPY_CODES + 1;
    return n / NW + (wave < n % NW ? 1 : 0);
}

// row of tile entry r (0..31) of compressed tile tau (CSA: kept list; HCA:
// every candidate, clamped to the last one)
__device__ __forceinline__ int mx8_row(bool sparse, const CSA_LDS int32_t* ssel, int base, int r,
                                       int nval) {
    return sparse ? ssel[base + r] : min(base + r, nval - 1);
}

template <int NW, bool SHARED>
__device__ __forceinline__ void mx8_issue_comp(int wave, int tau, int nval, bool sparse,
                                               const CSA_LDS int32_t* ssel, const uint8_t* ckb,
                                               const uint8_t* cvb, const uint8_t* ksb,
                                               const uint8_t* vsb, CSA_LDS uint8_t* stg) {
    using M = Mx8Geom;
    const int lane = threadIdx.x % 64;
    const int base = ATT_KT * tau;
    constexpr int NT = SHARED ? 1 : 2;
    constexpr int n = NT * M::NCOPY_CODES + 1;
#pragma unroll
    for (int c0 = 0; c0 < n; c0 += NW) {
        const int c = c0 + wave;
        if (c >= n) break;
        if (c < NT * M::NCOPY_CODES) {
            const int tensor = c / M::NCOPY_CODES, ins = c % M::NCOPY_CODES;
            const int r = ins * 8 + lane / 8;
            const uint32_t off = (uint32_t)mx8_row(sparse, ssel, base, r, nval) * M::D +
                                 (uint32_t)(lane % 8) * 16;
            __builtin_amdgcn_global_load_lds((tensor ? cvb : ckb) + off,
                                             (CSA_LDS void*)(stg + tensor * M::CODE_B + ins * 1024),
                                             16, 0, 0);
        } else {
            const int tensor = SHARED ? 0 : lane / 32;
            const uint32_t off = (uint32_t)mx8_row(sparse, ssel, base, lane % 32, nval) * 4;
            __builtin_amdgcn_global_load_lds((tensor ? vsb : ksb) + off,
                                             (CSA_LDS void*)(stg + M::SC_OFF), 4, 0, 0);
        }
    }
}

// staged tile -> bf16 tile buffers (every thread of the block takes items
// of 16 values: tensor, row r, 16-value group c)
template <int NW, bool SHARED>
__device__ __forceinline__ void mx8_convert(const CSA_LDS uint8_t* stg, CSA_LDS uint8_t* bk,
                                            CSA_LDS uint8_t* bv) {
    using M = Mx8Geom;
    using G = TileGeom<128>;
    constexpr int NTEN = SHARED ? 1 : 2;
    constexpr int ITEMS = NTEN * ATT_KT * 8;
#pragma unroll 1
    for (int it = threadIdx.x; it < ITEMS; it += NW * 64) {
        const int tensor = it / (ATT_KT * 8), r = (it / 8) % ATT_KT, c = it % 8;
        const u32x4 w = *reinterpret_cast<const CSA_LDS u32x4*>(stg + tensor * M::CODE_B +
                                                                r * M::D + c * 16);
        // the scale rows of the tile follow each other (4 bytes per row);
        // in SHARED mode lanes 32-63 of the scale copy held K rows again
        const uint32_t sb = stg[M::SC_OFF + (SHARED ? 0 : tensor * 128) + r * 4 + c / 2];
        const float sc = sb ? __uint_as_float(sb << 23) : 0x1p-127f;
        uint32_t o[8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            o[2 * j] = __builtin_bit_cast(uint32_t,
                                          __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[j], sc, false));
            o[2 * j + 1] = __builtin_bit_cast(uint32_t,
                                              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[j], sc, true));
        }
        CSA_LDS uint8_t* dst = (tensor ? bv : bk) + r * G::ROWB;
        *reinterpret_cast<CSA_LDS u32x4*>(dst + slot_of<128>(r, 2 * c) * 16) =
            u32x4{o[0], o[1], o[2], o[3]};
        *reinterpret_cast<CSA_LDS u32x4*>(dst + slot_of<128>(r, 2 * c + 1) * 16) =
            u32x4{o[4], o[5], o[6], o[7]};
    }
}

template <int NW, class E, bool SHARED>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
k_attend_mx8(AttnArgs<uint16_t, uint8_t> A, const uint8_t* __restrict__ cks,
             const uint8_t* __restrict__ cvs, const int32_t* __restrict__ topk,
             float* __restrict__ part, int64_t Tq, int64_t Nc, int64_t m, int64_t W, int k,
             int64_t q_pos0, float scale_log2, int64_t raw_pos0, int64_t raw_len, int splits) {
    constexpr int D = 128;
    using G = TileGeom<D>;
    using M = Mx8Geom;
    constexpr int NT = NW * 64;
    constexpr int H = NW * E::HPW;
    constexpr int KT = G::KT;
    // distinct arrays per stage, so the compiler can tell which stage an LDS
    // access touches
    __shared__ __attribute__((aligned(16))) uint8_t sS0[M::BYTES], sS1[M::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t sS2[M::BYTES], sS3[M::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t sK0[G::BYTES], sV0[G::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t sK1[G::BYTES], sV1[G::BYTES];
    __shared__ int32_t sSel[2048];
    __shared__ int sCnt[NW];

    const int i = (int)blockIdx.x;
    const int split = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
    const int64_t t = q_pos0 + i;
    const bool sparse = topk != nullptr;
    const int nc_t = (int)n_candidates(t, m, W);
    const int64_t w0 = t - W + 1 < 0 ? 0 : t - W + 1;
    const int nwin = (int)(t - w0 + 1), raw_first = (int)(w0 - raw_pos0);

    int nval = nc_t;
    if (sparse) {
        const int nsel = min(k, nc_t);
        const int32_t* sel = topk + (b * Tq + i) * k;
        nval = 0;
        int jn = tid < nsel ? sel[tid] : -1;
        for (int x0 = 0; x0 < nsel; x0 += NT) {
            const int j = jn;
            jn = x0 + NT + tid < nsel ? sel[x0 + NT + tid] : -1;
            const bool ok = j >= 0 && j < nc_t;
            const uint64_t bal = __ballot(ok);
            if (lane == 0) sCnt[wave] = __popcll(bal);
            __syncthreads();
            int before = nval, total = 0;
#pragma unroll
            for (int w = 0; w < NW; ++w) {
                const int c = sCnt[w];
                before += w < wave ? c : 0;
                total += c;
            }
            if (ok) sSel[before + __popcll(bal & ((1ull << lane) - 1ull))] = j;
            nval += total;
            __syncthreads();
        }
        for (int x = nval + tid; x < ((nval + KT - 1) & ~(KT - 1)); x += NT) sSel[x] = 0;
        __syncthreads();
    }
    const CSA_LDS int32_t* ssel = (const CSA_LDS int32_t*)sSel;

    const int ct = (nval + KT - 1) / KT;
    const int ntile = ct + (nwin + KT - 1) / KT;
    // the ntile tiles dealt evenly over the splits (they differ by at most one
    // tile, so the blocks of a decode launch finish together)
    const int tau0 = (int)((int64_t)split * ntile / splits);
    const int tau1 = (int)((int64_t)(split + 1) * ntile / splits);

    const uint8_t* ckb = A.ck + b * Nc * D;
    const uint8_t* cvb = A.cv + b * Nc * D;
    const uint8_t* ksb = cks + b * Nc * (D / 32);
    const uint8_t* vsb = cvs + b * Nc * (D / 32);
    const KvRows kv{nullptr, nullptr, reinterpret_cast<const char*>(A.rk + b * A.rks.ss),
                    reinterpret_cast<const char*>(A.rv + b * A.rvs.ss), 0u, 0u,
                    (uint32_t)(A.rks.rs * 2), (uint32_t)(A.rvs.rs * 2)};
    const int percomp = mx8_comp_copies<NW, SHARED>(wave);

    E eng;
    eng.init(A.q + b * A.qs.ss + i * A.qs.rs + wave * E::HPW * D);

    // staging copies of compressed tile tau (nothing for other tiles)
    auto stage = [&](int tau, uint8_t* stg) {
        if (tau < tau1 && tau < ct)
            mx8_issue_comp<NW, SHARED>(wave, tau, nval, sparse, ssel, ckb, cvb, ksb, vsb,
                                       (CSA_LDS uint8_t*)stg);
    };
    // bf16 tile tau: convert its staging slot, or copy its window rows
    auto fill = [&](int tau, const uint8_t* stg, uint8_t* bk, uint8_t* bv) {
        if (tau >= tau1) return;
        if (tau < ct)
            mx8_convert<NW, SHARED>((const CSA_LDS uint8_t*)stg, (CSA_LDS uint8_t*)bk,
                                    (CSA_LDS uint8_t*)bv);
        else
            issue_tile<NW, D, SHARED>(wave, tau, ct, nval, nwin, raw_first, false, ssel, kv,
                                      (CSA_LDS uint8_t*)bk, (CSA_LDS uint8_t*)bv);
    };
    // one step: wait, barrier (stage tau's bf16 tile complete everywhere; the
    // other bf16 buffer and staging slot of tau - 1 free), fill tile tau + 1,
    // stage tile tau + 3, compute tile tau
    auto step = [&](int tau, const uint8_t* stg1, uint8_t* stg3, uint8_t* ck_, uint8_t* cv_,
                    uint8_t* nk_, uint8_t* nv_) {
        // still in flight: the staging of tile tau + 2, issued after the
        // copies that tile tau and the conversion of tau + 1 need
        wait_vm_leaving(tau + 2 < tau1 && tau + 2 < ct ? percomp : 0);
        lds_barrier();
        // a window tile's copies go out first; a compressed tile is converted
        // after this tile's MFMA chain is issued, while it drains
        if (tau + 1 >= ct) fill(tau + 1, stg1, nk_, nv_);
        stage(tau + 3, stg3);
        __builtin_amdgcn_sched_barrier(0);
        const int nvalid = tau < ct ? nval - KT * tau : nwin - KT * (tau - ct);
        eng.tile((const CSA_LDS uint8_t*)ck_, (const CSA_LDS uint8_t*)(SHARED ? ck_ : cv_), nvalid,
                 scale_log2);
        if (tau + 1 < ct) fill(tau + 1, stg1, nk_, nv_);
    };

    // prologue: stage tau0 .. tau0 + 2, then tile tau0's bf16 buffer
    stage(tau0, sS0);
    stage(tau0 + 1, sS1);
    stage(tau0 + 2, sS2);
    if (tau0 < tau1 && tau0 < ct) {
        wait_vm_leaving((tau0 + 1 < tau1 && tau0 + 1 < ct ? percomp : 0) +
                        (tau0 + 2 < tau1 && tau0 + 2 < ct ? percomp : 0));
        lds_barrier();
    }
    fill(tau0, sS0, sK0, sV0);
    for (int tau = tau0; tau < tau1; tau += 4) {
        step(tau, sS1, sS3, sK0, sV0, sK1, sV1);
        if (tau + 1 >= tau1) break;
        step(tau + 1, sS2, sS0, sK1, sV1, sK0, sV0);
        if (tau + 2 >= tau1) break;
        step(tau + 2, sS3, sS1, sK0, sV0, sK1, sV1);
        if (tau + 3 >= tau1) break;
        step(tau + 3, sS0, sS2, sK1, sV1, sK0, sV0);
    }
    if (splits == 1) {
        eng.store(A.o + b * A.os.ss + i * A.os.rs + wave * E::HPW * D, nullptr, nullptr,
                  scale_log2);
    } else {
        const int64_t rec = ((b * Tq + i) * splits + split) * H + wave * E::HPW;
        const int64_t nrec = (int64_t)gridDim.x * gridDim.y * gridDim.z * H;
        uint16_t* po = reinterpret_cast<uint16_t*>(part);
        eng.store(nullptr, po + rec * D, reinterpret_cast<float*>(po + nrec * D) + rec * 2,
                  scale_log2);
    }
}

// Log-sum-exp merge of the split partials.  Grid (query, sequence, head
// group of 8); D/4 threads per head, 4 dims each.  The threads of a head
// read the splits' maxima and sums in parallel (at most 64 splits) and
// share the weights through LDS.  The partial outputs of the first
// CMB_PRE splits are loaded together with the maxima and sums (they do not
// depend on the weights), so a decode merge is one round trip to memory;
// further splits are loaded in batches of 8.
constexpr int CMB_MAXS = 64;
constexpr int CMB_PRE = 16;

template <typename TO>
__global__ void __launch_bounds__(256)
k_attend_combine(const uint16_t* __restrict__ po, const float* __restrict__ pml,
                 TO* __restrict__ o, RowStrides os, int64_t Tq, int H, int D, int splits) {
    __shared__ float sw[8][CMB_MAXS];
    const int64_t i = blockIdx.x, b = blockIdx.y;
    const int per_head = D / 4;                     // 32 or 16: a power of two <= 32
    const int hh = threadIdx.x / per_head, t = threadIdx.x % per_head;
    const int h = blockIdx.z * 8 + hh;
    const bool live = threadIdx.x < 8 * per_head && h < H;
    const int64_t rec0 = (b * Tq + i) * splits * (int64_t)H + (live ? h : 0);
    const int d0 = t * 4;
    const uint16_t* base = po + rec0 * D + d0;
    const int64_t sstride = (int64_t)H * D;
    u32x2 pre[CMB_PRE];
#pragma unroll
    for (int u = 0; u < CMB_PRE; ++u)
        pre[u] = live && u < splits ? *reinterpret_cast<const u32x2*>(base + u * sstride)
                                    : u32x2{0u, 0u};
    // maxima and sums of the splits t, t + per_head, ...
    float ms[CMB_MAXS / 16], ls[CMB_MAXS / 16];
    float M = -INFINITY;
#pragma unroll
    for (int x = 0; x < CMB_MAXS / 16; ++x) {
        const int sp = t + x * per_head;
        const bool ok = live && sp < splits;
        const float* r = pml + (rec0 + (int64_t)sp * H) * 2;
        ms[x] = ok ? r[0] : -INFINITY;
        ls[x] = ok ? r[1] : 0.f;
        M = fmaxf(M, ms[x]);
    }
    for (int off = per_head / 2; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off, 64));
    // weight of split s: 2^(m_s - M) l_s / sum over the splits of the same
    float wl[CMB_MAXS / 16];
    float L = 0.f;
#pragma unroll
    for (int x = 0; x < CMB_MAXS / 16; ++x) {
        wl[x] = ms[x] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(ms[x] - M) * ls[x];
        L += wl[x];
    }
    for (int off = per_head / 2; off > 0; off >>= 1) L += __shfl_xor(L, off, 64);
    const float invL = 1.f / L;
#pragma unroll
    for (int x = 0; x < CMB_MAXS / 16; ++x) {
        const int sp = t + x * per_head;
        if (live && sp < splits) sw[hh][sp] = wl[x] * invL;
    }
    __syncthreads();
    if (!live) return;
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int u = 0; u < CMB_PRE; ++u) {
        const float w = u < splits ? sw[hh][u] : 0.f;
        a[0] += bf16_bits_to_f32(pre[u][0] & 0xffffu) * w;
        a[1] += bf16_bits_to_f32(pre[u][0] >> 16) * w;
        a[2] += bf16_bits_to_f32(pre[u][1] & 0xffffu) * w;
        a[3] += bf16_bits_to_f32(pre[u][1] >> 16) * w;
    }
    constexpr int U = 8;
    for (int s0 = CMB_PRE; s0 < splits; s0 += U) {
        u32x2 v[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            v[u] = s0 + u < splits ? *reinterpret_cast<const u32x2*>(base + (s0 + u) * sstride)
                                   : u32x2{0u, 0u};
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const float w = s0 + u < splits ? sw[hh][s0 + u] : 0.f;
            a[0] += bf16_bits_to_f32(v[u][0] & 0xffffu) * w;
            a[1] += bf16_bits_to_f32(v[u][0] >> 16) * w;
            a[2] += bf16_bits_to_f32(v[u][1] & 0xffffu) * w;
            a[3] += bf16_bits_to_f32(v[u][1] >> 16) * w;
        }
    }
    TO* op = o + b * os.ss + i * os.rs + h * (int64_t)D + d0;
    if constexpr (sizeof(TO) == 2) {
        u32x2 w;
        w[0] = f32_to_bf16_bits(a[0]) | (f32_to_bf16_bits(a[1]) << 16);
        w[1] = f32_to_bf16_bits(a[2]) | (f32_to_bf16_bits(a[3]) << 16);
        *reinterpret_cast<u32x2*>(op) = w;
    } else {
        f32x4 w = {a[0], a[1], a[2], a[3]};
        *reinterpret_cast<f32x4*>(op) = w;
    }
}

// fp32 kernel: one wave per (query, head) at a time, keys in sequence, the
// D dims spread over the lanes; fp32 arithmetic with accurate expf.
__global__ void __launch_bounds__(256)
k_attend_f32(AttnArgs<float, float> A, const int32_t* __restrict__ topk, int64_t Tq, int H,
             int D, int64_t Nc, int64_t m, int64_t W, int k, int64_t q_pos0, float scale,
             int64_t raw_pos0, int64_t raw_len) {
    const int64_t i = blockIdx.x, b = blockIdx.y;
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
    const int64_t t = q_pos0 + i;
    const bool sparse = topk != nullptr;
    const KeyList L = key_list(t, m, W, k, sparse);
    const int64_t nc_t = n_candidates(t, m, W);
    const int32_t* sel = sparse ? topk + (b * Tq + i) * k : nullptr;
    constexpr int DPL = 4;                 // dims per lane (D <= 256)
    for (int h = wave; h < H; h += blockDim.x / 64) {
        const float* qh = A.q + b * A.qs.ss + i * A.qs.rs + h * (int64_t)D;
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
            const float* kr = row >= 0 ? A.ck + b * A.cks.ss + row * A.cks.rs
                                       : A.rk + b * A.rks.ss + (-row - 2) * A.rks.rs;
            const float* vr = row >= 0 ? A.cv + b * A.cvs.ss + row * A.cvs.rs
                                       : A.rv + b * A.rvs.ss + (-row - 2) * A.rvs.rs;
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
        float* oh = A.o + b * A.os.ss + i * A.os.rs + h * (int64_t)D;
#pragma unroll
        for (int e = 0; e < DPL; ++e) {
            const int d = lane + 64 * e;
            if (d < D) oh[d] = acc[e] / den;
        }
    }
}

// merge of the bf16 split partials in ws (the layout plan_attend sizes) into o
void launch_attend_combine(const void* ws, int64_t B, int64_t Tq, int H, int D, int splits,
                           void* o, RowStrides os, hipStream_t st) {
    const uint16_t* po = (const uint16_t*)ws;
    const float* pml = (const float*)(po + B * Tq * splits * H * D);
    hipLaunchKernelGGL(k_attend_combine<uint16_t>,
                       dim3((unsigned)Tq, (unsigned)B, (unsigned)((H + 7) / 8)), dim3(256), 0, st,
                       po, pml, (uint16_t*)o, os, Tq, H, D, splits);
}

AttendPlan plan_attend(int dt, int64_t B, int64_t Tq, int64_t H, int64_t D, int64_t max_keys) {
    AttendPlan p{};
    p.splits = 1;
    if (dt == 1) {
        const int64_t rows = B * Tq;
        const int64_t tiles = (max_keys + ATT_KT - 1) / ATT_KT;
        if (rows < 512 && tiles > 2) {
            int64_t want = (512 + rows - 1) / rows;            // ~2 blocks per CU
            int64_t cap = (tiles + 1) / 2;                     // >= 2 tiles per split
            p.splits = (int)min(min(want, cap), (int64_t)64);
            if (p.splits < 1) p.splits = 1;
        }
    }
    // per split and head: the normalised output in bf16, maximum and sum in fp32
    p.ws_bytes = p.splits > 1 ? (size_t)(B * Tq * p.splits * H) * (D * 2 + 8) : 0;
    return p;
}

// NW waves per block, E::HPW heads per wave
template <int D, int NW, class E>
static void launch_bf16(const AttendPlan& p, int64_t B, int64_t Tq, int64_t Nc, int64_t m,
                        int64_t W, int k, int64_t q_pos0, float scale, const AttendIO& io,
                        const int32_t* topk, int64_t raw_pos0, int64_t raw_len, void* ws,
                        hipStream_t st) {
    const float scale_log2 = scale * 1.4426950408889634f;
    const AttnArgs<uint16_t, uint16_t> A{
        (const uint16_t*)io.q,  (const uint16_t*)io.ck, (const uint16_t*)io.cv,
        (const uint16_t*)io.rk, (const uint16_t*)io.rv, (uint16_t*)io.o,
        io.qs, io.cks, io.cvs, io.rks, io.rvs, io.os};
    // the same rows passed as keys and values: copy them once
    const bool shared = io.ck == io.cv && io.rk == io.rv && io.cks.ss == io.cvs.ss &&
                        io.cks.rs == io.cvs.rs && io.rks.ss == io.rvs.ss && io.rks.rs == io.rvs.rs;
    auto kern = shared ? k_attend_bf16<NW, D, E, true> : k_attend_bf16<NW, D, E, false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)Tq, (unsigned)p.splits, (unsigned)B), dim3(NW * 64),
                       0, st, A, topk, (float*)ws, Tq, Nc, m, W, k, q_pos0, scale_log2, raw_pos0,
                       raw_len, p.splits);
    if (p.splits > 1) {
        const int H = NW * E::HPW;
        const uint16_t* po = (const uint16_t*)ws;
        const float* pml = (const float*)(po + B * Tq * p.splits * H * D);
        hipLaunchKernelGGL(k_attend_combine<uint16_t>,
                           dim3((unsigned)Tq, (unsigned)B, (unsigned)((H + 7) / 8)), dim3(256), 0,
                           st, po, pml, (uint16_t*)io.o, io.os, Tq, H, D, p.splits);
    }
}

hipError_t launch_attend(int dt, const AttendPlan& p, int64_t B, int64_t Tq, int64_t H,
                         int64_t D, int64_t Nc, int64_t m, int64_t W, int64_t k,
                         int64_t q_pos0, float scale, const AttendIO& io, const int32_t* topk,
                         int64_t raw_pos0, int64_t raw_len, void* ws, hipStream_t st) {
    if (B == 0 || Tq == 0) return hipSuccess;
    if (dt == 0) {
        const AttnArgs<float, float> A{(const float*)io.q,  (const float*)io.ck,
                                       (const float*)io.cv, (const float*)io.rk,
                                       (const float*)io.rv, (float*)io.o,
                                       io.qs, io.cks, io.cvs, io.rks, io.rvs, io.os};
        hipLaunchKernelGGL(k_attend_f32, dim3((unsigned)Tq, (unsigned)B), dim3(256), 0, st, A,
                           topk, Tq, (int)H, (int)D, Nc, m, W, (int)k, q_pos0, scale, raw_pos0,
                           raw_len);
        return hipGetLastError();
    }
    const int nw = (int)(H / 32);
#define CSA_ATT_CASE(DD, NN, EE)                                                               \
    launch_bf16<DD, NN, EE<DD>>(p, B, Tq, Nc, m, W, (int)k, q_pos0, scale, io, topk, raw_pos0, \
                                raw_len, ws, st)
    // 32 heads per wave.  (A 16-head engine on V_MFMA_F32_16X16X32_BF16 fits
    // four waves per SIMD but doubles the LDS operand reads per flop, and
    // measured slower.)
    if (D == 128) {
        switch (nw) {
            case 1: CSA_ATT_CASE(128, 1, Heads32); break;
            case 2: CSA_ATT_CASE(128, 2, Heads32); break;
            case 4: CSA_ATT_CASE(128, 4, Heads32); break;
            case 8: CSA_ATT_CASE(128, 8, Heads32); break;
            default: return hipErrorInvalidValue;
        }
    } else {
        switch (nw) {
            case 1: CSA_ATT_CASE(64, 1, Heads32); break;
            case 2: CSA_ATT_CASE(64, 2, Heads32); break;
            case 4: CSA_ATT_CASE(64, 4, Heads32); break;
            case 8: CSA_ATT_CASE(64, 8, Heads32); break;
            default: return hipErrorInvalidValue;
        }
    }
#undef CSA_ATT_CASE
    return hipGetLastError();
}

template <int NW>
static void launch_mx8_nw(const AttendPlan& p, int64_t B, int64_t Tq, int64_t Nc, int64_t m,
                          int64_t W, int k, int64_t q_pos0, float scale, const AttendIO& io,
                          const uint8_t* cks, const uint8_t* cvs, const int32_t* topk,
                          int64_t raw_pos0, int64_t raw_len, void* ws, hipStream_t st) {
    constexpr int D = 128;
    const float scale_log2 = scale * 1.4426950408889634f;
    const AttnArgs<uint16_t, uint8_t> A{
        (const uint16_t*)io.q,  (const uint8_t*)io.ck,  (const uint8_t*)io.cv,
        (const uint16_t*)io.rk, (const uint16_t*)io.rv, (uint16_t*)io.o,
        io.qs, io.cks, io.cvs, io.rks, io.rvs, io.os};
    const bool shared = io.ck == io.cv && cks == cvs && io.rk == io.rv &&
                        io.rks.ss == io.rvs.ss && io.rks.rs == io.rvs.rs;
    auto kern = shared ? k_attend_mx8<NW, Heads32<D>, true> : k_attend_mx8<NW, Heads32<D>, false>;
    hipLaunchKernelGGL(kern, dim3((unsigned)Tq, (unsigned)p.splits, (unsigned)B), dim3(NW * 64),
                       0, st, A, cks, cvs, topk, (float*)ws, Tq, Nc, m, W, k, q_pos0, scale_log2,
                       raw_pos0, raw_len, p.splits);
    if (p.splits > 1) {
        const int H = NW * 32;
        const uint16_t* po = (const uint16_t*)ws;
        const float* pml = (const float*)(po + B * Tq * p.splits * H * D);
        hipLaunchKernelGGL(k_attend_combine<uint16_t>,
                           dim3((unsigned)Tq, (unsigned)B, (unsigned)((H + 7) / 8)), dim3(256), 0,
                           st, po, pml, (uint16_t*)io.o, io.os, Tq, H, D, p.splits);
    }
}

hipError_t launch_attend_mx8(const AttendPlan& p, int64_t B, int64_t Tq, int64_t H, int64_t Nc,
                             int64_t m, int64_t W, int64_t k, int64_t q_pos0, float scale,
                             const AttendIO& io, const uint8_t* cks, const uint8_t* cvs,
                             const int32_t* topk, int64_t raw_pos0, int64_t raw_len, void* ws,
                             hipStream_t st) {
    if (B == 0 || Tq == 0) return hipSuccess;
#define CSA_MX8_CASE(NN)                                                                        \
    launch_mx8_nw<NN>(p, B, Tq, Nc, m, W, (int)k, q_pos0, scale, io, cks, cvs, topk, raw_pos0, \
                      raw_len, ws, st)
    switch (H / 32) {
        case 1: CSA_MX8_CASE(1); break;
        case 2: CSA_MX8_CASE(2); break;
        case 4: CSA_MX8_CASE(4); break;
        case 8: CSA_MX8_CASE(8); break;
        default: return hipErrorInvalidValue;
    }
#undef CSA_MX8_CASE
    return hipGetLastError();
}

}  // namespace csa
