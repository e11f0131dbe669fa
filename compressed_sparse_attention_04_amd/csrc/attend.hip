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
// per 32 heads) and one split of its key list, in tiles of 64 keys whose
// gathers for tile n+1 are in flight while tile n is computed.  Per tile:
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

#define CSA_LDS __attribute__((address_space(3)))

// Key rows of one tile are copied straight from global memory into LDS
// (global_load_lds, 16 bytes per lane, lane-contiguous).  A row of D bf16 is
// CH = D/8 chunks of 16 bytes; chunk c of tile row r sits in slot
// c ^ (r % CH) so that the 32 rows read by one MFMA operand load hit
// different LDS banks.
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

template <int D>
__device__ __forceinline__ int slot_of(int r, int c) { return c ^ (r & (TileGeom<D>::CH - 1)); }

// Row of key-list entry s (compressed row in ck/cv, or raw row in rk/rv) and
// whether it contributes.  Entries that contribute nothing point at the
// window's first raw row, which always exists.
__device__ __forceinline__ bool key_row(const KeyList& L, int64_t s, int64_t s_end, bool sparse,
                                        const CSA_LDS int32_t* ssel, int64_t nc_t,
                                        int64_t raw_pos0, bool* comp, int64_t* row) {
    *comp = false;
    *row = L.w0 - raw_pos0;
    if (s >= s_end) return false;
    if (s < L.nsel) {
        const int64_t j = sparse ? (int64_t)ssel[s] : s;
        if (j < 0 || j >= nc_t) return false;
        *comp = true;
        *row = j;
        return true;
    }
    *row = L.w0 + (s - L.nsel) - raw_pos0;
    return true;
}

// Issue this wave's copies of the K and V rows of the tile starting at key
// s0; returns the wave's bits of the tile's contribution mask.
template <int NW, int D>
__device__ __forceinline__ uint32_t issue_tile(int64_t s0, int64_t s_end, const KeyList& L,
                                               bool sparse, const CSA_LDS int32_t* ssel,
                                               int64_t nc_t,
                                               int64_t raw_pos0, const uint16_t* ckb,
                                               const uint16_t* cvb, const uint16_t* rkb,
                                               const uint16_t* rvb, CSA_LDS uint8_t* sk,
                                               CSA_LDS uint8_t* sv) {
    using G = TileGeom<D>;
    const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
    uint32_t mask = 0;
#pragma unroll
    for (int ins = wave; ins < G::NINS; ins += NW) {
        const int r = ins * G::RPI + lane / G::CH;
        const int c = slot_of<D>(r, lane % G::CH);   // slot <-> chunk is an involution
        bool comp;
        int64_t row;
        const bool ok = key_row(L, s0 + r, s_end, sparse, ssel, nc_t, raw_pos0, &comp, &row);
        const uint16_t* kp = (comp ? ckb : rkb) + row * D + c * 8;
        const uint16_t* vp = (comp ? cvb : rvb) + row * D + c * 8;
        __builtin_amdgcn_global_load_lds(kp, (CSA_LDS void*)(sk + ins * G::RPI * G::ROWB), 16, 0, 0);
        __builtin_amdgcn_global_load_lds(vp, (CSA_LDS void*)(sv + ins * G::RPI * G::ROWB), 16, 0, 0);
        const uint64_t bal = __ballot(ok && (lane % G::CH) == 0);
#pragma unroll
        for (int x = 0; x < G::RPI; ++x)
            mask |= (uint32_t)((bal >> (x * G::CH)) & 1ull) << (ins * G::RPI + x);
    }
    return mask;
}

// Running softmax state of one lane (one head, half of each key tile).
template <int D>
struct Online {
    f32x16 acc[D / 32];
    float m_run, l_run;
};

// One 32-key tile: S^T = K Q^T, online softmax, O^T += V^T P^T.  K and V
// are the tile's LDS copies; vmask marks the keys that contribute.
template <int D>
__device__ __forceinline__ void tile_compute(Online<D>& S, const bf16x8 (&qop)[D / 16],
                                             const CSA_LDS uint8_t* K, const CSA_LDS uint8_t* V,
                                             uint32_t vmask, float scale_log2) {
    using G = TileGeom<D>;
    const int lane = threadIdx.x % 64, col = lane & 31, kb = lane >> 5;
    // S^T: rows = keys (8*(r/4) + 4*kb + r%4), column = head
    f32x16 sacc = {};
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 a = *reinterpret_cast<const CSA_LDS bf16x8*>(
            K + col * G::ROWB + slot_of<D>(col, 2 * kk + kb) * 16);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qop[kk], sacc, 0, 0, 0);
    }
    if (vmask != ~0u) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int key = 8 * (r / 4) + 4 * kb + (r % 4);
            if (!((vmask >> key) & 1u)) sacc[r] = -INFINITY;
        }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, sacc[r]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float m_new = fmaxf(S.m_run, tmax);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f((S.m_run - m_use) * scale_log2);
    const float mb = -m_use * scale_log2;
    S.m_run = m_new;
    float psum = 0.f;
    uint32_t pb[8];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
        const float p0 = __builtin_amdgcn_exp2f(fmaf(sacc[r], scale_log2, mb));
        const float p1 = __builtin_amdgcn_exp2f(fmaf(sacc[r + 1], scale_log2, mb));
        psum += p0 + p1;
        pb[r / 2] = pack_bf16x2(p0, p1);
    }
    S.l_run = S.l_run * alpha + psum;
    if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int r = 0; r < 16; ++r) S.acc[dt][r] *= alpha;
    }
    // O^T += V^T P^T.  k-step u covers keys 16u..16u+15; k-slot s of lane
    // half kb is key 16u + 8*(s/4) + 4*kb + s%4 (the S^T register order).
    // Each half of the V^T operand is one transposing LDS read: lane
    // (16g + 4j + a) points at V[key 16u + 8h + 4kb + j][32dt + 16(g%2) + 4a].
    const int g = lane >> 4, wj = (lane >> 2) & 3, wa = lane & 3;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        bf16x8 pop;
        {
            u32x4 w = {pb[4 * u], pb[4 * u + 1], pb[4 * u + 2], pb[4 * u + 3]};
            pop = *reinterpret_cast<bf16x8*>(&w);
        }
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
            const int d = 32 * dt + 16 * (g & 1) + 4 * wa;
            const int key0 = 16 * u + 4 * (g >> 1) + wj;
            const int key1 = key0 + 8;
            const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((CSA_LDS bf16x4*)(
                V + key0 * G::ROWB + slot_of<D>(key0, d / 8) * 16 + (d % 8) * 2));
            const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((CSA_LDS bf16x4*)(
                V + key1 * G::ROWB + slot_of<D>(key1, d / 8) * 16 + (d % 8) * 2));
            const bf16x8 a = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            S.acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pop, S.acc[dt], 0, 0, 0);
        }
    }
}

// vmcnt wait (other counters untouched) leaving n copies in flight
#define CSA_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(0x3f70 | ((n) & 15) | (((n) >> 4) << 14))

// Block barrier without a memory fence: LDS writes are drained explicitly
// and the copies each wave waited for are complete, so no outstanding copy
// into another stage is waited for here.
__device__ __forceinline__ void lds_barrier() {
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    __builtin_amdgcn_s_waitcnt(0xc07f);            // lgkmcnt(0)
    __builtin_amdgcn_s_barrier();
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

template <int NW, int D>
__global__ void __launch_bounds__(NW * 64, 2)
k_attend_bf16(const uint16_t* __restrict__ q, const uint16_t* __restrict__ ck,
              const uint16_t* __restrict__ cv, const int32_t* __restrict__ topk,
              const uint16_t* __restrict__ rk, const uint16_t* __restrict__ rv,
              uint16_t* __restrict__ o, float* __restrict__ part, int64_t Tq, int64_t Nc,
              int64_t m, int64_t W, int k, int64_t q_pos0, float scale_log2, int64_t raw_pos0,
              int64_t raw_len, int splits) {
    using G = TileGeom<D>;
    constexpr int NT = NW * 64;
    constexpr int H = NW * 32;
    constexpr int KT = G::KT;
    constexpr int PER = 2 * ((G::NINS + NW - 1) / NW);   // copies per wave per tile
    // the stages live in distinct arrays, so the compiler can tell which
    // stage an LDS read touches and never waits on another stage's copies
    __shared__ __attribute__((aligned(16))) uint8_t sK0[G::BYTES], sV0[G::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t sK1[G::BYTES], sV1[G::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t sK2[G::BYTES], sV2[G::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t sK3[G::BYTES], sV3[G::BYTES];
    __shared__ uint32_t sM0[NW], sM1[NW], sM2[NW], sM3[NW];   // contribution masks
    __shared__ int32_t sSel[2048];                  // this query's kept indices (CSA)

    const int64_t i = blockIdx.x;
    const int split = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
    const int col = lane & 31, kb = lane >> 5;
    const int64_t t = q_pos0 + i;
    const bool sparse = topk != nullptr;
    const KeyList L = key_list(t, m, W, k, sparse);
    const int64_t nc_t = n_candidates(t, m, W);

    // this split's range of the key list, in whole tiles
    const int64_t ntile = (L.len + KT - 1) / KT;
    const int64_t tps = (ntile + splits - 1) / splits;
    const int64_t s_begin = split * tps * KT;
    const int64_t s_end = min(L.len, s_begin + tps * KT);

    const uint16_t* ckb = ck + b * Nc * D;
    const uint16_t* cvb = cv + b * Nc * D;
    const uint16_t* rkb = rk + b * raw_len * D;
    const uint16_t* rvb = rv + b * raw_len * D;

    if (sparse) {
        const int32_t* sel = topk + (b * Tq + i) * k;
        for (int x = tid; x < L.nsel; x += NT) sSel[x] = sel[x];
        __syncthreads();
    }
    const CSA_LDS int32_t* ssel = (const CSA_LDS int32_t*)sSel;

    // Q^T operand: head hq, d = 16*kk + 8*kb + 0..7
    const int hq = wave * 32 + col;
    bf16x8 qop[D / 16];
    {
        const uint16_t* qp = q + ((b * Tq + i) * H + hq) * D + 8 * kb;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
            qop[kk] = *reinterpret_cast<const bf16x8*>(qp + 16 * kk);
    }
    Online<D> S;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) S.acc[dt][r] = 0.f;
    S.m_run = -INFINITY;
    S.l_run = 0.f;

    auto issue = [&](int64_t s0, uint8_t* sk, uint8_t* sv, uint32_t* sm) {
        if (s0 < s_end) {
            const uint32_t mk = issue_tile<NW, D>(s0, s_end, L, sparse, ssel, nc_t, raw_pos0, ckb, cvb,
                                                  rkb, rvb, (CSA_LDS uint8_t*)sk,
                                                  (CSA_LDS uint8_t*)sv);
            if (lane == 0) sm[wave] = mk;
        }
    };
    // one tile: wait for its copies, barrier (the stage written next is then
    // free on every wave), issue the copies three tiles ahead, compute
    auto step = [&](int64_t s0, uint8_t* ck_, uint8_t* cv_, uint32_t* cm_, uint8_t* nk_,
                    uint8_t* nv_, uint32_t* nm_) {
        const int64_t after = min((int64_t)(G::NST - 2), (s_end - s0 - 1) / KT);
        if (after >= 2) CSA_WAIT_VM(2 * PER);
        else if (after == 1) CSA_WAIT_VM(PER);
        else CSA_WAIT_VM(0);
        lds_barrier();
        issue(s0 + (G::NST - 1) * KT, nk_, nv_, nm_);
        uint32_t vm = 0;
#pragma unroll
        for (int w = 0; w < NW; ++w) vm |= cm_[w];
        tile_compute<D>(S, qop, (const CSA_LDS uint8_t*)ck_, (const CSA_LDS uint8_t*)cv_, vm,
                        scale_log2);
    };

    issue(s_begin, sK0, sV0, sM0);
    issue(s_begin + KT, sK1, sV1, sM1);
    issue(s_begin + 2 * KT, sK2, sV2, sM2);
    for (int64_t s0 = s_begin; s0 < s_end; s0 += 4 * KT) {
        step(s0, sK0, sV0, sM0, sK3, sV3, sM3);
        if (s0 + KT >= s_end) break;
        step(s0 + KT, sK1, sV1, sM1, sK0, sV0, sM0);
        if (s0 + 2 * KT >= s_end) break;
        step(s0 + 2 * KT, sK2, sV2, sM2, sK1, sV1, sM1);
        if (s0 + 3 * KT >= s_end) break;
        step(s0 + 3 * KT, sK3, sV3, sM3, sK2, sV2, sM2);
    }
    const float l_tot = S.l_run + __shfl_xor(S.l_run, 32, 64);
    if (splits == 1) {
        const float inv = 1.f / l_tot;
        uint16_t* op = o + ((b * Tq + i) * H + hq) * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                const int d = 32 * dt + 8 * gg + 4 * kb;
                u32x2 w;
                w[0] = pack_bf16x2(S.acc[dt][4 * gg] * inv, S.acc[dt][4 * gg + 1] * inv);
                w[1] = pack_bf16x2(S.acc[dt][4 * gg + 2] * inv, S.acc[dt][4 * gg + 3] * inv);
                *reinterpret_cast<u32x2*>(op + d) = w;
            }
    } else {
        // partial record per (query, split, head): D accumulators, max, sum;
        // the max is stored in the exp2 domain of the combine kernel
        float* pr = part + (((b * Tq + i) * splits + split) * H + hq) * (D + 2);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                const int d = 32 * dt + 8 * gg + 4 * kb;
                f32x4 w = {S.acc[dt][4 * gg], S.acc[dt][4 * gg + 1], S.acc[dt][4 * gg + 2],
                           S.acc[dt][4 * gg + 3]};
                *reinterpret_cast<f32x4*>(pr + d) = w;
            }
        if (kb == 0) {
            pr[D] = S.m_run == -INFINITY ? -INFINITY : S.m_run * scale_log2;
            pr[D + 1] = l_tot;
        }
    }
}

// Log-sum-exp merge of the split partials.  Grid (query, sequence, head
// group of 8); one thread per (head, 4 dims).
template <typename TO>
__global__ void __launch_bounds__(256)
k_attend_combine(const float* __restrict__ part, TO* __restrict__ o, int64_t Tq, int H, int D,
                 int splits) {
    const int64_t i = blockIdx.x, b = blockIdx.y;
    const int per_head = D / 4;
    const int h = blockIdx.z * 8 + threadIdx.x / per_head;
    const int d0 = (threadIdx.x % per_head) * 4;
    if (threadIdx.x >= 8 * per_head || h >= H) return;
    const int64_t sstride = (int64_t)H * (D + 2);
    const float* base = part + ((b * Tq + i) * splits * H + h) * (int64_t)(D + 2);
    float M = -INFINITY;
    for (int s = 0; s < splits; ++s) M = fmaxf(M, base[s * sstride + D]);
    float Lsum = 0.f;
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < splits; ++s) {
        const float* pr = base + s * sstride;
        const float ms = pr[D];
        if (ms == -INFINITY) continue;
        const float wgt = __builtin_amdgcn_exp2f(ms - M);
        Lsum += pr[D + 1] * wgt;
        const f32x4 v = *reinterpret_cast<const f32x4*>(pr + d0);
        a[0] += v[0] * wgt; a[1] += v[1] * wgt; a[2] += v[2] * wgt; a[3] += v[3] * wgt;
    }
    const float inv = 1.f / Lsum;
    TO* op = o + ((b * Tq + i) * H + h) * (int64_t)D + d0;
    if constexpr (sizeof(TO) == 2) {
        u32x2 w;
        w[0] = f32_to_bf16_bits(a[0] * inv) | (f32_to_bf16_bits(a[1] * inv) << 16);
        w[1] = f32_to_bf16_bits(a[2] * inv) | (f32_to_bf16_bits(a[3] * inv) << 16);
        *reinterpret_cast<u32x2*>(op) = w;
    } else {
        f32x4 w = {a[0] * inv, a[1] * inv, a[2] * inv, a[3] * inv};
        *reinterpret_cast<f32x4*>(op) = w;
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
        const int64_t tiles = (max_keys + ATT_KT - 1) / ATT_KT;
        if (rows < 512 && tiles > 2) {
            int64_t want = (512 + rows - 1) / rows;            // ~2 blocks per CU
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
    hipLaunchKernelGGL((k_attend_bf16<NW, D>),
                       dim3((unsigned)Tq, (unsigned)p.splits, (unsigned)B), dim3(NW * 64), 0, st,
                       (const uint16_t*)q, (const uint16_t*)ck, (const uint16_t*)cv, topk,
                       (const uint16_t*)rk, (const uint16_t*)rv, (uint16_t*)o, (float*)ws, Tq, Nc,
                       m, W, k, q_pos0, scale_log2, raw_pos0, raw_len, p.splits);
    if (p.splits > 1) {
        const int H = NW * 32;
        hipLaunchKernelGGL(k_attend_combine<uint16_t>,
                           dim3((unsigned)Tq, (unsigned)B, (unsigned)((H + 7) / 8)), dim3(256), 0,
                           st, (const float*)ws, (uint16_t*)o, Tq, H, D, p.splits);
    }
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
