// indexer.hip -- Lightning Indexer scores and exact top-k selection
// (jiwasawa.github.io post, CSA indexer bullet: every query token scores the
// compressed entries with a light indexer and keeps the top k; studioglobal.ai
// answer, CSA bullet: FP4 indexer, 512 blocks per query; ai-papers.net,
// hybrid attention section: the indexer searches the already 4x shorter
// compressed sequence at FP4).
//
//   I(t, j) = sum_{h < HI} max(0, qhat[t][h] . khat[j])
//
// The dot products are a dense FP4 contraction, so they run on the gfx950
// scaled MFMA (V_MFMA_SCALE_F32_32X32X64_F8F6F4, e2m1 operands, E8M0 block
// scales).  One MFMA scores 32 keys against 32 (query, head) rows, i.e.
// 32/HI queries; products of e2m1 values are exact and every partial sum of
// N(0,1)-derived data fits fp32's 24-bit significand, so the fp32 scores are
// exact and the selection is bit-reproducible.
//
// Grid: (candidate chunk, query tile, sequence).  A block scores one chunk
// of <= CH candidates for the tile's queries into LDS, then selects each
// query's chunk-local top-k with the block-wide threshold search of
// select.h.  With one chunk the result is final; otherwise each chunk's
// list (key, index) goes to the workspace and k_topk_merge selects the top
// k of their union.  Chunks and lists are in ascending index order, so a
// selection that keeps position order yields ascending indices.
#include "internal.h"
#include "mxfp4.h"
#include "select.h"

namespace csa {

constexpr int IDX_NT = 256;
constexpr int SCORE_WORDS = 32768;          // 128 KB of LDS keys per block
constexpr int MERGE_MAX = 65536;            // largest union the merge handles

__device__ __forceinline__ uint32_t score_key(float s) {
    // +1 so that a +0 score still beats "not a candidate" (key 0)
    return (s == 0.f ? 0u : __float_as_uint(s)) + 1u;
}

template <typename T, int HI>
__global__ void __launch_bounds__(IDX_NT)
k_index_chunk(const T* __restrict__ q_idx, RowStrides qs, const uint8_t* __restrict__ kc,
              const uint8_t* __restrict__ ks, int32_t* __restrict__ topk,
              u32x2* __restrict__ part, int64_t Tq, int dI, int64_t Nc, int64_t m, int64_t W,
              int k, int64_t q_pos0, int ch, int64_t n_chunks) {
    constexpr int QT = 32 / HI;
    constexpr int EPT = SCORE_WORDS / QT / IDX_NT;     // keys per thread at selection
    extern __shared__ uint32_t skey[];                 // [qv][ch]
    __shared__ SelectSmem sm;

    const int chunk = blockIdx.x;
    const int64_t q0 = (int64_t)blockIdx.y * QT;
    const int64_t b = blockIdx.z;
    const int qv = (int)min((int64_t)QT, Tq - q0);
    const int64_t c0 = (int64_t)chunk * ch;
    const int64_t nc_last = n_candidates(q_pos0 + q0 + qv - 1, m, W);
    if (c0 >= nc_last) {                               // no query of the tile reaches here
        if (n_chunks == 1)                             // final rows: nothing kept
            for (int s = threadIdx.x; s < qv * k; s += IDX_NT) topk[(b * Tq + q0) * k + s] = -1;
        return;
    }
    const int nkeys = (int)min((int64_t)ch, nc_last - c0);

    const int tid = threadIdx.x, lane = tid % WAVE, wave = tid / WAVE;
    const int row = lane & 31, kb = lane >> 5;

    // A operand: MXFP4 encoding of query row (qi, h) = (row / HI, row % HI),
    // block kb of its dI values (dI = 32 leaves block 1 zero).
    i32x8 aop = {0, 0, 0, 0, 0, 0, 0, 0};
    int sa = 127;
    {
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
    // candidate counts of the queries this lane's output rows belong to
    const int kbq = kb * 4 / HI;                       // query offset of this lane half
    constexpr int NU = 16 / HI;                        // queries per lane
    int64_t ncq[NU];
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        // output rows 8g + 4kb + i, i < 4  ->  query (8g + i)/HI + kbq
        const int g = (u * HI) / 4, i = (u * HI) % 4;
        const int qi = (8 * g + i) / HI + kbq;
        ncq[u] = qi < qv ? n_candidates(q_pos0 + q0 + qi, m, W) : 0;
    }

    const int ntiles = (nkeys + 31) / 32;
    const int kbytes = dI / 2, kscales = dI / 32;
    for (int tile = wave; tile < ntiles; tile += IDX_NT / WAVE) {
        const int jj = tile * 32 + row;
        const int64_t j = c0 + jj;
        i32x8 bop = {0, 0, 0, 0, 0, 0, 0, 0};
        int sbk = 127;
        if (jj < nkeys && kb < kscales) {
            u32x4 w = __builtin_nontemporal_load(
                reinterpret_cast<const u32x4*>(kc + (b * Nc + j) * kbytes + kb * 16));
            bop[0] = (int)w[0]; bop[1] = (int)w[1]; bop[2] = (int)w[2]; bop[3] = (int)w[3];
            sbk = ks[(b * Nc + j) * kscales + kb];
        }
        f32x16 acc = {};
        acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop, bop, acc, 4, 4, 0, sa, 0, sbk);
        // acc[r] = row 8*(r/4) + 4*kb + r%4, key column `row`
#pragma unroll
        for (int u = 0; u < NU; ++u) {
            float s = 0.f;
#pragma unroll
            for (int hh = 0; hh < HI; ++hh) {
                const int r = u * HI + hh;             // rows of query u are consecutive
                s += fmaxf(acc[r], 0.f);
            }
            const int g = (u * HI) / 4, i = (u * HI) % 4;
            const int qi = (8 * g + i) / HI + kbq;
            if (qi < qv && jj < nkeys)
                skey[qi * ch + jj] = (j < ncq[u]) ? score_key(s) : 0u;
        }
    }
    __syncthreads();

    for (int qi = 0; qi < qv; ++qi) {
        const int64_t nc = n_candidates(q_pos0 + q0 + qi, m, W);
        if (c0 >= nc) {                                // the merge never reads this chunk
            if (n_chunks == 1)
                for (int s = tid; s < k; s += IDX_NT) topk[(b * Tq + q0 + qi) * k + s] = -1;
            continue;
        }
        const int nk = (int)min((int64_t)nkeys, nc - c0);
        uint32_t key[EPT];
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int p = tid * EPT + e;
            key[e] = p < nk ? skey[qi * ch + p] : 0u;
        }
        int base, total;
        uint32_t flags = block_topk_select<IDX_NT, EPT>(key, k, sm, &base, &total);
        const int64_t bq = b * Tq + q0 + qi;
        if (n_chunks == 1) {
            int32_t* out = topk + bq * k;
#pragma unroll
            for (int e = 0; e < EPT; ++e)
                if (flags & (1u << e)) out[base++] = (int32_t)(c0 + tid * EPT + e);
            for (int s = total + tid; s < k; s += IDX_NT) out[s] = -1;
        } else {
            u32x2* out = part + (bq * n_chunks + chunk) * k;
#pragma unroll
            for (int e = 0; e < EPT; ++e)
                if (flags & (1u << e)) {
                    u32x2 v = {key[e], (uint32_t)(c0 + tid * EPT + e)};
                    out[base++] = v;
                }
            for (int s = total + tid; s < k; s += IDX_NT) {
                u32x2 z = {0u, 0u};
                out[s] = z;
            }
        }
        __syncthreads();
    }
}

// Top k of the union of a query's chunk lists.
template <int NT, int EPT>
__global__ void __launch_bounds__(NT)
k_topk_merge(const u32x2* __restrict__ part, int32_t* __restrict__ topk, int64_t Tq,
             int64_t n_chunks, int k, int ch, int64_t q_pos0, int64_t m, int64_t W) {
    __shared__ SelectSmem sm;
    const int64_t q = blockIdx.x, b = blockIdx.y;
    const int64_t bq = b * Tq + q;
    const int64_t nc = n_candidates(q_pos0 + q, m, W);
    const int64_t nchk = (nc + ch - 1) / ch;
    const int64_t ne = nchk * k;                        // entries in the union
    const u32x2* src = part + bq * n_chunks * k;
    const int tid = threadIdx.x;
    uint32_t key[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        const int64_t p = (int64_t)tid * EPT + e;
        key[e] = p < ne ? src[p][0] : 0u;
    }
    int base, total;
    uint32_t flags = block_topk_select<NT, EPT>(key, k, sm, &base, &total);
    int32_t* out = topk + bq * k;
#pragma unroll
    for (int e = 0; e < EPT; ++e)
        if (flags & (1u << e)) out[base++] = (int32_t)src[(int64_t)tid * EPT + e][1];
    for (int s = total + tid; s < k; s += NT) out[s] = -1;
}

int stream_max_candidates();
int decode_max_candidates();
int decode_max_rows();
size_t decode_ws_bytes(int64_t B, int64_t Tq, int64_t ncap, int k);
hipError_t launch_index_stream(int dt, int64_t B, int64_t Tq, int HI, int dI, int64_t Nc,
                               int64_t m, int64_t W, int k, int64_t q_pos0, const void* q_idx,
                               RowStrides qs, const uint8_t* kc, const uint8_t* ks,
                               int32_t* topk, hipStream_t st);
hipError_t launch_index_decode(int dt, int64_t B, int64_t Tq, int HI, int dI, int64_t Nc,
                               int64_t m, int64_t W, int k, int64_t q_pos0, const void* q_idx,
                               RowStrides qs, const uint8_t* kc, const uint8_t* ks,
                               int32_t* topk, void* ws, hipStream_t st);

IndexPlan plan_index(int64_t B, int64_t Tq, int HI, int dI, int64_t Nc, int64_t m, int64_t W,
                     int k, int64_t q_pos0) {
    IndexPlan p{};
    p.qt = 32 / HI;
    p.ch = SCORE_WORDS / p.qt;
    p.n_qtiles = (Tq + p.qt - 1) / p.qt;
    int64_t maxc = Tq > 0 ? n_candidates(q_pos0 + Tq - 1, m, W) : 0;
    p.n_chunks = maxc > 0 ? (maxc + p.ch - 1) / p.ch : 1;
    if (Tq <= decode_max_rows() && maxc > 4096 && maxc <= decode_max_candidates()) {
        p.path = IDX_DECODE;
        p.ws_bytes = decode_ws_bytes(B, Tq, maxc, k);
    } else if (maxc <= stream_max_candidates()) {
        p.path = IDX_STREAM;
        p.ws_bytes = 0;
    } else {
        p.path = IDX_CHUNK;
        p.ws_bytes = p.n_chunks > 1 ? (size_t)(B * Tq * p.n_chunks * k) * sizeof(u32x2) : 0;
    }
    (void)Nc; (void)dI;
    return p;
}

int64_t index_merge_max() { return MERGE_MAX; }

template <typename T, int HI>
static hipError_t launch_chunk(const IndexPlan& p, int64_t B, int64_t Tq, int dI, int64_t Nc,
                               int64_t m, int64_t W, int k, int64_t q_pos0, const void* q_idx,
                               RowStrides qs, const uint8_t* kc, const uint8_t* ks,
                               int32_t* topk, void* ws, hipStream_t st) {
    const int qv = (int)min((int64_t)p.qt, Tq);
    size_t lds = (size_t)qv * p.ch * sizeof(uint32_t);
    auto kern = k_index_chunk<T, HI>;
    hipFuncSetAttribute((const void*)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                        (int)(SCORE_WORDS * sizeof(uint32_t)));
    dim3 grid((unsigned)p.n_chunks, (unsigned)p.n_qtiles, (unsigned)B);
    hipLaunchKernelGGL(kern, grid, dim3(IDX_NT), lds, st, (const T*)q_idx, qs, kc, ks, topk,
                       (u32x2*)ws, Tq, dI, Nc, m, W, k, q_pos0, p.ch, p.n_chunks);
    return hipGetLastError();
}

template <int NT, int EPT>
static void launch_merge(const IndexPlan& p, int64_t B, int64_t Tq, int k, int64_t q_pos0,
                         int64_t m, int64_t W, int32_t* topk, const void* ws, hipStream_t st) {
    hipLaunchKernelGGL((k_topk_merge<NT, EPT>), dim3((unsigned)Tq, (unsigned)B), dim3(NT), 0,
                       st, (const u32x2*)ws, topk, Tq, p.n_chunks, k, p.ch, q_pos0, m, W);
}

hipError_t launch_index_topk(int dt, const IndexPlan& p, int64_t B, int64_t Tq, int HI, int dI,
                             int64_t Nc, int64_t m, int64_t W, int k, int64_t q_pos0,
                             const void* q_idx, RowStrides qs, const uint8_t* kc,
                             const uint8_t* ks, int32_t* topk, void* ws, hipStream_t st) {
    if (B == 0 || Tq == 0) return hipSuccess;
    if (p.path == IDX_STREAM)
        return launch_index_stream(dt, B, Tq, HI, dI, Nc, m, W, k, q_pos0, q_idx, qs, kc, ks,
                                   topk, st);
    if (p.path == IDX_DECODE)
        return launch_index_decode(dt, B, Tq, HI, dI, Nc, m, W, k, q_pos0, q_idx, qs, kc, ks,
                                   topk, ws, st);
    hipError_t e;
#define CSA_IDX_CASE(TT, HH)                                                                  \
    e = launch_chunk<TT, HH>(p, B, Tq, dI, Nc, m, W, k, q_pos0, q_idx, qs, kc, ks, topk, ws, st)
    if (dt == 0) {
        if (HI == 1) CSA_IDX_CASE(float, 1);
        else if (HI == 2) CSA_IDX_CASE(float, 2);
        else CSA_IDX_CASE(float, 4);
    } else {
        if (HI == 1) CSA_IDX_CASE(uint16_t, 1);
        else if (HI == 2) CSA_IDX_CASE(uint16_t, 2);
        else CSA_IDX_CASE(uint16_t, 4);
    }
#undef CSA_IDX_CASE
    if (e != hipSuccess || p.n_chunks == 1) return e;
    const int64_t ne = p.n_chunks * (int64_t)k;
    if (ne <= 256 * 4) launch_merge<256, 4>(p, B, Tq, k, q_pos0, m, W, topk, ws, st);
    else if (ne <= 256 * 16) launch_merge<256, 16>(p, B, Tq, k, q_pos0, m, W, topk, ws, st);
    else if (ne <= 1024 * 16) launch_merge<1024, 16>(p, B, Tq, k, q_pos0, m, W, topk, ws, st);
    else if (ne <= 1024 * 32) launch_merge<1024, 32>(p, B, Tq, k, q_pos0, m, W, topk, ws, st);
    else launch_merge<1024, 64>(p, B, Tq, k, q_pos0, m, W, topk, ws, st);
    return hipGetLastError();
}

}  // namespace csa
