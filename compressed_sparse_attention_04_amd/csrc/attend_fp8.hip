// attend_fp8.hip -- shared-KV multi-query attention with FP8 arithmetic
// (ai-papers.net article, hybrid attention section: most KV entries are kept
// in FP8; jiwasawa.github.io post: CSA "Shared Key-Value MQA" over the
// selected entries, HCA dense attention over every compressed entry, SWA
// branch over the newest tokens).
//
// Every row the attention reads is an FP8 row: E4M3 codes with one scale 2^e
// per row of 128 values (a 32-bit word holding the fp32 bits of 2^e): the
// compressed K/V entries, the raw window K/V rows, and the query's head rows,
// which the kernel encodes itself with the same rule.
// The key list and its split into tiles are those of the bf16 kernel, with
// tiles of 64 keys.  Per tile and wave (32 heads):
//   S^T = K Q^T      2 halves x 2 V_MFMA_SCALE_F32_32X32X64_F8F6F4, the K and
//                    Q exponents as the MFMA's block scales
//   online softmax in fp32 (exp2 domain; the reference moves once a score
//   would give p > 4), row sums of the unrounded probabilities
//   O^T += V^T P^T   4 scaled FP8 MFMAs (one per 32 dims).  The product
//                    contracts over keys, so V's per-key exponent cannot be
//                    a block scale: it is folded into P, p' = p * 2^(eV - E
//                    + 6) with E the tile's largest V exponent (p' <= 256;
//                    2^(E - 6) becomes P's block scale; p * 2^eV is one
//                    multiply by the row's scale word), and p' is rounded to
//                    E4M3 for the MFMA.  p' stays in E4M3's normal range
//                    (relative error <= 2^-4) down to p = 2^(-12 + E - eV).
// V^T operands come from transposing LDS reads (ds_read_b64_tr_b8).  K and
// V codes of a tile are copied straight into LDS (global_load_lds) three
// tiles ahead, and the S^T products of a tile are issued one step before
// its softmax, so that they run while the previous tile's softmax takes the
// vector unit.  With splits, the bf16 partials go to the combine kernel of
// the bf16 path.
#include "attend_common.h"
#include "common.h"
#include "internal.h"

namespace csa {

typedef int i32x2 __attribute__((ext_vector_type(2)));

// One LDS stage: K codes [64][128] | V codes [64][128] (16-byte chunks
// swizzled by row) | K scale words [64] | V scale words [64].
struct F8Geom {
    static constexpr int D = 128;
    static constexpr int KT = 64;                    // keys per tile
    static constexpr int ROWB = 128;                 // code bytes per row
    static constexpr int CODE_B = KT * ROWB;         // 8192 per tensor
    static constexpr int KS_OFF = 2 * CODE_B;
    static constexpr int VS_OFF = KS_OFF + KT * 4;
    static constexpr int BYTES = VS_OFF + KT * 4;    // 16896
    static constexpr int NCODE = CODE_B / 1024;      // wave-wide code copies per tensor
    static constexpr int NCOPY = 2 * NCODE + 2;      // per tile: codes, then the scale words
};

// Chunk c of row r sits in slot c ^ f8_swz(r), f8_swz a bit permutation of
// q = (r / 2) mod 8 (bit 0 -> 1, bit 1 -> 0, bit 2 -> 2).  Rows 128 bytes
// apart alternate between the two halves of the 64 banks, so:
//   K operand read (16 lanes: rows 0..15 of a half-tile, one chunk): the
//     slots are distinct per row parity;
//   V^T transposing read (32 lanes: 8 rows 4h + {0..3, 8..11} + 16x, chunks
//     2b and 2b + 1): the 4 rows of one parity get swizzles of one parity
//     class with distinct upper bits, so the 8 (row, chunk) slots differ.
__device__ __forceinline__ int f8_swz(int r) {
    const int q = (r >> 1) & 7;
    return ((q & 1) << 1) | ((q >> 1) & 1) | (q & 4);
}

// Copies per tile: K codes (8 wave-wide copies of 8 rows), V codes (8), K
// scale words (1), V scale words (1).  Wave w of NW takes code copies w,
// w + NW, ... of each tensor and one scale copy: K's scale words on even
// waves, V's on odd ones (both on a lone wave).  Waves that copy the same
// scale words write the same bytes.  Every wave thus issues the same
// number of copies per tile, so the waits for them are constants.
template <int NW>
constexpr int f8_copies() {
    return 2 * (F8Geom::NCODE / NW) + (NW == 1 ? 2 : 1);
}

// LDS address of a stage, computed where it is used: the loop runs the four
// stages in turn, and addresses derived from four constant stage bases would
// otherwise be kept in registers across the loop.
__device__ __forceinline__ uint32_t f8_stage(const CSA_LDS uint8_t* stg) {
    uint32_t a = (uint32_t)(uintptr_t)stg;
    asm volatile("" : "+s"(a));
    return a;
}

// Rows of one sequence: codes (128 bytes per row) and scale words (4 bytes)
struct F8Rows {
    const uint8_t *ck, *cv, *cks, *cvs, *rk, *rv, *rks, *rvs;
};

// Copies of wave `wave` (uniform) for tile tau into stage stg, in two parts:
// f8_plan forms the lane's row offsets, f8_go issues the copies.  Tiles
// ct.. are window tiles; rows past the end of a part repeat an existing row
// (masked later).  Offsets fit 32 bits (rows * 128 < 2^31, checked on the
// host).  Every choice is uniform, so it compiles to scalar selects.  The
// prologue plans three tiles before issuing any copy: no address register
// is rewritten while a copy that used it may still be in flight, which the
// compiler would otherwise answer with a wait for every copy.
template <int NW>
struct F8Plan {
    uint32_t code[F8Geom::NCODE / NW];    // byte offset of the lane's 16-byte chunk
    uint32_t scale;                       // byte offset of row `lane`'s scale word
    bool comp;
};

template <int NW>
__device__ __forceinline__ F8Plan<NW> f8_plan(int wave, int tau, int ct, int nval, int nwin,
                                              int raw_first, bool sparse,
                                              const CSA_LDS int32_t* ssel) {
    using G = F8Geom;
    static_assert(G::NCODE % NW == 0, "code copies are dealt evenly");
    const int lane = threadIdx.x % 64;
    F8Plan<NW> p;
    p.comp = tau < ct;
    const bool gather = p.comp && sparse;
    const int base = G::KT * (p.comp ? tau : tau - ct);
    // rows of consecutive sources: off + min(base + r, lim)
    const int off = p.comp ? 0 : raw_first, lim = p.comp ? nval - 1 : nwin - 1;
    auto row_of = [&](int r) { return gather ? ssel[base + r] : off + min(base + r, lim); };
#pragma unroll
    for (int u = 0; u < G::NCODE / NW; ++u) {
        const int r = (wave + NW * u) * 8 + lane / 8;
        p.code[u] = (uint32_t)row_of(r) * G::ROWB + (((lane % 8) ^ f8_swz(r)) * 16);
    }
    p.scale = (uint32_t)row_of(lane) * 4;
    return p;
}

template <int NW>
__device__ __forceinline__ void f8_go(int wave, const F8Plan<NW>& p, F8Rows src,
                                      CSA_LDS uint8_t* stg) {
    using G = F8Geom;
    // selects between values (a select between member addresses would put
    // the struct in scratch memory)
    const bool c = p.comp;
    const uint8_t* kc = (const uint8_t*)(c ? (uintptr_t)src.ck : (uintptr_t)src.rk);
    const uint8_t* vc = (const uint8_t*)(c ? (uintptr_t)src.cv : (uintptr_t)src.rv);
    const uint8_t* ks = (const uint8_t*)(c ? (uintptr_t)src.cks : (uintptr_t)src.rks);
    const uint8_t* vs = (const uint8_t*)(c ? (uintptr_t)src.cvs : (uintptr_t)src.rvs);
#pragma unroll
    for (int u = 0; u < G::NCODE / NW; ++u) {
        const int ins = wave + NW * u;
        __builtin_amdgcn_global_load_lds(kc + p.code[u], (CSA_LDS void*)(stg + ins * 1024), 16,
                                         0, 0);
        __builtin_amdgcn_global_load_lds(vc + p.code[u],
                                         (CSA_LDS void*)(stg + G::CODE_B + ins * 1024), 16, 0, 0);
    }
    if (NW == 1 || wave % 2 == 0)
        __builtin_amdgcn_global_load_lds(ks + p.scale, (CSA_LDS void*)(stg + G::KS_OFF), 4, 0, 0);
    if (NW == 1 || wave % 2 == 1)
        __builtin_amdgcn_global_load_lds(vs + p.scale, (CSA_LDS void*)(stg + G::VS_OFF), 4, 0, 0);
}

// Per-wave engine for 32 heads of the block's query token.  Lane l holds
// head l % 32; h = l / 32 selects its half of every MFMA operand:
//   A/B operand bytes 0-15 of lane (x + 32h) are in block 0 of the 64-long
//   contraction, bytes 16-31 in block 1, and lane x + 32j gives the scale
//   of block j.  For QK (contraction over dims 64s..64s+63) lane x + 32h
//   holds dims 64s + 16h + 0..15 and 64s + 32 + 16h + 0..15.  For PV
//   (contraction over the tile's 64 keys) byte 16t + r holds key
//   32t + 8(r/4) + 4h + r%4, which is where S^T of half t leaves that key.
struct Fp8Heads {
    f32x16 acc[4];
    i32x8 qop[2];
    int qsc;                      // E8M0 exponent of this lane's head row
    float m_run, mb, l_run;

    u32x4 qraw[8];                // the lane's 64 query values (bf16), until encoded
    uint32_t ko[5], vo[5];        // the lane's LDS read offsets within a stage

    // K operand reads: chunk 4s + h (+ 2) of row 32t + rr (the two halves t
    // are 4 KB apart), and row rr's scale word.  V^T reads: group g = lane /
    // 16 reads dims 32b + 16 (g % 2) + 0..15 of 8 keys per read; lane 2j + a
    // of the group points at key 16x + 4h + 8 (j / 4) + j % 4, bytes
    // 8a..8a+7.  The swizzle of those keys does not depend on x, so the four
    // reads of one dim block are one address 16 key rows (2 KB) apart.  Then
    // the V scale words of the lane's keys 32t + 8q + 4h + 0..3.
    __device__ __forceinline__ void offsets() {
        using G = F8Geom;
        const int lane = threadIdx.x % 64, rr = lane & 31, h = lane >> 5;
        const int sw = f8_swz(rr);                  // = f8_swz(32 t + rr)
#pragma unroll
        for (int c = 0; c < 4; ++c) ko[c] = rr * G::ROWB + (((2 * c + h) ^ sw) * 16);
        ko[4] = G::KS_OFF + rr * 4;
        const int gi = lane & 15, j = gi >> 1, a = gi & 1, c16 = (lane >> 4) & 1;
        const int key0 = 4 * h + 8 * (j >> 2) + (j & 3);
        const int swv = f8_swz(key0);
#pragma unroll
        for (int c = 0; c < 4; ++c)
            vo[c] = G::CODE_B + key0 * G::ROWB + 8 * a + (((2 * c + c16) ^ swv) * 16);
        vo[4] = G::VS_OFF + 16 * h;
    }

    // qh: the query token's [H][128] bf16 rows, from this wave's first head;
    // lane (c + 32h) holds dims 16h + 32u + 0..15 (u = 0..3) of head c.  The
    // loads are one asm block that waits for them (and for every copy issued
    // before it), so the compiler does not wait for later copies at the
    // first use of the query values.
    __device__ __forceinline__ void load_q(const uint16_t* qh) {
        const int lane = threadIdx.x % 64, c = lane & 31, h = lane >> 5;
        const uint16_t* qp = qh + c * F8Geom::D + 16 * h;
        asm volatile(
            "global_load_dwordx4 %0, %8, off\n\t"
            "global_load_dwordx4 %1, %8, off offset:16\n\t"
            "global_load_dwordx4 %2, %8, off offset:64\n\t"
            "global_load_dwordx4 %3, %8, off offset:80\n\t"
            "global_load_dwordx4 %4, %8, off offset:128\n\t"
            "global_load_dwordx4 %5, %8, off offset:144\n\t"
            "global_load_dwordx4 %6, %8, off offset:192\n\t"
            "global_load_dwordx4 %7, %8, off offset:208\n\t"
            "s_waitcnt vmcnt(0)"
            : "=&v"(qraw[0]), "=&v"(qraw[1]), "=&v"(qraw[2]), "=&v"(qraw[3]), "=&v"(qraw[4]),
              "=&v"(qraw[5]), "=&v"(qraw[6]), "=&v"(qraw[7])
            : "v"(qp)
            : "memory");
    }

    // Encodes the head row: e = floor(log2 max|q|) - 8 (>= -127), and each
    // q * 2^-e (exact), clamped to +-448, rounded to the nearest E4M3 value
    // with ties to even by the hardware conversion -- the same code as
    // rounding first and saturating, since 448 is the largest finite value.
    __device__ __forceinline__ void encode_q() {
        float v[4][16];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int x = 0; x < 2; ++x)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    v[u][8 * x + 2 * j] = __uint_as_float(qraw[2 * u + x][j] << 16);
                    v[u][8 * x + 2 * j + 1] = __uint_as_float(qraw[2 * u + x][j] & 0xffff0000u);
                }
        float amax = 0.f;
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int i = 0; i < 16; ++i) amax = fmaxf(amax, fabsf(v[u][i]));
        amax = max_halves(amax);
        int e = (int)((__float_as_uint(amax) >> 23) & 0xff) - 127 - 8;
        e = e < -127 ? -127 : e;
        qsc = e + 127;
        typedef short s16x2 __attribute__((ext_vector_type(2)));
        // qop[s] word w: u = 2s + w / 4, dims 16h + 32u + 4 (w % 4) + 0..3
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int w = 0; w < 8; ++w) {
                const int u = 2 * s + w / 4, i0 = 4 * (w % 4);
                float y[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    y[i] = __builtin_amdgcn_fmed3f(ldexpf(v[u][i0 + i], -e), -448.f, 448.f);
                s16x2 pk = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s16x2{0, 0}, y[0], y[1], 1.f,
                                                                     false);
                pk = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(pk, y[2], y[3], 1.f, true);
                qop[s][w] = __builtin_bit_cast(int, pk);
            }
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[b][r] = 0.f;
        m_run = -INFINITY;
        mb = 0.f;
        l_run = 0.f;
    }

    // S^T of both halves of the tile in stage stg into s.  The K reads are
    // one asm block that waits for itself: the tile's copies are complete
    // (explicit vmcnt wait and barrier), and the compiler, which cannot
    // always tell a stage's reads from the copies in flight into the other
    // stages, would otherwise wait for every copy.  The products are left
    // running; the softmax of the previous tile overlaps them.
    __device__ __forceinline__ void qk(const CSA_LDS uint8_t* stg, f32x16 (&s)[2]) {
        const uint32_t sb = f8_stage(stg);
        const uint32_t a0 = sb + ko[0], a1 = sb + ko[1], a2 = sb + ko[2], a3 = sb + ko[3];
        const uint32_t as = sb + ko[4];
        u32x4 k[2][4];
        uint32_t ksw[2];
        asm volatile(
            "ds_read_b128 %0, %10\n\t"
            "ds_read_b128 %1, %11\n\t"
            "ds_read_b128 %2, %12\n\t"
            "ds_read_b128 %3, %13\n\t"
            "ds_read_b128 %4, %10 offset:4096\n\t"
            "ds_read_b128 %5, %11 offset:4096\n\t"
            "ds_read_b128 %6, %12 offset:4096\n\t"
            "ds_read_b128 %7, %13 offset:4096\n\t"
            "ds_read_b32 %8, %14\n\t"
            "ds_read_b32 %9, %14 offset:128\n\t"
            "s_waitcnt lgkmcnt(0)"
            : "=&v"(k[0][0]), "=&v"(k[0][1]), "=&v"(k[0][2]), "=&v"(k[0][3]), "=&v"(k[1][0]),
              "=&v"(k[1][1]), "=&v"(k[1][2]), "=&v"(k[1][3]), "=&v"(ksw[0]), "=&v"(ksw[1])
            : "v"(a0), "v"(a1), "v"(a2), "v"(a3), "v"(as));
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            f32x16 s_ = {};
#pragma unroll
            for (int q = 0; q < 2; ++q) {
                const u32x4 lo = k[t][2 * q], hi = k[t][2 * q + 1];
                const i32x8 kop = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3],
                                   (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
                // the row's E8M0 exponent for both blocks of the step
                s_ = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                    kop, qop[q], s_, 0, 0, 0, (int)(ksw[t] >> 23), 0, qsc);
            }
            s[t] = s_;
        }
    }

    // The tile in stage stg, whose S^T is in s: its V scale words and V^T
    // operands (one asm block that waits for itself, as the K reads), the
    // softmax (the first nvalid keys count), P folded with the V exponents
    // and rounded to E4M3, then O^T += V^T P^T.
    __device__ __forceinline__ void rest(const CSA_LDS uint8_t* stg, f32x16 (&s)[2], int nvalid,
                                         float scale_log2) {
        using G = F8Geom;
        const int lane = threadIdx.x % 64, h = lane >> 5;
        // V scale words of this lane's keys: 4 consecutive keys 32t + 8q + 4h + 0..3
        u32x4 ve[2][4];
        i32x2 rd[4][4];                             // V^T operands
        {
            const uint32_t sb = f8_stage(stg);
            const uint32_t v0 = sb + vo[0], v1 = sb + vo[1], v2 = sb + vo[2], v3 = sb + vo[3];
            const uint32_t av = sb + vo[4];
            asm volatile(
                "ds_read_b128 %0, %28\n\t"
                "ds_read_b128 %1, %28 offset:32\n\t"
                "ds_read_b128 %2, %28 offset:64\n\t"
                "ds_read_b128 %3, %28 offset:96\n\t"
                "ds_read_b128 %4, %28 offset:128\n\t"
                "ds_read_b128 %5, %28 offset:160\n\t"
                "ds_read_b128 %6, %28 offset:192\n\t"
                "ds_read_b128 %7, %28 offset:224\n\t"
                "ds_read_b64_tr_b8 %8, %24\n\t"
                "ds_read_b64_tr_b8 %9, %24 offset:2048\n\t"
                "ds_read_b64_tr_b8 %10, %24 offset:4096\n\t"
                "ds_read_b64_tr_b8 %11, %24 offset:6144\n\t"
                "ds_read_b64_tr_b8 %12, %25\n\t"
                "ds_read_b64_tr_b8 %13, %25 offset:2048\n\t"
                "ds_read_b64_tr_b8 %14, %25 offset:4096\n\t"
                "ds_read_b64_tr_b8 %15, %25 offset:6144\n\t"
                "ds_read_b64_tr_b8 %16, %26\n\t"
                "ds_read_b64_tr_b8 %17, %26 offset:2048\n\t"
                "ds_read_b64_tr_b8 %18, %26 offset:4096\n\t"
                "ds_read_b64_tr_b8 %19, %26 offset:6144\n\t"
                "ds_read_b64_tr_b8 %20, %27\n\t"
                "ds_read_b64_tr_b8 %21, %27 offset:2048\n\t"
                "ds_read_b64_tr_b8 %22, %27 offset:4096\n\t"
                "ds_read_b64_tr_b8 %23, %27 offset:6144\n\t"
                "s_waitcnt lgkmcnt(0)"
                : "=&v"(ve[0][0]), "=&v"(ve[0][1]), "=&v"(ve[0][2]), "=&v"(ve[0][3]),
                  "=&v"(ve[1][0]), "=&v"(ve[1][1]), "=&v"(ve[1][2]), "=&v"(ve[1][3]),
                  "=&v"(rd[0][0]), "=&v"(rd[0][1]), "=&v"(rd[0][2]), "=&v"(rd[0][3]),
                  "=&v"(rd[1][0]), "=&v"(rd[1][1]), "=&v"(rd[1][2]), "=&v"(rd[1][3]),
                  "=&v"(rd[2][0]), "=&v"(rd[2][1]), "=&v"(rd[2][2]), "=&v"(rd[2][3]),
                  "=&v"(rd[3][0]), "=&v"(rd[3][1]), "=&v"(rd[3][2]), "=&v"(rd[3][3])
                : "v"(v0), "v"(v1), "v"(v2), "v"(v3), "v"(av));
        }
        // mask, maximum, lazy rescaling (as the bf16 engine, with p <= 4 so
        // that P has 6 octaves of headroom below E4M3's largest value)
        if (nvalid < G::KT) {                           // wave-uniform
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const int lim = nvalid - 32 * t - 4 * h;
#pragma unroll
                for (int r = 0; r < 16; ++r)
                    if (8 * (r / 4) + (r % 4) >= lim) s[t][r] = -INFINITY;
            }
        }
        float tm = -INFINITY;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) tm = fmaxf(tm, s[t][r]);
        const float tmax = max_halves(tm);
        const bool grow = (tmax - m_run) * scale_log2 > 2.f;
        if (__ballot(grow)) {
            float alpha = 1.f;
            if (grow) {
                alpha = __builtin_amdgcn_exp2f((m_run - tmax) * scale_log2);   // 0 from -inf
                m_run = tmax;
                mb = -tmax * scale_log2;
            }
            l_run *= alpha;
#pragma unroll
            for (int b = 0; b < 4; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[b][r] *= alpha;
        }
        // probabilities (<= 4, in place of the scores), their sum, and the
        // largest V scale word
        uint32_t emax = 7u << 23;                    // E >= 7: the block scale E - 6 >= 1
        float ps[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                s[t][r] = __builtin_amdgcn_exp2f(fmaf(s[t][r], scale_log2, mb));
                ps[r % 4] += s[t][r];
                emax = max(emax, (uint32_t)ve[t][r / 4][r % 4]);
            }
        l_run += (ps[0] + ps[1]) + (ps[2] + ps[3]);
        {
            const auto sw = __builtin_amdgcn_permlane32_swap(emax, emax, false, false);
            emax = max((uint32_t)sw[0], (uint32_t)sw[1]);
        }
        // P^T operand: p * 2^(eV - 127) / 2^(E - 6 - 127) rounded to E4M3 (<= 256)
        emax -= 6u << 23;
        const float esc = __uint_as_float(emax);
        i32x8 pop;
#pragma unroll
        for (int w = 0; w < 8; ++w) {
            const int t = w / 4, r0 = 4 * (w % 4);
            const u32x4 f = ve[t][r0 / 4];            // scale words 2^eV
            const float a0 = s[t][r0] * __uint_as_float(f[0]);
            const float a1 = s[t][r0 + 1] * __uint_as_float(f[1]);
            const float a2 = s[t][r0 + 2] * __uint_as_float(f[2]);
            const float a3 = s[t][r0 + 3] * __uint_as_float(f[3]);
            typedef short s16x2 __attribute__((ext_vector_type(2)));
            s16x2 pk = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(s16x2{0, 0}, a0, a1, esc, false);
            pk = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(pk, a2, a3, esc, true);
            pop[w] = __builtin_bit_cast(int, pk);
        }
        const int psc = (int)(emax >> 23);
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const i32x8 vop = {rd[b][0][0], rd[b][0][1], rd[b][1][0], rd[b][1][1],
                               rd[b][2][0], rd[b][2][1], rd[b][3][0], rd[b][3][1]};
            acc[b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(vop, pop, acc[b], 0, 0, 0, 127,
                                                                   0, psc);
        }
    }

    // as the bf16 engine: output rows (splits == 1) or the split's record
    __device__ __forceinline__ void store(uint16_t* oh, uint16_t* po, float* pml,
                                          float scale_log2) {
        const int lane = threadIdx.x % 64, col = lane & 31, kb = lane >> 5;
        const float l_tot = sum_halves(l_run);
        const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
        uint16_t* op = (oh ? oh : po) + col * F8Geom::D;
#pragma unroll
        for (int dt = 0; dt < 4; ++dt)
#pragma unroll
            for (int gg = 0; gg < 4; ++gg) {
                const int d = 32 * dt + 8 * gg + 4 * kb;
                u32x2 w;
                w[0] = pack_bf16x2(acc[dt][4 * gg] * inv, acc[dt][4 * gg + 1] * inv);
                w[1] = pack_bf16x2(acc[dt][4 * gg + 2] * inv, acc[dt][4 * gg + 3] * inv);
                *reinterpret_cast<u32x2*>(op + d) = w;
            }
        if (!oh && kb == 0) {
            pml[2 * col] = m_run == -INFINITY ? -INFINITY : m_run * scale_log2;
            pml[2 * col + 1] = l_tot;
        }
    }
};

template <int NW>
__global__ void __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2)))
k_attend_fp8(Fp8IO A, const int32_t* __restrict__ topk, float* __restrict__ part, int64_t Tq,
             int64_t Nc, int64_t m, int64_t W, int k, int64_t q_pos0, float scale_log2,
             int64_t raw_pos0, int64_t raw_len, int splits) {
    using G = F8Geom;
    constexpr int D = G::D;
    constexpr int NT = NW * 64;
    constexpr int H = NW * 32;
    constexpr int KT = G::KT;
    // distinct arrays per stage, so the compiler can tell which stage an LDS
    // read touches and never waits on another stage's copies
    __shared__ __attribute__((aligned(16))) uint8_t sS0[G::BYTES], sS1[G::BYTES];
    __shared__ __attribute__((aligned(16))) uint8_t sS2[G::BYTES], sS3[G::BYTES];
    __shared__ int32_t sSel[2048];                  // kept indices (CSA), padded to tiles
    __shared__ int sCnt[NW];

    const int i = (int)blockIdx.x;
    const int split = blockIdx.y;
    const int64_t b = blockIdx.z;
    const int tid = threadIdx.x, lane = tid % 64;
    // uniform per wave: scalar registers and scalar branches for everything
    // derived from it (the copy plan, the key list bounds)
    const int wave = __builtin_amdgcn_readfirstlane(tid / 64);
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
        nval = __builtin_amdgcn_readfirstlane(nval);     // the same on every lane
    }
    const CSA_LDS int32_t* ssel = (const CSA_LDS int32_t*)sSel;

    // this split's range of tiles: the ntile tiles dealt evenly (the splits
    // differ by at most one tile, so the blocks of a launch finish together)
    const int ct = (nval + KT - 1) / KT;
    const int ntile = ct + (nwin + KT - 1) / KT;
    const int tau0 = (int)((int64_t)split * ntile / splits);
    const int tau1 = (int)((int64_t)(split + 1) * ntile / splits);

    const F8Rows src{A.ck + b * Nc * D,       A.cv + b * Nc * D,       A.cks + b * Nc * 4,
                     A.cvs + b * Nc * 4,      A.rk + b * raw_len * D,  A.rv + b * raw_len * D,
                     A.rks + b * raw_len * 4, A.rvs + b * raw_len * 4};
    constexpr int PER = f8_copies<NW>();

    auto plan = [&](int tau) {
        return f8_plan<NW>(wave, tau, ct, nval, nwin, raw_first, sparse, ssel);
    };
    auto issue = [&](int tau, uint8_t* stg) {
        if (tau < tau1) f8_go<NW>(wave, plan(tau), src, (CSA_LDS uint8_t*)stg);
    };
    // the first tile's copies and the query loads go out together (one
    // round trip), then the next two tiles' copies, which stay in flight
    // while the query is encoded.  The three tiles are planned before any
    // copy is issued, and every plan stays live until its copies are out: no
    // address register is rewritten while a copy that used it may still be
    // in flight (the compiler answers that with a wait for every copy).
    Fp8Heads eng;
    {
        const F8Plan<NW> p0 = plan(tau0), p1 = plan(tau0 + 1), p2 = plan(tau0 + 2);
        if (tau0 < tau1) f8_go<NW>(wave, p0, src, (CSA_LDS uint8_t*)sS0);
        eng.load_q(A.q + (b * Tq + i) * (int64_t)H * D + wave * 32 * D);
        if (tau0 + 1 < tau1) f8_go<NW>(wave, p1, src, (CSA_LDS uint8_t*)sS1);
        if (tau0 + 2 < tau1) f8_go<NW>(wave, p2, src, (CSA_LDS uint8_t*)sS2);
#pragma unroll
        for (int u = 0; u < F8Geom::NCODE / NW; ++u)
            asm volatile("" ::"v"(p0.code[u]), "v"(p1.code[u]), "v"(p2.code[u]));
        asm volatile("" ::"v"(p0.scale), "v"(p1.scale), "v"(p2.scale));
    }
    eng.encode_q();
    eng.offsets();
    // S^T of the first tile.  Then one step per tile tau: wait for tile
    // tau + 1's copies (tile tau + 2's stay in flight), barrier (every wave
    // is done with tile tau - 1, whose stage the copies for tile tau + 3
    // then overwrite), the products S^T of tile tau + 1 (on stale bytes of
    // its stage when tau is the last tile; never used), the copies, then
    // tile tau's softmax and PV, which overlap the S^T products.
    f32x16 sA[2], sB[2];
    if (tau0 + 2 < tau1) CSA_WAIT_VM(2 * PER);
    else if (tau0 + 1 < tau1) CSA_WAIT_VM(PER);
    else CSA_WAIT_VM(0);
    lds_barrier();
    eng.qk((const CSA_LDS uint8_t*)sS0, sA);
    auto step = [&](int tau, uint8_t* cur, uint8_t* nxt, uint8_t* cpy, f32x16 (&s_cur)[2],
                    f32x16 (&s_nxt)[2]) {
        if (tau + 2 < tau1) CSA_WAIT_VM(PER);
        else CSA_WAIT_VM(0);
        lds_barrier();
        const int nvalid = tau < ct ? nval - KT * tau : nwin - KT * (tau - ct);
        eng.qk((const CSA_LDS uint8_t*)nxt, s_nxt);
        // an empty asm naming the products: the compiler would otherwise
        // move them down to their first use, in the next step (it reads
        // nothing, so the wave does not wait for them here)
        asm volatile("" ::"v"(s_nxt[0]), "v"(s_nxt[1]));
        __builtin_amdgcn_sched_barrier(0);
        issue(tau + 3, cpy);
        __builtin_amdgcn_sched_barrier(0);
        eng.rest((const CSA_LDS uint8_t*)cur, s_cur, nvalid, scale_log2);
    };

    for (int tau = tau0; tau < tau1; tau += 4) {
        step(tau, sS0, sS1, sS3, sA, sB);
        if (tau + 1 >= tau1) break;
        step(tau + 1, sS1, sS2, sS0, sB, sA);
        if (tau + 2 >= tau1) break;
        step(tau + 2, sS2, sS3, sS1, sA, sB);
        if (tau + 3 >= tau1) break;
        step(tau + 3, sS3, sS0, sS2, sB, sA);
    }
    uint16_t* o_row = A.o + (b * Tq + i) * (int64_t)H * D + wave * 32 * D;
    if (splits == 1) {
        eng.store(o_row, nullptr, nullptr, scale_log2);
    } else {
        const int64_t rec = ((b * Tq + i) * splits + split) * H + wave * 32;
        const int64_t nrec = (int64_t)gridDim.x * gridDim.y * gridDim.z * H;
        uint16_t* po = reinterpret_cast<uint16_t*>(part);
        eng.store(nullptr, po + rec * D, reinterpret_cast<float*>(po + nrec * D) + rec * 2,
                  scale_log2);
    }
}

template <int NW>
static void launch_fp8_nw(const AttendPlan& p, int64_t B, int64_t Tq, int64_t Nc, int64_t m,
                          int64_t W, int k, int64_t q_pos0, float scale, const Fp8IO& io,
                          const int32_t* topk, int64_t raw_pos0, int64_t raw_len, void* ws,
                          hipStream_t st) {
    constexpr int D = F8Geom::D, H = NW * 32;
    const float scale_log2 = scale * 1.4426950408889634f;
    hipLaunchKernelGGL(k_attend_fp8<NW>, dim3((unsigned)Tq, (unsigned)p.splits, (unsigned)B),
                       dim3(NW * 64), 0, st, io, topk, (float*)ws, Tq, Nc, m, W, k, q_pos0,
                       scale_log2, raw_pos0, raw_len, p.splits);
    if (p.splits > 1)
        launch_attend_combine(ws, B, Tq, H, D, p.splits, io.o, RowStrides{Tq * H * D, H * D}, st);
}

hipError_t launch_attend_fp8(const AttendPlan& p, int64_t B, int64_t Tq, int64_t H, int64_t Nc,
                             int64_t m, int64_t W, int64_t k, int64_t q_pos0, float scale,
                             const Fp8IO& io, const int32_t* topk, int64_t raw_pos0,
                             int64_t raw_len, void* ws, hipStream_t st) {
    if (B == 0 || Tq == 0) return hipSuccess;
    switch (H / 32) {
        case 1: launch_fp8_nw<1>(p, B, Tq, Nc, m, W, (int)k, q_pos0, scale, io, topk, raw_pos0, raw_len, ws, st); break;
        case 2: launch_fp8_nw<2>(p, B, Tq, Nc, m, W, (int)k, q_pos0, scale, io, topk, raw_pos0, raw_len, ws, st); break;
        case 4: launch_fp8_nw<4>(p, B, Tq, Nc, m, W, (int)k, q_pos0, scale, io, topk, raw_pos0, raw_len, ws, st); break;
        case 8: launch_fp8_nw<8>(p, B, Tq, Nc, m, W, (int)k, q_pos0, scale, io, topk, raw_pos0, raw_len, ws, st); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace csa
