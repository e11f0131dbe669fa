// fp4_tiles.h -- streaming MXFP4 key tiles through the scaled FP4 MFMA for
// the Lightning Indexer kernels (jiwasawa.github.io post, CSA indexer
// bullet; studioglobal.ai answer: the indexer runs at FP4).
//
// A key tile is 32 consecutive candidates; one V_MFMA_SCALE_F32_32X32X64
// (FP4 x FP4, E8M0 scales) scores it against the block's 32 A-operand rows
// (query row x indexer head).
#pragma once
#include "common.h"

namespace csa {

// One wave's batches of UNR key tiles: virtual tiles v = 0..nv-1 map to
// key tiles v * stride; the wave takes batches wave, wave + NWV, ...  The
// next batch's key loads are in flight while the current one is processed.
struct TileSrc {
    const uint8_t* kcb;
    const uint8_t* ksb;
    int kbytes, kscales, nc_max, row, kb;
};

// Loads are unconditional (rows clamped to the last candidate; lanes past
// dI read a valid offset and get the neutral scale 2^0 against a zero A
// operand), so the compiler can count them: the current batch is waited
// for while the next one stays in flight.  STREAM: keys read once (decode)
// bypass the caches' normal retention.
// Offsets from the tile source's base are 32-bit, formed by 24-bit
// multiplies: a source holds at most 262,144 candidates of at most 32 code
// bytes (2^23 bytes).
template <int UNR, bool STREAM>
__device__ __forceinline__ void load_batch(const TileSrc& ts, int v0, int stride,
                                           u32x4 (&kw)[UNR], int (&ksv)[UNR]) {
    const uint32_t koff = (uint32_t)min(ts.kb * 16, ts.kbytes - 16);
    const uint32_t soff = (uint32_t)min(ts.kb, ts.kscales - 1);
#pragma unroll
    for (int x = 0; x < UNR; ++x) {
        const uint32_t j = (uint32_t)min((v0 + x) * stride * 32 + ts.row, ts.nc_max - 1);
        const u32x4* src =
            reinterpret_cast<const u32x4*>(ts.kcb + (__umul24(j, (uint32_t)ts.kbytes) + koff));
        kw[x] = STREAM ? __builtin_nontemporal_load(src) : *src;
        const int sc = ts.ksb[__umul24(j, (uint32_t)ts.kscales) + soff];
        ksv[x] = ts.kb < ts.kscales ? sc : 127;
    }
}

// f(acc, j0): MFMA scores of the tile whose first key is j0 (this lane's
// key is j0 + row for its S rows; see the callers).  kwA / ksA hold the
// wave's first batch, already requested by load_first (so a kernel can put
// the first key loads in flight before its own set-up work).
template <int NT, int UNR>
__device__ __forceinline__ int first_batch(int nv) {
    return (int)(threadIdx.x / WAVE) * UNR < nv;
}
template <int NT, int UNR, bool STREAM>
__device__ __forceinline__ void load_first(const TileSrc& ts, int nv, int stride,
                                           u32x4 (&kwA)[UNR], int (&ksA)[UNR]) {
    if (first_batch<NT, UNR>(nv))
        load_batch<UNR, STREAM>(ts, (int)(threadIdx.x / WAVE) * UNR, stride, kwA, ksA);
}

template <int NT, int UNR, bool STREAM = false, typename F>
__device__ __forceinline__ void stream_tiles_from(const TileSrc& ts, int nv, int stride,
                                                  const i32x8& aop, int sa, u32x4 (&kwA)[UNR],
                                                  int (&ksA)[UNR], F&& f) {
    constexpr int NWV = NT / WAVE;
    const int wave = threadIdx.x / WAVE;
    u32x4 kwB[UNR];
    int ksB[UNR];
    auto mfma = [&](const u32x4& kw, int ksv) {
        const i32x8 bop = {(int)kw[0], (int)kw[1], (int)kw[2], (int)kw[3], 0, 0, 0, 0};
        const f32x16 zero = {};
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop, bop, zero, 4, 4, 0, sa, 0,
                                                                ksv);
    };
    // the MFMA of tile x + 1 is issued before the scores of tile x are
    // used, so its latency is hidden behind f
    auto run = [&](const u32x4 (&kw)[UNR], const int (&ksv)[UNR], int v0) {
        f32x16 next = mfma(kw[0], ksv[0]);
#pragma unroll
        for (int x = 0; x < UNR; ++x) {
            if (v0 + x >= nv) break;
            const f32x16 acc = next;
            if (x + 1 < UNR) next = mfma(kw[x + 1], ksv[x + 1]);
            f(acc, (v0 + x) * stride * 32);
            // at most two tiles' scores live at a time
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    int v0 = wave * UNR;
    if (v0 >= nv) return;
    while (true) {
        load_batch<UNR, STREAM>(ts, v0 + NWV * UNR, stride, kwB, ksB);
        run(kwA, ksA, v0);
        v0 += NWV * UNR;
        if (v0 >= nv) break;
        load_batch<UNR, STREAM>(ts, v0 + NWV * UNR, stride, kwA, ksA);
        run(kwB, ksB, v0);
        v0 += NWV * UNR;
        if (v0 >= nv) break;
    }
}

// One query row (decode): its HI head scores are the A rows 0..HI-1, which
// the MFMA leaves in registers 0..HI-1 of lanes 0-31 only.  The tiles are
// therefore taken in pairs (stride 1): the scores of the pair's second tile
// are swapped into lanes 32-63 of the first tile's registers (a permlane32
// swap per head), so one pass of f covers 64 keys.  f(s, j, ok): head
// scores s[0..HI-1] of key j (lanes 0-31: the first tile's keys, lanes
// 32-63: the second's); ok is false on lanes 32-63 when the wave's last
// tile has no partner.  One pair's scores are live at a time (the register
// budget of four waves per SIMD), and they pass through an empty asm before
// f, whose branches depend on the lane.
template <int NT, int UNR, int HI, bool STREAM, typename F>
__device__ __forceinline__ void stream_tile_pairs(const TileSrc& ts, int nv, const i32x8& aop,
                                                  int sa, u32x4 (&kwA)[UNR], int (&ksA)[UNR],
                                                  F&& f) {
    static_assert(UNR % 2 == 0, "tiles go in pairs");
    constexpr int NWV = NT / WAVE;
    const int wave = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
    u32x4 kwB[UNR];
    int ksB[UNR];
    auto mfma = [&](const u32x4& kw, int ksv) {
        const i32x8 bop = {(int)kw[0], (int)kw[1], (int)kw[2], (int)kw[3], 0, 0, 0, 0};
        const f32x16 zero = {};
        return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(aop, bop, zero, 4, 4, 0, sa, 0,
                                                                ksv);
    };
    auto run = [&](const u32x4 (&kw)[UNR], const int (&ksv)[UNR], int v0) {
#pragma unroll
        for (int x = 0; x < UNR; x += 2) {
            if (v0 + x >= nv) break;
            const f32x16 a0 = mfma(kw[x], ksv[x]), a1 = mfma(kw[x + 1], ksv[x + 1]);
            float sc[HI];
#pragma unroll
            for (int h = 0; h < HI; ++h) {
                const auto r = __builtin_amdgcn_permlane32_swap(
                    __float_as_uint(a0[h]), __float_as_uint(a1[h]), false, false);
                uint32_t v = r[0];
                asm volatile("" : "+v"(v));
                sc[h] = __uint_as_float(v);
            }
            const int j = (v0 + x + (lane >> 5)) * 32 + (lane & 31);
            f(sc, j, lane < 32 || v0 + x + 1 < nv);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    int v0 = wave * UNR;
    if (v0 >= nv) return;
    while (true) {
        load_batch<UNR, STREAM>(ts, v0 + NWV * UNR, 1, kwB, ksB);
        run(kwA, ksA, v0);
        v0 += NWV * UNR;
        if (v0 >= nv) break;
        load_batch<UNR, STREAM>(ts, v0 + NWV * UNR, 1, kwA, ksA);
        run(kwB, ksB, v0);
        v0 += NWV * UNR;
        if (v0 >= nv) break;
    }
}

template <int NT, int UNR, bool STREAM = false, typename F>
__device__ __forceinline__ void stream_tiles(const TileSrc& ts, int nv, int stride,
                                             const i32x8& aop, int sa, F&& f) {
    u32x4 kwA[UNR];
    int ksA[UNR];
    load_first<NT, UNR, STREAM>(ts, nv, stride, kwA, ksA);
    stream_tiles_from<NT, UNR, STREAM>(ts, nv, stride, aop, sa, kwA, ksA, f);
}

// ReLU head sum of slot u of an MFMA tile as an order key.  ReLU is the
// signed-integer max of the bit pattern with 0 (negative floats, -0
// included, have negative patterns), so the sum of non-negative terms is
// never -0.  The MFMA outputs are finite (products of FP4 values).
template <int HI>
__device__ __forceinline__ uint32_t score_key(const f32x16& acc, int u) {
    float s = __int_as_float(max(__float_as_int(acc[u * HI]), 0));
#pragma unroll
    for (int hh = 1; hh < HI; ++hh) s += __int_as_float(max(__float_as_int(acc[u * HI + hh]), 0));
    return __float_as_uint(s);
}

// The order keys of every slot of a tile, formed by all lanes: each key
// passes through an empty asm statement before any lane-dependent branch of
// the caller, so the MFMA that produces the tile cannot be moved into a
// branch that only some lanes take (an MFMA issued with part of EXEC off
// does not give every lane its full result).
// Only the first nlive slots (wave-uniform) are formed; the others read 0.
template <int HI, int NU>
__device__ __forceinline__ void tile_keys(const f32x16& acc, uint32_t (&key)[NU],
                                          int nlive = NU) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        key[u] = 0u;
        if (u < nlive) {
            key[u] = score_key<HI>(acc, u);
            asm volatile("" : "+v"(key[u]));
        }
    }
}

// Slots of a tile that hold a query of the first qv (query qi of A row
// (qi, h) = (row / HI, row % HI) sits in slot u of the lanes with
// 8 (u HI / 4) + (u HI) % 4 + 4 kb = HI qi + h, h < HI).
template <int HI>
__host__ __device__ __forceinline__ int live_slots(int qv) {
    constexpr int NU = 16 / HI;
    int n = 0;
    for (int u = 0; u < NU; ++u)
        if ((8 * ((u * HI) / 4) + (u * HI) % 4) / HI < qv) n = u + 1;
    return n;
}

}  // namespace csa
