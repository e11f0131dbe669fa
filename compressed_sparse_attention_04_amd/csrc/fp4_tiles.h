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
template <int UNR, bool STREAM>
__device__ __forceinline__ void load_batch(const TileSrc& ts, int v0, int stride,
                                           u32x4 (&kw)[UNR], int (&ksv)[UNR]) {
    const int koff = min(ts.kb * 16, ts.kbytes - 16);
    const int soff = min(ts.kb, ts.kscales - 1);
#pragma unroll
    for (int x = 0; x < UNR; ++x) {
        const int j = min((v0 + x) * stride * 32 + ts.row, ts.nc_max - 1);
        const u32x4* src = reinterpret_cast<const u32x4*>(ts.kcb + (int64_t)j * ts.kbytes + koff);
        kw[x] = STREAM ? __builtin_nontemporal_load(src) : *src;
        const int sc = ts.ksb[(int64_t)j * ts.kscales + soff];
        ksv[x] = ts.kb < ts.kscales ? sc : 127;
    }
}

// f(acc, j0): MFMA scores of the tile whose first key is j0 (this lane's
// key is j0 + row for its S rows; see the callers)
template <int NT, int UNR, bool STREAM = false, typename F>
__device__ __forceinline__ void stream_tiles(const TileSrc& ts, int nv, int stride,
                                             const i32x8& aop, int sa, F&& f) {
    constexpr int NWV = NT / WAVE;
    const int wave = threadIdx.x / WAVE;
    u32x4 kwA[UNR], kwB[UNR];
    int ksA[UNR], ksB[UNR];
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
    load_batch<UNR, STREAM>(ts, v0, stride, kwA, ksA);
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
template <int HI, int NU>
__device__ __forceinline__ void tile_keys(const f32x16& acc, uint32_t (&key)[NU]) {
#pragma unroll
    for (int u = 0; u < NU; ++u) {
        key[u] = score_key<HI>(acc, u);
        asm volatile("" : "+v"(key[u]));
    }
}

}  // namespace csa
