// wave_select.h -- pieces of the streaming exact top-k used by the indexer
// kernels that never hold all of a query's scores at once.
//
// A query's candidates are ordered by key = fp32 bits of the (non-negative)
// score, larger first, equal keys broken toward the lower candidate index.
// The threshold is narrowed pass by pass over a key range [lo, hi):
//   level 1: 1024 fixed bins -- bin 0 = [0, 2^-6), bins 1..1022 split
//            [2^-6, ~2^10) into 1/64-octave ranges, bin 1023 = the rest;
//   level n: 1024 equal sub-ranges of the previous range.
// Keys >= hi are kept for sure (marked in a candidate bitmap); keys inside
// the final range are resolved exactly, either from a small collected
// buffer or, for a range holding one key value, by candidate order.  The
// kept set is read out of the bitmap in ascending candidate order.
#pragma once
#include "common.h"

namespace csa {

constexpr int SEL_NB = 1024;                       // histogram bins per level
constexpr uint32_t L1_BASE = 121u << 23;           // fp32 bits of 2^-6
constexpr uint32_t KEY_END = 0xFFFFFFFFu;          // exclusive top of key space

__host__ __device__ __forceinline__ int lvl1_bin(uint32_t key) {
    if (key < L1_BASE) return 0;
    uint32_t d = ((key - L1_BASE) >> 17) + 1u;
    return d > 1023u ? 1023 : (int)d;
}

__host__ __device__ __forceinline__ void lvl1_range(int d, uint32_t* lo, uint32_t* hi) {
    if (d == 0) {
        *lo = 0u;
        *hi = L1_BASE;
    } else {
        *lo = L1_BASE + ((uint32_t)(d - 1) << 17);
        *hi = d == 1023 ? KEY_END : L1_BASE + ((uint32_t)d << 17);
    }
}

// shift that splits [lo, hi) into at most SEL_NB sub-ranges
__host__ __device__ __forceinline__ int range_shift(uint32_t lo, uint32_t hi) {
    const uint32_t span = hi - lo - 1u;            // >= 1 when refining
    const int bits = span ? 32 - __builtin_clz(span) : 0;
    return bits > 10 ? bits - 10 : 0;
}

// Passes of the exact search.  A level-1 range is less than 2^32 keys wide;
// a narrowing pass over a range whose span needs b bits leaves a sub-range
// at most 2^max(b - 10, 0) wide, so widths go 2^32 -> 2^22 -> 2^12 -> 2^2
// -> 1 and NARROW_PASSES narrowing passes always end with a single key
// value (or fewer keys in range than the collection buffer holds, earlier).
// The search is then level 1, the narrowing passes and one collection pass.
__host__ __device__ constexpr int narrowing_passes_bound() {
    int bits = 32, n = 0;
    while (bits > 0) {
        bits = bits > 10 ? bits - 10 : 0;
        ++n;
    }
    return n;
}
constexpr int NARROW_PASSES = narrowing_passes_bound();
constexpr int EXACT_PASSES = 1 + NARROW_PASSES + 1;
static_assert(NARROW_PASSES == 4 && EXACT_PASSES == 6, "32-bit keys, 1024-bin passes");

// Wave-wide search of a SEL_NB-bin histogram (lane l owns bins 16l..16l+15):
// the largest bin d with count(bins > d) < need <= count(bins >= d).
// Returns d; *gt = count(bins > d), *in = count(bin d).  need >= 1 and the
// histogram must hold at least need entries.
__device__ __forceinline__ int wave_hist_find(const uint32_t* hist, int need, int* gt, int* in) {
    const int lane = threadIdx.x % WAVE;
    uint32_t c[16];
    int s = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        c[i] = hist[lane * 16 + i];
        s += (int)c[i];
    }
    int incl = wave_incl_scan(s);
    int total = __shfl(incl, WAVE - 1, WAVE);
    int suffix_excl = total - incl;                // count in lanes above this one
    int found = -1, fgt = 0, fin = 0;
    if (suffix_excl < need && suffix_excl + s >= need) {
        int acc = suffix_excl;
#pragma unroll
        for (int i = 15; i >= 0; --i) {
            if (found < 0 && acc + (int)c[i] >= need) {
                found = lane * 16 + i;
                fgt = acc;
                fin = (int)c[i];
            }
            acc += (int)c[i];
        }
    }
    uint64_t who = __ballot(found >= 0);
    int src = __ffsll((unsigned long long)who) - 1;
    *gt = __shfl(fgt, src, WAVE);
    *in = __shfl(fin, src, WAVE);
    return __shfl(found, src, WAVE);
}

// Exact threshold among n <= 64*EPT collected keys (wave-wide, keys in
// registers, 0xFFFFFFFF-free): the key T of the need-th largest and how many
// keys equal to T are kept (need_eq).  hist: 256 words of scratch LDS.
template <int EPT>
__device__ __forceinline__ void wave_radix_threshold(const uint32_t (&key)[EPT],
                                                     const bool (&valid)[EPT], int need,
                                                     uint32_t* hist, uint32_t* T_out,
                                                     int* need_eq_out) {
    const int lane = threadIdx.x % WAVE;
    uint32_t prefix = 0, mask = 0;
    int rem = need;
#pragma unroll 1
    for (int shift = 24; shift >= 0; shift -= 8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) hist[lane * 4 + i] = 0u;
        __builtin_amdgcn_wave_barrier();
#pragma unroll
        for (int e = 0; e < EPT; ++e)
            if (valid[e] && (key[e] & mask) == prefix) atomicAdd(&hist[(key[e] >> shift) & 255u], 1u);
        __builtin_amdgcn_wave_barrier();
        // lane l owns bins 4l..4l+3
        uint32_t c[4];
        int s = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            c[i] = hist[lane * 4 + i];
            s += (int)c[i];
        }
        int incl = wave_incl_scan(s);
        int total = __shfl(incl, WAVE - 1, WAVE);
        int above = total - incl;
        int found = -1, fgt = 0;
        if (above < rem && above + s >= rem) {
            int acc = above;
#pragma unroll
            for (int i = 3; i >= 0; --i) {
                if (found < 0 && acc + (int)c[i] >= rem) {
                    found = lane * 4 + i;
                    fgt = acc;
                }
                acc += (int)c[i];
            }
        }
        uint64_t who = __ballot(found >= 0);
        int src = __ffsll((unsigned long long)who) - 1;
        int d = __shfl(found, src, WAVE);
        rem -= __shfl(fgt, src, WAVE);
        prefix |= (uint32_t)d << shift;
        mask |= 255u << shift;
        __builtin_amdgcn_wave_barrier();
    }
    *T_out = prefix;
    *need_eq_out = rem;
}

// The same threshold without LDS: the bits of the need-th largest key are
// decided from the top, a bit kept when at least need keys reach the value
// with it set (counted with ballots).  The search covers only the bits in
// which the valid keys differ: it starts below the leading bits they all
// share and stops above the trailing ones (scores of FP4 products are
// multiples of a power of two, so the low bits of every key are often
// equal), which then take the shared values.  need >= 1 and at most the
// number of valid keys; keys below 0xFFFFFFFF.
template <int EPT>
__device__ __forceinline__ void wave_ballot_threshold(const uint32_t (&key)[EPT],
                                                      const bool (&valid)[EPT], int need,
                                                      uint32_t* T_out, int* need_eq_out) {
    // key + 1 for a valid key, 0 otherwise
    uint32_t kp[EPT];
    uint32_t hi = 0u, lo = 0xFFFFFFFFu;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        kp[e] = valid[e] ? key[e] + 1u : 0u;
        hi = max(hi, kp[e]);
        lo = valid[e] ? min(lo, kp[e]) : lo;
    }
    hi = wave_max_u32_sw(hi);
    lo = ~wave_max_u32_sw(~lo);
    const uint32_t diff = hi ^ lo;
    int top = diff ? 31 - __builtin_clz(diff) : -1;     // highest bit where valid keys differ
    // lowest bit where some valid key differs from the largest one
    uint32_t dif = 0u;
#pragma unroll
    for (int e = 0; e < EPT; ++e) dif |= valid[e] ? kp[e] ^ hi : 0u;
    dif = wave_or_u32_sw(dif);
    const int low = dif ? __builtin_ctz(dif) : 0;
    uint32_t t = top >= 31 ? 0u : hi & ~((2u << top) - 1u);
#pragma unroll 1
    for (int bit = top; bit >= low; --bit) {
        const uint32_t cand = t | (1u << bit);
        int cnt = 0;
#pragma unroll
        for (int e = 0; e < EPT; ++e) cnt += __popcll(__ballot(kp[e] >= cand));
        if (cnt >= need) t = cand;
    }
    // below bit low every valid key has the bits of the largest: fewer than
    // need keys lie above the decided prefix (else the search would have
    // taken a larger one), so the remaining bits follow the shared ones
    t |= hi & ((1u << low) - 1u);
    if (top < 0) t = hi;                                 // a single key value
    int gt = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) gt += __popcll(__ballot(kp[e] > t));
    *T_out = t - 1u;
    *need_eq_out = need - gt;
}

// Keep the first need_eq set bits of eq (in candidate order) by OR-ing them
// into sel; nw words, wave-wide (lane l owns words l*per .. l*per+per-1).
__device__ __forceinline__ void wave_merge_first_bits(uint32_t* sel, const uint32_t* eq, int nw,
                                                      int need_eq) {
    if (need_eq <= 0) return;
    const int lane = threadIdx.x % WAVE;
    const int per = (nw + WAVE - 1) / WAVE;
    const int w0 = lane * per, w1 = min(nw, w0 + per);
    int cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += __popc(eq[w]);
    int before = wave_incl_scan(cnt) - cnt;
    for (int w = w0; w < w1 && before < need_eq; ++w) {
        uint32_t bits = eq[w];
        int c = __popc(bits);
        if (before + c > need_eq) {              // keep only the lowest bits
            int keep = need_eq - before;
            uint32_t kept = 0;
            for (int i = 0; i < keep; ++i) {
                uint32_t low = bits & (0u - bits);
                kept |= low;
                bits ^= low;
            }
            bits = kept;
            c = keep;
        }
        sel[w] |= bits;
        before += c;
    }
}

// Write the set bits of sel (nw words) as ascending candidate indices into
// out[0..k), padding with -1.  Wave-wide.
__device__ __forceinline__ void wave_emit_bitmap(const uint32_t* sel, int nw, int32_t* out,
                                                 int k) {
    const int lane = threadIdx.x % WAVE;
    const int per = (nw + WAVE - 1) / WAVE;
    const int w0 = lane * per, w1 = min(nw, w0 + per);
    int cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += __popc(sel[w]);
    int pos = wave_incl_scan(cnt) - cnt;
    int total = __shfl(wave_incl_scan(cnt), WAVE - 1, WAVE);
    for (int w = w0; w < w1; ++w) {
        uint32_t bits = sel[w];
        while (bits) {
            int b = __ffs(bits) - 1;
            bits &= bits - 1u;
            if (pos < k) out[pos] = w * 32 + b;
            pos++;
        }
    }
    for (int s = total + lane; s < k; s += WAVE) out[s] = -1;
}

// wave_emit_bitmap through LDS: the indices are first written to stage
// (k ints of scratch LDS) in ascending order, then copied to out with
// consecutive lanes on consecutive entries.
__device__ __forceinline__ void wave_emit_bitmap_staged(const uint32_t* sel, int nw,
                                                        int32_t* stage, int32_t* out, int k) {
    const int lane = threadIdx.x % WAVE;
    const int per = (nw + WAVE - 1) / WAVE;
    const int w0 = lane * per, w1 = min(nw, w0 + per);
    int cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += __popc(sel[w]);
    const int incl = wave_incl_scan(cnt);
    int pos = incl - cnt;
    const int total = __shfl(incl, WAVE - 1, WAVE);
    for (int w = w0; w < w1 && pos < k; ++w) {
        uint32_t bits = sel[w];
        while (bits && pos < k) {
            const int b = __ffs(bits) - 1;
            bits &= bits - 1u;
            stage[pos++] = w * 32 + b;
        }
    }
    __builtin_amdgcn_wave_barrier();
    for (int x = lane; x < k; x += WAVE) out[x] = x < total ? stage[x] : -1;
}

// Block-wide versions of the two bitmap steps above, for long rows: every
// thread owns a contiguous run of words; scratch holds NT/64 + 1 ints.
template <int NT>
__device__ __forceinline__ int block_excl_scan_i(int v, int* scratch, int* total) {
    const int lane = threadIdx.x % WAVE, w = threadIdx.x / WAVE;
    const int inc = wave_incl_scan(v);
    __syncthreads();
    if (lane == WAVE - 1) scratch[w] = inc;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NT / WAVE; ++i) {
        const int x = scratch[i];
        base += i < w ? x : 0;
        tot += x;
    }
    *total = tot;
    return base + inc - v;
}

template <int NT>
__device__ __forceinline__ void block_merge_first_bits(uint32_t* sel, const uint32_t* eq, int nw,
                                                       int need_eq, int* scratch) {
    const int per = (nw + NT - 1) / NT;
    const int w0 = threadIdx.x * per, w1 = min(nw, w0 + per);
    int cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += __popc(eq[w]);
    int tot;
    int before = block_excl_scan_i<NT>(cnt, scratch, &tot);
    for (int w = w0; w < w1 && before < need_eq; ++w) {
        uint32_t bits = eq[w];
        int c = __popc(bits);
        if (before + c > need_eq) {
            const int keep = need_eq - before;
            uint32_t kept = 0;
            for (int i = 0; i < keep; ++i) {
                const uint32_t low = bits & (0u - bits);
                kept |= low;
                bits ^= low;
            }
            bits = kept;
            c = keep;
        }
        sel[w] |= bits;
        before += c;
    }
    __syncthreads();
}

// block_merge_first_bits and block_emit_bitmap in one pass over registers,
// segment by segment: in a segment of NT * 8 words thread t owns words
// 8t .. 8t + 7 (those from nw on read as empty), read once as two 16-byte
// vectors from sel and eq (both arrays hold whole segments).  The first
// need_eq set bits of eq (candidate order) join sel, and the set bits of
// the result go to out in ascending order (at most k), then -1 up to k.
template <int NT>
__device__ __forceinline__ void block_merge_emit8(const uint32_t* sel, const uint32_t* eq, int nw,
                                                  int need_eq, int32_t* out, int k,
                                                  int* scratch) {
    int pos_base = 0, eq_base = 0;          // bits emitted / tie bits passed in earlier segments
    for (int s0 = 0; s0 < nw; s0 += NT * 8) {
        const int w0 = s0 + 8 * (int)threadIdx.x;
        uint32_t s8[8], e8[8];
        {
            const u32x4 a = reinterpret_cast<const u32x4*>(sel + w0)[0];
            const u32x4 b = reinterpret_cast<const u32x4*>(sel + w0)[1];
            const u32x4 c = reinterpret_cast<const u32x4*>(eq + w0)[0];
            const u32x4 d = reinterpret_cast<const u32x4*>(eq + w0)[1];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                s8[i] = a[i]; s8[4 + i] = b[i];
                e8[i] = c[i]; e8[4 + i] = d[i];
            }
        }
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (w0 + i >= nw) s8[i] = e8[i] = 0u;
        int ceq = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) ceq += __popc(e8[i]);
        int tot_eq;
        int before = eq_base + block_excl_scan_i<NT>(ceq, scratch, &tot_eq);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t bits = before < need_eq ? e8[i] : 0u;
            const int c = __popc(bits);
            if (before + c > need_eq) {
                uint32_t kept = 0;
                for (int x = 0; x < need_eq - before; ++x) {
                    const uint32_t low = bits & (0u - bits);
                    kept |= low;
                    bits ^= low;
                }
                bits = kept;
            }
            s8[i] |= bits;
            before += c;
        }
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) cnt += __popc(s8[i]);
        int total;
        int pos = pos_base + block_excl_scan_i<NT>(cnt, scratch, &total);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            uint32_t bits = s8[i];
            while (bits) {
                const int b = __ffs(bits) - 1;
                bits &= bits - 1u;
                if (pos < k) out[pos] = (w0 + i) * 32 + b;
                pos++;
            }
        }
        pos_base += total;
        eq_base += tot_eq;
    }
    for (int x = pos_base + (int)threadIdx.x; x < k; x += NT) out[x] = -1;
}

template <int NT>
__device__ __forceinline__ void block_emit_bitmap(const uint32_t* sel, int nw, int32_t* out, int k,
                                                  int* scratch) {
    const int per = (nw + NT - 1) / NT;
    const int w0 = threadIdx.x * per, w1 = min(nw, w0 + per);
    int cnt = 0;
    for (int w = w0; w < w1; ++w) cnt += __popc(sel[w]);
    int total;
    int pos = block_excl_scan_i<NT>(cnt, scratch, &total);
    for (int w = w0; w < w1; ++w) {
        uint32_t bits = sel[w];
        while (bits) {
            const int b = __ffs(bits) - 1;
            bits &= bits - 1u;
            if (pos < k) out[pos] = w * 32 + b;
            pos++;
        }
    }
    for (int s = total + (int)threadIdx.x; s < k; s += NT) out[s] = -1;
}

}  // namespace csa
