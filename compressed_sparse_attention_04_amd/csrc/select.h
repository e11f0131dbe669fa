// select.h -- exact block-wide top-k selection on 32-bit keys.
//
// Keys order the candidates: key = fp32 bits of a non-negative score + 1 for
// a candidate (so +0 -> 1), 0 for "not a candidate".  Larger key = better;
// equal keys break toward the lower position.  Every thread holds EPT keys
// of one contiguous run of positions (thread t: t*EPT .. t*EPT+EPT-1), so
// a block-wide prefix sum in thread order is a prefix sum in position order.
//
// The routine finds the threshold key T and the number need_eq of keys
// equal to T that belong to the top kk: the selection is then
//   key > T  or  (key == T and rank among the keys equal to T < need_eq).
// First pass: a 256-bucket histogram of the score value (bucket
// floor(score * 256 / max_score)) spreads the keys evenly even when they
// share their exponent bits; the bucket holding the kk-th key is then
// resolved exactly by four 8-bit radix passes over its members only.
#pragma once
#include "common.h"

namespace csa {

struct SelectSmem {
    int hist[256];
    int scratch[32];
    int bcast[4];
};

template <int NT>
__device__ __forceinline__ int block_sum(int v, SelectSmem& sm) {
    v = wave_sum(v);
    const int w = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
    __syncthreads();
    if (lane == 0) sm.scratch[w] = v;
    __syncthreads();
    int t = 0;
#pragma unroll
    for (int i = 0; i < NT / WAVE; ++i) t += sm.scratch[i];
    return t;
}

template <int NT>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t v, SelectSmem& sm) {
    v = wave_max_u32(v);
    const int w = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
    __syncthreads();
    if (lane == 0) sm.scratch[w] = (int)v;
    __syncthreads();
    uint32_t t = 0;
#pragma unroll
    for (int i = 0; i < NT / WAVE; ++i) t = max(t, (uint32_t)sm.scratch[i]);
    return t;
}

// exclusive prefix sum in thread order; *total receives the block sum
template <int NT>
__device__ __forceinline__ int block_excl_scan(int v, SelectSmem& sm, int* total) {
    int inc = wave_incl_scan(v);
    const int w = threadIdx.x / WAVE, lane = threadIdx.x % WAVE;
    __syncthreads();
    if (lane == WAVE - 1) sm.scratch[w] = inc;
    __syncthreads();
    int base = 0, tot = 0;
#pragma unroll
    for (int i = 0; i < NT / WAVE; ++i) {
        int s = sm.scratch[i];
        base += (i < w) ? s : 0;
        tot += s;
    }
    *total = tot;
    return base + inc - v;
}

// Given sm.hist filled, find the largest bin d such that the number of keys
// in bins >= d reaches need; returns d and (in *above) the count in bins > d.
template <int NT>
__device__ __forceinline__ int hist_find(int need, SelectSmem& sm, int* above) {
    const int tid = threadIdx.x;
    int rev = (tid < 256) ? sm.hist[255 - tid] : 0;
    int tot;
    int excl = block_excl_scan<NT>(rev, sm, &tot);
    int incl = excl + rev;
    if (tid < 256 && rev > 0 && incl >= need && excl < need) {
        sm.bcast[0] = 255 - tid;
        sm.bcast[1] = excl;
    }
    __syncthreads();
    int d = sm.bcast[0];
    *above = sm.bcast[1];
    __syncthreads();
    return d;
}

__device__ __forceinline__ int value_bucket(uint32_t key, float inv) {
    float s = __uint_as_float(key - 1u);
    int b = (int)(s * inv);
    return b > 255 ? 255 : b;
}

// Threshold of the top kk (kk >= 1, kk <= number of keys != 0).
template <int NT, int EPT>
__device__ __forceinline__ void block_topk_threshold(const uint32_t (&key)[EPT], int kk,
                                                     SelectSmem& sm, uint32_t* T_out,
                                                     int* need_out) {
    const int tid = threadIdx.x;
    uint32_t kmax = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) kmax = max(kmax, key[e]);
    kmax = block_max_u32<NT>(kmax, sm);
    float smax = __uint_as_float(kmax - 1u);
    if (!(smax > 0.f)) {               // every candidate scores 0: all keys equal
        *T_out = 1u;
        *need_out = kk;
        return;
    }
    const float inv = 256.0f / smax;
    // pass 1: value buckets
    for (int i = tid; i < 256; i += NT) sm.hist[i] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < EPT; ++e)
        if (key[e]) atomicAdd(&sm.hist[value_bucket(key[e], inv)], 1);
    __syncthreads();
    int above;
    int bstar = hist_find<NT>(kk, sm, &above);
    int remaining = kk - above;
    // passes 2..5: exact radix over the members of bucket bstar
    uint32_t prefix = 0, mask = 0;
#pragma unroll 1
    for (int shift = 24; shift >= 0; shift -= 8) {
        for (int i = tid; i < 256; i += NT) sm.hist[i] = 0;
        __syncthreads();
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            uint32_t k = key[e];
            if (k && value_bucket(k, inv) == bstar && (k & mask) == prefix)
                atomicAdd(&sm.hist[(k >> shift) & 255u], 1);
        }
        __syncthreads();
        int ab;
        int d = hist_find<NT>(remaining, sm, &ab);
        remaining -= ab;
        prefix |= (uint32_t)d << shift;
        mask |= 255u << shift;
    }
    *T_out = prefix;
    *need_out = remaining;
}

// Selection flags for a known threshold: key > T, or key == T among the
// first need keys equal to T in position order.  Returns the thread's flags
// as a bitmask and its output offset; *total = number selected.
template <int NT, int EPT>
__device__ __forceinline__ uint32_t block_select_flags(const uint32_t (&key)[EPT], uint32_t T,
                                                       int need, SelectSmem& sm, int* out_base,
                                                       int* total) {
    int neq = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) neq += key[e] == T;
    int tot_eq;
    int eq_rank = block_excl_scan<NT>(neq, sm, &tot_eq);
    uint32_t flags = 0;
    int nsel = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        bool s = key[e] > T;
        if (key[e] == T) {
            s = eq_rank < need;
            eq_rank++;
        }
        if (s) { flags |= 1u << e; nsel++; }
    }
    *out_base = block_excl_scan<NT>(nsel, sm, total);
    return flags;
}

// Full selection: returns the selected flags as a bitmask per thread and
// the thread's output offset; *total = number selected (= kk).
template <int NT, int EPT>
__device__ __forceinline__ uint32_t block_topk_select(const uint32_t (&key)[EPT], int k,
                                                      SelectSmem& sm, int* out_base,
                                                      int* total) {
    int nv = 0;
#pragma unroll
    for (int e = 0; e < EPT; ++e) nv += key[e] != 0u;
    int nvalid = block_sum<NT>(nv, sm);
    uint32_t T;
    int need;
    if (nvalid <= k) {
        T = 1u;
        need = nvalid;              // every candidate (all keys >= 1)
        // keys > 1 are selected by "key > T"; keys == 1 by the rank rule
    } else {
        block_topk_threshold<NT, EPT>(key, k, sm, &T, &need);
    }
    return block_select_flags<NT, EPT>(key, T, need, sm, out_base, total);
}

}  // namespace csa
