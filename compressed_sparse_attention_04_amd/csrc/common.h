// common.h -- device helpers shared by the gfx950 kernels of libcsa.so.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int WAVE = 64;

// Element strides of a [B][rows][...] tensor whose rows are contiguous:
// element e of row r of sequence b sits at b * ss + r * rs + e.
struct RowStrides {
    int64_t ss, rs;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
    return __uint_as_float(h << 16);
}

// fp32 -> bf16 bits, round to nearest even (NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 (round to nearest even; v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    f32x2 v = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
}

// Storage element types: float (fp32) or uint16_t holding bf16 bits.
template <typename T> struct Elem;
template <> struct Elem<float> {
    __device__ static __forceinline__ void load8(const float* p, float (&v)[8]) {
        f32x4 a = *reinterpret_cast<const f32x4*>(p);
        f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
        v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
        v[4] = b[0]; v[5] = b[1]; v[6] = b[2]; v[7] = b[3];
    }
    __device__ static __forceinline__ void store8(float* p, const float (&v)[8]) {
        f32x4 a = {v[0], v[1], v[2], v[3]}, b = {v[4], v[5], v[6], v[7]};
        *reinterpret_cast<f32x4*>(p) = a;
        *reinterpret_cast<f32x4*>(p + 4) = b;
    }
    __device__ static __forceinline__ void load4(const float* p, float (&v)[4]) {
        f32x4 a = *reinterpret_cast<const f32x4*>(p);
        v[0] = a[0]; v[1] = a[1]; v[2] = a[2]; v[3] = a[3];
    }
    __device__ static __forceinline__ float load1(const float* p) { return *p; }
};
template <> struct Elem<uint16_t> {
    __device__ static __forceinline__ void load8(const uint16_t* p, float (&v)[8]) {
        u32x4 a = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(a[i] << 16);
            v[2 * i + 1] = __uint_as_float(a[i] & 0xffff0000u);
        }
    }
    __device__ static __forceinline__ void store8(uint16_t* p, const float (&v)[8]) {
        u32x4 a;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            a[i] = f32_to_bf16_bits(v[2 * i]) | (f32_to_bf16_bits(v[2 * i + 1]) << 16);
        *reinterpret_cast<u32x4*>(p) = a;
    }
    __device__ static __forceinline__ void load4(const uint16_t* p, float (&v)[4]) {
        u32x2 a = *reinterpret_cast<const u32x2*>(p);
        v[0] = __uint_as_float(a[0] << 16);
        v[1] = __uint_as_float(a[0] & 0xffff0000u);
        v[2] = __uint_as_float(a[1] << 16);
        v[3] = __uint_as_float(a[1] & 0xffff0000u);
    }
    __device__ static __forceinline__ float load1(const uint16_t* p) {
        return bf16_bits_to_f32(*p);
    }
};

// ---- wave / block reductions ------------------------------------------
__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, WAVE);
    return v;
}
// Lane exchanges with the pattern in the instruction (ds_swizzle bit mode:
// lane j reads lane j ^ x within its 32; permlane32_swap for the halves), so
// no lane-index register is formed (shuffle address registers computed once
// and kept across a kernel have cost spills)
template <int X>
__device__ __forceinline__ uint32_t swizzle_xor(uint32_t v) {
    static_assert(X > 0 && X < 32, "within 32 lanes");
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x1F | (X << 10));
}
__device__ __forceinline__ uint32_t wave_max_u32_sw(uint32_t v) {
    v = max(v, swizzle_xor<16>(v));
    v = max(v, swizzle_xor<8>(v));
    v = max(v, swizzle_xor<4>(v));
    v = max(v, swizzle_xor<2>(v));
    v = max(v, swizzle_xor<1>(v));
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return max((uint32_t)r[0], (uint32_t)r[1]);
}
__device__ __forceinline__ uint32_t wave_or_u32_sw(uint32_t v) {
    v |= swizzle_xor<16>(v);
    v |= swizzle_xor<8>(v);
    v |= swizzle_xor<4>(v);
    v |= swizzle_xor<2>(v);
    v |= swizzle_xor<1>(v);
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return (uint32_t)r[0] | (uint32_t)r[1];
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        uint32_t w = (uint32_t)__shfl_xor((int)v, o, WAVE);
        v = v > w ? v : w;
    }
    return v;
}
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
    return v;
}
// inclusive prefix sum over the lanes of a wave
__device__ __forceinline__ int wave_incl_scan(int v) {
    const int lane = threadIdx.x & (WAVE - 1);
#pragma unroll
    for (int o = 1; o < WAVE; o <<= 1) {
        int w = __shfl_up(v, o, WAVE);
        if (lane >= o) v += w;
    }
    return v;
}

// Number of compressed candidates of a query at position t (block j is a
// candidate iff m*j+m-1 <= t and m*j < w0, w0 = max(0, t-W+1)).
__host__ __device__ __forceinline__ int64_t n_candidates(int64_t t, int64_t m, int64_t W) {
    int64_t w0 = t - W + 1;
    if (w0 < 0) w0 = 0;
    int64_t a = (w0 + m - 1) / m;       // blocks starting before the window
    int64_t b = (t + 1) / m;            // complete, visible blocks
    return a < b ? a : b;
}

}  // namespace csa
