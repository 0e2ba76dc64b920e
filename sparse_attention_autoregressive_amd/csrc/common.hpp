// Device-side helpers shared by the FAST-AR kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fastar {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
// 16 bytes as a native vector: copies are vector loads/stores (HIP's uint4 is
// a struct whose copies become memcpy, which keeps register arrays of it in
// scratch memory).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// ---------------------------------------------------------------- bfloat16
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (inputs here are finite).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// 8 consecutive elements of a row -> fp32.  T = float or uint16_t (bf16 bits).
template <typename T>
__device__ __forceinline__ void load8_f32(const T* p, float (&v)[8]) {
    if constexpr (sizeof(T) == 2) {
        uint4 r = *reinterpret_cast<const uint4*>(p);
        uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    } else {
        float4 a = *reinterpret_cast<const float4*>(p);
        float4 b = *reinterpret_cast<const float4*>(p + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
}

// ---------------------------------------------------------------- lanes
__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t lanemask_lt() {
    return (uint64_t(1) << lane_id()) - 1;
}

// DPP butterfly within rows of 16 lanes: every lane of each group of
// ``width`` (8 or 16) lanes ends with the same sum.
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within 16

template <int WIDTH>
__device__ __forceinline__ float group_sum(float x) {
    static_assert(WIDTH == 8 || WIDTH == 16, "group width");
    x += dpp_f<kDppXor1>(x);
    x += dpp_f<kDppXor2>(x);
    x += dpp_f<kDppHalfMirror>(x);
    if constexpr (WIDTH == 16) x += dpp_f<kDppMirror>(x);
    return x;
}

// Inclusive prefix sum over the 64 lanes of a wave (V = int or uint32_t;
// unsigned sums wrap, which packed counters rely on).
template <typename V = int>
__device__ __forceinline__ V wave_inclusive_scan(V v) {
    const int l = lane_id();
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        V t = __shfl_up(v, off, kWave);
        if (l >= off) v += t;
    }
    return v;
}

// Exclusive prefix sum over a block of NT threads; ``total`` receives the sum.
// ``smem`` needs NT/64 elements.  Contains two __syncthreads.
template <int NT, typename V = int>
__device__ __forceinline__ V block_exclusive_scan(V v, V* smem, V& total) {
    constexpr int NW = NT / kWave;
    const int w = threadIdx.x / kWave;
    V inc = wave_inclusive_scan<V>(v);
    if (lane_id() == kWave - 1) smem[w] = inc;
    __syncthreads();
    V before = 0, sum = 0;
#pragma unroll
    for (int i = 0; i < NW; ++i) {
        V s = smem[i];
        before += (i < w) ? s : V(0);
        sum += s;
    }
    __syncthreads();
    total = sum;
    return before + inc - v;
}

__device__ __forceinline__ int clamp_n(const int32_t* n_valid, int h, int cap) {
    if (!n_valid) return 0;
    int n = n_valid[h];
    return n < 0 ? 0 : (n > cap ? cap : n);
}

}  // namespace fastar
