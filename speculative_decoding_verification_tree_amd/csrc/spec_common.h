// Device-side helpers shared by the gfx950 kernels of the verification step.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/spec_verify.h"

namespace specv {

constexpr int kWave = 64;
constexpr int kMaxNodes = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

template <typename T>
__device__ __forceinline__ T wave_max(T v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        T w = __shfl_xor(v, o, kWave);
        v = w > v ? w : v;
    }
    return v;
}

template <typename T>
__device__ __forceinline__ T wave_sum(T v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

// (value, index) argmax across a wavefront: largest value, lowest index on ties.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
        float w = __shfl_xor(v, o, kWave);
        int j = __shfl_xor(i, o, kWave);
        if (w > v || (w == v && j < i)) {
            v = w;
            i = j;
        }
    }
}

// Wait for this wave's LDS traffic and stop the compiler from moving memory
// operations across; sufficient for LDS exchange inside one wavefront.
__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Parent of node i (-1 for the root); parent == nullptr means a chain.
// Out-of-contract entries (p < 0 or p >= i for i > 0) are reported as -2.
__device__ __forceinline__ int tree_parent(const int32_t* parent, int N, int b, int i) {
    if (i <= 0) return -1;
    if (!parent) return i - 1;
    int p = parent[static_cast<size_t>(b) * N + i];
    return (p >= 0 && p < i) ? p : -2;
}

}  // namespace specv
