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

// 16-byte load with the non-temporal hint (global_load_dwordx4 ... nt), for
// data a kernel streams once from HBM: KV blocks, logits rows.  A read-only
// sweep of 4 GiB on MI355X reads 6.7-7.2 TB/s this way against 6.0-6.2 TB/s
// with plain loads, for flat, per-workgroup-range and KV-block access shapes.
__device__ __forceinline__ u32x4 ld_stream(const void* p) {
    return __builtin_nontemporal_load(static_cast<const u32x4*>(p));
}
__device__ __forceinline__ float4 ld_stream_f4(const float* p) {
    const u32x4 u = ld_stream(p);
    return make_float4(__uint_as_float(u[0]), __uint_as_float(u[1]), __uint_as_float(u[2]), __uint_as_float(u[3]));
}

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
    return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = __float_as_uint(f);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

// Two floats -> packed bf16 pair, round to nearest even (one v_cvt_pk_bf16_f32).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// ---- cross-lane exchange without the LDS crossbar -------------------------
// DPP moves within a 16-lane row, v_permlane16/32_swap across rows.  Each
// helper returns the value held by the partner lane (xor 1, xor 2, mirror in
// 8, mirror in 16) or, for the swaps, the pair whose combination pairs every
// lane with its xor-16 / xor-32 partner.
__device__ __forceinline__ uint32_t dpp_xor1(uint32_t v) { return __builtin_amdgcn_update_dpp(0, v, 0xB1, 0xF, 0xF, false); }
__device__ __forceinline__ uint32_t dpp_xor2(uint32_t v) { return __builtin_amdgcn_update_dpp(0, v, 0x4E, 0xF, 0xF, false); }
__device__ __forceinline__ uint32_t dpp_mirror8(uint32_t v) { return __builtin_amdgcn_update_dpp(0, v, 0x141, 0xF, 0xF, false); }
__device__ __forceinline__ uint32_t dpp_mirror16(uint32_t v) { return __builtin_amdgcn_update_dpp(0, v, 0x140, 0xF, 0xF, false); }

template <class F>
__device__ __forceinline__ float xrow_combine16(float v, F op) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
template <class F>
__device__ __forceinline__ float xrow_combine32(float v, F op) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Reduction over the four lanes n, n+16, n+32, n+48 (one per 16-lane row).
__device__ __forceinline__ float max_across_rows(float v) {
    auto mx = [](float x, float y) { return fmaxf(x, y); };
    return xrow_combine32(xrow_combine16(v, mx), mx);
}
__device__ __forceinline__ float sum_across_rows(float v) {
    auto ad = [](float x, float y) { return x + y; };
    return xrow_combine32(xrow_combine16(v, ad), ad);
}

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, __uint_as_float(dpp_xor1(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_xor2(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_mirror8(__float_as_uint(v))));
    v = fmaxf(v, __uint_as_float(dpp_mirror16(__float_as_uint(v))));
    return max_across_rows(v);
}

__device__ __forceinline__ float wave_sum(float v) {
    v += __uint_as_float(dpp_xor1(__float_as_uint(v)));
    v += __uint_as_float(dpp_xor2(__float_as_uint(v)));
    v += __uint_as_float(dpp_mirror8(__float_as_uint(v)));
    v += __uint_as_float(dpp_mirror16(__float_as_uint(v)));
    return sum_across_rows(v);
}

// 64-bit lane exchange: both halves through the same permutation.
template <uint32_t (*MOVE)(uint32_t)>
__device__ __forceinline__ double move_d(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint64_t lo = MOVE(static_cast<uint32_t>(u)), hi = MOVE(static_cast<uint32_t>(u >> 32));
    return __builtin_bit_cast(double, lo | (hi << 32));
}

__device__ __forceinline__ double wave_sum(double v) {
    v += move_d<dpp_xor1>(v);
    v += move_d<dpp_xor2>(v);
    v += move_d<dpp_mirror8>(v);
    v += move_d<dpp_mirror16>(v);
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    auto a = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(u), static_cast<uint32_t>(u), false, false);
    auto b = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(u >> 32), static_cast<uint32_t>(u >> 32), false, false);
    v = __builtin_bit_cast(double, static_cast<uint64_t>(a[0]) | (static_cast<uint64_t>(b[0]) << 32)) +
        __builtin_bit_cast(double, static_cast<uint64_t>(a[1]) | (static_cast<uint64_t>(b[1]) << 32));
    const uint64_t w = __builtin_bit_cast(uint64_t, v);
    a = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(w), static_cast<uint32_t>(w), false, false);
    b = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(w >> 32), static_cast<uint32_t>(w >> 32), false, false);
    return __builtin_bit_cast(double, static_cast<uint64_t>(a[0]) | (static_cast<uint64_t>(b[0]) << 32)) +
           __builtin_bit_cast(double, static_cast<uint64_t>(a[1]) | (static_cast<uint64_t>(b[1]) << 32));
}

__device__ __forceinline__ void argmax_step(float& v, int& i, float w, int j) {
    if (w > v || (w == v && j < i)) {
        v = w;
        i = j;
    }
}

// (value, index) argmax across a wavefront: largest value, lowest index on ties.
__device__ __forceinline__ void wave_argmax(float& v, int& i) {
    argmax_step(v, i, __uint_as_float(dpp_xor1(__float_as_uint(v))), static_cast<int>(dpp_xor1(i)));
    argmax_step(v, i, __uint_as_float(dpp_xor2(__float_as_uint(v))), static_cast<int>(dpp_xor2(i)));
    argmax_step(v, i, __uint_as_float(dpp_mirror8(__float_as_uint(v))), static_cast<int>(dpp_mirror8(i)));
    argmax_step(v, i, __uint_as_float(dpp_mirror16(__float_as_uint(v))), static_cast<int>(dpp_mirror16(i)));
    {
        const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        const auto b = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(i), static_cast<uint32_t>(i), false, false);
        float v0 = __uint_as_float(a[0]);
        int i0 = static_cast<int>(b[0]);
        argmax_step(v0, i0, __uint_as_float(a[1]), static_cast<int>(b[1]));
        v = v0;
        i = i0;
    }
    {
        const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
        const auto b = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(i), static_cast<uint32_t>(i), false, false);
        float v0 = __uint_as_float(a[0]);
        int i0 = static_cast<int>(b[0]);
        argmax_step(v0, i0, __uint_as_float(a[1]), static_cast<int>(b[1]));
        v = v0;
        i = i0;
    }
}

// ---- rotary embedding at depth positions -----------------------------------
// The pair (x_j, x_{j + D/2}) of a row at position pos turns by
// pos * base^(-2j/D) radians.  rev[j] = base^(-2j/D) / (2 pi), fp64 from the
// host: the angle in turns is frac(pos * rev[j]) in fp64, and the sine and
// cosine come from the hardware's fp32 sine and cosine of a fraction of a
// turn; the products are fp32.
constexpr int kRopeMaxPairs = 64;  // D / 2 for D <= 128
struct RopeTable {
    double rev[kRopeMaxPairs];
};

__device__ __forceinline__ void rope_cs(int pos, double rev, float& c, float& s) {
    double t = static_cast<double>(pos) * rev;
    t -= floor(t);
    const float f = static_cast<float>(t);
    s = __builtin_amdgcn_sinf(f);
    c = __builtin_amdgcn_cosf(f);
}

__device__ __forceinline__ void rope_pair(float& x, float& y, float c, float s) {
    const float xr = x * c - y * s, yr = x * s + y * c;
    x = xr;
    y = yr;
}

// Eight bf16 pairs: lo holds dims j0 .. j0 + 7 of a row, hi the dims D/2
// further; rev points at the table (LDS).  Rounded back to bf16 (nearest even).
__device__ __forceinline__ void rope_bf16x8(u32x4& lo, u32x4& hi, int pos, const double* rev, int j0) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        float x0 = __uint_as_float(lo[w] << 16), x1 = __uint_as_float(lo[w] & 0xFFFF0000u);
        float y0 = __uint_as_float(hi[w] << 16), y1 = __uint_as_float(hi[w] & 0xFFFF0000u);
        float c, s;
        rope_cs(pos, rev[j0 + 2 * w], c, s);
        rope_pair(x0, y0, c, s);
        rope_cs(pos, rev[j0 + 2 * w + 1], c, s);
        rope_pair(x1, y1, c, s);
        lo[w] = pack_bf16x2(x0, x1);
        hi[w] = pack_bf16x2(y0, y1);
    }
}

// Four fp32 pairs (dims j0 .. j0 + 3 and D/2 further).
__device__ __forceinline__ void rope_f32x4(u32x4& lo, u32x4& hi, int pos, const double* rev, int j0) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        float x = __uint_as_float(lo[w]), y = __uint_as_float(hi[w]);
        float c, s;
        rope_cs(pos, rev[j0 + w], c, s);
        rope_pair(x, y, c, s);
        lo[w] = __float_as_uint(x);
        hi[w] = __float_as_uint(y);
    }
}

// Wait for this wave's LDS traffic and stop the compiler from moving memory
// operations across; sufficient for LDS exchange inside one wavefront.
// Minimum of mn and maximum of mx over a wavefront, the two reductions
// interleaved (DPP within rows, permlane swaps across rows).
__device__ __forceinline__ void wave_min_max_i(int& mn, int& mx) {
    mn = min(mn, static_cast<int>(dpp_xor1(static_cast<uint32_t>(mn))));
    mx = max(mx, static_cast<int>(dpp_xor1(static_cast<uint32_t>(mx))));
    mn = min(mn, static_cast<int>(dpp_xor2(static_cast<uint32_t>(mn))));
    mx = max(mx, static_cast<int>(dpp_xor2(static_cast<uint32_t>(mx))));
    mn = min(mn, static_cast<int>(dpp_mirror8(static_cast<uint32_t>(mn))));
    mx = max(mx, static_cast<int>(dpp_mirror8(static_cast<uint32_t>(mx))));
    mn = min(mn, static_cast<int>(dpp_mirror16(static_cast<uint32_t>(mn))));
    mx = max(mx, static_cast<int>(dpp_mirror16(static_cast<uint32_t>(mx))));
    auto a = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(mn), static_cast<uint32_t>(mn), false, false);
    auto c = __builtin_amdgcn_permlane16_swap(static_cast<uint32_t>(mx), static_cast<uint32_t>(mx), false, false);
    mn = min(static_cast<int>(a[0]), static_cast<int>(a[1]));
    mx = max(static_cast<int>(c[0]), static_cast<int>(c[1]));
    a = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(mn), static_cast<uint32_t>(mn), false, false);
    c = __builtin_amdgcn_permlane32_swap(static_cast<uint32_t>(mx), static_cast<uint32_t>(mx), false, false);
    mn = min(static_cast<int>(a[0]), static_cast<int>(a[1]));
    mx = max(static_cast<int>(c[0]), static_cast<int>(c[1]));
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_d(double v) {
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = __builtin_amdgcn_update_dpp(0u, static_cast<uint32_t>(u), CTRL, ROW_MASK, 0xF, true);
    const uint32_t hi = __builtin_amdgcn_update_dpp(0u, static_cast<uint32_t>(u >> 32), CTRL, ROW_MASK, 0xF, true);
    return __builtin_bit_cast(double, static_cast<uint64_t>(lo) | (static_cast<uint64_t>(hi) << 32));
}

// Inclusive prefix sum over the lanes of a wavefront: shifts by 1, 2, 4, 8
// inside each 16-lane row, then the last lane of row 0 (row 2) is added to
// row 1 (row 3), and lane 31 to rows 2 and 3.
__device__ __forceinline__ double wave_incl_scan(double v) {
    v += dpp_d<0x111, 0xF>(v);  // row_shr:1
    v += dpp_d<0x112, 0xF>(v);  // row_shr:2
    v += dpp_d<0x114, 0xF>(v);  // row_shr:4
    v += dpp_d<0x118, 0xF>(v);  // row_shr:8
    v += dpp_d<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp_d<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

__device__ __forceinline__ void wave_lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Parent of node i (-1 for the root); parent == nullptr means a chain.
// Out-of-contract entries (p < 0 or p >= i for i > 0) are reported as -2.
// Device-scope (agent) relaxed 64-bit stores and loads: they bypass the
// caches that are not coherent across the XCDs, so workgroups on different
// XCDs can exchange records inside one launch (a store is complete, and
// visible to such loads, once the storing thread's vmcnt has drained).
__device__ __forceinline__ void agent_st64(void* p, uint64_t v) {
    __hip_atomic_store(static_cast<uint64_t*>(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t agent_ld64(const void* p) {
    return __hip_atomic_load(static_cast<uint64_t*>(const_cast<void*>(p)), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ int tree_parent(const int32_t* parent, int N, int b, int i) {
    if (i <= 0) return -1;
    if (!parent) return i - 1;
    int p = parent[static_cast<size_t>(b) * N + i];
    return (p >= 0 && p < i) ? p : -2;
}

}  // namespace specv
