// saga_device.hpp -- device-side building blocks shared by the SAGA kernels
// (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace saga {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Order-preserving map of an fp32 value to an unsigned key: a < b as floats
// (finite, -0 treated as its own bit pattern) iff key(a) < key(b) as integers.
__device__ __forceinline__ uint32_t fkey(float f) {
    uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float fkey_inv(uint32_t k) {
    uint32_t u = (k & 0x80000000u) ? (k & 0x7fffffffu) : ~k;
    return __uint_as_float(u);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

// Number of set bits of m strictly below this lane.
__device__ __forceinline__ int mbcnt_lt(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                     __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ u32x4 ld16(const void *p) { return *(const u32x4 *)p; }
__device__ __forceinline__ u32x4 ld16_stream(const void *p) {
    return __builtin_nontemporal_load((const u32x4 *)p);
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// bf16 pair packed in a 32-bit word -> two floats (exact widening).
__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float wave_max(float v) {
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    for (int o = 32; o > 0; o >>= 1) {
        uint32_t w = __shfl_xor(v, o);
        v = v > w ? v : w;
    }
    return v;
}
__device__ __forceinline__ int wave_sum_i32(int v) {
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

// DPP controls (GFX9 encoding).
constexpr int kDppRowShr1 = 0x111, kDppRowShr2 = 0x112, kDppRowShr4 = 0x114, kDppRowShr8 = 0x118;
constexpr int kDppRowBcast15 = 0x142, kDppRowBcast31 = 0x143;
constexpr int kDppSwapPairs = 0xB1;  // quad_perm [1,0,3,2]: lane l reads lane l ^ 1
constexpr int kDppQuadXor2 = 0x4E;   // quad_perm [2,3,0,1]: lane l reads lane l ^ 2
constexpr int kDppRowRor4 = 0x124, kDppRowRor8 = 0x128;  // rotations within 16-lane rows

// v of the lane a DPP control names (every lane valid).
template <int CTRL>
__device__ __forceinline__ int dppi(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xf, 0xf, false);
}
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
    return __int_as_float(dppi<CTRL>(__float_as_int(v)));
}

// The 16-byte vector of lane l ^ 1.
__device__ __forceinline__ u32x4 swap_pairs(u32x4 v) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = (uint32_t)dppi<kDppSwapPairs>((int)v[i]);
    return r;
}

// Maximum over the wave through DPP within 16-lane rows and four readlanes
// (no LDS); the result is wave-uniform.
__device__ __forceinline__ uint32_t wave_max_u32_dpp(uint32_t v) {
    auto mx = [](uint32_t x, uint32_t y) { return x > y ? x : y; };
    v = mx(v, (uint32_t)dppi<kDppSwapPairs>((int)v));
    v = mx(v, (uint32_t)dppi<kDppQuadXor2>((int)v));
    v = mx(v, (uint32_t)dppi<kDppRowRor4>((int)v));
    v = mx(v, (uint32_t)dppi<kDppRowRor8>((int)v));
    const int x = (int)v;
    return mx(mx((uint32_t)__builtin_amdgcn_readlane(x, 0), (uint32_t)__builtin_amdgcn_readlane(x, 16)),
              mx((uint32_t)__builtin_amdgcn_readlane(x, 32), (uint32_t)__builtin_amdgcn_readlane(x, 48)));
}

// Sum of v over the lanes of its 16-lane row whose index agrees with its own
// modulo P (P = 1, 2, 4 or 8); every lane receives its sum, in a fixed order.
template <int P>
__device__ __forceinline__ float row_sum_mod(float v) {
    static_assert(P == 1 || P == 2 || P == 4 || P == 8, "row_sum_mod");
    if constexpr (P == 1) v += dppf<kDppSwapPairs>(v);
    if constexpr (P <= 2) v += dppf<kDppQuadXor2>(v);
    if constexpr (P <= 4) v += dppf<kDppRowRor4>(v);
    v += dppf<kDppRowRor8>(v);
    return v;
}

typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// u of lane l ^ 16, through the gfx950 row-pair swap (no LDS): for a lane in
// 16-lane row R the swap's first result comes from row R & ~1, its second from
// row R | 1.
__device__ __forceinline__ unsigned from_xor16(unsigned u) {
    const u32x2 h = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return (threadIdx.x & 16) ? h[0] : h[1];
}
// u of lane l ^ 32, through the half swap: for a lane in row R the first
// result comes from row R & 1, the second from row 2 + (R & 1).
__device__ __forceinline__ unsigned from_xor32(unsigned u) {
    const u32x2 f = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return (threadIdx.x & 32) ? f[0] : f[1];
}
// v plus v of lane l ^ 16 (or ^ 32): the same sum as with __shfl_xor, one
// commutative add of the same two values.
__device__ __forceinline__ float add_xor16(float v) {
    return v + __uint_as_float(from_xor16(__float_as_uint(v)));
}
__device__ __forceinline__ float add_xor32(float v) {
    return v + __uint_as_float(from_xor32(__float_as_uint(v)));
}

// v plus v of lane l ^ O: within 16-lane rows by DPP (a rotation of a row by
// 8 is l ^ 8), across them by the row swaps; only O = 4 goes through LDS.
template <int O>
__device__ __forceinline__ float add_xor(float v) {
    static_assert(O == 1 || O == 2 || O == 4 || O == 8 || O == 16 || O == 32, "add_xor");
    if constexpr (O == 1) return v + dppf<kDppSwapPairs>(v);
    else if constexpr (O == 2) return v + dppf<kDppQuadXor2>(v);
    else if constexpr (O == 8) return v + dppf<kDppRowRor8>(v);
    else if constexpr (O == 16) return add_xor16(v);
    else if constexpr (O == 32) return add_xor32(v);
    else return v + __shfl_xor(v, O);
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP row shifts and
// row broadcasts (no LDS traffic).
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr1, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr2, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr4, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowShr8, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowBcast15, 0xa, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, kDppRowBcast31, 0xc, 0xf, false);
    return x;
}

// Block-wide exclusive scan of v over the NW*64 threads of a block; returns
// the prefix, *total receives the sum.  Uses red[NW] of LDS; contains two
// barriers, so every thread of the block must call it.
template <int NW>
__device__ __forceinline__ int block_excl_scan(int v, int *red, int *total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int x = wave_incl_scan(v);
    if (lane == 63) red[wave] = x;
    __syncthreads();
    int before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        before += (w < wave) ? red[w] : 0;
        tot += red[w];
    }
    __syncthreads();
    *total = tot;
    return before + x - v;
}

// First query head of key head g's group: ceil(g*h_q/h_k), so that
// floor(j*h_k/h_q) == g  <=>  group_lo(g) <= j < group_lo(g+1).
// 32-bit arithmetic: the plan admits h_q <= 32768, so g * h_q < 2^30.
__device__ __forceinline__ int group_lo(int g, int h_q, int h_k) {
    return (g * h_q + h_k - 1) / h_k;
}

}  // namespace saga
