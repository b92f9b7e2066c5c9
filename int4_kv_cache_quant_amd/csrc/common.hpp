// common.hpp - device helpers shared by the gfx950 kernels of libotq.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>
#include <utility>

namespace otq {

constexpr int kGroup = 32;  // elements per scale group
constexpr int kTile = 32;   // tokens per V tile
constexpr float kLog2e = 1.4426950408889634f;

// ------------------------------------------------------------ compile-time loops
template <typename F, int... Is>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, Is...>)
{
    (f(std::integral_constant<int, Is>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f)
{
    static_for_impl(static_cast<F&&>(f), std::make_integer_sequence<int, N>{});
}

// ------------------------------------------------------------ 16-bit inputs
__device__ __forceinline__ float f16_bits_to_f32(uint16_t b)
{
    return (float)__builtin_bit_cast(_Float16, b);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b)
{
    return __builtin_bit_cast(float, (uint32_t)b << 16);
}
__device__ __forceinline__ float widen(uint16_t b, int dtype)
{
    return dtype == 0 ? f16_bits_to_f32(b) : bf16_bits_to_f32(b);
}

// ------------------------------------------------------------ cross-lane
// Broadcast lane K (0..15) of each row of 16 lanes to the whole row (DPP
// row_newbcast, gfx90a and later).  bound_ctrl is set (every source lane is
// valid anyway) so that the move can fold into a consuming v_mul / v_add.
template <int K>
__device__ __forceinline__ float row_bcast(float v)
{
    static_assert(K >= 0 && K < 16, "row lane");
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x150 + K, 0xF, 0xF, true));
}

__device__ __forceinline__ float shfl_xor(float v, int m)
{
    return __shfl_xor(v, m, 64);
}

// Cross-row exchanges without LDS: v_permlane16_swap pairs rows (0,1) and
// (2,3) of the wave, v_permlane32_swap its two halves; applied to two copies
// of a value, each lane ends up with its own value and its partner's, one in
// each register.  Written as inline asm (a register move, no memory access):
// the compiler builtin's two results are treated as equal when both inputs
// are one value, which would drop the partner's.  The s_nop covers the wait
// states between a VALU write and the swap reading it.
__device__ __forceinline__ void swap_rows16(unsigned& a, unsigned& b)
{
    asm volatile("s_nop 1\n\tv_permlane16_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ void swap_rows32(unsigned& a, unsigned& b)
{
    asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
}
template <bool XOR16>
__device__ __forceinline__ void pair_values(float v, float& x, float& y)
{
    unsigned a = __builtin_bit_cast(unsigned, v), b = a;
    if constexpr (XOR16) swap_rows16(a, b);
    else swap_rows32(a, b);
    x = __builtin_bit_cast(float, a);
    y = __builtin_bit_cast(float, b);
}
__device__ __forceinline__ float max_xor16(float v)
{
    float x, y;
    pair_values<true>(v, x, y);
    return fmaxf(x, y);
}
__device__ __forceinline__ float max_xor32(float v)
{
    float x, y;
    pair_values<false>(v, x, y);
    return fmaxf(x, y);
}
__device__ __forceinline__ float sum_xor16(float v)
{
    float x, y;
    pair_values<true>(v, x, y);
    return x + y;
}
__device__ __forceinline__ float sum_xor32(float v)
{
    float x, y;
    pair_values<false>(v, x, y);
    return x + y;
}

// Other DPP lane moves (bound_ctrl set: every source lane is valid), which the
// compiler folds into the consuming v_max / v_add: quad_perm swaps of lanes
// 1 and 2 apart, the mirror of each half-row of 8 and of each row of 16, and
// the rotation of a row by 8 (lane i reads lane i ^ 8).
constexpr int kDppXor1 = 0xB1, kDppXor2 = 0x4E, kDppHalfMirror = 0x141, kDppMirror = 0x140,
              kDppRor8 = 0x128;
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v)
{
    return __builtin_bit_cast(float,
                              __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, true));
}

// Maximum / sum over each aligned group of N lanes (N = 1, 2, 4, ..., 64),
// every lane of the group getting the result; all 64 lanes must be active.
template <int N>
__device__ __forceinline__ float group_max(float v)
{
    static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "group size");
    if constexpr (N >= 2) v = fmaxf(v, dpp_mov<kDppXor1>(v));
    if constexpr (N >= 4) v = fmaxf(v, dpp_mov<kDppXor2>(v));
    if constexpr (N >= 8) v = fmaxf(v, dpp_mov<kDppHalfMirror>(v));
    if constexpr (N >= 16) v = fmaxf(v, dpp_mov<kDppMirror>(v));
    if constexpr (N >= 32) v = max_xor16(v);
    if constexpr (N >= 64) v = max_xor32(v);
    return v;
}
template <int N>
__device__ __forceinline__ float group_sum(float v)
{
    static_assert(N >= 1 && N <= 64 && (N & (N - 1)) == 0, "group size");
    if constexpr (N >= 2) v += dpp_mov<kDppXor1>(v);
    if constexpr (N >= 4) v += dpp_mov<kDppXor2>(v);
    if constexpr (N >= 8) v += dpp_mov<kDppHalfMirror>(v);
    if constexpr (N >= 16) v += dpp_mov<kDppMirror>(v);
    if constexpr (N >= 32) v = sum_xor16(v);
    if constexpr (N >= 64) v = sum_xor32(v);
    return v;
}

// Signed int4 nibble k (0..7) of a 32-bit word, as fp32.
template <int K>
__device__ __forceinline__ float nib_f32(uint32_t w)
{
    return (float)(((int32_t)(w << (28 - 4 * K))) >> 28);
}

// ------------------------------------------------------------ contract violations
// Bits of the library's device error word (otq_last_device_error): set with
// a device-scope atomic or, only on the rare path where a kernel meets an
// argument outside the caller's contract (the kernel then clamps or skips as
// documented and carries on).
constexpr unsigned kErrPos = 1u;   // an append position outside [0, capacity - n_new]
constexpr unsigned kErrLens = 2u;  // a length outside [0, max_len]
__device__ __forceinline__ void report_error(unsigned* err, unsigned flag)
{
    __hip_atomic_fetch_or(err, flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ float exp2_approx(float x)
{
    return __builtin_amdgcn_exp2f(x);  // v_exp_f32; exp2(-inf) = 0
}

}  // namespace otq
