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

// Signed int4 nibble k (0..7) of a 32-bit word, as fp32.
template <int K>
__device__ __forceinline__ float nib_f32(uint32_t w)
{
    return (float)(((int32_t)(w << (28 - 4 * K))) >> 28);
}

__device__ __forceinline__ float exp2_approx(float x)
{
    return __builtin_amdgcn_exp2f(x);  // v_exp_f32; exp2(-inf) = 0
}

}  // namespace otq
