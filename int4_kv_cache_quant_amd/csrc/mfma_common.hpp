// mfma_common.hpp - pieces shared by the MFMA split passes (the int4 one and
// the 2-bit one): operand types, the softmax-reference and value-exponent
// constants, the hi/lo split of the value operand, and DPP lane moves.
#pragma once

#include "common.hpp"

namespace otq {
namespace mfma {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_huge_valf();
// Headroom (base-2 exponent) the softmax reference keeps above the largest
// score seen when it has to move: 4 makes the moves (and their rescale of
// every accumulator) rare after the first tiles; every p stays <= 1.
constexpr float kHeadroom = 4.0f;
// The value operand x = p * s_v * 2^E: E puts the largest V scale seen so
// far at [2^11, 2^12) when it is set, and moves again only once a V scale
// passes 2^15 / 2^E, so x (p <= 1) never leaves fp16's range while the
// dominant terms keep fp16's normal precision.  The bounds cover every fp32
// scale (2^-149 .. 2^128); the partial written at the end splits 2^E
// between l and o (see the merge), which keeps both inside fp32's range.
constexpr int kVTarget = 12;
constexpr int kVLimit = 15;
constexpr int kEMin = -120, kEMax = 165;

// fp16 (x0 - h0, x1 - h1) packed, where (h0, h1) = h2 are x0, x1 rounded to
// fp16: the differences are exact in fp32 and rounded once (v_fma_mix with
// an fp16 operand; register-only instructions).  The results feed an MFMA,
// which must not read a VGPR within 2 wait states of a VALU write; the
// compiler counts no wait states for instructions inside inline asm (without
// them the MFMA read the registers' previous contents: measured, the lo half
// of p * s_v was lost).  The MFMA reads the four pairs of a group together,
// so only the last of them (LAST) ends with the two wait states: the others
// were written earlier still.
typedef uint32_t v4u_t __attribute__((ext_vector_type(4)));
template <bool LAST>
__device__ __forceinline__ uint32_t lo_pair(float x0, float x1, uint32_t h2)
{
    uint32_t r;
    if constexpr (LAST) {
        asm volatile("v_fma_mixlo_f16 %0, %1, 1.0, -%3 op_sel_hi:[0,0,1]\n\t"
                     "v_fma_mixhi_f16 %0, %2, 1.0, -%3 op_sel:[0,0,1] op_sel_hi:[0,0,1]\n\t"
                     "s_nop 1"
                     : "=&v"(r)
                     : "v"(x0), "v"(x1), "v"(h2));
    } else {
        asm volatile("v_fma_mixlo_f16 %0, %1, 1.0, -%3 op_sel_hi:[0,0,1]\n\t"
                     "v_fma_mixhi_f16 %0, %2, 1.0, -%3 op_sel:[0,0,1] op_sel_hi:[0,0,1]"
                     : "=&v"(r)
                     : "v"(x0), "v"(x1), "v"(h2));
    }
    return r;
}

// Lane K (0..3) of each quad of lanes, broadcast to the quad (DPP quad_perm).
template <int K>
__device__ __forceinline__ float quad_bcast(float v)
{
    static_assert(K >= 0 && K < 4, "quad lane");
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), K * 0x55, 0xF, 0xF, true));
}

// Value of lane 4 r + I of the lane's own row (r = lane / 16), by DPP row
// broadcasts: the source differs per row, so the four candidates are selected.
template <int I>
__device__ __forceinline__ float row_quad_gather(float v, int r)
{
    const float v0 = row_bcast<I>(v), v1 = row_bcast<4 + I>(v);
    const float v2 = row_bcast<8 + I>(v), v3 = row_bcast<12 + I>(v);
    return r == 0 ? v0 : r == 1 ? v1 : r == 2 ? v2 : v3;
}

}  // namespace mfma
}  // namespace otq
