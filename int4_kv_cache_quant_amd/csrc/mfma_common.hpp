// mfma_common.hpp - pieces shared by the MFMA split passes (the int4 one and
// the b-bit one): operand types, the softmax-reference and value-exponent
// constants, the hi/lo split of the value operand, DPP lane moves, and the
// rotations of the query in the passes' register layout.
#pragma once

#include "common.hpp"
#include "srft.hpp"

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

// Butterfly across lane bit 4 (XOR16) or bit 5 (XOR32 = false): the lane with
// that bit clear gets lo + hi, its partner lo - hi.  first_lo says whether the
// swap's first register holds the value of the lane with the bit clear (told
// by swapping the lane's own row index once).
template <bool XOR16>
__device__ __forceinline__ float butterfly_lanes(float v, bool first_lo, bool upper)
{
    float x, y;
    pair_values<XOR16>(v, x, y);
    const float lo = first_lo ? x : y, hi = first_lo ? y : x;
    return upper ? lo - hi : lo + hi;
}

// The query's FFT rotation (without rot_norm, which the score multiplier
// carries) in the split kernel's query layout: lane (n16, r) holds channels
// 32 g + 8 r + e in qx[g][e], i.e. complex number j = 16 g + 4 r + e / 2,
// component e % 2.  Decimation-in-frequency stages of half-size h: h >= 16
// pair g with g + h / 16 in the lane, h = 8 and 4 pair lanes 32 and 16
// apart, h = 2 and 1 pair complex numbers inside an 8-channel run.
template <int NG>
__device__ __forceinline__ void srft_query(float (&qx)[NG][8], int r)
{
    constexpr int N = 16 * NG;
    auto bfly = [](float& ar, float& ai, float& br, float& bi, int u) {
        const float wr = srft_detail::kTw.re[u], wi = srft_detail::kTw.im[u];
        const float dr = ar - br, di = ai - bi;
        ar = ar + br;
        ai = ai + bi;
        br = dr * wr - di * wi;
        bi = dr * wi + di * wr;
    };
#pragma unroll
    for (int h = N / 2; h >= 16; h >>= 1) {
        const int gm = h / 16;
#pragma unroll
        for (int g = 0; g < NG; ++g)
            if ((g & gm) == 0)
#pragma unroll
                for (int cp = 0; cp < 4; ++cp)
                    bfly(qx[g][2 * cp], qx[g][2 * cp + 1], qx[g + gm][2 * cp], qx[g + gm][2 * cp + 1],
                         (16 * (g % gm) + 4 * r + cp) * (64 / h));
    }
#pragma unroll
    for (int h = 8; h >= 4; h >>= 1) {  // lanes 32 (r bit 1) and 16 (r bit 0) apart
        const int m = h == 8 ? 32 : 16;
        const bool upper = (r & (h / 4)) != 0;
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int cp = 0; cp < 4; ++cp) {
                const float ore = shfl_xor(qx[g][2 * cp], m), oim = shfl_xor(qx[g][2 * cp + 1], m);
                const int u = ((4 * r + cp) & (h - 1)) * (64 / h);
                const float wr = srft_detail::kTw.re[u], wi = srft_detail::kTw.im[u];
                const float dr = ore - qx[g][2 * cp], di = oim - qx[g][2 * cp + 1];
                const float ur = dr * wr - di * wi, ui = dr * wi + di * wr;
                qx[g][2 * cp] = upper ? ur : qx[g][2 * cp] + ore;
                qx[g][2 * cp + 1] = upper ? ui : qx[g][2 * cp + 1] + oim;
            }
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        // h = 2: complex 0 with 2, 1 with 3; h = 1: 0 with 1, 2 with 3
        bfly(qx[g][0], qx[g][1], qx[g][4], qx[g][5], 0);
        bfly(qx[g][2], qx[g][3], qx[g][6], qx[g][7], 32);
        bfly(qx[g][0], qx[g][1], qx[g][2], qx[g][3], 0);
        bfly(qx[g][4], qx[g][5], qx[g][6], qx[g][7], 0);
    }
}

// The query's mixed-radix FFT at head_dim 192 (N = 96 = 3 * 32 complex
// numbers; without rot_norm) in the same layout, complex j = 16 g + 4 r +
// e / 2 in qx[g][e], g < 6.  The radix-3 stage combines j, j + 32, j + 64:
// groups g, g + 2, g + 4 of the lane, its outputs m = 0, 1, 2 going to
// groups g + 2 m.  Inside each block of 32 (groups 2 m, 2 m + 1) the radix-2
// stages of half-size 16 pair the block's two groups, 8 and 4 pair lanes 32
// and 16 apart, 2 and 1 stay in the 8-channel run; twiddle index (j mod h)
// 96 / (2 h).
__device__ __forceinline__ void srft_query192(float (&qx)[6][8], int r)
{
    using srft_detail::kC3;
    using srft_detail::kTw96;
    auto cmul = [](float& xr, float& xi, int u) {
        const float wr = kTw96.re[u], wi = kTw96.im[u];
        const float pr = xr * wr - xi * wi, pi = xr * wi + xi * wr;
        xr = pr;
        xi = pi;
    };
    auto bfly = [&](float& ar, float& ai, float& br, float& bi, int u) {
        float dr = ar - br, di = ai - bi;
        ar = ar + br;
        ai = ai + bi;
        cmul(dr, di, u);
        br = dr;
        bi = di;
    };
#pragma unroll
    for (int g0 = 0; g0 < 2; ++g0)
#pragma unroll
        for (int cp = 0; cp < 4; ++cp) {
            const int j = 16 * g0 + 4 * r + cp;
            float& a0r = qx[g0][2 * cp];
            float& a0i = qx[g0][2 * cp + 1];
            float& a1r = qx[g0 + 2][2 * cp];
            float& a1i = qx[g0 + 2][2 * cp + 1];
            float& a2r = qx[g0 + 4][2 * cp];
            float& a2i = qx[g0 + 4][2 * cp + 1];
            const float sr = a1r + a2r, si = a1i + a2i, dr = a1r - a2r, di = a1i - a2i;
            const float mr = a0r - 0.5f * sr, mi = a0i - 0.5f * si;
            const float tr = kC3 * dr, ti = kC3 * di;
            a0r = a0r + sr;
            a0i = a0i + si;
            a1r = mr + ti;  // (m - i t) W^j
            a1i = mi - tr;
            cmul(a1r, a1i, j);
            a2r = mr - ti;  // (m + i t) W^2j
            a2i = mi + tr;
            cmul(a2r, a2i, 2 * j);
        }
#pragma unroll
    for (int m = 0; m < 3; ++m)
#pragma unroll
        for (int cp = 0; cp < 4; ++cp)  // h = 16: block position 4 r + cp with 16 + 4 r + cp
            bfly(qx[2 * m][2 * cp], qx[2 * m][2 * cp + 1], qx[2 * m + 1][2 * cp], qx[2 * m + 1][2 * cp + 1],
                 3 * (4 * r + cp));
#pragma unroll
    for (int h = 8; h >= 4; h >>= 1) {  // lanes 32 (r bit 1) and 16 (r bit 0) apart
        const int lm = h == 8 ? 32 : 16;
        const bool upper = (r & (h / 4)) != 0;
#pragma unroll
        for (int g = 0; g < 6; ++g)
#pragma unroll
            for (int cp = 0; cp < 4; ++cp) {
                const float ore = shfl_xor(qx[g][2 * cp], lm), oim = shfl_xor(qx[g][2 * cp + 1], lm);
                float dr = ore - qx[g][2 * cp], di = oim - qx[g][2 * cp + 1];
                cmul(dr, di, ((4 * r + cp) & (h - 1)) * (96 / (2 * h)));
                qx[g][2 * cp] = upper ? dr : qx[g][2 * cp] + ore;
                qx[g][2 * cp + 1] = upper ? di : qx[g][2 * cp + 1] + oim;
            }
    }
#pragma unroll
    for (int g = 0; g < 6; ++g) {
        // h = 2: complex 0 with 2, 1 with 3 (W^24 for the odd pair); h = 1
        bfly(qx[g][0], qx[g][1], qx[g][4], qx[g][5], 0);
        bfly(qx[g][2], qx[g][3], qx[g][6], qx[g][7], 24);
        bfly(qx[g][0], qx[g][1], qx[g][2], qx[g][3], 0);
        bfly(qx[g][4], qx[g][5], qx[g][6], qx[g][7], 0);
    }
}

// The query's Walsh-Hadamard rotation (without rot_norm, which the score
// multiplier carries) in the split kernels' query layout: lane (n16, r)
// holds channels 32 g + 8 r + e in qx[g][e].  The butterflies over channel
// bits 0-2 stay in the lane, bits 3 and 4 pair lanes 16 and 32 apart, bits
// 5.. pair the lane's groups (the stages of the transform commute).
template <int NG>
__device__ __forceinline__ void fwht_query(float (&qx)[NG][8], int r)
{
#pragma clang fp contract(off)
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int h = 1; h < 8; h <<= 1)
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if ((e & h) == 0) {
                    const float lo = qx[g][e], hi = qx[g][e + h];
                    qx[g][e] = lo + hi;
                    qx[g][e + h] = lo - hi;
                }
    unsigned ra = (unsigned)r, rb = ra;
    swap_rows16(ra, rb);
    const bool lo16 = (ra & 1u) == 0;
    ra = (unsigned)r; rb = ra;
    swap_rows32(ra, rb);
    const bool lo32 = (ra & 2u) == 0;
#pragma unroll
    for (int g = 0; g < NG; ++g)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            qx[g][e] = butterfly_lanes<true>(qx[g][e], lo16, (r & 1) != 0);
            qx[g][e] = butterfly_lanes<false>(qx[g][e], lo32, (r & 2) != 0);
        }
#pragma unroll
    for (int h = 1; h < NG; h <<= 1)
#pragma unroll
        for (int g = 0; g < NG; ++g)
            if ((g & h) == 0)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float lo = qx[g][e], hi = qx[g + h][e];
                    qx[g][e] = lo + hi;
                    qx[g + h][e] = lo - hi;
                }
}

// MFMA k-slot e of an unpacked word holds element kSlot[e] (0..7) of the
// word, scaled by 2^kShift[e] (times 2^-24 for the subnormal form):
// registers are (0,4), (1,5), (2,6), (3,7), each one mask of the word or of
// the word shifted by 8 bits.
constexpr int kSlot[8] = {0, 4, 1, 5, 2, 6, 3, 7};
constexpr int kShift[8] = {0, 0, 4, 4, 0, 0, 4, 4};

// 8 signed nibbles -> 8 fp16 subnormals (c + 8) * 2^(kShift[e] - 24) (the K
// operand of the score products).
__device__ __forceinline__ half8_t unpack_codes_sub(uint32_t w)
{
    const uint32_t w8 = w >> 8;
    uint32_t r[4];
    r[0] = (w ^ 0x88888888u) & 0x000F000Fu;
    r[1] = (w ^ 0x88888888u) & 0x00F000F0u;
    r[2] = (w8 ^ 0x00888888u) & 0x000F000Fu;
    r[3] = (w8 ^ 0x00888888u) & 0x00F000F0u;
    half8_t out;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const half2_t p = __builtin_bit_cast(half2_t, r[m]);
        out[2 * m] = p[0];
        out[2 * m + 1] = p[1];
    }
    return out;
}

// 8 signed nibbles -> 8 normal fp16 values c * 2^kShift[e] (exact): the
// offset-binary value n = c + 8 of a nibble goes into the mantissa of 1024.0
// (0x6400, ulp 1), at bit 0 (1024 + n) or bit 4 (1024 + 16 n); one packed
// subtraction of 1032 or 1152 then leaves c or 16 c.  One and-xor per
// register, as for the subnormal form, plus one packed fp16 subtraction.
__device__ __forceinline__ half8_t unpack_codes_signed(uint32_t w)
{
    const uint32_t w8 = w >> 8;
    const half2_t b0 = half2_t{(_Float16)1032.0f, (_Float16)1032.0f};
    const half2_t b4 = half2_t{(_Float16)1152.0f, (_Float16)1152.0f};
    half2_t h[4];
    h[0] = __builtin_bit_cast(half2_t, (w & 0x000F000Fu) ^ 0x64086408u) - b0;   // elements 0, 4
    h[1] = __builtin_bit_cast(half2_t, (w & 0x00F000F0u) ^ 0x64806480u) - b4;   // elements 1, 5
    h[2] = __builtin_bit_cast(half2_t, (w8 & 0x000F000Fu) ^ 0x64086408u) - b0;  // elements 2, 6
    h[3] = __builtin_bit_cast(half2_t, (w8 & 0x00F000F0u) ^ 0x64806480u) - b4;  // elements 3, 7
    half8_t out;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        out[2 * m] = h[m][0];
        out[2 * m + 1] = h[m][1];
    }
    return out;
}

}  // namespace mfma
}  // namespace otq
