// quant_lane.hpp - the int4 quantiser of a vector spread over a group of
// lanes, and the byte positions of the cache layouts.  Shared by the append
// kernel and by the combine's fused one-token append, so both write
// identical codes.
//
// Every step is one IEEE fp32 operation with round-to-nearest-even (the
// bodies forbid contraction into FMAs whatever the file's flags), so the codes
// and scales are bit-identical to any correct evaluation of the same steps
// (quantize_word8 reaches the same correctly rounded quotients by another
// sequence of exactly rounded operations).
#pragma once

#include "common.hpp"

namespace otq {

// E consecutive elements per lane, a scale group spanning the 32 / E
// consecutive lanes of an aligned lane group: returns codes in [-8, 7] in
// c[] and the scale of the lane's group.
template <int E>
__device__ __forceinline__ float quantize_elems(float (&x)[E], int (&c)[E])
{
#pragma clang fp contract(off)
    constexpr int LANES_PER_GROUP = kGroup / E;
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < E; ++e) a = fmaxf(a, fabsf(x[e]));
    a = group_max<LANES_PER_GROUP>(a);  // exact in any order
    const float s = a / 7.0f;  // correctly rounded IEEE division
    // branch-free: with s == 0 the quotient is infinite or NaN, the clamp
    // turns it into -8 or 7 (fmax ignores a NaN operand), and the select
    // gives 0
#pragma unroll
    for (int e = 0; e < E; ++e) {
        float r = rintf(x[e] / s);  // correctly rounded IEEE division, then v_rndne_f32: half to even
        r = fminf(fmaxf(r, -8.0f), 7.0f);
        c[e] = s != 0.0f ? (int)r : 0;
    }
    return s;
}

// Eight consecutive elements per lane, a scale group spanning an aligned quad
// of lanes: returns the 8 codes packed as one word (nibble e = code of x[e],
// two's complement) and the group's scale in `scale`.  The same codes and
// scale as quantize_elems, with fewer operations:
//  - a / 7 and the lane's 8 quotients x / s are rounded correctly by
//    Markstein's division (P. Markstein, IBM J. Res. Dev. 34(1), 1990) from
//    one correctly rounded reciprocal y = RN(1 / b) per divisor b: q =
//    RN(x y) is within 1.5 ulp of x / b; a correction q <- RN(q + RN(x - q
//    b) y) makes it faithful, and from a faithful q the remainder x - q b is
//    exact, so a second correction rounds it correctly (Markstein's theorem,
//    y within half an ulp of 1 / b).  The bounds on a keep every reciprocal
//    normal and every remainder above the subnormal range whenever |x / s| >=
//    2^-13; smaller quotients are not exact but stay far below 1/2, so their
//    code (0) is unchanged.
//  - |x| <= a and s = RN(a / 7) give |x / s| <= 7 (1 + 2^-23): the clamp
//    never acts.  Adding 1.5 * 2^23 + 8 rounds q to an integer, half to even
//    (the constant is even and the sum's ulp is 1), and leaves code + 8, in
//    1..15, in the low nibble of the sum's encoding above a constant part:
//    the shifted encodings add up without carries between nibbles, the sum of
//    the constant parts is cancelled by the accumulator's start value, and
//    an exclusive or with 8 per nibble turns code + 8 into the code's two's
//    complement nibble.
// Other group maxima (zero, below 2^-80, above 2^100, infinite, NaN) divide
// element by element as quantize_elems does.
namespace detail {
constexpr float kRecip7 = 1.0f / 7.0f;  // RN(1/7)
static_assert(__builtin_bit_cast(uint32_t, kRecip7) == 0x3E124925u, "RN(1/7)");
constexpr float kRoundBias = 0x1.8p23f + 8.0f;  // 1.5 * 2^23 + 8
constexpr uint32_t kRoundBiasHigh = 0x4B400000u;  // its encoding less the 8
constexpr uint32_t pack_start()
{
    uint32_t j = 0;
    for (int e = 0; e < 8; ++e) j += kRoundBiasHigh << (4 * e);
    return 0u - j;
}
}  // namespace detail

__device__ __forceinline__ uint32_t quantize_word8(const float (&x)[8], float& scale)
{
#pragma clang fp contract(off)
    float a = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(x[e]));
    a = group_max<4>(a);  // exact in any order
    if (a >= 0x1p-80f && a <= 0x1p100f) {
        constexpr float y7 = detail::kRecip7;
        float s = a * y7;
        s = __builtin_fmaf(__builtin_fmaf(-s, 7.0f, a), y7, s);
        s = __builtin_fmaf(__builtin_fmaf(-s, 7.0f, a), y7, s);  // RN(a / 7)
        scale = s;
        const float y = 1.0f / s;  // correctly rounded IEEE division
        uint32_t acc = detail::pack_start();
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            float q = x[e] * y;
            q = __builtin_fmaf(__builtin_fmaf(-q, s, x[e]), y, q);
            q = __builtin_fmaf(__builtin_fmaf(-q, s, x[e]), y, q);  // RN(x / s)
            acc += __builtin_bit_cast(uint32_t, q + detail::kRoundBias) << (4 * e);
        }
        return acc ^ 0x88888888u;
    }
    const float s = a / 7.0f;  // correctly rounded IEEE division
    scale = s;
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float r = rintf(x[e] / s);  // correctly rounded IEEE division, then half to even
        r = fminf(fmaxf(r, -8.0f), 7.0f);
        word |= ((uint32_t)(s != 0.0f ? (int)r : 0) & 0xFu) << (4 * e);
    }
    return word;
}

// One wave quantises one vector of D elements; lane l owns elements
// [l*E, l*E + E), E = D / 64.
template <int D>
__device__ __forceinline__ float quantize_lane(float (&x)[D / 64], int (&c)[D / 64], int /*lane*/)
{
    return quantize_elems<D / 64>(x, c);
}

// One element per lane, b-bit codes (b = 2 or 3): the group of 32 lanes
// shares s = abs-max / (2^(b-1) - 1) (IEEE division), c = clamp(rint(x / s),
// -2^(b-1), 2^(b-1) - 1), 0 when s == 0 -- the steps of the b-bit append.
__device__ __forceinline__ float quantize_lane_bits(float x, int& c, int bits)
{
#pragma clang fp contract(off)
    const float qmax = (float)((1 << (bits - 1)) - 1), qmin = -(float)(1 << (bits - 1));
    const float a = group_max<kGroup>(fabsf(x));  // exact in any order
    const float s = a / qmax;                     // correctly rounded IEEE division
    float r = rintf(x / s);
    r = fminf(fmaxf(r, qmin), qmax);
    c = s != 0.0f ? (int)r : 0;
    return s;
}

// y <- rot_norm * H y (y already multiplied by the signs), Sylvester order,
// stages in ascending stride; a butterfly replaces (lower, upper) with
// (lower + upper, lower - upper) exactly as the in-place fast Walsh-Hadamard
// transform does.  A vector of D elements spread over D / E consecutive
// lanes (an aligned lane group), E consecutive elements per lane; `lane` is
// the lane's index within its group.
template <int D, int E>
__device__ __forceinline__ void rotate_signed(float (&y)[E], float rot_norm, int lane)
{
#pragma clang fp contract(off)
#pragma unroll
    for (int h = 1; h < E; h <<= 1) {
#pragma unroll
        for (int e = 0; e < E; ++e) {
            if ((e & h) == 0) {
                const float lo = y[e], hi = y[e + h];
                y[e] = lo + hi;
                y[e + h] = lo - hi;
            }
        }
    }
#pragma unroll
    for (int h = E; h < D; h <<= 1) {
        const int m = h / E;
        const bool upper = (lane & m) != 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float o = shfl_xor(y[e], m);
            y[e] = upper ? (o - y[e]) : (y[e] + o);
        }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) y[e] = y[e] * rot_norm;
}

// y <- rot_norm * H (signs (.) y), the signs read for the lane's elements.
template <int D, int E>
__device__ __forceinline__ void rotate_elems(float (&y)[E], const float* __restrict__ signs,
                                             float rot_norm, int lane)
{
#pragma clang fp contract(off)
#pragma unroll
    for (int e = 0; e < E; ++e) y[e] = y[e] * signs[lane * E + e];
    rotate_signed<D, E>(y, rot_norm, lane);
}

// One wave rotates one vector: lane l owns elements [l*E, l*E + E), E = D / 64.
template <int D>
__device__ __forceinline__ void rotate_lane(float (&y)[D / 64], const float* __restrict__ signs,
                                            float rot_norm, int lane)
{
    rotate_elems<D, D / 64>(y, signs, rot_norm, lane);
}

// Byte offset, inside one K row, of the byte holding even channel c and
// channel c + 1: word (r * NG + g) holds channels 32 g + 8 r + 0..7.
template <int D>
__device__ __forceinline__ int k_row_byte(int c)
{
    constexpr int NG = D / kGroup;
    const int g = c >> 5, r = (c >> 3) & 3, k = c & 7;
    return (r * NG + g) * 4 + (k >> 1);
}

// Byte offset, inside one V tile, of the byte holding (channel c, token pair
// starting at even tile-relative token u).
template <int D>
__device__ __forceinline__ int v_tile_byte(int c, int u)
{
    const int r = (u & 15) >> 2;
    const int j = 4 * (u >> 4) + (u & 3);
    const int cb = c >> 4, n = c & 15, a = cb >> 2, b = cb & 3;
    const int word = ((a * 4 + r) * 16 + n) * 4 + b;
    return word * 4 + (j >> 1);
}

}  // namespace otq
