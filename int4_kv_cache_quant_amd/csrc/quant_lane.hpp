// quant_lane.hpp - the int4 quantiser of a vector spread over a group of
// lanes, and the byte positions of the cache layouts.  Shared by the append
// kernel and by the combine's fused one-token append, so both write
// identical codes.
//
// Every step is one IEEE fp32 operation with round-to-nearest-even (the
// bodies forbid contraction into FMAs whatever the file's flags), so the codes
// and scales are bit-identical to any correct evaluation of the same steps.
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

// One wave quantises one vector of D elements; lane l owns elements
// [l*E, l*E + E), E = D / 64.
template <int D>
__device__ __forceinline__ float quantize_lane(float (&x)[D / 64], int (&c)[D / 64], int /*lane*/)
{
    return quantize_elems<D / 64>(x, c);
}

// y <- rot_norm * H (signs (.) y), Sylvester order, stages in ascending
// stride; a butterfly replaces (lower, upper) with (lower + upper,
// lower - upper) exactly as the in-place fast Walsh-Hadamard transform does.
// A vector of D elements spread over D / E consecutive lanes (an aligned
// lane group), E consecutive elements per lane; `lane` is the lane's index
// within its group.
template <int D, int E>
__device__ __forceinline__ void rotate_elems(float (&y)[E], const float* __restrict__ signs,
                                             float rot_norm, int lane)
{
#pragma clang fp contract(off)
#pragma unroll
    for (int e = 0; e < E; ++e) y[e] = y[e] * signs[lane * E + e];
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
