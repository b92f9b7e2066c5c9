// bits_layout.hpp - the V tile layout of 2- and 3-bit caches.
//
// V codes of a b-bit cache are stored per tile of 32 tokens (tile t of a
// (sequence, KV head) holds tokens 32 t .. 32 t + 31, 32 D b / 8 bytes, the
// same bytes as 32 plain rows), regrouped so that the matrix-core split pass
// reads its value operands with one wide load per lane.  Tile-relative token
// u has half h = u / 16, quarter r = (u % 16) / 4 and slot m = u % 4; channel
// c has block cb = c / 16 and column n = c % 16; lane l = 16 r + n.  Every
// field is the code's two's complement b bits.
//
//  2 bits: lane l owns the D / 32 words l (D / 32) + j, j = cb / 2; the field
//          of (u, c) sits at bit 16 h + 8 (cb % 2) + 2 m of word j.
//  3 bits: lane l owns 3 D / 64 words, three per quad qd = cb / 4 of channel
//          blocks: l (3 D / 64) + 3 qd + w.  For cb % 4 = w < 3 the field of
//          (u, c) sits at bit 16 h + 3 m of word w (bits 0..11 and 16..27);
//          the 24 bits of block 4 qd + 3 fill the top nibbles: bit i (0..2)
//          of its field for slot m is chunk bit p = 3 m + i, held at bit
//          16 h + 12 + p % 4 of word p / 4.
//
// So the two codes of an MFMA k-slot pair (tokens 4 r + m and 16 + 4 r + m,
// one channel) lie in the two 16-bit halves of one word at the same offset,
// ready for the and-xor masks that turn them into fp16 operands.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace otq {

template <int D, int BITS>
struct VBitsTile {
    static_assert(BITS == 2 || BITS == 3, "2- or 3-bit codes");
    static constexpr int WPL = BITS == 2 ? D / 32 : 3 * D / 64;  // words per lane
    static constexpr int WORDS = 64 * WPL;                       // per tile: 2 D or 3 D
    static constexpr int TOKEN_WORDS = 16 * WPL;                 // words holding one token's fields
};

// Calls f(u, c, pos, width, shift) for each piece of a field in tile word
// W: bits [pos, pos + width) of the word hold bits [shift, shift + width) of
// the code of (token u, channel c).
template <int D, int BITS, typename F>
__device__ __forceinline__ void vtile_fields(int W, F&& f)
{
    using T = VBitsTile<D, BITS>;
    const int l = W / T::WPL, k = W % T::WPL, r = l >> 4, n = l & 15;
    if constexpr (BITS == 2) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int m = 0; m < 4; ++m)
                    f(16 * h + 4 * r + m, 16 * (2 * k + t) + n, 16 * h + 8 * t + 2 * m, 2, 0);
    } else {
        const int qd = k / 3, w = k % 3;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
#pragma unroll
            for (int m = 0; m < 4; ++m) f(16 * h + 4 * r + m, 16 * (4 * qd + w) + n, 16 * h + 3 * m, 3, 0);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int p = 4 * w + i;
                f(16 * h + 4 * r + p / 3, 16 * (4 * qd + 3) + n, 16 * h + 12 + i, 1, p % 3);
            }
        }
    }
}

// Tile word index of the x-th word (x < TOKEN_WORDS) that holds fields of
// tile-relative token u.
template <int D, int BITS>
__device__ __forceinline__ int vtile_token_word(int u, int x)
{
    using T = VBitsTile<D, BITS>;
    const int r = (u >> 2) & 3, n = x & 15, k = x >> 4;
    return (16 * r + n) * T::WPL + k;
}

// Signed code of (token u, channel c) in a tile's words.
template <int D, int BITS>
__device__ __forceinline__ int vtile_code(const uint32_t* tw, int u, int c)
{
    using T = VBitsTile<D, BITS>;
    const int h = u >> 4, r = (u >> 2) & 3, m = u & 3, cb = c >> 4, n = c & 15;
    const uint32_t* lw = tw + (16 * r + n) * T::WPL;
    uint32_t f;
    if constexpr (BITS == 2) {
        f = (lw[cb >> 1] >> (16 * h + 8 * (cb & 1) + 2 * m)) & 3u;
    } else {
        const uint32_t* qw = lw + 3 * (cb >> 2);
        if ((cb & 3) < 3) {
            f = (qw[cb & 3] >> (16 * h + 3 * m)) & 7u;
        } else {
            f = 0;
#pragma unroll
            for (int i = 0; i < 3; ++i) {
                const int p = 3 * m + i;
                f |= ((qw[p >> 2] >> (16 * h + 12 + (p & 3))) & 1u) << i;
            }
        }
    }
    return (int)(f << (32 - BITS)) >> (32 - BITS);
}

}  // namespace otq
