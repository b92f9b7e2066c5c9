// quantize.hip - on-the-fly int4 quantisation of new K/V vectors into the
// cache (Open-TQ-Metal abstract: the KV cache is quantised to int4 as it is
// produced).  One fused pass per vector: optional sign-randomised Hadamard
// rotation of K, group abs-max, scale, round, clamp and nibble pack, as the
// agents-report "SRFT + int4 KV-cache" page describes for its single-dispatch
// quantiser (core-method section), here with the Walsh-Hadamard rotation of
// the AdapTQ page (section on Fast Hadamard Rotation).
//
// Built with -ffp-contract=off: every step is one IEEE fp32 operation with
// round-to-nearest-even, so the codes and scales are bit-identical to any
// correct evaluation of the same steps.
#include "common.hpp"
#include "kernels.hpp"
#include "quant_lane.hpp"

namespace otq {

namespace {

// Appends of fewer tokens take the one-pair-per-wave kernel.
constexpr int kPairKernelMaxTokens = 8;

// Small appends (a decode step's token): one wave per pair of positions,
// E = D / 64 elements per lane, so that a lone token's quantisation is a
// short chain.
template <int D>
__global__ __launch_bounds__(256) void quantize_pair_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int dtype, int n_new,
    int H, int cap, uint8_t* __restrict__ kc, float* __restrict__ ks, uint8_t* __restrict__ vc,
    float* __restrict__ vs, const float* __restrict__ signs, float rot_norm,
    const int32_t* __restrict__ pos, int pair_slots)
{
    constexpr int E = D / 64;
    constexpr int NG = D / kGroup;
    const int lane = threadIdx.x & 63;
    const int slot = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (slot >= pair_slots) return;
    const int h = blockIdx.y, b = blockIdx.z;
    const int p0 = pos[b];
    const int t0 = ((p0 >> 1) + slot) * 2;  // even absolute position
    const size_t head = (size_t)b * H + h;

    bool fresh[2];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int t = t0 + s;
        fresh[s] = t >= p0 && t < p0 + n_new && t >= 0 && t < cap;
    }
    if (!fresh[0] && !fresh[1]) return;  // wave-uniform

    // Tokens t0 and t0 + 1 share one V byte per channel.  When only one of
    // them is new, the other's nibbles are read first, so that the read
    // overlaps the K/V loads instead of following the quantisation (t0 + 1 <
    // cap: cap is even).
    const int tile = t0 / kTile;
    uint8_t* vt = vc + (head * (cap / kTile) + tile) * (size_t)(16 * D);
    uint8_t old[E];
    const bool partial = fresh[0] != fresh[1];
    if (partial) {
#pragma unroll
        for (int e = 0; e < E; ++e) old[e] = vt[v_tile_byte<D>(lane * E + e, t0 % kTile)];
    }

    int vcode[2][E];
#pragma unroll
    for (int s = 0; s < 2; ++s) {
        const int t = t0 + s;
#pragma unroll
        for (int e = 0; e < E; ++e) vcode[s][e] = 0;
        if (!fresh[s]) continue;  // wave-uniform
        const size_t src = (head * n_new + (t - p0)) * D + (size_t)lane * E;
        const size_t row = head * cap + t;

        // K: widen, rotate, quantise, store row + scales
        float x[E];
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] = widen(k[src + e], dtype);
        if (signs) rotate_lane<D>(x, signs, rot_norm, lane);
        int c[E];
        float sk = quantize_lane<D>(x, c, lane);
        uint8_t* krow = kc + row * (D / 2);
        if constexpr (E == 1) {
            const int other = __shfl_xor(c[0], 1, 64);
            if ((lane & 1) == 0)
                krow[k_row_byte<D>(lane)] = (uint8_t)((c[0] & 0xF) | ((other & 0xF) << 4));
        } else {
#pragma unroll
            for (int e = 0; e < E; e += 2)
                krow[k_row_byte<D>(lane * E + e)] = (uint8_t)((c[e] & 0xF) | ((c[e + 1] & 0xF) << 4));
        }
        if (lane % (kGroup / E) == 0) ks[row * NG + (lane * E) / kGroup] = sk;

        // V: widen, quantise, store scales; nibbles are stored per pair below
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] = widen(v[src + e], dtype);
        float sv = quantize_lane<D>(x, vcode[s], lane);
        if (lane % (kGroup / E) == 0) vs[row * NG + (lane * E) / kGroup] = sv;
    }
    // V nibbles of the pair
#pragma unroll
    for (int e = 0; e < E; ++e) {
        const int ch = lane * E + e;
        uint32_t lo = vcode[0][e] & 0xF, hi = vcode[1][e] & 0xF;
        if (partial) {
            if (!fresh[0]) lo = old[e] & 0xF;
            if (!fresh[1]) hi = old[e] >> 4;
        }
        vt[v_tile_byte<D>(ch, t0 % kTile)] = (uint8_t)(lo | (hi << 4));
    }
}

// Lane layout: each token of the wave occupies LT = D / 8 consecutive lanes,
// and lane j of a token holds its 8 consecutive channels 8 j .. 8 j + 7 (one
// 16-byte load).  A scale group (32 channels) is then one aligned quad of
// lanes, and a lane's 8 codes are exactly one 32-bit word of the K row
// (quarter-interleaved: word r NG + g holds channels 32 g + 8 r + 0..7).
// A wave covers TW = 64 / LT tokens starting at an even position, so the two
// tokens sharing a V byte are in the wave, LT lanes apart.
template <int D>
__global__ __launch_bounds__(256) void quantize_append_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int dtype, int n_new,
    int H, int cap, uint8_t* __restrict__ kc, float* __restrict__ ks, uint8_t* __restrict__ vc,
    float* __restrict__ vs, const float* __restrict__ signs, float rot_norm,
    const int32_t* __restrict__ pos, int wave_slots)
{
    constexpr int NG = D / kGroup;
    constexpr int LT = D / 8;   // lanes per token
    constexpr int TW = 64 / LT;  // tokens per wave
    const int lane = threadIdx.x & 63;
    const int slot = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (slot >= wave_slots) return;
    const int h = blockIdx.y, b = blockIdx.z;
    const int p0 = pos[b];
    const int tw = lane / LT, j = lane % LT;  // token of the wave, channel block
    const int t = (p0 & ~1) + slot * TW + tw;  // absolute position (the wave starts even)
    const size_t head = (size_t)b * H + h;
    const bool fresh = t >= p0 && t < p0 + n_new && t >= 0 && t < cap;
    if (__ballot(fresh) == 0) return;  // wave-uniform
    const bool fresh_pair = __shfl_xor(fresh ? 1 : 0, LT, 64) != 0;  // the token sharing t's V byte
    const size_t row = head * cap + t;
    const size_t src = (head * n_new + (t - p0)) * D + 8 * j;
    const int c0 = 8 * j, g = j / 4, r = j % 4;

    // Where only one token of a pair is new, the byte keeps the other's
    // nibble: both lanes of the pair read the old bytes of the 4 channels
    // they write (before the quantisation, so that the loads overlap).  Pairs
    // are aligned to even positions and capacity is even, so both tokens of
    // a partial pair lie inside the cache.
    const bool partial = fresh != fresh_pair;
    const int tt = t >= 0 ? t : 0;
    uint8_t* vt = vc + (head * (cap / kTile) + tt / kTile) * (size_t)(16 * D);
    const int u = (tt % kTile) & ~1;  // tile-relative even token of the pair
    const int half = t & 1;           // writes channels c0 + 4 half .. + 3
    uint32_t old4 = 0;
    if (partial) {
#pragma unroll
        for (int e = 0; e < 4; ++e)
            old4 |= (uint32_t)vt[v_tile_byte<D>(c0 + 4 * half + e, u)] << (8 * e);
    }

    uint4 kraw = make_uint4(0, 0, 0, 0), vraw = make_uint4(0, 0, 0, 0);
    if (fresh) {
        kraw = *reinterpret_cast<const uint4*>(k + src);
        vraw = *reinterpret_cast<const uint4*>(v + src);
    }
    auto widen8 = [&](const uint4& w, float (&x)[8]) {
        const uint32_t ww[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = widen((uint16_t)(ww[e / 2] >> (16 * (e % 2))), dtype);
    };

    // K: widen, rotate, quantise; one code word and (per group) one scale
    float x[8];
    widen8(kraw, x);
    if (signs) rotate_elems<D, 8>(x, signs, rot_norm, j);
    int c[8];
    const float sk = quantize_elems<8>(x, c);
    uint32_t word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) word |= ((uint32_t)c[e] & 0xFu) << (4 * e);
    if (fresh) {
        reinterpret_cast<uint32_t*>(kc + row * (D / 2))[r * NG + g] = word;
        if (r == 0) ks[row * NG + g] = sk;
    }

    // V: widen, quantise; scales, then the nibbles of the pair
    widen8(vraw, x);
    const float sv = quantize_elems<8>(x, c);
    if (fresh && r == 0) vs[row * NG + g] = sv;
    word = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) word |= ((uint32_t)c[e] & 0xFu) << (4 * e);
    const uint32_t other = (uint32_t)__shfl_xor((int)word, LT, 64);
    const uint32_t even_w = half ? other : word, odd_w = half ? word : other;
    const bool even_fresh = half ? fresh_pair : fresh, odd_fresh = half ? fresh : fresh_pair;
    if (even_fresh || odd_fresh) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int ch = 4 * half + e;
            const uint32_t ob = (old4 >> (8 * e)) & 0xFF;
            const uint32_t lo = even_fresh ? (even_w >> (4 * ch)) & 0xF : ob & 0xF;
            const uint32_t hi = odd_fresh ? (odd_w >> (4 * ch)) & 0xF : ob >> 4;
            vt[v_tile_byte<D>(c0 + ch, u)] = (uint8_t)(lo | (hi << 4));
        }
    }
}

}  // namespace

hipError_t launch_quantize_append(const void* k, const void* v, int dtype, int n_new, int B, int H,
                                  int D, int cap, uint8_t* kc, float* ks, uint8_t* vc, float* vs,
                                  const float* signs, float rot_norm, const int32_t* pos,
                                  hipStream_t stream)
{
    if (D != 64 && D != 128 && D != 256) return hipErrorInvalidValue;
    const auto* kk = static_cast<const uint16_t*>(k);
    const auto* vv = static_cast<const uint16_t*>(v);
    if (n_new < kPairKernelMaxTokens) {
        const int pair_slots = (n_new + 2) / 2;
        dim3 grid((pair_slots + 3) / 4, H, B), block(256);
        auto kern = D == 64 ? quantize_pair_kernel<64> : D == 128 ? quantize_pair_kernel<128> : quantize_pair_kernel<256>;
        kern<<<grid, block, 0, stream>>>(kk, vv, dtype, n_new, H, cap, kc, ks, vc, vs, signs, rot_norm, pos,
                                         pair_slots);
    } else {
        // waves of 512 / D tokens starting at pos & ~1: n_new + 1 positions at most
        const int tw = 512 / D;
        const int wave_slots = (n_new + 1 + tw - 1) / tw;
        dim3 grid((wave_slots + 3) / 4, H, B), block(256);
        auto kern = D == 64 ? quantize_append_kernel<64> : D == 128 ? quantize_append_kernel<128>
                                                                    : quantize_append_kernel<256>;
        kern<<<grid, block, 0, stream>>>(kk, vv, dtype, n_new, H, cap, kc, ks, vc, vs, signs, rot_norm, pos,
                                         wave_slots);
    }
    return hipGetLastError();
}

}  // namespace otq
