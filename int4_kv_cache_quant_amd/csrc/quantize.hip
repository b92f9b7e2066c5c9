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

template <int D>
__global__ __launch_bounds__(256) void quantize_append_kernel(
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

}  // namespace

hipError_t launch_quantize_append(const void* k, const void* v, int dtype, int n_new, int B, int H,
                                  int D, int cap, uint8_t* kc, float* ks, uint8_t* vc, float* vs,
                                  const float* signs, float rot_norm, const int32_t* pos,
                                  hipStream_t stream)
{
    const int pair_slots = (n_new + 2) / 2;
    dim3 grid((pair_slots + 3) / 4, H, B), block(256);
    const auto* kk = static_cast<const uint16_t*>(k);
    const auto* vv = static_cast<const uint16_t*>(v);
    switch (D) {
    case 64:
        quantize_append_kernel<64><<<grid, block, 0, stream>>>(kk, vv, dtype, n_new, H, cap, kc, ks,
                                                               vc, vs, signs, rot_norm, pos, pair_slots);
        break;
    case 128:
        quantize_append_kernel<128><<<grid, block, 0, stream>>>(kk, vv, dtype, n_new, H, cap, kc, ks,
                                                                vc, vs, signs, rot_norm, pos, pair_slots);
        break;
    case 256:
        quantize_append_kernel<256><<<grid, block, 0, stream>>>(kk, vv, dtype, n_new, H, cap, kc, ks,
                                                                vc, vs, signs, rot_norm, pos, pair_slots);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace otq
