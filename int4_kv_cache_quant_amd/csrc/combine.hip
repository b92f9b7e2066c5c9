// combine.hip - merge the split partials of decode attention.
//
// Each split s of a (sequence, query head) row carries (m_s, l_s, o_s): its
// running max (log2 domain), its sum of 2^(S_t - m_s), and its unnormalised
// value sum.  The exact softmax over the union of splits is
//   M = max_s m_s,  L = sum_s l_s 2^(m_s - M),  out = sum_s 2^(m_s - M) o_s / L
// evaluated in fp32 (the high-precision accumulation the zingnex
// Open-TQ-Metal page asks for in its section on numerical stability).
// A row with lens == 0 has no splits and gets zeros.
#include "common.hpp"
#include "kernels.hpp"

namespace otq {

namespace {

template <int D>
__global__ __launch_bounds__(64) void lse_combine_kernel(const float* __restrict__ part_o,
                                                         const float2* __restrict__ part_ml,
                                                         const int32_t* __restrict__ lens,
                                                         int max_len, int chunk, int S, int Hq,
                                                         float* __restrict__ out)
{
    constexpr int PER = D / 64;
    const int row = blockIdx.x, lane = threadIdx.x;
    const int b = row / Hq;
    const int len = min(max(lens[b], 0), max_len);
    const int ns = (len + chunk - 1) / chunk;
    float* o = out + (size_t)row * D;
    if (ns == 0) {
#pragma unroll
        for (int e = 0; e < PER; ++e) o[lane + 64 * e] = 0.0f;
        return;
    }
    const float2* ml = part_ml + (size_t)row * S;
    float M = -__builtin_huge_valf();
    for (int s = lane; s < ns; s += 64) M = fmaxf(M, ml[s].x);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) M = fmaxf(M, shfl_xor(M, m));
    float L = 0.0f;
    for (int s = lane; s < ns; s += 64) L += ml[s].y * exp2_approx(ml[s].x - M);
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) L += shfl_xor(L, m);

    float acc[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = 0.0f;
    const float* po = part_o + (size_t)row * S * D;
    for (int s = 0; s < ns; ++s) {
        const float f = exp2_approx(ml[s].x - M);
#pragma unroll
        for (int e = 0; e < PER; ++e) acc[e] += f * po[(size_t)s * D + lane + 64 * e];
    }
    const float inv = 1.0f / L;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[lane + 64 * e] = acc[e] * inv;
}

}  // namespace

hipError_t launch_lse_combine(const float* part_o, const float2* part_ml, const int32_t* lens,
                              int max_len, int chunk, int num_splits, int B, int Hq, int D,
                              float* out, hipStream_t stream)
{
    dim3 grid(B * Hq), block(64);
    switch (D) {
    case 64:
        lse_combine_kernel<64><<<grid, block, 0, stream>>>(part_o, part_ml, lens, max_len, chunk,
                                                           num_splits, Hq, out);
        break;
    case 128:
        lse_combine_kernel<128><<<grid, block, 0, stream>>>(part_o, part_ml, lens, max_len, chunk,
                                                            num_splits, Hq, out);
        break;
    case 256:
        lse_combine_kernel<256><<<grid, block, 0, stream>>>(part_o, part_ml, lens, max_len, chunk,
                                                            num_splits, Hq, out);
        break;
    default:
        return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace otq
