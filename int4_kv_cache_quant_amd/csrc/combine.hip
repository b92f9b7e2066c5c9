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

constexpr int kThreads = 256;

__device__ __forceinline__ float block_reduce(float v, bool is_max, float* red)
{
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
        const float o = shfl_xor(v, m);
        v = is_max ? fmaxf(v, o) : v + o;
    }
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[wave] = v;
    __syncthreads();
    float r = red[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) r = is_max ? fmaxf(r, red[w]) : r + red[w];
    return r;
}

// Block (row, c0): row = b * Hq + h, channels [64 * c0, 64 * c0 + 64).
// Thread t owns channel 64 * c0 + (t % 64) and the splits s = t / 64 (mod 4),
// so the per-split loads of 64 consecutive floats are coalesced and four
// splits are in flight per channel.
__global__ __launch_bounds__(kThreads) void lse_combine_kernel(const float* __restrict__ part_o,
                                                               const float2* __restrict__ part_ml,
                                                               const int32_t* __restrict__ lens,
                                                               int max_len, int chunk, int S,
                                                               int Hq, int D,
                                                               float* __restrict__ out)
{
    extern __shared__ float w_lds[];  // [S] split weights, then [4][64] partial sums
    __shared__ float red[kThreads / 64];
    const int row = blockIdx.x, tid = threadIdx.x;
    const int b = row / Hq;
    const int c = 64 * blockIdx.y + (tid & 63);
    const int ph = tid >> 6;
    const int len = min(max(lens[b], 0), max_len);
    const int ns = (len + chunk - 1) / chunk;
    if (ns == 0) {
        if (ph == 0) out[(size_t)row * D + c] = 0.0f;
        return;
    }
    const float2* ml = part_ml + (size_t)row * S;
    float M = -__builtin_huge_valf();
    for (int s = tid; s < ns; s += kThreads) M = fmaxf(M, ml[s].x);
    M = block_reduce(M, true, red);
    float L = 0.0f;
    for (int s = tid; s < ns; s += kThreads) {
        const float2 v = ml[s];
        const float w = exp2_approx(v.x - M);
        w_lds[s] = w;
        L += v.y * w;
    }
    L = block_reduce(L, false, red);  // its barriers also publish w_lds

    const float* po = part_o + (size_t)row * S * D + c;
    float acc0 = 0.0f, acc1 = 0.0f;
    int s = ph;
    for (; s + 4 < ns; s += 8) {
        acc0 += w_lds[s] * po[(size_t)s * D];
        acc1 += w_lds[s + 4] * po[(size_t)(s + 4) * D];
    }
    if (s < ns) acc0 += w_lds[s] * po[(size_t)s * D];
    float* part = w_lds + S;
    part[ph * 64 + (tid & 63)] = acc0 + acc1;
    __syncthreads();
    if (ph == 0) {
        const float o = part[tid] + part[64 + tid] + part[128 + tid] + part[192 + tid];
        out[(size_t)row * D + c] = o / L;
    }
}

}  // namespace

hipError_t launch_lse_combine(const float* part_o, const float2* part_ml, const int32_t* lens,
                              int max_len, int chunk, int num_splits, int B, int Hq, int D,
                              float* out, hipStream_t stream)
{
    if (D % 64 != 0) return hipErrorInvalidValue;
    dim3 grid(B * Hq, D / 64), block(kThreads);
    const size_t lds = ((size_t)num_splits + 4 * 64) * sizeof(float);
    lse_combine_kernel<<<grid, block, lds, stream>>>(part_o, part_ml, lens, max_len, chunk,
                                                     num_splits, Hq, D, out);
    return hipGetLastError();
}

}  // namespace otq
