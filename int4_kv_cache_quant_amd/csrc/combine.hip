// combine.hip - merge the split partials of decode attention.
//
// Each split s of a (sequence, query head) row carries (m_s, l_s, o_s): its
// softmax reference (log2 domain; any value at or above its largest score),
// its sum of 2^(S_t - m_s), and its unnormalised value sum.  The exact
// softmax over the union of splits is
//   M = max_s m_s,  L = sum_s l_s 2^(m_s - M),  out = sum_s 2^(m_s - M) o_s / L
// evaluated in fp32 (the high-precision accumulation the zingnex
// Open-TQ-Metal page asks for in its section on numerical stability).
// A row with lens == 0 has no splits and gets zeros.
#include "common.hpp"
#include "kernels.hpp"

namespace otq {

namespace {

constexpr int kThreads = 256;
constexpr int kCh = 32;                       // channels per block
constexpr int kQuads = kCh / 4;               // threads sharing one split (a float4 each)
constexpr int kLanesS = kThreads / kQuads;    // splits read side by side

// Block (row, c0): row = b * Hq + h, channels [32 c0, 32 c0 + 32).  Thread
// t reads channels 32 c0 + 4 (t % 8) .. + 3 of the splits s = t / 8 (mod 32),
// so 32 splits stream in side by side; each thread folds its splits into a
// running (m, l, o) (the same merge rule as above), then the block merges the
// threads' triples: one pass over the partials.
__global__ __launch_bounds__(kThreads) void lse_combine_kernel(const float* __restrict__ part_o,
                                                               const float2* __restrict__ part_ml,
                                                               const int32_t* __restrict__ lens,
                                                               int max_len, int chunk, int S,
                                                               int Hq, int D,
                                                               float* __restrict__ out)
{
    __shared__ float red_m[kThreads / 64];
    __shared__ float4 red_o[kThreads / 64][kQuads];
    __shared__ float red_l[kThreads / 64];
    const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = row / Hq;
    const int q = tid % kQuads, g = tid / kQuads;
    const int c = kCh * blockIdx.y + 4 * q;
    const int len = min(max(lens[b], 0), max_len);
    const int ns = (len + chunk - 1) / chunk;
    float4* dst = reinterpret_cast<float4*>(out + (size_t)row * D + c);
    if (ns == 0) {
        if (tid < kQuads) *dst = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        return;
    }
    const float2* ml = part_ml + (size_t)row * S;
    const float* po = part_o + (size_t)row * S * D + c;

    const float kNegInf = -__builtin_huge_valf();
    float m = kNegInf, l = 0.0f;
    float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    auto fold = [&](float2 v, float4 x) {  // every written partial has a finite m
        const float mn = fmaxf(m, v.x);
        const float a = exp2_approx(m - mn), w = exp2_approx(v.x - mn);
        o = make_float4(o.x * a + x.x * w, o.y * a + x.y * w, o.z * a + x.z * w, o.w * a + x.w * w);
        l = l * a + v.y * w;
        m = mn;
    };
    int s = g;
    for (; s + kLanesS < ns; s += 2 * kLanesS) {  // two splits in flight per thread
        const float2 v0 = ml[s], v1 = ml[s + kLanesS];
        const float4 x0 = *reinterpret_cast<const float4*>(po + (size_t)s * D);
        const float4 x1 = *reinterpret_cast<const float4*>(po + (size_t)(s + kLanesS) * D);
        fold(v0, x0);
        fold(v1, x1);
    }
    if (s < ns) fold(ml[s], *reinterpret_cast<const float4*>(po + (size_t)s * D));

    // block maximum of the threads' references
    float M = m;
#pragma unroll
    for (int k = 1; k < 64; k <<= 1) M = fmaxf(M, shfl_xor(M, k));
    if (lane == 0) red_m[wave] = M;
    __syncthreads();
    M = red_m[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) M = fmaxf(M, red_m[w]);
    const float f = (m == kNegInf) ? 0.0f : exp2_approx(m - M);
    o = make_float4(o.x * f, o.y * f, o.z * f, o.w * f);
    l = (q == 0) ? l * f : 0.0f;  // the kQuads threads of a split group hold the same l
    // sum over the threads of one channel quad: lanes 8 apart, then waves
#pragma unroll
    for (int k = kQuads; k < 64; k <<= 1) {
        o.x += shfl_xor(o.x, k);
        o.y += shfl_xor(o.y, k);
        o.z += shfl_xor(o.z, k);
        o.w += shfl_xor(o.w, k);
        l += shfl_xor(l, k);
    }
    if (lane < kQuads) red_o[wave][lane] = o;
    if (lane == 0) red_l[wave] = l;
    __syncthreads();
    if (tid < kQuads) {
        float4 r = red_o[0][tid];
        float L = red_l[0];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) {
            const float4 x = red_o[w][tid];
            r.x += x.x; r.y += x.y; r.z += x.z; r.w += x.w;
            L += red_l[w];
        }
        *dst = make_float4(r.x / L, r.y / L, r.z / L, r.w / L);
    }
}

}  // namespace

hipError_t launch_lse_combine(const float* part_o, const float2* part_ml, const int32_t* lens,
                              int max_len, int chunk, int num_splits, int B, int Hq, int D,
                              float* out, hipStream_t stream)
{
    if (D % kCh != 0) return hipErrorInvalidValue;
    dim3 grid(B * Hq, D / kCh), block(kThreads);
    lse_combine_kernel<<<grid, block, 0, stream>>>(part_o, part_ml, lens, max_len, chunk,
                                                   num_splits, Hq, D, out);
    return hipGetLastError();
}

}  // namespace otq
