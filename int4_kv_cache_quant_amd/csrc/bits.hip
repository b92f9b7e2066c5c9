// bits.hip - 2- and 3-bit codes: quantise-append and the split pass over
// caches whose rows are plain little-endian bit streams.
//
// The code widths the AdapTQ page lists beside 4-bit (its section on the
// core mechanisms: 2-, 3- and 4-bit quantisation): b-bit codes take the
// int4 steps with the symmetric range of b bits, s = abs-max / (2^(b-1) - 1)
// in IEEE fp32 and c = clamp(rint(x / s), -2^(b-1), 2^(b-1) - 1), s == 0
// giving zero codes; element i of a row occupies bits [b i, b i + b) of the
// row's little-endian bit stream, two's complement.  K and V rows have the
// same layout, [B][H][capacity][D b / 8] bytes, scales as for int4.
//
// A first path, for correctness: the split kernel computes scores and the
// value sum with fp32 vector arithmetic, one token per thread for the
// scores and one channel per thread for the value sum, and writes the same
// (m, l, o) partials as the int4 kernels, so the same combine merges them.
#include "common.hpp"
#include "kernels.hpp"
#include "quant_lane.hpp"
#include "srft.hpp"

namespace otq {

namespace {

constexpr float kNegInfB = -__builtin_huge_valf();
constexpr int kVecsPerWave = 8;  // vectors one wave of a bulk append quantises (one for short appends)

// Signed b-bit code of element i of a row held as 32-bit words (the bits
// may straddle two words).
template <int BITS>
__device__ __forceinline__ int code_in_words(const uint32_t* w, int i)
{
    const int pos = i * BITS, k = pos >> 5, sh = pos & 31;
    uint32_t u = w[k] >> sh;
    if (sh + BITS > 32) u |= w[k + 1] << (32 - sh);
    // sign-extend the low BITS bits
    return (int)(u << (32 - BITS)) >> (32 - BITS);
}

// One wave per new vector (K tokens, then V tokens), E = D / 64 elements per
// lane; the codes pass through LDS so that D b / 32 lanes assemble the row's
// 32-bit words.
template <int D, int BITS>
__global__ __launch_bounds__(256) void quantize_bits_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int dtype, int n_new, int H, int cap,
    uint8_t* __restrict__ kc, float* __restrict__ ks, uint8_t* __restrict__ vc, float* __restrict__ vs,
    const int32_t* __restrict__ pos, int vpw, const float* __restrict__ signs, float rot_norm, int rot_kind,
    const float* __restrict__ lam, const float* __restrict__ vsigns)
{
#pragma clang fp contract(off)
    constexpr int E = D / 64, NG = D / kGroup, RB = D * BITS / 8, NWORD = RB / 4;
    constexpr float qmax = (float)((1 << (BITS - 1)) - 1), qmin = -(float)(1 << (BITS - 1));
    static_assert(RB % 4 == 0, "whole words per row");
    __shared__ int8_t cs[4][D];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int h = blockIdx.y, b = blockIdx.z;
    const int p0 = pos[b];
    SrftLaneTw<D, E> stw;  // the FFT rotation's twiddles of this lane
    if ((signs || vsigns) && rot_kind) stw.load(lane);
    // each wave takes vpw vectors in turn (the block's barrier count is the
    // same for all its threads)
    for (int iv = 0; iv < vpw; ++iv) {
    const int vec = (blockIdx.x * 4 + wave) * vpw + iv;
    const bool is_v = vec >= n_new;
    const int tok = is_v ? vec - n_new : vec;
    const int t = p0 + tok;
    // every thread reaches the barrier; inactive waves do no memory access
    const bool active = vec < 2 * n_new && t >= 0 && t < cap;
    const size_t head = (size_t)b * H + h;
    float sc = 0.0f;
    if (active) {
        const uint16_t* src = (is_v ? v : k) + (head * n_new + tok) * D + lane * E;
        float x[E];
        float a = 0.0f;
#pragma unroll
        for (int e = 0; e < E; ++e) x[e] = widen(src[e], dtype);
        // the same rotation and channel scale as the int4 appends (K: signs,
        // then lambda; V: its own signs)
        const float* sg = is_v ? vsigns : signs;
        if (sg) {
            if (rot_kind) {
#pragma unroll
                for (int e = 0; e < E; ++e) x[e] = x[e] * sg[lane * E + e];
                srft_signed<D, E>(x, rot_norm, lane, stw);
            } else {
                rotate_lane<D>(x, sg, rot_norm, lane);
            }
        }
        if (!is_v && lam) {
#pragma unroll
            for (int e = 0; e < E; ++e) x[e] = x[e] * lam[lane * E + e];
        }
#pragma unroll
        for (int e = 0; e < E; ++e) a = fmaxf(a, fabsf(x[e]));
        a = group_max<kGroup / E>(a);  // exact in any order
        sc = a / qmax;                 // correctly rounded IEEE division
#pragma unroll
        for (int e = 0; e < E; ++e) {
            float r = rintf(x[e] / sc);  // IEEE division, then half to even
            r = fminf(fmaxf(r, qmin), qmax);
            cs[wave][lane * E + e] = (int8_t)(sc != 0.0f ? (int)r : 0);
        }
    }
    __syncthreads();
    if (active) {
        const size_t row = head * cap + t;
        if (lane % (kGroup / E) == 0) (is_v ? vs : ks)[row * NG + (lane * E) / kGroup] = sc;
        if (lane < NWORD) {  // word w holds bits [32 w, 32 w + 32) of the row
            uint32_t word = 0;
            const int i0 = (32 * lane) / BITS, i1 = min((32 * lane + 31) / BITS, D - 1);
            for (int i = i0; i <= i1; ++i) {
                const uint32_t u = (uint32_t)cs[wave][i] & ((1u << BITS) - 1u);
                const int off = i * BITS - 32 * lane;  // may be negative for the first element
                word |= off >= 0 ? u << off : u >> -off;
            }
            reinterpret_cast<uint32_t*>((is_v ? vc : kc) + row * RB)[lane] = word;
        }
    }
    __syncthreads();  // cs is rewritten by the next vector
    }
}

// One block per (split, KV head, sequence): q of the G heads in LDS (scaled
// by scale log2(e)); per 256-token tile, one token per thread scores all G
// heads, then per head 16 threads find the tile maximum and turn the scores
// into probabilities, and one channel per thread accumulates p * V for the
// G heads.
template <int D, int BITS, int GT>
__global__ __launch_bounds__(256) void split_bits_kernel(SplitArgs a)
{
    // GT: the query heads per KV head when fixed at compile time, else 0
    constexpr int NG = D / kGroup, RB = D * BITS / 8, RW = RB / 4, TT = 256;
    constexpr int GM = GT > 0 ? GT : 16;  // loop bound over heads
    __shared__ __align__(16) float q_lds[16][D];
    __shared__ float p_lds[16][TT];
    __shared__ float3 step[16];  // per head: (rescale of the old state, new reference, tile sum)
    __shared__ uint32_t v_lds[TT * RW];  // the tile's V rows
    __shared__ float vs_lds[TT * NG];    // and their scales

    const int tid = threadIdx.x;
    int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
    if (a.items) {  // a batch: the block's item in longest-first order
        const int kk = blockIdx.x + a.num_splits * (blockIdx.y + a.H * blockIdx.z);
        const int2 it = a.items[kk];
        if (it.x < 0) return;  // block-uniform: no item
        split = it.x;
        b = it.y;
        hk = kk % a.H;
    }
    const int G = GT > 0 ? GT : a.Hq / a.H;
    const int len = min(max(a.lens[b] - a.lens_offset, 0), a.max_len);
    const int start = split * a.chunk;
    if (start >= len) return;  // block-uniform: no partial for empty chunks
    const int end = min(start + a.chunk, len);

    const uint16_t* qsrc = static_cast<const uint16_t*>(a.q) + ((size_t)b * a.Hq + hk * G) * D;
    for (int i = tid; i < G * D; i += TT) {
        float x = widen(qsrc[i], a.dtype) * a.qscale;
        if (a.signs) x *= a.signs[i % D];
        q_lds[i / D][i % D] = x;
    }
    __syncthreads();
    // the query rotated as K is (then rot_norm), and divided by K's channel scale
    if (a.signs) {
        if (a.rot_kind) {  // FFT stages over the (even, odd) complex pairs
            for (int h = D / 4; h >= 1; h >>= 1) {
                for (int i = tid; i < G * D / 4; i += TT) {
                    const int hh = i / (D / 4), kk = i % (D / 4);
                    const int j = (kk / h) * 2 * h + (kk % h);
                    const int u = (kk % h) * (64 / h);
                    const float wr = srft_detail::kTw.re[u], wi = srft_detail::kTw.im[u];
                    const float ar = q_lds[hh][2 * j], ai = q_lds[hh][2 * j + 1];
                    const float br = q_lds[hh][2 * (j + h)], bi = q_lds[hh][2 * (j + h) + 1];
                    const float dr = ar - br, di = ai - bi;
                    q_lds[hh][2 * j] = ar + br;
                    q_lds[hh][2 * j + 1] = ai + bi;
                    q_lds[hh][2 * (j + h)] = dr * wr - di * wi;
                    q_lds[hh][2 * (j + h) + 1] = dr * wi + di * wr;
                }
                __syncthreads();
            }
        } else {  // Walsh-Hadamard butterflies
            for (int h = 1; h < D; h <<= 1) {
                for (int i = tid; i < G * D / 2; i += TT) {
                    const int hh = i / (D / 2), kk = i % (D / 2);
                    const int j = (kk / h) * 2 * h + (kk % h);
                    const float lo = q_lds[hh][j], hi = q_lds[hh][j + h];
                    q_lds[hh][j] = lo + hi;
                    q_lds[hh][j + h] = lo - hi;
                }
                __syncthreads();
            }
        }
    }
    if (a.signs || a.lam) {
        for (int i = tid; i < G * D; i += TT) {
            float x = q_lds[i / D][i % D];
            if (a.signs) x *= a.rot_norm;
            if (a.lam) x /= a.lam[i % D];
            q_lds[i / D][i % D] = x;
        }
        __syncthreads();
    }

    const size_t head = (size_t)b * a.H + hk;
    const uint8_t* krows = a.kc + head * a.cap * RB;
    const uint8_t* vrows = a.vc + head * a.cap * RB;
    const float* kscl = a.ks + head * a.cap * NG;
    const float* vscl = a.vs + head * a.cap * NG;

    float m[GM], l[GM], o[GM];
#pragma unroll
    for (int g = 0; g < GM; ++g) {
        m[g] = kNegInfB;
        l[g] = 0.0f;
        o[g] = 0.0f;
    }
    const int hg = tid / 16, hl = tid % 16;  // reduction role: head hg, 16 threads per head
    constexpr int TS = TT / D;                // value role: channel vc_, token subset vts of TS
    const int vc_ = tid % D, vts = tid / D;
    for (int t0 = start; t0 < end; t0 += TT) {
        const int n = min(TT, end - t0);
        // scores, one token per thread
        {
            float acc[GM];
#pragma unroll
            for (int g = 0; g < GM; ++g) acc[g] = 0.0f;
            if (tid < n) {
                uint32_t kw[RW];  // the token's K row, read 16 or 8 bytes at a time
                const uint32_t* row = reinterpret_cast<const uint32_t*>(krows + (size_t)(t0 + tid) * RB);
                if constexpr (RW % 4 == 0) {
#pragma unroll
                    for (int k = 0; k < RW; k += 4) {
                        const uint4 w4 = *reinterpret_cast<const uint4*>(row + k);
                        kw[k] = w4.x; kw[k + 1] = w4.y; kw[k + 2] = w4.z; kw[k + 3] = w4.w;
                    }
                } else {
#pragma unroll
                    for (int k = 0; k < RW; k += 2) {
                        const uint2 w2 = *reinterpret_cast<const uint2*>(row + k);
                        kw[k] = w2.x; kw[k + 1] = w2.y;
                    }
                }
#pragma unroll
                for (int gr = 0; gr < NG; ++gr) {
                    const float s = kscl[(size_t)(t0 + tid) * NG + gr];
#pragma unroll
                    for (int i = 32 * gr; i < 32 * gr + 32; i += 4) {
                        float kd[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) kd[e] = (float)code_in_words<BITS>(kw, i + e) * s;
#pragma unroll
                        for (int g = 0; g < GM; ++g) {
                            if (g < G) {
                                const float4 qv = *reinterpret_cast<const float4*>(&q_lds[g][i]);
                                acc[g] += qv.x * kd[0] + qv.y * kd[1] + qv.z * kd[2] + qv.w * kd[3];
                            }
                        }
                    }
                }
            }
            // the tile's V rows and scales into LDS (coalesced)
            {
                const uint32_t* vsrc = reinterpret_cast<const uint32_t*>(vrows + (size_t)t0 * RB);
                for (int k = tid; k < n * RW; k += TT) v_lds[k] = vsrc[k];
                for (int k = tid; k < n * NG; k += TT) vs_lds[k] = vscl[(size_t)t0 * NG + k];
            }
#pragma unroll
            for (int g = 0; g < GM; ++g)
                if (g < G) p_lds[g][tid] = tid < n ? acc[g] : kNegInfB;
        }
        __syncthreads();
        // per head: the tile's maximum, the probabilities and their sum
        if (hg < G) {
            float mx = kNegInfB;
            for (int j = hl; j < TT; j += 16) mx = fmaxf(mx, p_lds[hg][j]);
#pragma unroll
            for (int s = 8; s >= 1; s >>= 1) mx = fmaxf(mx, shfl_xor(mx, s));
            const float old = m[hg];
            const float mn = fmaxf(old, mx);
            float sum = 0.0f;
            for (int j = hl; j < TT; j += 16) {
                const float p = j < n ? exp2_approx(p_lds[hg][j] - mn) : 0.0f;
                p_lds[hg][j] = p;
                sum += p;
            }
#pragma unroll
            for (int s = 8; s >= 1; s >>= 1) sum += shfl_xor(sum, s);
            if (hl == 0) step[hg] = make_float3(old == kNegInfB ? 0.0f : exp2_approx(old - mn), mn, sum);
        }
        __syncthreads();
#pragma unroll
        for (int g = 0; g < GM; ++g) {
            if (g < G) {
                const float3 st = step[g];
                l[g] = l[g] * st.x + st.z;
                m[g] = st.y;
                o[g] *= st.x;
            }
        }
        // value sum: channel c of every TS-th token of the tile per thread
        {
            const int gr = vc_ / kGroup;
#pragma unroll 4
            for (int j = vts; j < n; j += TS) {
                const float vd = (float)code_in_words<BITS>(&v_lds[j * RW], vc_) * vs_lds[j * NG + gr];
#pragma unroll
                for (int g = 0; g < GM; ++g)
                    if (g < G) o[g] += p_lds[g][j] * vd;
            }
        }
        __syncthreads();  // p_lds and step are rewritten by the next tile
    }
    // the TS token subsets of each channel, added through LDS (p_lds is free)
#pragma unroll
    for (int g = 0; g < GM; ++g) {
        if (g < G) {
            float* red = &p_lds[0][0];
            if (TS > 1) {
                red[vts * D + vc_] = o[g];
                __syncthreads();
                if (vts == 0)
                    for (int k = 1; k < TS; ++k) o[g] += red[k * D + vc_];
                __syncthreads();
            }
            const size_t prow = ((size_t)b * a.Hq + hk * G + g) * a.num_splits + split;
            if (vts == 0) a.part_o[prow * D + vc_] = o[g];
            if (tid == 0) a.part_ml[prow] = make_float2(m[g], l[g]);
        }
    }
}

template <int D, int BITS>
hipError_t launch_q(const void* k, const void* v, int dtype, int n_new, int B, int H, int cap,
                    uint8_t* kc, float* ks, uint8_t* vc, float* vs, const int32_t* pos, const BitsRot& r,
                    hipStream_t s)
{
    const int vpw = n_new >= 64 ? kVecsPerWave : 1;
    dim3 grid((2 * n_new + 4 * vpw - 1) / (4 * vpw), H, B), block(256);
    quantize_bits_kernel<D, BITS><<<grid, block, 0, s>>>(static_cast<const uint16_t*>(k),
                                                          static_cast<const uint16_t*>(v), dtype, n_new,
                                                          H, cap, kc, ks, vc, vs, pos, vpw, r.signs,
                                                          r.rot_norm, r.rot_kind, r.lam, r.vsigns);
    return hipGetLastError();
}

template <int D, int BITS>
hipError_t launch_s(const SplitArgs& a, hipStream_t s)
{
    dim3 grid(a.num_splits, a.H, a.B), block(256);
    switch (a.Hq / a.H) {
    case 1: split_bits_kernel<D, BITS, 1><<<grid, block, 0, s>>>(a); break;
    case 2: split_bits_kernel<D, BITS, 2><<<grid, block, 0, s>>>(a); break;
    case 4: split_bits_kernel<D, BITS, 4><<<grid, block, 0, s>>>(a); break;
    case 8: split_bits_kernel<D, BITS, 8><<<grid, block, 0, s>>>(a); break;
    default: split_bits_kernel<D, BITS, 0><<<grid, block, 0, s>>>(a); break;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_bits(const void* k, const void* v, int dtype, int n_new, int B, int H, int D,
                                int cap, int bits, uint8_t* kc, float* ks, uint8_t* vc, float* vs,
                                const int32_t* pos, const BitsRot& r, hipStream_t s)
{
    switch (D * 10 + bits) {
    case 642: return launch_q<64, 2>(k, v, dtype, n_new, B, H, cap, kc, ks, vc, vs, pos, r, s);
    case 643: return launch_q<64, 3>(k, v, dtype, n_new, B, H, cap, kc, ks, vc, vs, pos, r, s);
    case 1282: return launch_q<128, 2>(k, v, dtype, n_new, B, H, cap, kc, ks, vc, vs, pos, r, s);
    case 1283: return launch_q<128, 3>(k, v, dtype, n_new, B, H, cap, kc, ks, vc, vs, pos, r, s);
    case 2562: return launch_q<256, 2>(k, v, dtype, n_new, B, H, cap, kc, ks, vc, vs, pos, r, s);
    case 2563: return launch_q<256, 3>(k, v, dtype, n_new, B, H, cap, kc, ks, vc, vs, pos, r, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_split_bits(const SplitArgs& a, int bits, hipStream_t s)
{
    if (a.Hq / a.H > 16) return hipErrorInvalidValue;
    switch (a.D * 10 + bits) {
    case 642: return launch_s<64, 2>(a, s);
    case 643: return launch_s<64, 3>(a, s);
    case 1282: return launch_s<128, 2>(a, s);
    case 1283: return launch_s<128, 3>(a, s);
    case 2562: return launch_s<256, 2>(a, s);
    case 2563: return launch_s<256, 3>(a, s);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace otq
