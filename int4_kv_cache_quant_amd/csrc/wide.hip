// wide.hip - head widths that are multiples of 64 but not powers of two
// (192): the quantise-append and the split pass, with K (optionally) rotated
// by the mixed-radix SRFT.
//
// The FFT form of the rotation is not tied to powers of two, which is its
// advantage over the Hadamard form on the "SRFT + int4 KV-cache" page (core
// method; comparison of methods).  For D = 192 the D reals are N = 96
// complex numbers z_j = (y_2j, y_2j+1), N = 3 M with M = 32: after the signs,
// one radix-3 decimation-in-frequency stage over (a0, a1, a2) = (z_j, z_j+M,
// z_j+2M), j < M -- with s = a1 + a2, d = a1 - a2, m = a0 - 0.5 s and
// t = c3 d (c3 = fp32(sqrt(3)/2)): b0 = a0 + s, b1 = m - i t, b2 = m + i t,
// then z_j = b0, z_j+M = b1 W^j, z_j+2M = b2 W^2j (W = exp(-2 pi i / N)) --
// then the radix-2 stages of half-size 16, ..., 1 inside each block of M
// ((a, b) -> (a + b, (a - b) W^t), t = (j mod h) N / (2h)), then the product
// by rot_norm = fp32(1/sqrt(N)).  Every step is one IEEE fp32 operation in
// that order (no contraction; complex products (dr wr - di wi, dr wi + di
// wr) with the products rounded first; the twiddles correctly rounded), so
// the rotated values, and the codes quantised from them, are the same bits
// as in any other evaluation of those steps.
//
// The cache layouts are the int4 ones of every width (include/otq.h): the
// quarter-interleaved K rows (word r NG + g, NG = 6) and the V tiles of 32
// tokens (channel block cb = c / 16 = 4 a + b, a < 3).
//
// These paths favour plainness over speed: one block of D threads per token
// for the append (the transform through LDS, V nibbles placed with atomics),
// and for the split pass vector arithmetic with one token per thread for the
// scores and one channel per thread for the value sum.
#include "common.hpp"
#include "kernels.hpp"
#include "quant_lane.hpp"
#include "srft.hpp"

namespace otq {

namespace {

constexpr float kNegInfW = -__builtin_huge_valf();
using srft_detail::kC3;
using srft_detail::kTw96;

// One block of D threads per (token, KV head, sequence): quantises the
// token's K and V (each rotated when its signs are given; K scaled by its
// channel scale after the rotation) with the per-lane quantiser of the
// other append kernels, and stores both rows.  K bytes are whole bytes of
// one token; a V byte holds two tokens, so each thread replaces its own
// nibble with two atomics on the containing word.
template <int D>
__global__ __launch_bounds__(D) void quantize_wide_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int dtype, int n_new, int H, int cap,
    uint8_t* __restrict__ kc, float* __restrict__ ks, uint8_t* __restrict__ vc, float* __restrict__ vs,
    const float* __restrict__ signs, float rot_norm, const float* __restrict__ lam,
    const float* __restrict__ vsigns, const int32_t* __restrict__ pos, unsigned* __restrict__ err)
{
#pragma clang fp contract(off)
    constexpr int NG = D / kGroup;
    __shared__ float xch[D];
    const int tok = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
    const int ch = threadIdx.x, lane = ch & 63;
    const int p0 = pos[b];
    if (ch == 0 && tok == 0 && h == 0 && (p0 < 0 || p0 > cap - n_new)) report_error(err, kErrPos);
    const int t = p0 + tok;
    if (t < 0 || t >= cap) return;  // block-uniform: outside the cache
    const size_t head = (size_t)b * H + h;
    const size_t src = (head * n_new + tok) * D + ch;
    const size_t row = head * cap + t;
#pragma unroll
    for (int which = 0; which < 2; ++which) {  // K, then V
        const float* sg = which ? vsigns : signs;
        float x = widen((which ? v : k)[src], dtype);
        if (sg) {
            x = x * sg[ch];
            x = srft_mixed_block<D>(x, xch);
            x = x * rot_norm;
        }
        if (!which && lam) x = x * lam[ch];
        float xv[1] = {x};
        int cv[1];
        const float s = quantize_lane<64>(xv, cv, lane);  // 32-lane groups: this vector's groups
        if (ch % kGroup == 0) (which ? vs : ks)[row * NG + ch / kGroup] = s;
        if (!which) {
            const int cnext = __shfl_xor(cv[0], 1, 64);
            if ((ch & 1) == 0) kc[row * (D / 2) + k_row_byte<D>(ch)] = (uint8_t)((cv[0] & 0xF) | ((cnext & 0xF) << 4));
        } else {
            const size_t vbyte =
                (head * (cap / kTile) + t / kTile) * (size_t)(16 * D) + v_tile_byte<D>(ch, (t % kTile) & ~1);
            const int shift = 8 * (int)(vbyte & 3) + 4 * (t & 1);
            unsigned* vword = reinterpret_cast<unsigned*>(vc + (vbyte & ~(size_t)3));
            __hip_atomic_fetch_and(vword, ~(0xFu << shift), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_or(vword, ((unsigned)cv[0] & 0xFu) << shift, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Signed nibble at bit offset sh of a word.
__device__ __forceinline__ int nibble_at(uint32_t w, int sh) { return (int)(w << (28 - sh)) >> 28; }

// One block per (split, KV head, sequence), 256 threads; per step of 256
// tokens (8 V tiles): one token per thread scores all G heads against q in
// LDS, 16 threads per head turn the scores into probabilities, and one
// channel per thread (threads < D) adds p * V for the G heads.
template <int D, int GT>
__global__ __launch_bounds__(256) void split_wide_kernel(SplitArgs a)
{
    constexpr int N = D / 2, NG = D / kGroup, TT = 256, NTILE = TT / kTile;
    constexpr int RW = D / 8;                   // 32-bit words of a K row
    constexpr int TW = 4 * D;                   // 32-bit words of a V tile
    constexpr int GM = GT > 0 ? GT : 16;
    __shared__ __align__(16) float q_lds[16][D];
    __shared__ float p_lds[16][TT];
    __shared__ float3 step[16];
    __shared__ uint32_t v_lds[NTILE * TW];
    __shared__ float vs_lds[TT * NG];

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
    const int raw_len = a.lens[b];
    const int len = max(min(max(raw_len, 0), a.max_len) - a.lens_offset, 0);
    if (tid == 0 && split == 0 && hk == 0 && (raw_len < 0 || raw_len > a.max_len)) report_error(a.err, kErrLens);
    const int start = split * a.chunk;
    if (start >= len) return;  // block-uniform
    const int end = min(start + a.chunk, len);

    // ---- the query: widened, rotated as K is (signs, transform, rot_norm),
    //      divided by K's channel scale, times scale log2(e)
    const uint16_t* qsrc = static_cast<const uint16_t*>(a.q) + ((size_t)b * a.Hq + hk * G) * D;
    for (int i = tid; i < G * D; i += TT) {
        float x = widen(qsrc[i], a.dtype);
        if (a.signs) x *= a.signs[i % D];
        q_lds[i / D][i % D] = x;
    }
    __syncthreads();
    if (a.signs) {
        // the transform on every head's row, stage by stage; each thread
        // computes up to QPT outputs (complex numbers) into registers, then
        // writes them after a barrier
        constexpr int M = N / 3, QPT = (16 * N + TT - 1) / TT;
        float2 out[QPT];
        // radix-3 stage
#pragma unroll
        for (int k = 0; k < QPT; ++k) {
            const int idx = tid + k * TT;
            if (idx < G * N) {
                const int hh = idx / N, Pq = idx % N, m = Pq / M, j = Pq % M;
                const float* z = q_lds[hh];
                const float a0r = z[2 * j], a0i = z[2 * j + 1];
                const float a1r = z[2 * (j + M)], a1i = z[2 * (j + M) + 1];
                const float a2r = z[2 * (j + 2 * M)], a2i = z[2 * (j + 2 * M) + 1];
                const float sr = a1r + a2r, si = a1i + a2i, dr = a1r - a2r, di = a1i - a2i;
                const float mr = a0r - 0.5f * sr, mi = a0i - 0.5f * si;
                const float tr = kC3 * dr, ti = kC3 * di;
                if (m == 0) {
                    out[k] = make_float2(a0r + sr, a0i + si);
                } else {
                    const int u = m * j;
                    const float br = m == 1 ? mr + ti : mr - ti, bi = m == 1 ? mi - tr : mi + tr;
                    out[k] = make_float2(br * kTw96.re[u] - bi * kTw96.im[u], br * kTw96.im[u] + bi * kTw96.re[u]);
                }
            }
        }
        __syncthreads();
#pragma unroll
        for (int k = 0; k < QPT; ++k) {
            const int idx = tid + k * TT;
            if (idx < G * N) {
                q_lds[idx / N][2 * (idx % N)] = out[k].x;
                q_lds[idx / N][2 * (idx % N) + 1] = out[k].y;
            }
        }
        for (int h = M / 2; h >= 1; h >>= 1) {
            __syncthreads();
#pragma unroll
            for (int k = 0; k < QPT; ++k) {
                const int idx = tid + k * TT;
                if (idx < G * N) {
                    const int hh = idx / N, Pq = idx % N, w = (Pq % M) & (2 * h - 1);
                    const float* z = q_lds[hh];
                    if (w < h) {
                        out[k] = make_float2(z[2 * Pq] + z[2 * (Pq + h)], z[2 * Pq + 1] + z[2 * (Pq + h) + 1]);
                    } else {
                        const int lo = Pq - h, u = (w - h) * (N / (2 * h));
                        const float dr = z[2 * lo] - z[2 * Pq], di = z[2 * lo + 1] - z[2 * Pq + 1];
                        out[k] = make_float2(dr * kTw96.re[u] - di * kTw96.im[u],
                                             dr * kTw96.im[u] + di * kTw96.re[u]);
                    }
                }
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < QPT; ++k) {
                const int idx = tid + k * TT;
                if (idx < G * N) {
                    q_lds[idx / N][2 * (idx % N)] = out[k].x;
                    q_lds[idx / N][2 * (idx % N) + 1] = out[k].y;
                }
            }
        }
        __syncthreads();
    }
    for (int i = tid; i < G * D; i += TT) {
        float x = q_lds[i / D][i % D];
        if (a.signs) x *= a.rot_norm;
        if (a.lam) x /= a.lam[i % D];
        q_lds[i / D][i % D] = x * a.qscale;
    }
    __syncthreads();

    const size_t head = (size_t)b * a.H + hk;
    const uint32_t* krows = reinterpret_cast<const uint32_t*>(a.kc + head * a.cap * (D / 2));
    const uint32_t* vtiles = reinterpret_cast<const uint32_t*>(a.vc + head * a.cap * (D / 2));
    const float* kscl = a.ks + head * a.cap * NG;
    const float* vscl = a.vs + head * a.cap * NG;

    float m[GM], l[GM], o[GM];
#pragma unroll
    for (int g = 0; g < GM; ++g) {
        m[g] = kNegInfW;
        l[g] = 0.0f;
        o[g] = 0.0f;
    }
    const int hg = tid / 16, hl = tid % 16;  // reduction role: head hg, 16 threads per head
    // value role: channel tid (tid < D) and its place in the V tile layout
    const int vch = tid < D ? tid : 0;
    const int vcb = vch >> 4, vn = vch & 15, va = vcb >> 2, vb = vcb & 3;
    for (int t0 = start; t0 < end; t0 += TT) {
        const int n = min(TT, end - t0);
        {  // scores, one token per thread
            float acc[GM];
#pragma unroll
            for (int g = 0; g < GM; ++g) acc[g] = 0.0f;
            if (tid < n) {
                uint32_t kw[RW];
                const uint4* row = reinterpret_cast<const uint4*>(krows + (size_t)(t0 + tid) * RW);
#pragma unroll
                for (int k4 = 0; k4 < RW / 4; ++k4) {
                    const uint4 w4 = row[k4];
                    kw[4 * k4] = w4.x; kw[4 * k4 + 1] = w4.y; kw[4 * k4 + 2] = w4.z; kw[4 * k4 + 3] = w4.w;
                }
#pragma unroll
                for (int gr = 0; gr < NG; ++gr) {
                    const float s = kscl[(size_t)(t0 + tid) * NG + gr];
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const uint32_t w = kw[r * NG + gr];  // channels 32 gr + 8 r + 0..7
                        float kd[8];
#pragma unroll
                        for (int e = 0; e < 8; ++e) kd[e] = (float)nibble_at(w, 4 * e) * s;
                        const int c0 = 32 * gr + 8 * r;
#pragma unroll
                        for (int g = 0; g < GM; ++g) {
                            if (g < G) {
                                const float4 qa = *reinterpret_cast<const float4*>(&q_lds[g][c0]);
                                const float4 qb = *reinterpret_cast<const float4*>(&q_lds[g][c0 + 4]);
                                acc[g] += qa.x * kd[0] + qa.y * kd[1] + qa.z * kd[2] + qa.w * kd[3] +
                                          qb.x * kd[4] + qb.y * kd[5] + qb.z * kd[6] + qb.w * kd[7];
                            }
                        }
                    }
                }
            }
            // the step's V tiles (whole tiles up to the one holding token n - 1)
            // and V scales into LDS
            {
                const int ntile = (n + kTile - 1) / kTile;
                const uint32_t* vsrc = vtiles + (size_t)(t0 / kTile) * TW;
                for (int k = tid; k < ntile * TW; k += TT) v_lds[k] = vsrc[k];
                for (int k = tid; k < n * NG; k += TT) vs_lds[k] = vscl[(size_t)t0 * NG + k];
            }
#pragma unroll
            for (int g = 0; g < GM; ++g)
                if (g < G) p_lds[g][tid] = tid < n ? acc[g] : kNegInfW;
        }
        __syncthreads();
        if (hg < G) {  // per head: the step's maximum, the probabilities, their sum
            float mx = kNegInfW;
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
            if (hl == 0) step[hg] = make_float3(old == kNegInfW ? 0.0f : exp2_approx(old - mn), mn, sum);
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
        if (tid < D) {  // value sum: channel tid over the step's tokens
            const int gr = vch / kGroup;
            for (int j = 0; j < n; ++j) {
                const int tile = j / kTile, u = j % kTile;
                const int r = (u & 15) >> 2, slot = 4 * (u >> 4) + (u & 3);
                const uint32_t w = v_lds[tile * TW + ((va * 4 + r) * 16 + vn) * 4 + vb];
                const float vd = (float)nibble_at(w, 4 * slot) * vs_lds[j * NG + gr];
#pragma unroll
                for (int g = 0; g < GM; ++g)
                    if (g < G) o[g] += p_lds[g][j] * vd;
            }
        }
        __syncthreads();  // p_lds, step and v_lds are rewritten by the next step
    }
#pragma unroll
    for (int g = 0; g < GM; ++g) {
        if (g < G) {
            const size_t prow = ((size_t)b * a.Hq + hk * G + g) * a.num_splits + split;
            if (tid < D) a.part_o[prow * D + tid] = o[g];
            if (tid == 0) a.part_ml[prow] = make_float2(m[g], l[g]);
        }
    }
}

}  // namespace

bool wide_supported_dim(int D) { return D == 192; }

hipError_t launch_quantize_wide(const void* k, const void* v, int dtype, int n_new, int B, int H, int D,
                                int cap, uint8_t* kc, float* ks, uint8_t* vc, float* vs, const float* signs,
                                float rot_norm, const float* lam, const float* vsigns, const int32_t* pos,
                                unsigned* err, hipStream_t stream)
{
    if (D != 192) return hipErrorInvalidValue;
    if (quantize_tile_wide_supports(D, n_new, vsigns != nullptr))  // one block per tile
        return launch_quantize_tile_wide(k, v, dtype, n_new, B, H, D, cap, kc, ks, vc, vs, signs, rot_norm, lam, pos,
                                         err, stream);
    dim3 grid(n_new, H, B), block(192);
    quantize_wide_kernel<192><<<grid, block, 0, stream>>>(static_cast<const uint16_t*>(k),
                                                           static_cast<const uint16_t*>(v), dtype, n_new, H,
                                                           cap, kc, ks, vc, vs, signs, rot_norm, lam, vsigns,
                                                           pos, err);
    return hipGetLastError();
}

hipError_t launch_split_wide(const SplitArgs& a, hipStream_t stream)
{
    if (a.D != 192 || a.Hq / a.H > 16) return hipErrorInvalidValue;
    dim3 grid(a.num_splits, a.H, a.B), block(256);
    switch (a.Hq / a.H) {
    case 1: split_wide_kernel<192, 1><<<grid, block, 0, stream>>>(a); break;
    case 2: split_wide_kernel<192, 2><<<grid, block, 0, stream>>>(a); break;
    case 4: split_wide_kernel<192, 4><<<grid, block, 0, stream>>>(a); break;
    case 8: split_wide_kernel<192, 8><<<grid, block, 0, stream>>>(a); break;
    default: split_wide_kernel<192, 0><<<grid, block, 0, stream>>>(a); break;
    }
    return hipGetLastError();
}

}  // namespace otq
