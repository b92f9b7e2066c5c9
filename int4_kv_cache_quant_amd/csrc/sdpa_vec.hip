// sdpa_vec.hip - split pass of decode attention on the packed int4 cache,
// fp32 vector variant (used when few query heads share a KV head).
//
// Attention is evaluated straight from the nibbles and group scales, with no
// dequantised K/V written anywhere (Open-TQ-Metal abstract; zingnex
// Open-TQ-Metal page, sections on compressed-domain attention and on
// eliminating intermediate matrices).  Numerical stability follows the same
// page's section on numerical stability: running-max (online) softmax with
// fp32 accumulators.
//
// One workgroup (4 waves) owns one chunk of tokens of one (sequence, KV head)
// and produces, for each of the G query heads of that KV head, the
// unnormalised partial (m, l, o) that the LSE-combine kernel merges.
//
// Wave layout per 32-token tile (two sub-tiles of 16 tokens):
//  * score role: lane = 4 * t + q, t = token of the sub-tile, q = quarter of
//    the K row.  One 128-bit load gives the lane 8 channels of every scale
//    group of one token (the K row layout interleaves quarters of groups);
//    it multiplies them by q in fp32, applies each group's scale and the
//    4 lanes of a token sum with two xor shuffles.
//  * value role: lane = 16 * r + n.  One 128-bit load of the V tile gives
//    4 channels x 8 tokens; the 8 tokens are those whose scores live in the
//    same row of 16 lanes, so each probability reaches the value lanes by a
//    DPP row broadcast instead of LDS.
//  Each row of 16 lanes keeps its own running max; rows, then waves, are
//  merged at the end (LDS is used only for that cross-wave merge).
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"
#include "srft.hpp"

namespace otq {

namespace {

constexpr float kNegInf = -__builtin_huge_valf();

// Groups a score lane covers, and the row-lane / register that holds the
// probability of (token i of the row, group g).
template <int D>
struct VecGeom {
    static constexpr int NG = D / kGroup;
    static constexpr int QC = D / 4;             // channels per score lane
    static constexpr int NW = QC / 8;            // 32-bit code words per score lane (one per group)
    static constexpr int PG = (D >= 128) ? D / 128 : 1;  // groups whose p * s_v a score lane supplies
    static constexpr int NA = D / 64;            // 128-bit V loads per lane per tile
    static constexpr int src_lane(int i, int g)
    {
        return 4 * i + (D == 64 ? 2 * g : (D == 128 ? g : g / 2));
    }
    static constexpr int src_reg(int g) { return D == 256 ? (g & 1) : 0; }
};

template <int D, int G>
__global__ __launch_bounds__(256) void split_vec_kernel(SplitArgs a)
{
    using Geo = VecGeom<D>;
    constexpr int NG = Geo::NG, QC = Geo::QC, NW = Geo::NW, PG = Geo::PG, NA = Geo::NA;
    __shared__ float q_lds[G][D];
    __shared__ float2 merge_ml[4][G];
    __shared__ float merge_o[4][G][D];

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar loop control
    int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
    if (a.items) {  // a batch: the block's item in longest-first order
        const int k = blockIdx.x + a.num_splits * (blockIdx.y + a.H * blockIdx.z);
        const int2 it = a.items[k];
        if (it.x < 0) return;  // block-uniform: no item
        split = it.x;
        b = it.y;
        hk = k % a.H;
    }
    // lens clamped to [0, max_len] first, as the combine does, then the
    // fused append's token (lens_offset = 1) left to the combine
    const int raw_len = a.lens[b];
    const int len = max(min(max(raw_len, 0), a.max_len) - a.lens_offset, 0);
    if (tid == 0 && split == 0 && hk == 0 && (raw_len < 0 || raw_len > a.max_len)) report_error(a.err, kErrLens);
    const int start = split * a.chunk;
    if (start >= len) return;  // block-uniform: no partial for empty chunks
    const int end = min(start + a.chunk, len);
    const int ntiles = (end - start + kTile - 1) / kTile;

    // ---- query prologue: widen, rotate like K if the cache is rotated, scale
    const uint16_t* qsrc = static_cast<const uint16_t*>(a.q) + ((size_t)b * a.Hq + hk * G) * D;
    for (int i = tid; i < G * D; i += 256) {
        float x = widen(qsrc[i], a.dtype);
        if (a.signs) x *= a.signs[i % D];
        q_lds[i / D][i % D] = x;
    }
    __syncthreads();
    if (a.signs && a.rot_kind) {  // the FFT rotation: complex pairs (2j, 2j + 1), DIF stages
        for (int h = D / 4; h >= 1; h >>= 1) {
            for (int i = tid; i < G * D / 4; i += 256) {
                const int hh = i / (D / 4), kk = i % (D / 4);
                const int j = (kk / h) * 2 * h + (kk % h);  // the pair's lower complex index
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
    } else if (a.signs) {
        for (int h = 1; h < D; h <<= 1) {
            for (int i = tid; i < G * D / 2; i += 256) {
                const int hh = i / (D / 2), kk = i % (D / 2);
                const int j = (kk / h) * 2 * h + (kk % h);
                const float lo = q_lds[hh][j], hi = q_lds[hh][j + h];
                q_lds[hh][j] = lo + hi;
                q_lds[hh][j + h] = lo - hi;
            }
            __syncthreads();
        }
    }
    const int tq = lane >> 2, q4 = lane & 3, r = lane >> 4, n = lane & 15;
    const float qmul = a.signs ? a.qscale * a.rot_norm : a.qscale;
    float qr[G][QC];
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int i = 0; i < QC; ++i) qr[hh][i] = q_lds[hh][32 * (i / 8) + 8 * q4 + i % 8];
    if (a.lam) {  // K holds lambda (.) k: divide q by K's channel scale
#pragma unroll
        for (int hh = 0; hh < G; ++hh)
#pragma unroll
            for (int i = 0; i < QC; ++i) qr[hh][i] = qr[hh][i] / a.lam[32 * (i / 8) + 8 * q4 + i % 8];
    }
#pragma unroll
    for (int hh = 0; hh < G; ++hh)
#pragma unroll
        for (int i = 0; i < QC; ++i) qr[hh][i] = qr[hh][i] * qmul;

    const size_t head = (size_t)b * a.H + hk;
    const uint8_t* kbase = a.kc + head * a.cap * (D / 2) + q4 * (D / 8);
    const float* ksb = a.ks + head * a.cap * NG;
    const uint8_t* vbase = a.vc + head * (a.cap / kTile) * (16 * D);
    const float* vsb = a.vs + head * a.cap * NG;
    // group index of register gi of this score lane
    const int g_first = (D == 64) ? (q4 >> 1) : q4 * PG;

    float m_run[G], l_lane[G], acc[G][NA][4];
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        m_run[hh] = kNegInf;
        l_lane[hh] = 0.0f;
#pragma unroll
        for (int x = 0; x < NA; ++x)
#pragma unroll
            for (int y = 0; y < 4; ++y) acc[hh][x][y] = 0.0f;
    }

    for (int it = wave; it < ntiles; it += 4) {
        const int tok0 = start + it * kTile;
        float S[2][G], pv[2][G][PG];
        float svr[2][PG];
        bool valid[2];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int row = tok0 + 16 * s + tq;
            valid[s] = row < end;
            const int rowc = valid[s] ? row : tok0;  // stay inside written rows
            uint32_t kw[NW];
            const uint32_t* kp = reinterpret_cast<const uint32_t*>(kbase + (size_t)rowc * (D / 2));
            if constexpr (NW == 2) {
                const uint2 t = *reinterpret_cast<const uint2*>(kp);
                kw[0] = t.x; kw[1] = t.y;
            } else {
#pragma unroll
                for (int w4 = 0; w4 < NW / 4; ++w4) {
                    const uint4 t = reinterpret_cast<const uint4*>(kp)[w4];
                    kw[4 * w4 + 0] = t.x; kw[4 * w4 + 1] = t.y;
                    kw[4 * w4 + 2] = t.z; kw[4 * w4 + 3] = t.w;
                }
            }
            float skr[NG];
#pragma unroll
            for (int g = 0; g < NG; ++g) skr[g] = ksb[(size_t)rowc * NG + g];
#pragma unroll
            for (int gi = 0; gi < PG; ++gi) svr[s][gi] = vsb[(size_t)rowc * NG + g_first + gi];
            float part[G];
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                float tot = 0.0f;
                // word g holds channels 32 g + 8 q4 + 0..7
                static_for<NG>([&](auto gI) {
                    constexpr int g = decltype(gI)::value;
                    const uint32_t word = kw[g];
                    float dot = 0.0f;
                    static_for<8>([&](auto kI) {
                        constexpr int kb = decltype(kI)::value;
                        dot += qr[hh][g * 8 + kb] * nib_f32<kb>(word);
                    });
                    tot += skr[g] * dot;
                });
                part[hh] = tot;
            }
#pragma unroll
            for (int hh = 0; hh < G; ++hh) {
                float v = part[hh];
                v += shfl_xor(v, 1);
                v += shfl_xor(v, 2);
                S[s][hh] = valid[s] ? v : kNegInf;
            }
        }

        // ---- online softmax, one running max per row of 16 lanes
#pragma unroll
        for (int hh = 0; hh < G; ++hh) {
            float mt = fmaxf(S[0][hh], S[1][hh]);
            mt = fmaxf(mt, shfl_xor(mt, 4));
            mt = fmaxf(mt, shfl_xor(mt, 8));
            const float m_new = fmaxf(m_run[hh], mt);
            const bool none = m_new == kNegInf;
            const float base = none ? 0.0f : m_new;
            const float alpha = none ? 1.0f : exp2_approx(m_run[hh] - m_new);
            const float p0 = exp2_approx(S[0][hh] - base);
            const float p1 = exp2_approx(S[1][hh] - base);
            l_lane[hh] = l_lane[hh] * alpha + p0 + p1;
            m_run[hh] = m_new;
#pragma unroll
            for (int x = 0; x < NA; ++x)
#pragma unroll
                for (int y = 0; y < 4; ++y) acc[hh][x][y] *= alpha;
#pragma unroll
            for (int gi = 0; gi < PG; ++gi) {
                pv[0][hh][gi] = valid[0] ? p0 * svr[0][gi] : 0.0f;
                pv[1][hh][gi] = valid[1] ? p1 * svr[1][gi] : 0.0f;
            }
        }

        // ---- P.V straight from the tiled nibbles
        const uint8_t* vt = vbase + (size_t)(tok0 / kTile) * (16 * D);
        static_for<NA>([&](auto aI) {
            constexpr int av = decltype(aI)::value;
            const uint4 w4 = *reinterpret_cast<const uint4*>(vt + (((av * 4 + r) * 16 + n) * 16));
            const uint32_t words[4] = {w4.x, w4.y, w4.z, w4.w};
            static_for<4>([&](auto bI) {
                constexpr int bv = decltype(bI)::value;
                constexpr int g = (4 * av + bv) / 2;
                const uint32_t word = words[bv];
                static_for<8>([&](auto jI) {
                    constexpr int j = decltype(jI)::value;
                    constexpr int s = j / 4, i = j % 4;
                    constexpr int src = Geo::src_lane(i, g);
                    constexpr int reg = Geo::src_reg(g);
                    const float c = nib_f32<j>(word);
#pragma unroll
                    for (int hh = 0; hh < G; ++hh)
                        acc[hh][av][bv] += row_bcast<src>(pv[s][hh][reg]) * c;
                });
            });
        });
    }

    // ---- merge the 4 rows of the wave, then the 4 waves of the block
#pragma unroll
    for (int hh = 0; hh < G; ++hh) {
        float M = m_run[hh];
        M = fmaxf(M, shfl_xor(M, 16));
        M = fmaxf(M, shfl_xor(M, 32));
        const float al = (m_run[hh] == kNegInf) ? 0.0f : exp2_approx(m_run[hh] - M);
        float L = l_lane[hh];
        L += shfl_xor(L, 1);
        L += shfl_xor(L, 2);
        L += shfl_xor(L, 4);
        L += shfl_xor(L, 8);
        L *= al;
        L += shfl_xor(L, 16);
        L += shfl_xor(L, 32);
#pragma unroll
        for (int x = 0; x < NA; ++x)
#pragma unroll
            for (int y = 0; y < 4; ++y) {
                float o = acc[hh][x][y] * al;
                o += shfl_xor(o, 16);
                o += shfl_xor(o, 32);
                if (lane < 16) merge_o[wave][hh][16 * (4 * x + y) + n] = o;
            }
        // every token's probability sits in 4 score lanes
        if (lane == 0) merge_ml[wave][hh] = make_float2(M, L * 0.25f);
    }
    __syncthreads();

    for (int i = tid; i < G * D; i += 256) {
        const int hh = i / D, c = i % D;
        float Mb = kNegInf;
#pragma unroll
        for (int w = 0; w < 4; ++w) Mb = fmaxf(Mb, merge_ml[w][hh].x);
        float o = 0.0f, L = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float mw = merge_ml[w][hh].x;
            const float f = (mw == kNegInf) ? 0.0f : exp2_approx(mw - Mb);
            o += f * merge_o[w][hh][c];
            L += f * merge_ml[w][hh].y;
        }
        const size_t prow = ((size_t)b * a.Hq + hk * G + hh) * a.num_splits + split;
        a.part_o[prow * D + c] = o;
        if (c == 0) a.part_ml[prow] = make_float2(Mb, L);
    }
}

template <int D, int G>
hipError_t launch_vec(const SplitArgs& a, hipStream_t stream)
{
    dim3 grid(a.num_splits, a.H, a.B), block(256);
    split_vec_kernel<D, G><<<grid, block, 0, stream>>>(a);
    return hipGetLastError();
}

template <int D>
hipError_t dispatch_g(const SplitArgs& a, int G, hipStream_t stream)
{
    switch (G) {
    case 1: return launch_vec<D, 1>(a, stream);
    case 2: return launch_vec<D, 2>(a, stream);
    case 4:
        if constexpr (D != 256) return launch_vec<D, 4>(a, stream);
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
    }
}

}  // namespace

bool split_vector_supports(int D, int G)
{
    if (D == 256) return G == 1 || G == 2;  // G = 4 at D = 256 exceeds the register file
    return (D == 64 || D == 128) && (G == 1 || G == 2 || G == 4);
}

hipError_t launch_split_vector(const SplitArgs& a, hipStream_t stream)
{
    const int G = a.Hq / a.H;
    switch (a.D) {
    case 64: return dispatch_g<64>(a, G, stream);
    case 128: return dispatch_g<128>(a, G, stream);
    case 256: return dispatch_g<256>(a, G, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace otq
