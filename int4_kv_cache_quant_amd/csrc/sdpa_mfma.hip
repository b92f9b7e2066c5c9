// sdpa_mfma.hip - split pass of decode attention on the packed int4 cache,
// MFMA variant for grouped-query attention (G >= 4 query heads per KV head).
//
// With G heads sharing one KV head, scoring a tile of tokens and weighting
// its values are both genuine matrix products (G x D by D x tokens, then
// G x tokens by tokens x D), so they run on the gfx950 matrix cores
// (v_mfma_f32_16x16x32_f16, fp32 accumulation); everything else stays in
// fp32 VALU.  As in the vector variant, attention reads only the nibbles and
// the group scales (Open-TQ-Metal abstract; zingnex Open-TQ-Metal page,
// sections on compressed-domain attention and eliminating intermediate
// matrices) and keeps a running-max softmax with fp32 accumulators (same
// page, section on numerical stability).
//
// Exactness of the products:
//  * V codes are integers in [-8, 7], exact in fp16 (built with the 1024 + n
//    magic constant and one packed fp16 subtraction); K codes enter as the
//    fp16 subnormals n * 2^-24 of their offset-binary value n = c + 8 (one
//    byte permute per pair, no arithmetic), the MFMA accumulator starts at
//    -8 * 2^-24 * sum(q) so that it ends at 2^-24 * q.c, and 2^24 is folded
//    into the softmax scale (the matrix cores keep fp16 subnormals);
//  * q is converted to fp16 (bf16 values convert exactly in fp16's normal
//    range); a rotated q is split into fp16 hi + lo parts and both are
//    multiplied, so the score keeps ~22 bits of q;
//  * the per-token, per-group K scale is applied in fp32 after the MFMA,
//    since one MFMA of K = 32 covers exactly one scale group;
//  * for P.V the V scale depends on the contracted token, so it is folded
//    into the probability operand, x = p * s_v in fp32, and x enters as two
//    fp16 MFMA operands hi = fp16(x), lo = fp16(x - hi) (~22 significant
//    bits); fp16(x) alone (2^-11 relative) is too coarse when a handful of
//    tokens carry the softmax and a channel is an outlier.
//
// Wave layout per 32-token tile (sub-tiles s = 0, 1 of 16 tokens), lane
// l = 16 r + n:
//  scores  A = K codes (row = token 16 s + n, k = 8 channels of quarter r of
//          the group), B = q (column = head n), C = S[token 16 s + 4 r + i][head n]
//  values  A = p * s_v (row = head n, k = the 8 tokens 4 r + i of both
//          sub-tiles, exactly the tokens whose scores this lane holds),
//          B = V codes (column = channel, k = the same 8 tokens, one 32-bit
//          word of the V tile layout), C = O[head 4 r + i][channel]
//  scales  each lane loads one (or two) of the sub-tile's fp32 scales and
//          the row of 16 lanes shares them by DPP row broadcast.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"

namespace otq {

namespace {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));

constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kWaves = 4;

// MFMA k-slot e of an unpacked word holds element kSlot[e] (0..7) of the word:
// registers are (0,2), (4,6), (1,3), (5,7) so that each is one byte permute.
constexpr int kSlot[8] = {0, 2, 4, 6, 1, 3, 5, 7};

// 8 signed nibbles -> 8 exact fp16 integers in MFMA operand order.
__device__ __forceinline__ half8_t unpack_codes(uint32_t w)
{
    const uint32_t x = w ^ 0x88888888u;          // offset binary: n = c + 8
    const uint32_t lo = x & 0x0F0F0F0Fu;         // elements 0,2,4,6
    const uint32_t hi = (x >> 4) & 0x0F0F0F0Fu;  // elements 1,3,5,7
    const uint32_t K = 0x64646464u;              // fp16 0x64nn = 1024 + nn
    uint32_t r[4];
    r[0] = __builtin_amdgcn_perm(K, lo, 0x04010400u);
    r[1] = __builtin_amdgcn_perm(K, lo, 0x04030402u);
    r[2] = __builtin_amdgcn_perm(K, hi, 0x04010400u);
    r[3] = __builtin_amdgcn_perm(K, hi, 0x04030402u);
    const half2_t bias = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    half8_t out;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        half2_t p = __builtin_bit_cast(half2_t, r[m]) + bias;  // exact: 1024 + n - 1032
        out[2 * m] = p[0];
        out[2 * m + 1] = p[1];
    }
    return out;
}

// 8 signed nibbles -> 8 fp16 subnormals (c + 8) * 2^-24, same operand order.
__device__ __forceinline__ half8_t unpack_codes_offset(uint32_t w)
{
    const uint32_t x = w ^ 0x88888888u;
    const uint32_t lo = x & 0x0F0F0F0Fu;
    const uint32_t hi = (x >> 4) & 0x0F0F0F0Fu;
    uint32_t r[4];
    r[0] = __builtin_amdgcn_perm(0u, lo, 0x04010400u);
    r[1] = __builtin_amdgcn_perm(0u, lo, 0x04030402u);
    r[2] = __builtin_amdgcn_perm(0u, hi, 0x04010400u);
    r[3] = __builtin_amdgcn_perm(0u, hi, 0x04030402u);
    half8_t out;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const half2_t p = __builtin_bit_cast(half2_t, r[m]);
        out[2 * m] = p[0];
        out[2 * m + 1] = p[1];
    }
    return out;
}

template <int D>
struct TileLoads {
    static constexpr int NG = D / kGroup;
    static constexpr int SPL = NG >= 4 ? NG / 4 : 1;
    uint32_t kw[2][NG];
    float sk[2][SPL], sv[2][SPL];
    uint4 vw[D / 64];
};

template <int D>
struct MfmaGeom {
    static constexpr int NG = D / kGroup;           // scale groups per vector
    static constexpr int NA = D / 64;               // 128-bit V loads per lane per tile
    static constexpr int NCB = D / 16;              // 16-channel output blocks
    static constexpr int SPL = NG >= 4 ? NG / 4 : 1;  // scale floats per lane per sub-tile
    // lane (within the row) and register holding scale (token i of the row, group g)
    static constexpr int src_lane(int i, int g) { return (NG * i + g) / SPL; }
    static constexpr int src_reg(int i, int g) { return (NG * i + g) % SPL; }
};

// Waves per SIMD the register allocation must allow (occupancy floor).
#ifndef OTQ_MFMA_WAVES_PER_EU
#define OTQ_MFMA_WAVES_PER_EU 2
#endif

template <int D, bool ROT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(OTQ_MFMA_WAVES_PER_EU)))
void split_mfma_kernel(SplitArgs a)
{
    using Geo = MfmaGeom<D>;
    constexpr int NG = Geo::NG, NA = Geo::NA, NCB = Geo::NCB, SPL = Geo::SPL;
    extern __shared__ float lds[];  // q: [16][D]; later merge: [4][G][D] + ml [4][G]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int split = blockIdx.x, hk = blockIdx.y, b = blockIdx.z;
    const int G = a.Hq / a.H;
    const int len = min(max(a.lens[b], 0), a.max_len);
    const int start = split * a.chunk;
    if (start >= len) return;  // block-uniform
    const int end = min(start + a.chunk, len);
    const int ntiles = (end - start + kTile - 1) / kTile;
    const int n16 = lane & 15, r = lane >> 4;

    // ---- query prologue: fp32 in LDS, rotated like K when the cache is
    float* q_lds = lds;
    const uint16_t* qsrc = static_cast<const uint16_t*>(a.q) + ((size_t)b * a.Hq + hk * G) * D;
    for (int i = tid; i < 16 * D; i += 256) {
        const int h = i / D, c = i % D;
        float x = 0.0f;
        if (h < G) {
            x = widen(qsrc[h * D + c], a.dtype);
            if (ROT) x *= a.signs[c];
        }
        q_lds[i] = x;
    }
    __syncthreads();
    if (ROT) {
        for (int h = 1; h < D; h <<= 1) {
            for (int i = tid; i < 16 * D / 2; i += 256) {
                const int hh = i / (D / 2), kk = i % (D / 2);
                const int j = hh * D + (kk / h) * 2 * h + (kk % h);
                const float lo = q_lds[j], hi = q_lds[j + h];
                q_lds[j] = lo + hi;
                q_lds[j + h] = lo - hi;
            }
            __syncthreads();
        }
    }
    // B operands of the score MFMAs: column = head n16, k slot e = channel
    // 32 g + 8 r + kSlot[e]
    half8_t qb[NG], qb_lo[ROT ? NG : 1];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = q_lds[n16 * D + 32 * g + 8 * r + kSlot[e]];
            const _Float16 h16 = (_Float16)x;
            qb[g][e] = h16;
            if (ROT) qb_lo[g][e] = (_Float16)(x - (float)h16);
        }
    }
    // accumulator start of the score MFMAs: -8 * 2^-24 * sum of the fp16 q
    // values of head n16 in group g (summed over the whole group by lanes
    // of the four quarters)
    float qinit[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        float t = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            t += (float)qb[g][e];
            if (ROT) t += (float)qb_lo[g][e];
        }
        t += shfl_xor(t, 16);
        t += shfl_xor(t, 32);
        qinit[g] = -8.0f * 0x1p-24f * t;
    }
    const float qmul = (ROT ? a.qscale * a.rot_norm : a.qscale) * 0x1p24f;
    __syncthreads();  // q_lds is reused for the final merge

    const size_t head = (size_t)b * a.H + hk;
    const uint8_t* kbase = a.kc + head * a.cap * (D / 2);
    const float* ksb = a.ks + head * a.cap * NG;
    const uint8_t* vbase = a.vc + head * (a.cap / kTile) * (16 * D);
    const float* vsb = a.vs + head * a.cap * NG;

    float m_run = kNegInf;  // running max of head n16 (log2 domain), same in all rows
    float l_lane = 0.0f;    // sum of this lane's probabilities (head n16)
    floatx4_t acc[NCB];
#pragma unroll
    for (int cb = 0; cb < NCB; ++cb) acc[cb] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

    auto load_tile = [&](TileLoads<D>& t, int it) {
        const int tok0 = start + it * kTile;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const uint8_t* krow = kbase + (size_t)(tok0 + 16 * s + n16) * (D / 2) + 4 * r;
#pragma unroll
            for (int g = 0; g < NG; ++g) t.kw[s][g] = *reinterpret_cast<const uint32_t*>(krow + 16 * g);
            const size_t sbase = (size_t)(tok0 + 16 * s) * NG + 4 * r * NG;
#pragma unroll
            for (int e = 0; e < SPL; ++e) {
                const int off = (n16 * SPL + e) % (4 * NG);
                t.sk[s][e] = ksb[sbase + off];
                t.sv[s][e] = vsb[sbase + off];
            }
        }
        const uint8_t* vt = vbase + (size_t)(tok0 / kTile) * (16 * D);
#pragma unroll
        for (int av = 0; av < NA; ++av)
            t.vw[av] = *reinterpret_cast<const uint4*>(vt + ((av * 4 + r) * 16 + n16) * 16);
    };

    auto compute_tile = [&](const TileLoads<D>& t, int it) {
        const int tok0 = start + it * kTile;
        // ---- scores
        float S[2][4];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            floatx4_t tot = {0.0f, 0.0f, 0.0f, 0.0f};
            static_for<NG>([&](auto gI) {
                constexpr int g = decltype(gI)::value;
                const half8_t A = unpack_codes_offset(t.kw[s][g]);
                floatx4_t d = {qinit[g], qinit[g], qinit[g], qinit[g]};
                d = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qb[g], d, 0, 0, 0);
                if constexpr (ROT) d = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qb_lo[g], d, 0, 0, 0);
                static_for<4>([&](auto iI) {
                    constexpr int i = decltype(iI)::value;
                    const float scl = row_bcast<Geo::src_lane(i, g)>(t.sk[s][Geo::src_reg(i, g)]);
                    tot[i] += scl * d[i];
                });
            });
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tk = tok0 + 16 * s + 4 * r + i;
                S[s][i] = (tk < end) ? tot[i] * qmul : kNegInf;
            }
        }

        // ---- online softmax for head n16 over the tile's 32 tokens
        float mt = kNegInf;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) mt = fmaxf(mt, S[s][i]);
        mt = fmaxf(mt, shfl_xor(mt, 16));
        mt = fmaxf(mt, shfl_xor(mt, 32));
        const float m_new = fmaxf(m_run, mt);  // finite: the tile has a valid token
        // alpha is computed by every lane (1 where the max did not move, 0 on
        // the first tile); the rescale runs only when some head's max moved,
        // decided for the whole wave so that the shuffles see every lane.
        const float alpha = exp2_approx(m_run - m_new);
        if (__any(m_new != m_run)) {
            l_lane *= alpha;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float ai = __shfl(alpha, 20 * r + i, 64);  // alpha of head 4 r + i
#pragma unroll
                for (int cb = 0; cb < NCB; ++cb) acc[cb][i] *= ai;
            }
        }
        m_run = m_new;
        float p[2][4];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[s][i] = exp2_approx(S[s][i] - m_run);
                l_lane += p[s][i];
            }

        // ---- values, one scale group (two 16-channel blocks) at a time:
        //      A_g = p * s_v[token][g] as fp16 hi + lo, B = V codes
        static_for<NG>([&](auto gI) {
            constexpr int g = decltype(gI)::value;
            half8_t pa, pl;
            static_for<8>([&](auto eI) {
                constexpr int e = decltype(eI)::value;
                constexpr int j = kSlot[e], s = j / 4, i = j % 4;
                const float scl = row_bcast<Geo::src_lane(i, g)>(t.sv[s][Geo::src_reg(i, g)]);
                const float x = p[s][i] * scl;
                const _Float16 hi = (_Float16)x;
                pa[e] = hi;
                pl[e] = (_Float16)(x - (float)hi);
            });
            static_for<2>([&](auto hI) {
                constexpr int cb = 2 * g + decltype(hI)::value;
                constexpr int av = cb / 4, bv = cb % 4;
                const uint32_t word = bv == 0 ? t.vw[av].x : bv == 1 ? t.vw[av].y
                                    : bv == 2 ? t.vw[av].z : t.vw[av].w;
                const half8_t B = unpack_codes(word);
                acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, B, acc[cb], 0, 0, 0);
                acc[cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl, B, acc[cb], 0, 0, 0);
            });
        });
    };

    // two register sets: the next tile's loads are in flight while the
    // current one is computed
    TileLoads<D> bufA, bufB;
    int it = wave;
    if (it < ntiles) load_tile(bufA, it);
    while (it < ntiles) {
        if (it + kWaves < ntiles) load_tile(bufB, it + kWaves);
        compute_tile(bufA, it);
        it += kWaves;
        if (it >= ntiles) break;
        if (it + kWaves < ntiles) load_tile(bufA, it + kWaves);
        compute_tile(bufB, it);
        it += kWaves;
    }

    // ---- merge the 4 rows (l only: m and O are already wave-wide), then waves
    float L = l_lane;
    L += shfl_xor(L, 16);
    L += shfl_xor(L, 32);
    float* merge_o = lds;                       // [4][G][D]
    float2* merge_ml = reinterpret_cast<float2*>(lds + kWaves * G * D);  // [4][G]
    if (lane < 16 && lane < G) merge_ml[wave * G + lane] = make_float2(m_run, L);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int h = 4 * r + i;
        if (h < G) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) merge_o[(wave * G + h) * D + 16 * cb + n16] = acc[cb][i];
        }
    }
    __syncthreads();
    for (int i = tid; i < G * D; i += 256) {
        const int h = i / D, c = i % D;
        float Mb = kNegInf;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) Mb = fmaxf(Mb, merge_ml[w * G + h].x);
        float o = 0.0f, Ls = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float mw = merge_ml[w * G + h].x;
            const float f = (mw == kNegInf) ? 0.0f : exp2_approx(mw - Mb);
            o += f * merge_o[(w * G + h) * D + c];
            Ls += f * merge_ml[w * G + h].y;
        }
        const size_t prow = ((size_t)b * a.Hq + hk * G + h) * a.num_splits + split;
        a.part_o[prow * D + c] = o;
        if (c == 0) a.part_ml[prow] = make_float2(Mb, Ls);
    }
}

template <int D, bool ROT>
hipError_t launch(const SplitArgs& a, hipStream_t stream)
{
    const int G = a.Hq / a.H;
    const size_t q_bytes = 16 * D * sizeof(float);
    const size_t merge_bytes = kWaves * G * (D * sizeof(float) + sizeof(float2));
    const size_t lds = q_bytes > merge_bytes ? q_bytes : merge_bytes;
    dim3 grid(a.num_splits, a.H, a.B), block(256);
    split_mfma_kernel<D, ROT><<<grid, block, lds, stream>>>(a);
    return hipGetLastError();
}

template <int D>
hipError_t dispatch_rot(const SplitArgs& a, hipStream_t stream)
{
    return a.signs ? launch<D, true>(a, stream) : launch<D, false>(a, stream);
}

}  // namespace

bool split_mfma_supports(int D, int G)
{
    return (D == 64 || D == 128 || D == 256) && G >= 4 && G <= 16;
}

hipError_t launch_split_mfma(const SplitArgs& a, hipStream_t stream)
{
    switch (a.D) {
    case 64: return dispatch_rot<64>(a, stream);
    case 128: return dispatch_rot<128>(a, stream);
    case 256: return dispatch_rot<256>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace otq
