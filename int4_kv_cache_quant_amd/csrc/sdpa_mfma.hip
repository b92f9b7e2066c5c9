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
// One wave serves P = 16 / G KV heads at once (P = 2 for G = 8): MFMA column
// n is query head n of the block, which belongs to KV head n / G, so no
// column of the 16-wide products is padding.  Per 32-token tile (sub-tiles
// s = 0, 1 of 16 tokens), lane l = 16 r + n:
//  scores  for each KV head j: A = K_j codes (row = token 16 s + n, k = 8
//          channels of quarter r of the group, all groups in one 16-byte load
//          thanks to the quarter-interleaved K row), B = q masked to the columns
//          of head j; all P products accumulate into one C = S[token
//          16 s + 4 r + i][column n] since the other heads' B columns are 0
//  values  A = p * s_v (row = column n, k = the 8 tokens 4 r + i of both
//          sub-tiles, exactly the tokens whose scores this lane holds),
//          B = V_j codes (column = channel, k = the same 8 tokens, one 32-bit
//          word of the V tile layout), C_j = O[column 4 r + i][channel]; one
//          accumulator set per KV head, of which only the rows of head j
//          are kept
//  scales  lane k of each quad loads the fp32 scales of token 4 r + k of its
//          head and DPP quad broadcasts hand them to the quad (every quad
//          lies inside one head, as G >= 4).
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

// Lane K (0..3) of each quad of lanes, broadcast to the quad (DPP quad_perm).
template <int K>
__device__ __forceinline__ float quad_bcast(float v)
{
    static_assert(K >= 0 && K < 4, "quad lane");
    return __builtin_bit_cast(
        float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), K * 0x55, 0xF, 0xF, false));
}

template <int NG>
__device__ __forceinline__ void load_scales(float (&dst)[NG], const float* __restrict__ src)
{
    if constexpr (NG == 2) {
        const float2 v = *reinterpret_cast<const float2*>(src);
        dst[0] = v.x; dst[1] = v.y;
    } else {
#pragma unroll
        for (int q = 0; q < NG / 4; ++q) {
            const float4 v = reinterpret_cast<const float4*>(src)[q];
            dst[4 * q + 0] = v.x; dst[4 * q + 1] = v.y;
            dst[4 * q + 2] = v.z; dst[4 * q + 3] = v.w;
        }
    }
}

// One tile's loads for the P KV heads of the block.
template <int D, int P>
struct TileLoads {
    static constexpr int NG = D / kGroup;
    uint32_t kw[P][2][NG];   // K code words: head, sub-tile, group
    uint4 vw[P][D / 64];     // V tile words: head, 128-bit load
    float sk[2][NG];         // K scales of token 4 r + (lane % 4) of the lane's head
    float sv[2][NG];         // V scales, same token
};

// Waves per SIMD the register allocation must allow: 2 (up to 256 VGPRs)
// except at head_dim 256, whose accumulators alone take 64 VGPRs per head.
template <int D>
constexpr int kWavesPerEU = D == 256 ? 1 : 2;

template <int D, int P, bool ROT, bool PF>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(kWavesPerEU<D>)))
void split_mfma_kernel(SplitArgs a)
{
    constexpr int NG = D / kGroup, NA = D / 64, NCB = D / 16;
    extern __shared__ float lds[];  // q: [16][D]; later merge: [4][P*G][D] + ml [4][P*G]

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int split = blockIdx.x, hk0 = blockIdx.y * P, b = blockIdx.z;
    const int G = a.Hq / a.H;
    const int PG = P * G;  // query heads served by the block (<= 16)
    const int len = min(max(a.lens[b], 0), a.max_len);
    const int start = split * a.chunk;
    if (start >= len) return;  // block-uniform
    const int end = min(start + a.chunk, len);
    const int ntiles = (end - start + kTile - 1) / kTile;
    const int n16 = lane & 15, r = lane >> 4, slot = lane & 3;
    const bool col_valid = n16 < PG;
    const int jl = col_valid ? n16 / G : P - 1;  // KV head of this lane's column

    // ---- query prologue: fp32 in LDS, rotated like K when the cache is
    float* q_lds = lds;
    const uint16_t* qsrc = static_cast<const uint16_t*>(a.q) + ((size_t)b * a.Hq + hk0 * G) * D;
    for (int i = tid; i < 16 * D; i += 256) {
        const int h = i / D, c = i % D;
        float x = 0.0f;
        if (h < PG) {
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
    // B operands of the score MFMAs, one per KV head: column n16 holds q of
    // query head n16 in the set of head jl and zeros in the others; k slot e
    // = channel 32 g + 8 r + kSlot[e].
    half8_t qb[P][NG], qb_lo[ROT ? P : 1][ROT ? NG : 1];
    float qinit[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        half8_t hv, lv;
        float t = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = q_lds[n16 * D + 32 * g + 8 * r + kSlot[e]];
            const _Float16 h16 = (_Float16)x;
            hv[e] = h16;
            t += (float)h16;
            if (ROT) {
                lv[e] = (_Float16)(x - (float)h16);
                t += (float)lv[e];
            }
        }
#pragma unroll
        for (int j = 0; j < P; ++j) {
            const bool mine = col_valid && j == jl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                qb[j][g][e] = mine ? hv[e] : (_Float16)0.0f;
                if (ROT) qb_lo[j][g][e] = mine ? lv[e] : (_Float16)0.0f;
            }
        }
        // the score accumulator starts at -8 * 2^-24 * sum(q over the group)
        t += shfl_xor(t, 16);
        t += shfl_xor(t, 32);
        qinit[g] = -8.0f * 0x1p-24f * t;
    }
    const float qmul = (ROT ? a.qscale * a.rot_norm : a.qscale) * 0x1p24f;
    __syncthreads();  // q_lds is reused for the final merge

    const uint8_t* kbase[P];
    const uint8_t* vbase[P];
#pragma unroll
    for (int j = 0; j < P; ++j) {
        const size_t head = (size_t)b * a.H + hk0 + j;
        kbase[j] = a.kc + head * a.cap * (D / 2) + r * (D / 8);  // row quarter r
        vbase[j] = a.vc + head * (a.cap / kTile) * (16 * D) + ((size_t)r * 16 + n16) * 16;
    }
    const size_t head_l = (size_t)b * a.H + hk0 + jl;
    const float* ks_l = a.ks + head_l * a.cap * NG;
    const float* vs_l = a.vs + head_l * a.cap * NG;

    float m_run = kNegInf;  // running max of column n16 (log2 domain)
    float l_lane = 0.0f;    // sum of this lane's probabilities (column n16)
    floatx4_t acc[P][NCB];
#pragma unroll
    for (int j = 0; j < P; ++j)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[j][cb] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

    auto load_tile = [&](TileLoads<D, P>& t, int it) {
        const int tok0 = start + it * kTile;
#pragma unroll
        for (int j = 0; j < P; ++j) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                // quarter r of the row: word g = channels 32 g + 8 r + 0..7
                const uint8_t* krow = kbase[j] + (size_t)(tok0 + 16 * s + n16) * (D / 2);
                if constexpr (NG == 2) {
                    const uint2 w = *reinterpret_cast<const uint2*>(krow);
                    t.kw[j][s][0] = w.x; t.kw[j][s][1] = w.y;
                } else {
#pragma unroll
                    for (int q = 0; q < NG / 4; ++q) {
                        const uint4 w = reinterpret_cast<const uint4*>(krow)[q];
                        t.kw[j][s][4 * q + 0] = w.x; t.kw[j][s][4 * q + 1] = w.y;
                        t.kw[j][s][4 * q + 2] = w.z; t.kw[j][s][4 * q + 3] = w.w;
                    }
                }
            }
            const uint8_t* vt = vbase[j] + (size_t)(tok0 / kTile) * (16 * D);
#pragma unroll
            for (int av = 0; av < NA; ++av) t.vw[j][av] = *reinterpret_cast<const uint4*>(vt + av * 1024);
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const size_t tok = (size_t)(tok0 + 16 * s + 4 * r + slot) * NG;
            load_scales<NG>(t.sk[s], ks_l + tok);
            load_scales<NG>(t.sv[s], vs_l + tok);
        }
    };

    auto compute_tile = [&](const TileLoads<D, P>& t, int it) {
        const int tok0 = start + it * kTile;
        // ---- scores
        float S[2][4];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            floatx4_t tot = {0.0f, 0.0f, 0.0f, 0.0f};
            static_for<NG>([&](auto gI) {
                constexpr int g = decltype(gI)::value;
                floatx4_t d = {qinit[g], qinit[g], qinit[g], qinit[g]};
#pragma unroll
                for (int j = 0; j < P; ++j) {
                    const half8_t A = unpack_codes_offset(t.kw[j][s][g]);
                    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qb[j][g], d, 0, 0, 0);
                    if constexpr (ROT) d = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qb_lo[j][g], d, 0, 0, 0);
                }
                static_for<4>([&](auto iI) {
                    constexpr int i = decltype(iI)::value;
                    tot[i] += quad_bcast<i>(t.sk[s][g]) * d[i];
                });
            });
            const bool full = tok0 + 16 * s + 16 <= end;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int tk = tok0 + 16 * s + 4 * r + i;
                S[s][i] = (full || tk < end) ? tot[i] * qmul : kNegInf;
            }
        }

        // ---- online softmax for column n16 over the tile's 32 tokens
        float mt = kNegInf;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) mt = fmaxf(mt, S[s][i]);
        mt = fmaxf(mt, shfl_xor(mt, 16));
        mt = fmaxf(mt, shfl_xor(mt, 32));
        const float m_new = fmaxf(m_run, mt);  // finite: the tile has a valid token
        // alpha is computed by every lane (1 where the max did not move, 0 on
        // the first tile); the rescale runs only when some column's max
        // moved, decided for the whole wave so that the shuffles see every lane.
        const float alpha = exp2_approx(m_run - m_new);
        if (__any(m_new != m_run)) {
            l_lane *= alpha;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float ai = __shfl(alpha, 20 * r + i, 64);  // alpha of column 4 r + i
#pragma unroll
                for (int j = 0; j < P; ++j)
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) acc[j][cb][i] *= ai;
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
        //      A_g = p * s_v[token][g] as fp16 hi + lo, B = V_j codes
        static_for<NG>([&](auto gI) {
            constexpr int g = decltype(gI)::value;
            half8_t pa, pl;
            static_for<8>([&](auto eI) {
                constexpr int e = decltype(eI)::value;
                constexpr int js = kSlot[e], s = js / 4, i = js % 4;
                const float x = p[s][i] * quad_bcast<i>(t.sv[s][g]);
                const _Float16 hi = (_Float16)x;
                pa[e] = hi;
                pl[e] = (_Float16)(x - (float)hi);
            });
#pragma unroll
            for (int j = 0; j < P; ++j) {
                static_for<2>([&](auto hI) {
                    constexpr int cb = 2 * g + decltype(hI)::value;
                    constexpr int av = cb / 4, bv = cb % 4;
                    const uint32_t word = bv == 0 ? t.vw[j][av].x : bv == 1 ? t.vw[j][av].y
                                        : bv == 2 ? t.vw[j][av].z : t.vw[j][av].w;
                    const half8_t B = unpack_codes(word);
                    acc[j][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, B, acc[j][cb], 0, 0, 0);
                    acc[j][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl, B, acc[j][cb], 0, 0, 0);
                });
            }
        });
    };

    if constexpr (PF) {
        // two register sets: the next tile's loads are in flight while the
        // current one is computed
        TileLoads<D, P> bufA, bufB;
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
    } else {
        for (int it = wave; it < ntiles; it += kWaves) {
            TileLoads<D, P> buf;
            load_tile(buf, it);
            compute_tile(buf, it);
        }
    }

    // ---- merge the 4 rows (l only: m and O are already wave-wide), then waves
    float L = l_lane;
    L += shfl_xor(L, 16);
    L += shfl_xor(L, 32);
    float* merge_o = lds;                                                  // [4][PG][D]
    float2* merge_ml = reinterpret_cast<float2*>(lds + kWaves * PG * D);  // [4][PG]
    if (lane < PG) merge_ml[wave * PG + lane] = make_float2(m_run, L);
    // rows 4 r .. 4 r + 3 of O lie in one KV head (G >= 4): keep that head's set
    const int jr = min(4 * r / G, P - 1);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int h = 4 * r + i;
        if (h < PG) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                float v = acc[0][cb][i];
#pragma unroll
                for (int j = 1; j < P; ++j) v = (jr == j) ? acc[j][cb][i] : v;
                merge_o[(wave * PG + h) * D + 16 * cb + n16] = v;
            }
        }
    }
    __syncthreads();
    for (int i = tid; i < PG * D; i += 256) {
        const int h = i / D, c = i % D;
        float Mb = kNegInf;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) Mb = fmaxf(Mb, merge_ml[w * PG + h].x);
        float o = 0.0f, Ls = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
            const float mw = merge_ml[w * PG + h].x;
            const float f = (mw == kNegInf) ? 0.0f : exp2_approx(mw - Mb);
            o += f * merge_o[(w * PG + h) * D + c];
            Ls += f * merge_ml[w * PG + h].y;
        }
        const size_t prow = ((size_t)b * a.Hq + hk0 * G + h) * a.num_splits + split;
        a.part_o[prow * D + c] = o;
        if (c == 0) a.part_ml[prow] = make_float2(Mb, Ls);
    }
}


// Prefetching the next tile needs a second register set; it is used only
// where that set still fits without spilling.
template <int D, int P>
constexpr bool kPrefetch = (D == 64) || (D == 128 && P == 1);

template <int D, int P, bool ROT>
hipError_t launch(const SplitArgs& a, hipStream_t stream)
{
    const int G = a.Hq / a.H;
    const size_t q_bytes = 16 * D * sizeof(float);
    const size_t merge_bytes = (size_t)kWaves * P * G * (D * sizeof(float) + sizeof(float2));
    const size_t lds = q_bytes > merge_bytes ? q_bytes : merge_bytes;
    dim3 grid(a.num_splits, a.H / P, a.B), block(256);
    split_mfma_kernel<D, P, ROT, kPrefetch<D, P>><<<grid, block, lds, stream>>>(a);
    return hipGetLastError();
}

template <int D>
hipError_t dispatch(const SplitArgs& a, hipStream_t stream)
{
    const int P = split_mfma_heads_per_wave(a.D, a.Hq / a.H, a.H);
    if (P == 2) return a.signs ? launch<D, 2, true>(a, stream) : launch<D, 2, false>(a, stream);
    return a.signs ? launch<D, 1, true>(a, stream) : launch<D, 1, false>(a, stream);
}

}  // namespace

// KV heads per wave: two (filling 16 MFMA columns at G = 8) when the head
// count allows it and the registers suffice, else one.
int split_mfma_heads_per_wave(int D, int G, int H)
{
    return (D != 256 && G <= 8 && H % 2 == 0) ? 2 : 1;
}

bool split_mfma_supports(int D, int G)
{
    return (D == 64 || D == 128 || D == 256) && G >= 4 && G <= 16;
}

hipError_t launch_split_mfma(const SplitArgs& a, hipStream_t stream)
{
    switch (a.D) {
    case 64: return dispatch<64>(a, stream);
    case 128: return dispatch<128>(a, stream);
    case 256: return dispatch<256>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace otq
