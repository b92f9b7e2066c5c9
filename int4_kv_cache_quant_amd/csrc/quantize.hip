// quantize.hip - on-the-fly int4 quantisation of new K/V vectors into the
// cache (Open-TQ-Metal abstract: the KV cache is quantised to int4 as it is
// produced).  One fused pass per vector: optional sign-randomised Hadamard
// rotation of K, group abs-max, scale, round, clamp and nibble pack, as the
// agents-report "SRFT + int4 KV-cache" page describes for its single-dispatch
// quantiser (core-method section), here with the Walsh-Hadamard rotation of
// the AdapTQ page (section on Fast Hadamard Rotation).
//
// Built with -ffp-contract=off: every step is one IEEE fp32 operation with
// round-to-nearest-even (or, in the bulk kernel, an exact sequence that
// reaches the same correctly rounded results), so the codes and scales are
// bit-identical to any correct evaluation of the same steps.
//
// Fewer than 8 new tokens take quantize_pair_kernel (one wave per token
// pair); more take quantize_tile_kernel (one block per 32-token V tile).
#include "common.hpp"
#include "kernels.hpp"
#include "quant_lane.hpp"
#include "srft.hpp"

namespace otq {

namespace {

// Streaming accesses of the bulk kernel: its inputs are read once, and the
// K rows, K scales and whole V words it writes are not read again by this
// pass (measured: non-temporal forms for those take 16384-token appends at
// head_dim 128 from 20.7 to 18.7 us, at 256 from 69 to 63 us; the V scales,
// written by a quarter of the lanes, went slower that way and stay plain).
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint16_t* p)
{
    const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}
template <typename T>
__device__ __forceinline__ void store_stream(T* p, T x)
{
    __builtin_nontemporal_store(x, p);
}

// Appends of fewer tokens take the one-pair-per-wave kernel.
constexpr int kPairKernelMaxTokens = 8;

// Small appends (a decode step's token): one wave per pair of positions,
// E = D / 64 elements per lane, so that a lone token's quantisation is a
// short chain.
template <int D>
__global__ __launch_bounds__(256) void quantize_pair_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int dtype, int n_new,
    int H, int cap, uint8_t* __restrict__ kc, float* __restrict__ ks, uint8_t* __restrict__ vc,
    float* __restrict__ vs, const float* __restrict__ signs, float rot_norm, int rot_kind,
    const float* __restrict__ lam, const float* __restrict__ vsigns, const int32_t* __restrict__ pos,
    int pair_slots, unsigned* __restrict__ err)
{
    constexpr int E = D / 64;
    constexpr int NG = D / kGroup;
    const int lane = threadIdx.x & 63;
    const int slot = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (slot >= pair_slots) return;
    const int h = blockIdx.y, b = blockIdx.z;
    const int p0 = pos[b];
    if (threadIdx.x == 0 && blockIdx.x == 0 && h == 0 && (p0 < 0 || p0 > cap - n_new))
        report_error(err, kErrPos);  // the tokens outside [0, cap) are skipped below
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

    SrftLaneTw<D, E> stw;  // the FFT rotation's twiddles of this lane
    if ((signs || vsigns) && rot_kind) stw.load(lane);

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
        if (signs) {
            if (rot_kind) {  // the FFT rotation
#pragma unroll
                for (int e = 0; e < E; ++e) x[e] = x[e] * signs[lane * E + e];
                srft_signed<D, E>(x, rot_norm, lane, stw);
            } else {
                rotate_lane<D>(x, signs, rot_norm, lane);
            }
        }
        if (lam) {  // K's per-channel scale, after the rotation
#pragma unroll
            for (int e = 0; e < E; ++e) x[e] = x[e] * lam[lane * E + e];
        }
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
        if (vsigns) {
            if (rot_kind) {
#pragma unroll
                for (int e = 0; e < E; ++e) x[e] = x[e] * vsigns[lane * E + e];
                srft_signed<D, E>(x, rot_norm, lane, stw);
            } else {
                rotate_lane<D>(x, vsigns, rot_norm, lane);
            }
        }
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

// The mixed-radix FFT of one K vector at head_dim 192 (N = 96 = 3 * 32
// complex numbers), in the bulk kernel's layout: lane j (0..23) of the
// token holds reals 8 j .. 8 j + 7, complex numbers 4 j + c (c < 4), and zr
// is the token's row (after the signs) in LDS.  The radix-3 stage (output
// 32 m + q from complex q, q + 32, q + 64, m = j / 8) reads the row; the
// radix-2 stages of half-size 16, 8 and 4 inside each block of 32 pair lanes
// 4, 2 and 1 apart (an aligned group of 8 lanes, never split by a wave),
// those of 2 and 1 stay in the lane.  The fp32 operations and their order
// are those of the per-token form in wide.hip, so the codes are the same.
// tw is the 96-point twiddle table in LDS (re[96], then im[96]): the indices
// differ from lane to lane.
__device__ __forceinline__ void srft192_lane(float (&x)[8], const float* zr, int j, const float* tw)
{
#pragma clang fp contract(off)
    using srft_detail::kC3;
    auto cmul = [tw](float& re, float& im, int u) {
        const float wr = tw[u], wi = tw[96 + u];
        const float p1 = re * wr, p2 = im * wi, p3 = re * wi, p4 = im * wr;
        re = p1 - p2;
        im = p3 + p4;
    };
    const int jm = j & 7, m = j >> 3;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int q = 4 * jm + c;
        const float a0r = zr[2 * q], a0i = zr[2 * q + 1];
        const float a1r = zr[2 * (q + 32)], a1i = zr[2 * (q + 32) + 1];
        const float a2r = zr[2 * (q + 64)], a2i = zr[2 * (q + 64) + 1];
        const float sr = a1r + a2r, si = a1i + a2i;
        const float dr = a1r - a2r, di = a1i - a2i;
        const float hr = 0.5f * sr, hi = 0.5f * si;
        const float mr = a0r - hr, mi = a0i - hi;
        const float tr = kC3 * dr, ti = kC3 * di;
        float yr, yi;
        if (m == 0) {
            yr = a0r + sr;
            yi = a0i + si;
        } else if (m == 1) {  // (m - i t) W^q
            yr = mr + ti;
            yi = mi - tr;
            cmul(yr, yi, q);
        } else {  // (m + i t) W^2q
            yr = mr - ti;
            yi = mi + tr;
            cmul(yr, yi, 2 * q);
        }
        x[2 * c] = yr;
        x[2 * c + 1] = yi;
    }
#pragma unroll
    for (int h = 16; h >= 4; h >>= 1) {
        const int lm = h / 4;  // lane distance
        const bool upper = (jm & lm) != 0;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
            const float ore = shfl_xor(x[2 * c], lm), oim = shfl_xor(x[2 * c + 1], lm);
            if (upper) {
                float dr = ore - x[2 * c], di = oim - x[2 * c + 1];
                cmul(dr, di, (((4 * jm + c) & (2 * h - 1)) - h) * (96 / (2 * h)));
                x[2 * c] = dr;
                x[2 * c + 1] = di;
            } else {
                x[2 * c] = x[2 * c] + ore;
                x[2 * c + 1] = x[2 * c + 1] + oim;
            }
        }
    }
#pragma unroll
    for (int h = 2; h >= 1; h >>= 1)
#pragma unroll
        for (int c = 0; c < 4; ++c)
            if ((c & h) == 0) {
                const float lr = x[2 * c], li = x[2 * c + 1], ur = x[2 * (c + h)], ui = x[2 * (c + h) + 1];
                float dr = lr - ur, di = li - ui;
                cmul(dr, di, (((c + h) & (2 * h - 1)) - h) * (96 / (2 * h)));
                x[2 * c] = lr + ur;
                x[2 * c + 1] = li + ui;
                x[2 * (c + h)] = dr;
                x[2 * (c + h) + 1] = di;
            }
}

// One block per 32-token V tile of one head, so that every byte of the tile,
// of its 32 K rows and of their scales is written from one CU (one L2) as
// whole words.
//
// K: each token occupies LT = D / 8 consecutive lanes, lane j of a token
// holding its channels 8 j .. 8 j + 7 (one 16-byte load).  A scale group
// (32 channels) is then one aligned quad of lanes, and a lane's 8 codes are
// exactly one 32-bit word of the K row (quarter-interleaved: word r NG + g
// holds channels 32 g + 8 r + 0..7).
//
// V: a V word holds one channel of the 8 tokens 4 r + {0..3, 16..19} of a
// tile (nibble m for token 4 r + (m & 3) + 16 (m >> 2)).  A wave takes one r
// and 64 channels: lane bits 0-1 pick the channel block within a group (so a
// group is still a quad), bits 2-4 the token m, bit 5 the group of the pair.
// After the quantisation lane m holds token m's 8 codes of its channel block;
// a transpose of the 8 x 8 nibbles across the lanes m (three exchange stages,
// blocks of 4, 2 and 1 nibbles) leaves lane m with channel 8 j + m of the 8
// tokens: an output word, the wave's 64 words filling 256 contiguous bytes.
//
// A rotated V (VROT) mixes all of a token's channels, which this V layout
// spreads over several waves: then V is read, rotated and quantised in the K
// layout instead, and its code words pass through LDS to the V layout.
//
// quantize_tile is one tile's work; FULL when every token of the tile is
// appended (no freshness tests, no merge with older V nibbles).
template <int D, int DTYPE, bool FULL, bool VROT, bool SRFT>
__device__ __forceinline__ void quantize_tile(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                              int n_new, int cap, size_t head, int p0, int t_tile, int t_end,
                                              uint8_t* __restrict__ kc, float* __restrict__ ks,
                                              uint8_t* __restrict__ vc, float* __restrict__ vs,
                                              const float* __restrict__ signs, float rot_norm,
                                              const float* __restrict__ lam,
                                              const float* __restrict__ vsigns, uint32_t* vstage, float* krot)
{
    constexpr int NG = D / kGroup;
    constexpr int LT = D / 8;  // K lanes per token
    constexpr int U = D / 64;  // K units and V units per thread
    // at head_dim 192 (24 lanes per token, which may straddle two waves) K's
    // FFT rotation goes through LDS (srft192_lane) and V is not rotated
    constexpr bool kRotates = (D & (D - 1)) == 0;
    constexpr bool kSrft192 = D == 192 && SRFT;
    static_assert(kRotates || (!VROT && (!SRFT || D == 192)), "head_dim 192: K's FFT rotation only");
    const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
    auto fresh_at = [&](int t) { return FULL || (t >= p0 && t < t_end && t >= 0); };
    auto widen8 = [&](const uint4& q, float (&x)[8]) {
        const uint32_t ww[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = widen((uint16_t)(ww[e / 2] >> (16 * (e % 2))), DTYPE);
    };

    // V lane roles, and the nibble mask of the tokens a word takes (the same
    // for the whole wave, which has one r)
    const int jl = lane & 3, m = (lane >> 2) & 7, jh = lane >> 5;
    auto v_token = [&](int r, int mm) { return 4 * r + (mm & 3) + 16 * (mm >> 2); };
    auto v_mask = [&](int r) {
        uint32_t mask = 0;
#pragma unroll
        for (int mm = 0; mm < 8; ++mm) mask |= fresh_at(t_tile + v_token(r, mm)) ? 0xFu << (4 * mm) : 0u;
        return mask;
    };

    // issue every load first; the K signs and channel scales of a lane are
    // the same in every unit when a token's lanes divide the block (LT | 256),
    // else (head_dim 192) the channel scales are loaded per unit
    constexpr bool kSameJ = 256 % LT == 0;
    float sg[kSameJ ? 1 : U][8], lm[kSameJ ? 1 : U][8], vsg[VROT ? 8 : 1];
    if (signs) {
#pragma unroll
        for (int i = 0; i < (kSameJ ? 1 : U); ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) sg[i][e] = signs[8 * ((i * 256 + tid) % LT) + e];
    }
    // the FFT rotation's twiddles: the lane's position in its token, hence
    // its twiddles, is the same in every unit
    [[maybe_unused]] SrftLaneTw<kRotates ? D : 64, 8> stw;
    if constexpr (SRFT && kRotates) stw.load(tid % LT);
    if constexpr (VROT) {
#pragma unroll
        for (int e = 0; e < 8; ++e) vsg[e] = vsigns[8 * (tid % LT) + e];
    }
    if (lam) {
#pragma unroll
        for (int i = 0; i < (kSameJ ? 1 : U); ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) lm[i][e] = lam[8 * ((i * 256 + tid) % LT) + e];
    }
    uint4 kraw[U], vraw[U];
#pragma unroll
    for (int i = 0; i < U; ++i) {
        const int L = i * 256 + tid, t = t_tile + L / LT;
        kraw[i] = make_uint4(0, 0, 0, 0);
        if (fresh_at(t)) kraw[i] = load_stream(k + (head * n_new + (t - p0)) * D + 8 * (L % LT));
    }
#pragma unroll
    for (int i = 0; i < U; ++i) {
        vraw[i] = make_uint4(0, 0, 0, 0);
        if constexpr (VROT) {  // the K layout
            const int L = i * 256 + tid, t = t_tile + L / LT;
            if (fresh_at(t)) vraw[i] = load_stream(v + (head * n_new + (t - p0)) * D + 8 * (L % LT));
        } else {
            const int vt = i * 4 + w, gp = vt >> 2, r = vt & 3;
            const int t = t_tile + v_token(r, m), g = 2 * gp + jh;
            if (fresh_at(t)) vraw[i] = load_stream(v + (head * n_new + (t - p0)) * D + 32 * g + 8 * jl);
        }
    }
    uint32_t* vtile = reinterpret_cast<uint32_t*>(vc + (head * (cap / kTile) + t_tile / kTile) * (size_t)(16 * D));
    auto v_word = [&](int gp, int r) { return ((gp * 4 + r) * 16 + 8 * (jl & 1) + m) * 4 + 2 * jh + (jl >> 1); };
    uint32_t vold[U];  // older nibbles of words the range shares at its ends
#pragma unroll
    for (int i = 0; i < U; ++i) {
        vold[i] = 0;
        if constexpr (!FULL) {
            const int vt = i * 4 + w, gp = vt >> 2, r = vt & 3;
            const uint32_t mask = v_mask(r);
            if (mask != 0 && mask != 0xFFFFFFFFu) vold[i] = vtile[v_word(gp, r)];
        }
    }

    // head_dim 192, K FFT-rotated: the tile's K rows, signs applied, in LDS
    // (krot, kTile x D floats) for the radix-3 stage, which reads lanes of
    // other waves, followed by the 96-point twiddles (re, then im)
    if constexpr (kSrft192) {
        if (tid < 192) krot[kTile * D + tid] = tid < 96 ? srft_detail::kTw96.re[tid] : srft_detail::kTw96.im[tid - 96];
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int L = i * 256 + tid;
            float x[8];
            widen8(kraw[i], x);
#pragma unroll
            for (int e = 0; e < 8; ++e) krot[(L / LT) * D + 8 * (L % LT) + e] = x[e] * sg[i][e];
        }
        __syncthreads();
    }

    // K: widen, rotate, quantise; one code word and (per group) one scale
#pragma unroll
    for (int i = 0; i < U; ++i) {
        const int L = i * 256 + tid, t = t_tile + L / LT, j = L % LT;
        float x[8];
        widen8(kraw[i], x);
        if constexpr (kSrft192) {  // the row staged in LDS (signs applied) above
            srft192_lane(x, krot + (L / LT) * D, j, krot + kTile * D);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = x[e] * rot_norm;
        } else if constexpr (kRotates) {
            if (signs) {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = x[e] * sg[0][e];
                if constexpr (SRFT)
                    srft_signed<D, 8>(x, rot_norm, j, stw);
                else
                    rotate_signed<D, 8>(x, rot_norm, j);
            }
        }
        if (lam) {  // K's per-channel scale, after the rotation
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = x[e] * lm[kSameJ ? 0 : i][e];
        }
        float sk;
        const uint32_t word = quantize_word8(x, sk);
        if (fresh_at(t)) {
            const size_t row = head * cap + t;
            store_stream(reinterpret_cast<uint32_t*>(kc + row * (D / 2)) + (j & 3) * NG + (j >> 2), word);
            if ((j & 3) == 0) store_stream(ks + row * NG + (j >> 2), sk);
        }
    }

    // V rotated: widen, rotate, quantise and store the scales in the K
    // layout, then stage the code words in LDS (vstage, kTile x LT words:
    // token u, channel block j)
    if constexpr (VROT) {
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int L = i * 256 + tid, u = L / LT, t = t_tile + u, j = L % LT;
            float x[8];
            widen8(vraw[i], x);
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = x[e] * vsg[e];
            if constexpr (SRFT)
                srft_signed<D, 8>(x, rot_norm, j, stw);
            else
                rotate_signed<D, 8>(x, rot_norm, j);
            float sv;
            vstage[u * LT + j] = quantize_word8(x, sv);
            if (fresh_at(t) && (j & 3) == 0) vs[(head * cap + t) * NG + (j >> 2)] = sv;
        }
        __syncthreads();
    }

    // V: widen, quantise, scales (or the staged words of a rotated V);
    // transpose the nibbles and store whole words
#pragma unroll
    for (int i = 0; i < U; ++i) {
        const int vt = i * 4 + w, gp = vt >> 2, r = vt & 3;
        uint32_t word;
        if constexpr (VROT) {
            word = vstage[v_token(r, m) * LT + 8 * gp + 4 * jh + jl];
        } else {
            const int t = t_tile + v_token(r, m), g = 2 * gp + jh;
            float x[8];
            widen8(vraw[i], x);
            float sv;
            word = quantize_word8(x, sv);
            if (fresh_at(t) && jl == 0) vs[(head * cap + t) * NG + g] = sv;
        }
#pragma unroll
        for (int s = 1; s <= 4; s <<= 1) {
            const uint32_t keep = s == 1 ? 0x0F0F0F0Fu : s == 2 ? 0x00FF00FFu : 0x0000FFFFu;
            const uint32_t other = (uint32_t)__shfl_xor((int)word, 4 * s, 64);
            word = (m & s) ? (((other >> (4 * s)) & keep) | (word & ~keep))
                           : ((word & keep) | ((other & keep) << (4 * s)));
        }
        // the mask is wave-uniform: whole words inside the appended range,
        // merged with the old word at its ends, nothing outside it
        if constexpr (FULL) {
            store_stream(vtile + v_word(gp, r), word);
        } else {
            const uint32_t mask = v_mask(r);
            if (mask == 0xFFFFFFFFu) vtile[v_word(gp, r)] = word;
            else if (mask != 0) vtile[v_word(gp, r)] = (vold[i] & ~mask) | (word & mask);
        }
    }
}

template <int D, int DTYPE, bool VROT, bool SRFT>
__global__ __launch_bounds__(256) void quantize_tile_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int n_new,
    int H, int cap, uint8_t* __restrict__ kc, float* __restrict__ ks, uint8_t* __restrict__ vc,
    float* __restrict__ vs, const float* __restrict__ signs, float rot_norm,
    const float* __restrict__ lam, const float* __restrict__ vsigns, const int32_t* __restrict__ pos,
    unsigned* __restrict__ err)
{
    const int h = blockIdx.y, b = blockIdx.z;
    const int p0 = pos[b];
    if (threadIdx.x == 0 && blockIdx.x == 0 && h == 0 && (p0 < 0 || p0 > cap - n_new))
        report_error(err, kErrPos);  // the tokens outside [0, cap) are skipped below
    const int t_tile = (p0 / kTile + (int)blockIdx.x) * kTile;
    const int t_end = min(p0 + n_new, cap);
    if (t_tile >= t_end) return;  // block-uniform
    const size_t head = (size_t)b * H + h;
    // LDS of the rotated forms (one array for both instances below)
    constexpr bool kSrft192 = D == 192 && SRFT;
    __shared__ uint32_t vstage[VROT ? kTile * (D / 8) : 1];
    __shared__ float krot[kSrft192 ? kTile * D + 192 : 1];
    if (t_tile >= 0 && t_tile >= p0 && t_tile + kTile <= t_end)
        quantize_tile<D, DTYPE, true, VROT, SRFT>(k, v, n_new, cap, head, p0, t_tile, t_end, kc, ks, vc, vs,
                                            signs, rot_norm, lam, vsigns, vstage, krot);
    else
        quantize_tile<D, DTYPE, false, VROT, SRFT>(k, v, n_new, cap, head, p0, t_tile, t_end, kc, ks, vc, vs,
                                             signs, rot_norm, lam, vsigns, vstage, krot);
}

}  // namespace

bool quantize_tile_wide_supports(int D, int n_new, bool v_rotated)
{
    return D == 192 && n_new >= kPairKernelMaxTokens && !v_rotated;
}

hipError_t launch_quantize_tile_wide(const void* k, const void* v, int dtype, int n_new, int B, int H, int D,
                                     int cap, uint8_t* kc, float* ks, uint8_t* vc, float* vs,
                                     const float* signs, float rot_norm, const float* lam, const int32_t* pos,
                                     unsigned* err, hipStream_t stream)
{
    if (!quantize_tile_wide_supports(D, n_new, false)) return hipErrorInvalidValue;
    const int tiles = (n_new + 2 * kTile - 2) / kTile;  // the range may start inside a tile
    dim3 grid(tiles, H, B), block(256);
    const auto* kk = static_cast<const uint16_t*>(k);
    const auto* vv = static_cast<const uint16_t*>(v);
    // a K rotation at this width is the FFT kind
    auto kern = signs ? (dtype == 0 ? quantize_tile_kernel<192, 0, false, true> : quantize_tile_kernel<192, 1, false, true>)
                      : (dtype == 0 ? quantize_tile_kernel<192, 0, false, false> : quantize_tile_kernel<192, 1, false, false>);
    kern<<<grid, block, 0, stream>>>(kk, vv, n_new, H, cap, kc, ks, vc, vs, signs, rot_norm, lam, nullptr, pos, err);
    return hipGetLastError();
}

hipError_t launch_quantize_append(const void* k, const void* v, int dtype, int n_new, int B, int H,
                                  int D, int cap, uint8_t* kc, float* ks, uint8_t* vc, float* vs,
                                  const float* signs, float rot_norm, int rot_kind, const float* lam,
                                  const float* vsigns, const int32_t* pos, unsigned* err,
                                  hipStream_t stream)
{
    if (D != 64 && D != 128 && D != 256) return hipErrorInvalidValue;
    const auto* kk = static_cast<const uint16_t*>(k);
    const auto* vv = static_cast<const uint16_t*>(v);
    if (n_new < kPairKernelMaxTokens) {
        const int pair_slots = (n_new + 2) / 2;
        dim3 grid((pair_slots + 3) / 4, H, B), block(256);
        auto kern = D == 64 ? quantize_pair_kernel<64> : D == 128 ? quantize_pair_kernel<128> : quantize_pair_kernel<256>;
        kern<<<grid, block, 0, stream>>>(kk, vv, dtype, n_new, H, cap, kc, ks, vc, vs, signs, rot_norm,
                                         (signs || vsigns) ? rot_kind : 0, lam, vsigns, pos, pair_slots, err);
    } else {
        // one block per tile touched: the range may start inside a tile
        const int tiles = (n_new + 2 * kTile - 2) / kTile;
        dim3 grid(tiles, H, B), block(256);
        using K = void (*)(const uint16_t*, const uint16_t*, int, int, int, uint8_t*, float*, uint8_t*, float*,
                           const float*, float, const float*, const float*, const int32_t*, unsigned*);
        auto pick = [&](auto d) -> K {
            constexpr int DD = decltype(d)::value;
            if (vsigns && rot_kind)
                return dtype == 0 ? quantize_tile_kernel<DD, 0, true, true> : quantize_tile_kernel<DD, 1, true, true>;
            if (vsigns)
                return dtype == 0 ? quantize_tile_kernel<DD, 0, true, false> : quantize_tile_kernel<DD, 1, true, false>;
            if (signs && rot_kind)
                return dtype == 0 ? quantize_tile_kernel<DD, 0, false, true> : quantize_tile_kernel<DD, 1, false, true>;
            return dtype == 0 ? quantize_tile_kernel<DD, 0, false, false> : quantize_tile_kernel<DD, 1, false, false>;
        };
        const K kern = D == 64 ? pick(std::integral_constant<int, 64>{})
                     : D == 128 ? pick(std::integral_constant<int, 128>{})
                                : pick(std::integral_constant<int, 256>{});
        kern<<<grid, block, 0, stream>>>(kk, vv, n_new, H, cap, kc, ks, vc, vs, signs, rot_norm, lam, vsigns,
                                         pos, err);
    }
    return hipGetLastError();
}

}  // namespace otq
