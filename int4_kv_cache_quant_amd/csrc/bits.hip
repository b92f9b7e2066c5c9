// bits.hip - 2- and 3-bit codes: quantise-append and the vector split pass.
//
// The code widths the AdapTQ page lists beside 4-bit (its section on the
// core mechanisms: 2-, 3- and 4-bit quantisation): b-bit codes take the
// int4 steps with the symmetric range of b bits, s = abs-max / (2^(b-1) - 1)
// in IEEE fp32 and c = clamp(rint(x / s), -2^(b-1), 2^(b-1) - 1), s == 0
// giving zero codes, two's complement.  A K row is a plain little-endian bit
// stream (element i at bits [b i, b i + b)), [B][H][capacity][D b / 8]
// bytes; V codes are regrouped per tile of 32 tokens (bits_layout.hpp), the
// same bytes per tile; scales as for int4.
//
// The vector split pass (for caches whose K is rotated or channel-scaled,
// and 3-bit codes at head_dim 256) computes scores and the value sum with
// fp32 vector arithmetic, one token per thread for the scores and one
// channel per thread for the value sum, and writes the same (m, l, o)
// partials as the int4 kernels, so the same combine merges them.
#include "bits_layout.hpp"
#include "common.hpp"
#include "kernels.hpp"
#include "quant_lane.hpp"
#include "srft.hpp"

namespace otq {

namespace {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr float kNegInfB = -__builtin_huge_valf();

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

constexpr int kBitsSmallAppend = 8;

// Appends of fewer than kBitsSmallAppend tokens (a decode step's token): one
// block per (32-token tile touched, KV head, sequence) whose waves quantise
// the tile's new K and V vectors in turn (one wave per vector, E = D / 64
// elements per lane), a short dependency chain per token.  A K row is written whole from the
// wave's codes (D b / 32 lanes assemble its 32-bit words); the V codes of
// the tile are staged in LDS and the tile's V words are written whole, merged
// with the old words under a mask where only part of the tile is new (only
// this block writes the tile in this launch).
template <int D, int BITS>
__global__ __launch_bounds__(256) void quantize_bits_small_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int dtype, int n_new, int H, int cap,
    uint8_t* __restrict__ kc, float* __restrict__ ks, uint8_t* __restrict__ vc, float* __restrict__ vs,
    const int32_t* __restrict__ pos, const float* __restrict__ signs, float rot_norm, int rot_kind,
    const float* __restrict__ lam, const float* __restrict__ vsigns, unsigned* __restrict__ err)
{
#pragma clang fp contract(off)
    constexpr int E = D / 64, NG = D / kGroup, RB = D * BITS / 8, NWORD = RB / 4;
    constexpr float qmax = (float)((1 << (BITS - 1)) - 1), qmin = -(float)(1 << (BITS - 1));
    using VT = VBitsTile<D, BITS>;
    static_assert(RB % 4 == 0, "whole words per row");
    __shared__ int8_t cs[4][D];       // a wave's K codes
    __shared__ int8_t cvt[kTile][D];  // the tile's V codes
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int h = blockIdx.y, b = blockIdx.z;
    const int p0 = pos[b];
    if (tid == 0 && blockIdx.x == 0 && h == 0 && (p0 < 0 || p0 > cap - n_new))
        report_error(err, kErrPos);  // the tokens outside [0, cap) are skipped below
    // the block's tile: the appended range clipped to [0, cap), tiles counted
    // from the one holding its first token
    const long long lo_all = max((long long)p0, 0LL), hi_all = min((long long)p0 + n_new, (long long)cap);
    if (lo_all >= hi_all) return;  // block-uniform: nothing inside the cache
    const int tile = (int)(lo_all / kTile) + blockIdx.x;
    const int lo = (int)max(lo_all, (long long)kTile * tile), hi = (int)min(hi_all, (long long)kTile * tile + kTile);
    if (lo >= hi) return;  // block-uniform: past the range
    const int nt = hi - lo, u0 = lo - kTile * tile;
    SrftLaneTw<D, E> stw;  // the FFT rotation's twiddles of this lane
    if ((signs || vsigns) && rot_kind) stw.load(lane);
    const size_t head = (size_t)b * H + h;
    // 2 nt vectors (the K tokens, then the V tokens), four at a time (the
    // block's barrier count is the same for all its threads)
    const int iters = (2 * nt + 3) / 4;
    for (int it = 0; it < iters; ++it) {
        const int vec = 4 * it + wave;
        const bool active = vec < 2 * nt;
        const bool is_v = vec >= nt;
        const int tr = is_v ? vec - nt : vec;  // token lo + tr
        const int t = lo + tr;
        float sc = 0.0f;
        if (active) {
            const uint16_t* src = (is_v ? v : k) + (head * n_new + (t - p0)) * D + lane * E;
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
            int8_t* dst = is_v ? &cvt[u0 + tr][0] : &cs[wave][0];
#pragma unroll
            for (int e = 0; e < E; ++e) {
                float r = rintf(x[e] / sc);  // IEEE division, then half to even
                r = fminf(fmaxf(r, qmin), qmax);
                dst[lane * E + e] = (int8_t)(sc != 0.0f ? (int)r : 0);
            }
        }
        __syncthreads();
        if (active) {
            const size_t row = head * cap + t;
            if (lane % (kGroup / E) == 0) (is_v ? vs : ks)[row * NG + (lane * E) / kGroup] = sc;
            if (!is_v && lane < NWORD) {  // word w holds bits [32 w, 32 w + 32) of the K row
                uint32_t word = 0;
                const int i0 = (32 * lane) / BITS, i1 = min((32 * lane + 31) / BITS, D - 1);
                for (int i = i0; i <= i1; ++i) {
                    const uint32_t u = (uint32_t)cs[wave][i] & ((1u << BITS) - 1u);
                    const int off = i * BITS - 32 * lane;  // may be negative for the first element
                    word |= off >= 0 ? u << off : u >> -off;
                }
                reinterpret_cast<uint32_t*>(kc + row * RB)[lane] = word;
            }
        }
        __syncthreads();  // cs is rewritten by the next vectors
    }
    // the tile's V words: the new tokens' fields from the staged codes
    uint32_t* vt = reinterpret_cast<uint32_t*>(vc + (head * (cap / kTile) + tile) * (size_t)(kTile * RB));
    for (int W = tid; W < VT::WORDS; W += 256) {
        uint32_t val = 0, mask = 0;
        vtile_fields<D, BITS>(W, [&](int u, int c, int bpos, int width, int shift) {
            if (u >= u0 && u < u0 + nt) {
                const uint32_t fm = (1u << width) - 1u;
                val |= (((uint32_t)(int)cvt[u][c] >> shift) & fm) << bpos;
                mask |= fm << bpos;
            }
        });
        if (mask == 0) continue;
        if (mask != 0xFFFFFFFFu) val |= vt[W] & ~mask;
        vt[W] = val;
    }
}

// Bulk appends: one block per (32-token tile touched by the append, KV
// head, sequence).  K and V alike: a token occupies LT = D / 8 consecutive threads, thread j of
// a token holding its channels 8 j .. 8 j + 7 (one 16-byte load), so a scale
// group is one aligned quad of lanes; every load of the block is issued
// before any arithmetic.  Each vector is widened, rotated (its own signs, in
// the same order of operations as the other append kernels), K scaled by its
// channel scale, and quantised: s = abs-max / (2^(b-1) - 1) and c =
// clamp(rint(x / s)), the quotients correctly rounded (by reciprocal and
// Markstein corrections for group maxima in [2^-80, 2^100], else by IEEE
// division).  K rows are written whole from registers (a lane's 8 fields
// with its neighbours' make whole words); V codes pass through LDS, then the
// block writes the tile's V words whole, merging them with their old
// contents under a mask where only part of the tile is new (only this block
// writes the tile in this launch).
template <int D, int BITS, bool SRFT>
__global__ __launch_bounds__(256) void quantize_bits_kernel(
    const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, int dtype, int n_new, int H, int cap,
    uint8_t* __restrict__ kc, float* __restrict__ ks, uint8_t* __restrict__ vc, float* __restrict__ vs,
    const int32_t* __restrict__ pos, const float* __restrict__ signs, float rot_norm,
    const float* __restrict__ lam, const float* __restrict__ vsigns, unsigned* __restrict__ err)
{
#pragma clang fp contract(off)
    constexpr int NG = D / kGroup, RB = D * BITS / 8;
    constexpr int LT = D / 8;           // threads per token
    constexpr int U = kTile * LT / 256;  // units (16-byte pieces) per thread, of K and of V
    constexpr float qmax = (float)((1 << (BITS - 1)) - 1), qmin = -(float)(1 << (BITS - 1));
    using VT = VBitsTile<D, BITS>;
    static_assert(RB % 4 == 0, "whole words per row");
    // the tile's V codes, channel-major (a channel's 32 tokens in a row of
    // TS bytes: four tokens of a quarter are one aligned word, and the
    // padding spreads the rows over the banks)
    constexpr int TS = kTile + 4;
    __shared__ __align__(4) int8_t ccs[D * TS];
    const int tid = threadIdx.x, j = tid % LT;
    const int h = blockIdx.y, b = blockIdx.z;
    const int p0 = pos[b];
    if (tid == 0 && blockIdx.x == 0 && h == 0 && (p0 < 0 || p0 > cap - n_new))
        report_error(err, kErrPos);  // the tokens outside [0, cap) are skipped below
    // the block's tile: the appended range clipped to [0, cap), tiles counted
    // from the one holding its first token
    const long long lo_all = max((long long)p0, 0LL), hi_all = min((long long)p0 + n_new, (long long)cap);
    if (lo_all >= hi_all) return;  // block-uniform: nothing inside the cache
    const int tile = (int)(lo_all / kTile) + blockIdx.x;
    const int t0 = kTile * tile;
    const int lo = (int)max(lo_all, (long long)t0), hi = (int)min(hi_all, (long long)t0 + kTile);
    if (lo >= hi) return;  // block-uniform: past the range
    const int u0 = lo - t0, nt = hi - lo;
    auto fresh = [&](int u) { return u >= u0 && u < u0 + nt; };
    const size_t head = (size_t)b * H + h;

    // every load first: unit i of this thread is token u = (256 i + tid) / LT
    // of the tile, channels 8 j .. 8 j + 7
    u32x4_t raw[2][U];
#pragma unroll
    for (int w = 0; w < 2; ++w)
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int u = (256 * i + tid) / LT;
            raw[w][i] = u32x4_t{0u, 0u, 0u, 0u};
            if (fresh(u))
                raw[w][i] = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(
                    (w ? v : k) + (head * n_new + (t0 + u - p0)) * D + 8 * j));
        }
    float sg[8], vsg[8], lm[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        sg[e] = signs ? signs[8 * j + e] : 1.0f;
        vsg[e] = vsigns ? vsigns[8 * j + e] : 1.0f;
        lm[e] = lam ? lam[8 * j + e] : 1.0f;
    }
    [[maybe_unused]] SrftLaneTw<D, 8> stw;  // the FFT rotation's twiddles of this lane position
    if constexpr (SRFT) stw.load(j);

#pragma unroll
    for (int w = 0; w < 2; ++w) {
        const bool rot = w ? vsigns != nullptr : signs != nullptr;
#pragma unroll
        for (int i = 0; i < U; ++i) {
            const int u = (256 * i + tid) / LT;
            // the same for the LT lanes of a token, which alone exchange values
            if (!fresh(u)) continue;
            float x[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) x[e] = widen((uint16_t)(raw[w][i][e / 2] >> (16 * (e % 2))), dtype);
            if (rot) {
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = x[e] * (w ? vsg[e] : sg[e]);
                if constexpr (SRFT)
                    srft_signed<D, 8>(x, rot_norm, j, stw);
                else
                    rotate_signed<D, 8>(x, rot_norm, j);
            }
            if (w == 0 && lam) {  // K's per-channel scale, after the rotation
#pragma unroll
                for (int e = 0; e < 8; ++e) x[e] = x[e] * lm[e];
            }
            float a = 0.0f;
#pragma unroll
            for (int e = 0; e < 8; ++e) a = fmaxf(a, fabsf(x[e]));
            a = group_max<4>(a);        // exact in any order
            const float sc = a / qmax;  // correctly rounded IEEE division
            int cd[8];
            if (a >= 0x1p-80f && a <= 0x1p100f) {
                // RN(x / sc) from one correctly rounded reciprocal and two
                // Markstein corrections: the int4 quantiser's argument
                // (quant_lane.hpp) holds for any qmax <= 7, since |x / sc| <=
                // qmax (1 + 2^-23) and sc >= a / 7; the same quotients as the
                // division, hence the same codes
                const float y = 1.0f / sc;  // correctly rounded IEEE division
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float q = x[e] * y;
                    q = __builtin_fmaf(__builtin_fmaf(-q, sc, x[e]), y, q);
                    q = __builtin_fmaf(__builtin_fmaf(-q, sc, x[e]), y, q);  // RN(x / sc)
                    const float r = fminf(fmaxf(rintf(q), qmin), qmax);
                    cd[e] = (int)r;
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float r = rintf(x[e] / sc);  // IEEE division, then half to even
                    r = fminf(fmaxf(r, qmin), qmax);
                    cd[e] = sc != 0.0f ? (int)r : 0;
                }
            }
            if (w == 0) {
                // K: the lane's 8 fields are bits [8 b j, 8 b j + 8 b) of the
                // row; whole words from the token's neighbouring lanes (a
                // pair at 2 bits, the group's quad at 3)
                uint32_t f = 0;
#pragma unroll
                for (int e = 0; e < 8; ++e) f |= ((uint32_t)cd[e] & ((1u << BITS) - 1u)) << (BITS * e);
                uint32_t* krow = reinterpret_cast<uint32_t*>(kc + (head * cap + t0 + u) * RB);
                if constexpr (BITS == 2) {
                    const uint32_t other = (uint32_t)__shfl_xor((int)f, 1, 64);
                    if ((j & 1) == 0) __builtin_nontemporal_store(f | (other << 16), krow + j / 2);
                } else {
                    const int jj = j & 3;
                    const uint32_t nx = (uint32_t)__shfl_down((int)f, 1, 4);  // lane j + 1 of the quad
                    const uint32_t word = jj == 0 ? (f | (nx << 24)) : jj == 1 ? ((f >> 8) | (nx << 16))
                                                                               : ((f >> 16) | (nx << 8));
                    if (jj < 3) __builtin_nontemporal_store(word, krow + 3 * (j >> 2) + jj);
                }
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) ccs[(8 * j + e) * TS + u] = (int8_t)cd[e];
            }
            if ((j & 3) == 0) (w ? vs : ks)[(head * cap + t0 + u) * NG + j / 4] = sc;
        }
    }
    __syncthreads();
    // the tile's V words: the new tokens' fields
    uint32_t* vt = reinterpret_cast<uint32_t*>(vc + (head * (cap / kTile) + tile) * (size_t)(kTile * RB));
    if (nt == kTile) {  // block-uniform: every token of the tile is new
        // the b-bit fields of the four tokens 4 r + m (m = 0..3) of channel
        // c, quarter r, half h: one LDS word of four codes, packed at b m
        auto quad = [&](int c, int h, int r) {
            const uint32_t v = *reinterpret_cast<const uint32_t*>(&ccs[c * TS + 16 * h + 4 * r]);
            constexpr uint32_t m = (1u << BITS) - 1u;
            return (v & m) | ((v >> (8 - BITS)) & (m << BITS)) | ((v >> (16 - 2 * BITS)) & (m << (2 * BITS))) |
                   ((v >> (24 - 3 * BITS)) & (m << (3 * BITS)));
        };
        for (int W = tid; W < VT::WORDS; W += 256) {
            const int l = W / VT::WPL, k = W % VT::WPL, r = l >> 4, n = l & 15;
            uint32_t val = 0;
            if constexpr (BITS == 2) {  // blocks 2 k + t at bit 16 h + 8 t
#pragma unroll
                for (int t = 0; t < 2; ++t)
#pragma unroll
                    for (int h = 0; h < 2; ++h) val |= quad(16 * (2 * k + t) + n, h, r) << (16 * h + 8 * t);
            } else {  // block 4 qd + w at bit 16 h, and bits 4 w .. 4 w + 3 of block 4 qd + 3 at 16 h + 12
                const int qd = k / 3, w = k % 3;
#pragma unroll
                for (int h = 0; h < 2; ++h)
                    val |= (quad(16 * (4 * qd + w) + n, h, r) | (((quad(16 * (4 * qd + 3) + n, h, r) >> (4 * w)) & 0xFu)
                                                                << 12))
                           << (16 * h);
            }
            vt[W] = val;
        }
        return;
    }
    for (int W = tid; W < VT::WORDS; W += 256) {
        uint32_t val = 0, mask = 0;
        vtile_fields<D, BITS>(W, [&](int u, int c, int bpos, int width, int shift) {
            if (fresh(u)) {
                const uint32_t fm = (1u << width) - 1u;
                val |= (((uint32_t)(int)ccs[c * TS + u] >> shift) & fm) << bpos;
                mask |= fm << bpos;
            }
        });
        if (mask == 0) continue;
        if (mask != 0xFFFFFFFFu) val |= vt[W] & ~mask;
        vt[W] = val;
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
    // lens clamped to [0, max_len] first, as the combine does, then the
    // fused append's token (lens_offset = 1) left to the combine
    const int raw_len = a.lens[b];
    const int len = max(min(max(raw_len, 0), a.max_len) - a.lens_offset, 0);
    if (tid == 0 && split == 0 && hk == 0 && (raw_len < 0 || raw_len > a.max_len)) report_error(a.err, kErrLens);
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
            // the step's V tiles (whole: the fields of a token spread over
            // its tile) and scales into LDS (coalesced); t0 is tile-aligned
            {
                const uint32_t* vsrc = reinterpret_cast<const uint32_t*>(vrows + (size_t)t0 * RB);
                const int nw = (n + kTile - 1) / kTile * kTile * RW;
                for (int k = tid; k < nw; k += TT) v_lds[k] = vsrc[k];
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
                const float vd = (float)vtile_code<D, BITS>(&v_lds[(j / kTile) * (kTile * RW)], j % kTile, vc_) *
                                 vs_lds[j * NG + gr];
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
                    unsigned* err, hipStream_t s)
{
    // an unaligned range of n_new tokens touches at most n_new / 32 + 2 tiles
    dim3 grid(n_new / kTile + 2, H, B), block(256);
    if (n_new < kBitsSmallAppend) {
        quantize_bits_small_kernel<D, BITS><<<grid, block, 0, s>>>(
            static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), dtype, n_new, H, cap, kc, ks, vc, vs,
            pos, r.signs, r.rot_norm, r.rot_kind, r.lam, r.vsigns, err);
        return hipGetLastError();
    }
    auto kern = (r.signs || r.vsigns) && r.rot_kind ? quantize_bits_kernel<D, BITS, true>
                                                    : quantize_bits_kernel<D, BITS, false>;
    kern<<<grid, block, 0, s>>>(static_cast<const uint16_t*>(k), static_cast<const uint16_t*>(v), dtype, n_new, H,
                                cap, kc, ks, vc, vs, pos, r.signs, r.rot_norm, r.lam, r.vsigns, err);
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
                                const int32_t* pos, const BitsRot& r, unsigned* err, hipStream_t s)
{
    switch (D * 10 + bits) {
    case 642: return launch_q<64, 2>(k, v, dtype, n_new, B, H, cap, kc, ks, vc, vs, pos, r, err, s);
    case 643: return launch_q<64, 3>(k, v, dtype, n_new, B, H, cap, kc, ks, vc, vs, pos, r, err, s);
    case 1282: return launch_q<128, 2>(k, v, dtype, n_new, B, H, cap, kc, ks, vc, vs, pos, r, err, s);
    case 1283: return launch_q<128, 3>(k, v, dtype, n_new, B, H, cap, kc, ks, vc, vs, pos, r, err, s);
    case 2562: return launch_q<256, 2>(k, v, dtype, n_new, B, H, cap, kc, ks, vc, vs, pos, r, err, s);
    case 2563: return launch_q<256, 3>(k, v, dtype, n_new, B, H, cap, kc, ks, vc, vs, pos, r, err, s);
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
