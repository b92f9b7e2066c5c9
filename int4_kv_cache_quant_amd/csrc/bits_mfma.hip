// bits_mfma.hip - split pass of decode attention on 2- and 3-bit caches, on
// the matrix cores.
//
// The 2- and 3-bit codes of the AdapTQ page (its core-mechanism section
// lists 2-, 3- and 4-bit quantisation behind one pipeline) go through the same kind of
// products as the int4 cache: G query heads sharing a KV head make scoring a
// tile and weighting its values two genuine matrix products, run here as
// v_mfma_f32_16x16x32_f16 with fp32 accumulation.  K rows are plain b-bit
// rows (element i at bits [b i, b i + b) of the row's little-endian bit
// stream); V codes are regrouped per 32-token tile (bits_layout.hpp) so that
// each lane's value operands come from its own words of the tile; fp32 group
// scales.
//
// Exactness, as in the int4 split pass:
//  * K codes enter as fp16 subnormals n 2^(e_k - 24) of their offset-binary
//    value n = c + 2^(b-1): the 8 codes of one lane's k slots (channels
//    32 g + 8 r + 0..7, 8b consecutive bits of the row) are brought to bit 0
//    (a byte permute at 2 bits, a funnel shift at 3), channels 4..7 are
//    moved to the upper half, and and-xor masks give the four half pairs
//    (channel 8 r + k, 8 r + k + 4) at a position e_k (2k at 2 bits; 0, 3, 6
//    and, after a shift, 0 at 3); 2^e_k is cancelled by q's operand, the
//    offset by starting each group's accumulator at -2^(b-1) 2^-24 sum(q),
//    2^24 is folded into the softmax scale;
//  * V codes enter as signed normal fp16 integers: the two codes of a k-slot
//    pair sit at the same offset e_m of the two halves of one tile word
//    (2 m at 2 bits; 3 m, and 0 after a shift, at 3), so one and-xor mask
//    puts 1024 + (c + 2^(b-1)) 2^e_m in each half (0x6400 is the exponent of
//    1024, the flipped top bit of the field the offset) and one packed
//    subtraction leaves c 2^e_m exactly; 2^-e_m goes onto p.  The value
//    products are exact and their sums plain fp32;
//  * q rows are scaled by a power of two that puts the largest |element| in
//    [2^14, 2^15) before the fp16 conversion (bf16 and fp16 inputs convert
//    exactly), undone in the softmax scale;
//  * x = p * s_v * 2^E is split into fp16 hi + lo operands; E follows the
//    largest V scale seen, as in the int4 pass.
// A rotated or channel-scaled K (head_dim up to 192) takes q rotated as K
// was and divided by the channel scale, as fp16 hi + lo operands (two score
// products per group, one KV head per wave); at head_dim 256 such caches take
// the vector split pass.  A rotated V is undone by the combine.
//
// Int4 caches at head_dim 192 (six groups, twelve channel blocks; the FFT
// rotation of that width is mixed radix) take this kernel as well: K words
// are the int4 rows' words (word 6 r + g holds channels 32 g + 8 r + 0..7),
// unpacked to subnormals as in the int4 pass, and V words the int4 tile
// words (tokens 4 r + m and 16 + 4 r + m in nibbles m and 4 + m), with
// 2^(4 (k & 1)) as the k-slot powers; one KV head per wave.
//
// Block = 4 waves, one (split, P KV heads, sequence): P = 2 when 4 <= G <= 8
// and head_dim is 64 or 128 (the two heads' query heads fill the 16 MFMA
// columns), else 1; wave w takes the tiles w, w + 4, ... of the split (32
// tokens each).  Each tile (per head: K rows, the V tile, K and V scales:
// (8 b + 8) D bytes) is loaded into registers ahead (two tiles; one at head_dim
// 256, for two heads per wave and for the hi + lo query at 192), written to
// the wave's LDS stage when its turn comes, and read back
// in the operand layouts below.  Lane l = 16 r + n:
//  scores  A = K codes of head j (row = token 16 s + n, k = channels
//          32 g + 8 r + the slot order), B = q of query head n masked to
//          head j's columns (columns >= P G are zero); the P products
//          accumulate into C = S[token 16 s + 4 r + i][head n]
//  values  A = x (row = head n, k slots (2m, 2m + 1) = tokens 4 r + m and
//          16 + 4 r + m: the tokens whose scores this lane holds), B = V codes
//          (column = channel 16 cb + n, the same tokens), one accumulator set
//          per KV head, C_j = O[head 4 r + i][channel 16 cb + n], of which
//          the rows of head j are kept.
#include "bits_layout.hpp"
#include "common.hpp"
#include "kernels.hpp"
#include "mfma_common.hpp"

namespace otq {

namespace {

using namespace mfma;

constexpr int kB2Waves = 4;  // waves per block
// Tiles each wave holds in registers ahead of the one it computes (one at
// head_dim 256, for two KV heads per wave, whose tiles take twice the
// registers, and for the hi + lo query at head_dim 192).
template <int D, int P, bool HILO>
constexpr int kB2Ahead = (D == 256 || P == 2 || (D == 192 && HILO)) ? 1 : 2;
// Where the score accumulator starts at the offset correction (a register
// quad per group, live through the loop) rather than taking it after the
// MFMA: everywhere but head_dim 256 and two heads per wave, whose registers
// are full.
template <int D, int P, bool HILO>
constexpr bool kB2QinitInAcc = D != 256 && D != 192 && P == 1 && !HILO;

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// One tile of a KV head in a wave's LDS stage: K rows, the V tile (32 x RB bytes
// each, as in the cache), then the K and V scales (32 x NG fp32 each).
template <int D, int BITS>
struct BTile {
    static constexpr int RB = D * BITS / 8;  // bytes per row
    static constexpr int NG = D / kGroup;
    static constexpr int KOFF = 0, VOFF = 32 * RB, KSOFF = 64 * RB, VSOFF = KSOFF + 32 * NG * 4;
    static constexpr int BYTES = VSOFF + 32 * NG * 4;  // (8 BITS + 8) D
    static constexpr int SLOTS = BYTES / 16;            // 16-byte pieces
    static constexpr int LOADS = (SLOTS + 63) / 64;     // pieces per lane
    // the merge of the block's waves reuses the stages: 16 O rows padded by
    // 4 floats, then 16 (m, l) pairs
    static constexpr int RS = D + 4;
    static constexpr int MERGE = 16 * RS * 4 + 16 * 8;
    static constexpr int STAGE = BYTES > MERGE ? BYTES : MERGE;
};

// A wave's LDS stage for P KV heads: their tiles one after the other (head j
// at j BYTES); the merge reuses it.
template <int D, int BITS, int P>
struct BStage {
    using T = BTile<D, BITS>;
    static constexpr int SLOTS = P * T::SLOTS;
    static constexpr int LOADS = (SLOTS + 63) / 64;
    static constexpr int BYTES = P * T::BYTES > T::MERGE ? P * T::BYTES : T::MERGE;
};

// K: 8 codes (16 bits of a row, the lane's channels 32 g + 8 r + 0..7 at bit
// 2e) -> 8 fp16 subnormals (c + 2) 2^(2k - 24); k slot (2k, 2k + 1) holds
// channels (8 r + k, 8 r + k + 4).  sel moves the row word's half r & 1 to
// bytes 0 and 2.
__device__ __forceinline__ half8_t unpack_k2(uint32_t w, uint32_t sel)
{
    const uint32_t x = __builtin_amdgcn_perm(w, w, sel);
    uint32_t h[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t m = 0x00030003u << (2 * k), f = 0x00020002u << (2 * k);
        h[k] = (x & m) ^ f;  // one v_bitop3: the sign bit flip makes c + 2
    }
    half8_t out;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const half2_t p = __builtin_bit_cast(half2_t, h[k]);
        out[2 * k] = p[0];
        out[2 * k + 1] = p[1];
    }
    return out;
}

// K, 3-bit: 8 codes (24 bits from bit 0 of f, the lane's channels 32 g +
// 8 r + 0..7 at bit 3e) -> 8 fp16 subnormals (c + 4) 2^(kK3Exp[k] - 24); k
// slot (2k, 2k + 1) holds channels (8 r + k, 8 r + k + 4).  The channels
// 4..7 are first moved to bit 16; the fourth pair (bits 9..11 and 25..27)
// is shifted down, as it would reach into the fp16 exponent.
constexpr int kK3Exp[4] = {0, 3, 6, 0};
__device__ __forceinline__ half8_t unpack_k3(uint32_t f)
{
    const uint32_t x = (f & 0x00000FFFu) | ((f << 4) & 0x0FFF0000u);
    uint32_t h[4];
#pragma unroll
    for (int k = 0; k < 3; ++k) {
        const uint32_t m = 0x00070007u << (3 * k), fl = 0x00040004u << (3 * k);
        h[k] = (x & m) ^ fl;  // the sign bit flip makes c + 4
    }
    h[3] = ((x >> 9) & 0x00070007u) ^ 0x00040004u;
    half8_t out;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const half2_t p = __builtin_bit_cast(half2_t, h[k]);
        out[2 * k] = p[0];
        out[2 * k + 1] = p[1];
    }
    return out;
}

// V, 2 bits: one word of the lane (fields at bit 2 m of each half: tokens
// 4 r + m below, 16 + 4 r + m above) -> k slots (2 m, 2 m + 1) as exact fp16
// values c 4^m: 1024 + (c + 2) 4^m in each half (the flip of the field's top
// bit is the offset, 0x6400 the exponent of 1024), less 1024 + 2 4^m.
__device__ __forceinline__ half8_t unpack_v2(uint32_t w)
{
    half8_t out;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const uint32_t u = (w & (0x00030003u << (2 * m))) ^ (0x64006400u | (0x00020002u << (2 * m)));
        const _Float16 off = (_Float16)(1024.0f + 2.0f * (float)(1 << (2 * m)));
        const half2_t h = __builtin_bit_cast(half2_t, u) - half2_t{off, off};
        out[2 * m] = h[0];
        out[2 * m + 1] = h[1];
    }
    return out;
}

// V, 3 bits: 12 bits per half (fields at bit 3 m) -> k slots (2 m, 2 m + 1)
// as exact fp16 values c 2^kVExp<3>[m]; the slot-3 fields are shifted down
// first, as they would reach into the fp16 exponent.
__device__ __forceinline__ half8_t unpack_v3(uint32_t x)
{
    half8_t out;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
        const uint32_t u = m < 3 ? (x & (0x00070007u << (3 * m))) ^ (0x64006400u | (0x00040004u << (3 * m)))
                                 : ((x >> 9) & 0x00070007u) ^ 0x64046404u;
        const _Float16 off = (_Float16)(1024.0f + 4.0f * (float)(1 << (m < 3 ? 3 * m : 0)));
        const half2_t h = __builtin_bit_cast(half2_t, u) - half2_t{off, off};
        out[2 * m] = h[0];
        out[2 * m + 1] = h[1];
    }
    return out;
}

// The power of two (log2) that slot pair m of an unpacked V word carries.
template <int BITS>
constexpr int kVExp[4] = {0, BITS == 2 ? 2 : BITS == 3 ? 3 : 4, BITS == 2 ? 4 : BITS == 3 ? 6 : 0,
                          BITS == 2 ? 6 : BITS == 3 ? 0 : 4};

template <int D, int BITS, int P, bool HILO>
__global__ __launch_bounds__(64 * kB2Waves) __attribute__((amdgpu_waves_per_eu(2, D == 64 ? 4 : 2)))
void split_bits_mfma_kernel(SplitArgs a)
{
    static_assert(BITS == 2 || BITS == 3 || (BITS == 4 && D == 192), "2- or 3-bit codes, or int4 at 192");
    using T = BTile<D, BITS>;
    using SG = BStage<D, BITS, P>;
    using VT = VBitsTile<D, BITS == 4 ? 2 : BITS>;  // (b-bit V tiles only)
    constexpr int NG = T::NG, NCB = D / 16, RB = T::RB, W = kB2Waves;
    extern __shared__ __align__(16) char lds[];  // W stages of SG::BYTES

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    int split = blockIdx.x, hk0 = blockIdx.y * P, b = blockIdx.z;
    if (a.items) {  // a batch: the block's item in longest-first order
        const int groups = a.H / P;
        const int k = blockIdx.x + a.num_splits * (blockIdx.y + groups * blockIdx.z);
        const int2 it = a.items[k];
        if (it.x < 0) return;  // block-uniform: no item
        split = it.x;
        b = it.y;
        hk0 = (k % groups) * P;
    }
    const int G = a.Hq / a.H;
    const int PG = P * G;  // query heads served by the block (<= 16)
    const int n16 = lane & 15, r = lane >> 4;
    const bool col_valid = n16 < PG;
    const int jl = col_valid ? n16 / G : 0;  // KV head (of the block's P) of this lane's column
    char* stage = lds + wave * SG::BYTES;

    // lens clamped to [0, max_len], then the fused append's token left to
    // the combine
    const int raw_len = a.lens[b];
    const int len = max(min(max(raw_len, 0), a.max_len) - a.lens_offset, 0);
    if (tid == 0 && split == 0 && hk0 == 0 && (raw_len < 0 || raw_len > a.max_len)) report_error(a.err, kErrLens);
    const int start = split * a.chunk;
    if (start >= len) return;  // block-uniform: no partial for an empty split
    const int end = min(start + a.chunk, len);
    const int ntiles = (end - start + kTile - 1) / kTile;

    // ---- per-lane sources of the tile's 16-byte pieces: per KV head, K rows,
    //      the V tile, K scales, V scales, each contiguous for the tile's 32
    //      tokens
    const char* src_base[SG::LOADS];
    int src_stride[SG::LOADS];
    bool src_on[SG::LOADS];
#pragma unroll
    for (int k = 0; k < SG::LOADS; ++k) {
        const int i = 64 * k + lane;
        src_on[k] = i < SG::SLOTS;
        const size_t head = (size_t)b * a.H + hk0 + min(i / T::SLOTS, P - 1);
        const int o = 16 * (i % T::SLOTS);
        if (o < T::VOFF) {
            src_base[k] = reinterpret_cast<const char*>(a.kc) + head * a.cap * RB + o;
            src_stride[k] = RB;
        } else if (o < T::KSOFF) {
            src_base[k] = reinterpret_cast<const char*>(a.vc) + head * a.cap * RB + (o - T::VOFF);
            src_stride[k] = RB;
        } else if (o < T::VSOFF) {
            src_base[k] = reinterpret_cast<const char*>(a.ks + head * a.cap * NG) + (o - T::KSOFF);
            src_stride[k] = NG * 4;
        } else {
            src_base[k] = reinterpret_cast<const char*>(a.vs + head * a.cap * NG) + (o - T::VSOFF);
            src_stride[k] = NG * 4;
        }
    }
    constexpr int AH = kB2Ahead<D, P, HILO>;
    u32x4_t pf[AH][SG::LOADS];
    auto load_tile = [&](u32x4_t (&dst)[SG::LOADS], int it) {
        const int tok0 = start + it * kTile;
#pragma unroll
        for (int k = 0; k < SG::LOADS; ++k)
            if (src_on[k])
                dst[k] = __builtin_nontemporal_load(
                    reinterpret_cast<const u32x4_t*>(src_base[k] + (size_t)tok0 * src_stride[k]));
    };
#pragma unroll
    for (int k = 0; k < AH; ++k)
        if (wave + k * W < ntiles) load_tile(pf[k], wave + k * W);

    // ---- q: column n16 = query head hk0 G + n16, lane r holds channels
    //      32 g + 8 r + 0..7; scaled by 2^qk (largest |q| in [2^14, 2^15))
    float qx[NG][8];
    {
        const uint16_t* qsrc =
            static_cast<const uint16_t*>(a.q) + ((size_t)b * a.Hq + hk0 * G + (col_valid ? n16 : 0)) * D;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const uint4 raw = *reinterpret_cast<const uint4*>(qsrc + 32 * g + 8 * r);
            const uint32_t w4[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                qx[g][e] = col_valid ? widen((uint16_t)(w4[e / 2] >> (16 * (e % 2))), a.dtype) : 0.0f;
        }
    }
    // HILO (K rotated or channel-scaled): q rotated as K was (its signs, then
    // the cache's transform; rot_norm goes into qmul), then divided by K's
    // channel scale; such a q is not exact in fp16 and enters as hi + lo
    const bool rot = HILO && a.signs != nullptr;
    if constexpr (HILO) {
        if (rot) {
#pragma unroll
            for (int g = 0; g < NG; ++g)
#pragma unroll
                for (int e = 0; e < 8; ++e) qx[g][e] *= a.signs[32 * g + 8 * r + e];
            if constexpr (D == 192) {
                srft_query192(qx, r);  // the FFT kind only at this width
            } else {
                if (a.rot_kind) srft_query<NG>(qx, r);
                else fwht_query<NG>(qx, r);
            }
        }
        if (a.lam) {
#pragma unroll
            for (int g = 0; g < NG; ++g)
#pragma unroll
                for (int e = 0; e < 8; ++e) qx[g][e] = qx[g][e] / a.lam[32 * g + 8 * r + e];
        }
    }
    int qk = 0;
    {
        float qa = 0.0f;
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) qa = fmaxf(qa, fabsf(qx[g][e]));
        qa = max_xor32(max_xor16(qa));
        qk = qa > 0.0f ? 15 - __builtin_amdgcn_frexp_expf(qa) : 0;  // qa = f 2^e, f in [0.5, 1)
    }
    // B operands: k slot (2k, 2k + 1) = channels (8 r + k, 8 r + k + 4) of the
    // group, divided by the code's positional power of two (4^k at 2 bits,
    // kK3Exp at 3); the accumulator starts at -2^(b-1) * 2^-24 * sum(q over
    // the group).  With two KV heads per wave, head j's products take q
    // masked to its columns (qbj[j]), so both accumulate into one C.
    half8_t qb[NG], qbl[HILO ? NG : 1];
    floatx4_t qinit4[kB2QinitInAcc<D, P, HILO> ? NG : 1];
    float qinit1[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        float tq = 0.0f;
#pragma unroll
        for (int k = 0; k < 4; ++k)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const float xs = __builtin_ldexpf(qx[g][k + 4 * h], qk);
                const _Float16 v = (_Float16)xs;
                const int pe = BITS == 2 ? 2 * k : BITS == 3 ? kK3Exp[k] : 4 * (k & 1);
                qb[g][2 * k + h] = (_Float16)((float)v * __builtin_ldexpf(1.0f, -pe));
                tq += (float)v;
                if constexpr (HILO) {
                    const _Float16 lo = (_Float16)(xs - (float)v);
                    qbl[g][2 * k + h] = (_Float16)((float)lo * __builtin_ldexpf(1.0f, -pe));
                    tq += (float)lo;
                }
            }
        const float qi = -(float)(1 << (BITS - 1)) * 0x1p-24f * sum_xor32(sum_xor16(tq));
        if constexpr (kB2QinitInAcc<D, P, HILO>) qinit4[g] = floatx4_t{qi, qi, qi, qi};
        qinit1[g] = qi;
    }
    half8_t qbj[P][NG];
#pragma unroll
    for (int j = 0; j < P; ++j)
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const half8_t zero = {};
            qbj[j][g] = (P == 1 || jl == j) ? qb[g] : zero;
        }
    const float qmul = __builtin_ldexpf((rot ? a.qscale * a.rot_norm : a.qscale) * 0x1p24f, -qk);
    // 2 bits: the lane's K field is half r & 1 of word 2 g + r / 2 of a row;
    // 3 bits: it starts at bit 24 r of the group's three words
    const uint32_t ksel = (r & 1) ? 0x0C030C02u : 0x0C010C00u;
    const int k3w = (24 * r) >> 5, k3s = (24 * r) & 31;

    float m_run = kNegInf;  // softmax reference of column n16
    int e_v = 0;            // E (wave-uniform): the value operand carries 2^E
    float v_lim = 0.0f;     // V scales above this move E
    float l_lane = 0.0f;    // sum of this lane's probabilities (column n16)
    floatx4_t acc[P][NCB];  // per KV head: O[query head 4 r + i][channel 16 cb + n16]
#pragma unroll
    for (int j = 0; j < P; ++j)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[j][cb] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // one tile: its registers (rg) into the wave's stage, the tile AH rounds
    // ahead into rg, then the tile's products
    auto tile_step = [&](int it, u32x4_t (&rg)[SG::LOADS]) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < SG::LOADS; ++k)
            if (src_on[k]) *reinterpret_cast<u32x4_t*>(stage + 16 * (64 * k + lane)) = rg[k];
        if (it + AH * W < ntiles) load_tile(rg, it + AH * W);
        const int tok0 = start + it * kTile;

        // the scales of the lane's tokens 16 s + 4 r + i, group g, in its
        // column's KV head
        const float* ksc = reinterpret_cast<const float*>(stage + jl * T::BYTES + T::KSOFF);
        const float* vsc = reinterpret_cast<const float*>(stage + jl * T::BYTES + T::VSOFF);
        auto tok_of = [&](int s, int i) { return 16 * s + 4 * r + i; };
        // a token past the end (only in the split's last tile) counts as
        // absent: its score is -inf and its V scale 0 (set after the loads,
        // so that no load is predicated)
        const int nvalid = end - tok0;  // >= 32 but in the split's last tile
        const bool tail = nvalid < kTile;  // wave-uniform
        bool valid[2][4];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) valid[s][i] = tok_of(s, i) < nvalid;
        // the V scales of the lane's token 16 s + 4 r + slot (slot = lane % 4),
        // every group, zero past the end (whatever the cache holds there);
        // DPP quad broadcasts hand token 4 r + m's to the quad
        const int slot = lane & 3;
        float sv[2][NG];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const float* src = vsc + tok_of(s, slot) * NG;
            const bool in = !tail || tok_of(s, slot) < nvalid;
#pragma unroll
            for (int g = 0; g < NG; ++g) sv[s][g] = in ? src[g] : 0.0f;
        }

        // ---- scores T[s][i] (token 16 s + 4 r + i, column n16), / qmul
        float Tt[2][4];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            floatx4_t tot = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                floatx4_t d = kB2QinitInAcc<D, P, HILO> ? qinit4[kB2QinitInAcc<D, P, HILO> ? g : 0]
                                                  : floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int j = 0; j < P; ++j) {
                    const char* krow = stage + j * T::BYTES + T::KOFF + (16 * s + n16) * RB;
                    half8_t A;
                    if constexpr (BITS == 4) {  // quarter-interleaved int4 row: word r NG + g
                        A = unpack_codes_sub(*reinterpret_cast<const uint32_t*>(krow + 4 * (r * NG + g)));
                    } else if constexpr (BITS == 2) {
                        A = unpack_k2(*reinterpret_cast<const uint32_t*>(krow + 4 * (2 * g + (r >> 1))), ksel);
                    } else {
                        // the word after the field's first lies inside the stage
                        // even for the tile's last row (the V tile follows)
                        const uint32_t* kw = reinterpret_cast<const uint32_t*>(krow) + 3 * g + k3w;
                        A = unpack_k3(__builtin_amdgcn_alignbit(kw[1], kw[0], k3s));
                    }
                    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qbj[j][g], d, 0, 0, 0);
                    if constexpr (HILO) d = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qbl[g], d, 0, 0, 0);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float di = kB2QinitInAcc<D, P, HILO> ? d[i] : d[i] + qinit1[g];
                    const float term = ksc[tok_of(s, i) * NG + g] * di;
                    tot[i] = (g == 0) ? term : tot[i] + term;
                }
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) Tt[s][i] = tot[i];
        }
        if (tail) {
#pragma unroll
            for (int s = 0; s < 2; ++s)
#pragma unroll
                for (int i = 0; i < 4; ++i) Tt[s][i] = valid[s][i] ? Tt[s][i] : kNegInf;
        }

        // ---- online softmax of column n16 (base 2), reference with headroom
        float mt = kNegInf;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) mt = fmaxf(mt, Tt[s][i]);
        mt = max_xor32(max_xor16(mt)) * qmul;  // finite: the tile has a valid token
        // the largest V scale of the lane's tokens (whatever the cache holds
        // past the end is left out)
        float svm = 0.0f;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int g = 0; g < NG; ++g) svm = fmaxf(svm, sv[s][g]);
        const bool vmove = __any(svm > v_lim);
        if (__any(mt > m_run) || vmove) {
            const float m_new = (mt > m_run) ? mt + kHeadroom : m_run;
            int e_new = e_v;
            if (vmove) {  // wave-uniform: E from the wave's largest V scale
                const int ve = __builtin_amdgcn_frexp_expf(group_max<64>(svm));
                const int en = min(max(kVTarget - ve, kEMin), kEMax);
                e_new = en;
                v_lim = __builtin_ldexpf(1.0f, kVLimit - en);
            }
            const float alpha = exp2_approx(m_run - m_new);  // 0 on the first tile
            const float alpha_o = __builtin_ldexpf(alpha, e_new - e_v);
            l_lane *= alpha;
            static_for<4>([&](auto iI) {
                constexpr int i = decltype(iI)::value;
                const float ai = row_quad_gather<i>(alpha_o, r);  // of column 4 r + i
#pragma unroll
                for (int j = 0; j < P; ++j)
#pragma unroll
                    for (int cb = 0; cb < NCB; ++cb) acc[j][cb][i] *= ai;
            });
            m_run = m_new;
            e_v = e_new;
        }
        // the tile's V scales carry 2^E (exact)
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int g = 0; g < NG; ++g) sv[s][g] = __builtin_ldexpf(sv[s][g], e_v);
        // p of the lane's tokens; the V codes of slot pair i carry
        // 2^kVExp<BITS>[i], taken off p here (exact), after l has taken p
        float p[2][4];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float pf = exp2_approx(__builtin_fmaf(Tt[s][i], qmul, -m_run));
                l_lane += pf;
                p[s][i] = kVExp<BITS>[i] ? __builtin_ldexpf(pf, -kVExp<BITS>[i]) : pf;
            }

        // ---- values: the lane's words of the V tile (channel column n16 of
        //      every block, tokens 4 r + m and 16 + 4 r + m in the two halves)
        constexpr int VW = BITS == 4 ? NCB : VT::WPL;  // words per lane and head
        uint32_t vw[P][VW];
#pragma unroll
        for (int j = 0; j < P; ++j) {
            const char* src = stage + j * T::BYTES + T::VOFF + lane * 4 * VT::WPL;
            if constexpr (BITS == 4) {  // int4 V tile: block cb = 4 a + b in word ((4 a + r) 16 + n) 4 + b
#pragma unroll
                for (int a4 = 0; a4 < NCB / 4; ++a4) {
                    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(stage + j * T::BYTES + T::VOFF +
                                                                         16 * ((a4 * 4 + r) * 16 + n16));
                    vw[j][4 * a4] = w.x; vw[j][4 * a4 + 1] = w.y; vw[j][4 * a4 + 2] = w.z; vw[j][4 * a4 + 3] = w.w;
                }
            } else if constexpr (VT::WPL % 4 == 0) {
#pragma unroll
                for (int k = 0; k < VT::WPL; k += 4) {
                    const u32x4_t w = *reinterpret_cast<const u32x4_t*>(src + 4 * k);
                    vw[j][k] = w.x; vw[j][k + 1] = w.y; vw[j][k + 2] = w.z; vw[j][k + 3] = w.w;
                }
            } else if constexpr (VT::WPL % 2 == 0) {
#pragma unroll
                for (int k = 0; k < VT::WPL; k += 2) {
                    const uint2 w = *reinterpret_cast<const uint2*>(src + 4 * k);
                    vw[j][k] = w.x; vw[j][k + 1] = w.y;
                }
            } else {
#pragma unroll
                for (int k = 0; k < VT::WPL; ++k) vw[j][k] = reinterpret_cast<const uint32_t*>(src)[k];
            }
        }
        static_for<NG>([&](auto gI) {
            constexpr int g = decltype(gI)::value;  // scale group: channel blocks 2 g, 2 g + 1
            v4u_t ha, la;
            static_for<4>([&](auto mI) {
#pragma clang fp contract(off)
                constexpr int m = decltype(mI)::value;
                // one product per element, consumed by both halves, so the
                // broadcast folds into v_mul_f32_dpp
                const float x0 = p[0][m] * quad_bcast<m>(sv[0][g]);
                const float x1 = p[1][m] * quad_bcast<m>(sv[1][g]);
                ha[m] = __builtin_bit_cast(uint32_t, half2_t{(_Float16)x0, (_Float16)x1});
                la[m] = lo_pair<m == 3>(x0, x1, ha[m]);
            });
            const half8_t pa = __builtin_bit_cast(half8_t, ha), pl = __builtin_bit_cast(half8_t, la);
#pragma unroll
            for (int j = 0; j < P; ++j) {
                static_for<2>([&](auto hI) {
                    constexpr int cb = 2 * g + decltype(hI)::value;
                    half8_t B;
                    if constexpr (BITS == 4) {
                        B = unpack_codes_signed(vw[j][cb]);
                    } else if constexpr (BITS == 2) {
                        B = unpack_v2((cb & 1) ? (vw[j][cb >> 1] >> 8) : vw[j][cb >> 1]);
                    } else {
                        constexpr int qd = cb >> 2, t = cb & 3;
                        if constexpr (t < 3) {
                            B = unpack_v3(vw[j][3 * qd + t]);
                        } else {  // the block held in the top nibbles of the quad's words
                            B = unpack_v3(((vw[j][3 * qd] >> 12) & 0x000F000Fu) |
                                          ((vw[j][3 * qd + 1] >> 8) & 0x00F000F0u) |
                                          ((vw[j][3 * qd + 2] >> 4) & 0x0F000F00u));
                        }
                    }
                    acc[j][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, B, acc[j][cb], 0, 0, 0);
                    acc[j][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl, B, acc[j][cb], 0, 0, 0);
                });
            }
        });
    };
    // the register sets in turn, each index fixed at compile time
    for (int it = wave; it < ntiles; it += AH * W) {
        tile_step(it, pf[0]);
        static_for<AH - 1>([&](auto kI) {
            constexpr int k = decltype(kI)::value + 1;
            if (it + k * W < ntiles) tile_step(it + k * W, pf[k]);
        });
    }

    // ---- merge of the W waves (each writes its share into its own stage,
    //      which it no longer reads), then the block's partial
    auto merge_o = [&](int w) { return reinterpret_cast<float*>(lds + w * SG::BYTES); };
    auto merge_ml = [&](int w) { return reinterpret_cast<float2*>(merge_o(w) + 16 * T::RS); };
    const float L = sum_xor32(sum_xor16(l_lane));
    // acc carries 2^E: (M - F, l 2^F, acc 2^(F - E)) with F = floor(E / 2)
    // keeps both sums inside fp32's range
    const int f_e = e_v >> 1;
    if (lane < 16) merge_ml(wave)[lane] = make_float2(m_run - (float)f_e, __builtin_ldexpf(L, f_e));
    float* own = merge_o(wave);
    // rows 4 r .. 4 r + 3 lie in one KV head (two heads per wave only when
    // G >= 4): keep that head's accumulators
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
                own[h * T::RS + 16 * cb + n16] = __builtin_ldexpf(v, f_e - e_v);
            }
        }
    }
    __syncthreads();
    constexpr int kMergeIters = (16 * (D / 4) + 64 * W - 1) / (64 * W);
#pragma unroll
    for (int k = 0; k < kMergeIters; ++k) {
        const int i = tid + k * 64 * W;
        if (i >= PG * (D / 4)) break;
        const int h = i / (D / 4), c = 4 * (i % (D / 4));
        float2 ml[W];
        float Mb = kNegInf;
#pragma unroll
        for (int w = 0; w < W; ++w) {  // a wave without tiles left m = -inf, l = 0, O = 0
            ml[w] = merge_ml(w)[h];
            Mb = fmaxf(Mb, ml[w].x);
        }
        float4 o = {0.0f, 0.0f, 0.0f, 0.0f};
        float Ls = 0.0f;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const float f = (ml[w].x == kNegInf) ? 0.0f : exp2_approx(ml[w].x - Mb);
            const float4 x = *reinterpret_cast<const float4*>(merge_o(w) + h * T::RS + c);
            o.x += f * x.x; o.y += f * x.y; o.z += f * x.z; o.w += f * x.w;
            Ls += f * ml[w].y;
        }
        const size_t prow = ((size_t)b * a.Hq + hk0 * G + h) * a.num_splits + split;
        *reinterpret_cast<float4*>(a.part_o + prow * D + c) = o;
        if (c == 0) a.part_ml[prow] = make_float2(Mb, Ls);
    }
}

}  // namespace

// KV heads per wave: two (filling 16 MFMA columns at G = 8) when 4 <= G <= 8,
// the head count is even and the registers suffice (head_dim 64 or 128),
// else one.
int split_bits_mfma_heads_per_wave(int D, int G, int H, bool hilo)
{
    if (hilo) return 1;  // the hi + lo query takes the registers of a second head
    return (D != 256 && D != 192 && G >= 4 && G <= 8 && H % 2 == 0) ? 2 : 1;
}

bool split_bits_mfma_supports(int D, int G, int bits, bool rotated_k, bool scaled_k)
{
    if (G < 1 || G > 16) return false;
    // int4 codes at head_dim 192 (a rotated K there is FFT-rotated)
    if (D == 192) return bits == 4;
    // a rotated or channel-scaled K (hi + lo query) up to head_dim 128, whose
    // registers leave room for it
    return (D == 64 || D == 128 || D == 256) && (bits == 2 || bits == 3) && !((rotated_k || scaled_k) && D == 256);
}

namespace {

template <int D, int BITS, int P, bool HILO>
hipError_t launch_bp(const SplitArgs& a, hipStream_t stream)
{
    const size_t lds = (size_t)kB2Waves * BStage<D, BITS, P>::BYTES;
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&split_bits_mfma_kernel<D, BITS, P, HILO>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (attr != hipSuccess) return attr;
    dim3 grid(a.num_splits, a.H / P, a.B), block(64 * kB2Waves);
    split_bits_mfma_kernel<D, BITS, P, HILO><<<grid, block, lds, stream>>>(a);
    return hipGetLastError();
}

template <int D, int BITS>
hipError_t launch_b(const SplitArgs& a, hipStream_t stream)
{
    if constexpr (D != 256) {
        if (a.signs || a.lam) return launch_bp<D, BITS, 1, true>(a, stream);
    }
    if constexpr (D != 256 && D != 192) {
        if (split_bits_mfma_heads_per_wave(D, a.Hq / a.H, a.H, false) == 2)
            return launch_bp<D, BITS, 2, false>(a, stream);
    }
    return launch_bp<D, BITS, 1, false>(a, stream);
}

}  // namespace

hipError_t launch_split_bits_mfma(const SplitArgs& a, int bits, hipStream_t stream)
{
    if (((a.signs || a.lam) && a.D == 256) || (a.signs && a.D == 192 && a.rot_kind != 1) || a.Hq / a.H > 16 ||
        (a.D == 192) != (bits == 4))
        return hipErrorInvalidValue;
    switch (a.D * 10 + bits) {
    case 642: return launch_b<64, 2>(a, stream);
    case 643: return launch_b<64, 3>(a, stream);
    case 1282: return launch_b<128, 2>(a, stream);
    case 1283: return launch_b<128, 3>(a, stream);
    case 2562: return launch_b<256, 2>(a, stream);
    case 2563: return launch_b<256, 3>(a, stream);
    case 1924: return launch_b<192, 4>(a, stream);  // int4 codes at head_dim 192
    default: return hipErrorInvalidValue;
    }
}

}  // namespace otq
