// sdpa_mfma.hip - split pass of decode attention on the packed int4 cache,
// MFMA variant (any G = query heads per KV head up to 16).
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
//  * K codes enter the score MFMAs as fp16 subnormals of their offset-binary
//    value n = c + 8: a nibble left at bit 0 (or bit 4) of a 16-bit half
//    reads as n * 2^-24 (or n * 2^-20), so one shift and four masks give all
//    eight operands of a 32-bit word; the 2^4 of the bit-4 nibbles is
//    cancelled exactly by a power of two on the q operand, the +8 by starting
//    the score accumulator at -8 * 2^-24 * sum(q) (a shift shared by every
//    token of a query head's score), and 2^24 is folded into the softmax
//    scale.  The score's rounding is per token and does not accumulate;
//  * V codes enter the value MFMAs as signed normal fp16 integers: a
//    nibble's offset-binary value goes into the mantissa of 1024.0 (whose
//    ulp is 1) and one packed fp16 subtraction per pair leaves c (or 16 c for
//    a bit-4 nibble) exactly, so every value product is exact and the sums
//    are plain fp32: no offset term whose rounding would grow with the
//    context (the 16 of the bit-4 nibbles is cancelled on p);
//  * q is converted to fp16 after each query head's row is scaled by a power
//    of two that puts its largest |element| in [2^14, 2^15) (bf16 inputs of
//    any magnitude fit, and the factor is undone in the softmax scale); bf16
//    values then convert exactly; a rotated q (or one divided by K's
//    per-channel scale) is split into fp16 hi + lo parts and both are
//    multiplied, so the score keeps ~22 bits of q;
//  * the per-token, per-group K scale is applied in fp32 after the MFMA,
//    since one MFMA of K = 32 covers exactly one scale group;
//  * for P.V the V scale depends on the contracted token, so it is folded
//    into the probability operand, x = p * s_v in fp32, and x enters as two
//    fp16 MFMA operands hi = fp16(x), lo = fp16(x - hi) (~22 significant
//    bits); fp16(x) alone (2^-11 relative) is too coarse when a handful of
//    tokens carry the softmax and a channel is an outlier.  p carries a
//    power of two 2^E chosen from the largest V scale seen so far (moved like
//    the softmax reference, and folded into it), so that x stays inside
//    fp16's normal range for V of any magnitude.
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
//          lies inside one head: two heads per wave only when G >= 4).
// With G < 16 and one KV head per wave, columns G..15 are idle: the matrix
// cores have room to spare, while the VALU work per token (unpacking, scale
// products) is the same as for full columns and far below that of
// per-channel fp32 dot products.
#include <math.h>

#include "common.hpp"
#include "kernels.hpp"
#include "mfma_common.hpp"
#include "srft.hpp"

namespace otq {

namespace {

using namespace mfma;

// s_waitcnt lgkmcnt(0) with the vector-memory and export counters left
// unconstrained (gfx9 encoding: vmcnt [3:0] + [15:14], expcnt [6:4],
// lgkmcnt [11:8]).
constexpr int kWaitLgkm0 = 0xC07F;
// s_waitcnt vmcnt(N) with the other counters unconstrained.
constexpr int wait_vm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
constexpr int kWaitVm0 = wait_vm(0);

// Buffer resource (4 SGPRs): base, no stride, size in bytes, 32-bit data
// format; reads past the size return 0.
typedef int v4i_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ v4i_t make_rsrc(const void* base, uint32_t bytes)
{
    const uint64_t p = reinterpret_cast<uint64_t>(base);
    return v4i_t{(int)(uint32_t)p, (int)((p >> 32) & 0xFFFF), (int)bytes, 0x00020000};
}

// Direct buffer -> LDS copy of 16 bytes per lane: lane l reads the resource
// at voffset + soffset and its bytes land at LDS address lds_addr + 16 l
// (every operand but voffset wave-uniform).  Issued as inline asm (M0, the
// LDS base, saved and restored around it) so that the compiler does not
// follow it with a wait for every copy in flight before each later LDS read;
// the kernel waits on the vector-memory counter itself, one tile at a time,
// which lets a second tile stream in while the first is consumed.
typedef __attribute__((address_space(3))) char lds_char_t;
__device__ __forceinline__ uint32_t lds_address(void* p)
{
    return (uint32_t)(uintptr_t)(lds_char_t*)p;
}
// All copies of one tile in one asm statement.  M0 (the LDS destination
// base) is saved once and restored at the end; each run of 1 KB pieces of
// one head and array shares one lane offset and one M0 value and steps by the
// instruction's offset field, which moves the global and the LDS address
// alike.  The V-scale resource starts 1 KB before the V scales, so that its
// piece lands 1 KB after the K-scale piece under the same M0.  At one wave
// per SIMD every instruction costs an issue slot: this takes 2 + 2 runs + the
// copies, against 5 per copy with M0 saved around each.
#define OTQ_M0(M) "s_mov_b32 m0, %[" M "]\n\ts_nop 0\n\t"
// nt: the cache streams through once per step, so its lines are marked
// non-temporal (measured on workload 3: the split from 34.4 to 32.2 us).
#define OTQ_LD(VO, RS, SO, OFF) "buffer_load_dwordx4 %[" VO "], %[" RS "], %[" SO "] offen offset:" OFF " nt lds\n\t"
#define OTQ_RUN1(M, VO, RS) OTQ_M0(M) OTQ_LD(VO, RS, "soc", "0")
#define OTQ_RUN2(M, VO, RS) OTQ_RUN1(M, VO, RS) OTQ_LD(VO, RS, "soc", "1024")
#define OTQ_RUN4(M, VO, RS) OTQ_RUN2(M, VO, RS) OTQ_LD(VO, RS, "soc", "2048") OTQ_LD(VO, RS, "soc", "3072")
#define OTQ_SCALES OTQ_M0("ms") OTQ_LD("vs", "rks", "sos", "0") OTQ_LD("vs", "rvs", "sos", "1024")
#define OTQ_DMA_OPS                                                                     \
    : [sv] "=&s"(saved)                                                                 \
    : [vk0] "v"(vk[0]), [vk1] "v"(vk[P - 1]), [vv0] "v"(vv[0]), [vv1] "v"(vv[P - 1]),  \
      [vs] "v"(vs), [rk] "s"(rk), [rv] "s"(rv), [rks] "s"(rks), [rvs] "s"(rvs),        \
      [soc] "s"(so_code), [sos] "s"(so_scale), [mk0] "s"(mk[0]), [mk1] "s"(mk[P - 1]), \
      [mv0] "s"(mv[0]), [mv1] "s"(mv[P - 1]), [ms] "s"(ms)                             \
    : "memory"
template <int NA, int P>
__device__ __forceinline__ void dma_tile_asm(const v4i_t& rk, const v4i_t& rv, const v4i_t& rks,
                                             const v4i_t& rvs, const int (&vk)[P], const int (&vv)[P],
                                             int vs, int so_code, int so_scale, const uint32_t (&mk)[P],
                                             const uint32_t (&mv)[P], uint32_t ms)
{
    int saved;
    if constexpr (NA == 1 && P == 1) {
        asm volatile("s_mov_b32 %[sv], m0\n\t" OTQ_RUN1("mk0", "vk0", "rk") OTQ_RUN1("mv0", "vv0", "rv")
                     OTQ_SCALES "s_mov_b32 m0, %[sv]" OTQ_DMA_OPS);
    } else if constexpr (NA == 1 && P == 2) {
        asm volatile("s_mov_b32 %[sv], m0\n\t" OTQ_RUN1("mk0", "vk0", "rk") OTQ_RUN1("mk1", "vk1", "rk")
                     OTQ_RUN1("mv0", "vv0", "rv") OTQ_RUN1("mv1", "vv1", "rv")
                     OTQ_SCALES "s_mov_b32 m0, %[sv]" OTQ_DMA_OPS);
    } else if constexpr (NA == 2 && P == 1) {
        asm volatile("s_mov_b32 %[sv], m0\n\t" OTQ_RUN2("mk0", "vk0", "rk") OTQ_RUN2("mv0", "vv0", "rv")
                     OTQ_SCALES "s_mov_b32 m0, %[sv]" OTQ_DMA_OPS);
    } else if constexpr (NA == 2 && P == 2) {
        asm volatile("s_mov_b32 %[sv], m0\n\t" OTQ_RUN2("mk0", "vk0", "rk") OTQ_RUN2("mk1", "vk1", "rk")
                     OTQ_RUN2("mv0", "vv0", "rv") OTQ_RUN2("mv1", "vv1", "rv")
                     OTQ_SCALES "s_mov_b32 m0, %[sv]" OTQ_DMA_OPS);
    } else {
        static_assert(NA == 4 && P == 1, "tiles: head_dim 64 or 128 with one or two heads, 256 with one");
        asm volatile("s_mov_b32 %[sv], m0\n\t" OTQ_RUN4("mk0", "vk0", "rk") OTQ_RUN4("mv0", "vv0", "rv")
                     OTQ_SCALES "s_mov_b32 m0, %[sv]" OTQ_DMA_OPS);
    }
}
#undef OTQ_DMA_OPS
#undef OTQ_SCALES
#undef OTQ_RUN4
#undef OTQ_RUN2
#undef OTQ_RUN1
#undef OTQ_LD
#undef OTQ_M0

// One tile of the P KV heads, staged in LDS:
//  [K_0 .. K_{P-1}][V_0 .. V_{P-1}][scales]
// K_j: 32 rows x D/2 bytes as 16-byte chunks, chunk c of row t at slot
//      k_slot(t, c) (a rotation within the row that spreads the 16 lanes
//      reading one quarter over distinct banks);
// V_j: the V tile as stored in memory;
// scales: [K, V][head][32 tokens][D/32] fp32.
template <int D, int P>
struct Stage {
    static constexpr int KB = 16 * D;               // K or V bytes per head per tile
    static constexpr int SRAW = P * 4 * D;          // K (or V) scale bytes, all heads
    static constexpr int SPAD = SRAW < 1024 ? 1024 : SRAW;
    static constexpr int BYTES = 2 * P * KB + 2 * SPAD;
    static constexpr int koff(int j) { return j * KB; }
    static constexpr int voff(int j) { return (P + j) * KB; }
    static constexpr int KSOFF = 2 * P * KB;        // K scales [head][32 tokens][D/32]
    static constexpr int VSOFF = KSOFF + SPAD;      // V scales, same layout
    // copy instructions per tile (one per 1 KB)
    static constexpr int COPIES = 2 * P * (D / 64) + 2 * (SPAD / 1024);
};

template <int D>
__device__ __forceinline__ int k_slot(int t, int c)
{
    if constexpr (D == 128) return 4 * t + ((c + (t >> 2)) & 3);
    else if constexpr (D == 256) return 8 * t + (c ^ (((t >> 1) & 3) << 1));
    else return 2 * t + c;
}
template <int D>
__device__ __forceinline__ void k_unslot(int slot, int& t, int& c)
{
    if constexpr (D == 128) {
        t = slot >> 2;
        c = ((slot & 3) - (t >> 2)) & 3;
    } else if constexpr (D == 256) {
        t = slot >> 3;
        c = (slot & 7) ^ (((t >> 1) & 3) << 1);
    } else {
        t = slot >> 1;
        c = slot & 1;
    }
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

// One tile's loads for the P KV heads of the block.  K scales: with ROWS,
// those of tokens 4 r + 0..3 of the lane's head (every lane of a row reads
// the same 16 bytes, so no broadcast instruction is needed); otherwise only
// token 4 r + (lane % 4), handed out by DPP quad broadcasts (fewer registers).
template <int D, int P, bool ROWS>
struct TileLoads {
    static constexpr int NG = D / kGroup;
    uint32_t kw[P][2][NG];       // K code words: head, sub-tile, group
    uint4 vw[P][D / 64];         // V tile words: head, 128-bit load
    float sk[2][ROWS ? 4 : 1][NG];
    float sv[2][NG];             // V scales of token 4 r + (lane % 4)
};

// HILO: the query is not exact in fp16 (a rotated cache, or K's per-channel
// scale divides it), so each q operand is an fp16 hi + lo pair and every
// score MFMA is issued twice.
//
// K scales loaded per row where the registers allow it: not at head_dim 256
// (eight groups per token) nor for two heads with hi + lo q operands, which
// already fill the register file.
template <int D, int P, bool HILO>
constexpr bool kScaleRows = D <= 128 && !(HILO && P == 2);

// Waves per SIMD the register allocation must allow: 2 (up to 256 VGPRs),
// so that a second block on the CU can hide the first one's latencies.
template <int D>
constexpr int kWavesPerEU = 2;

// Where the score accumulator starts at the offset correction (a register
// quad per group, live through the loop) rather than taking it after the
// MFMA (four adds per group and sub-tile): everywhere but head_dim 256 with
// hi + lo q operands, whose registers are full.
template <int D, bool HILO>
constexpr bool kQinitInAcc = !(D == 256 && HILO);

// Whether the query prologue loads K's channel scales together with q and the
// rotation signs (before the first tile's copies), or only once the rotation
// is done: at head_dim 256 the three sets (192 registers) do not fit beside
// each other.
template <int D>
constexpr bool kLamEarly = D < 256;

// LDS stages per wave: two where the copies a block keeps in flight stay
// within 80 KB, else one (measured: deeper queues per CU slow the stream).
template <int D, int P, int W>
constexpr int kStages = 2 * W * Stage<D, P>::BYTES <= 80 * 1024 ? 2 : 1;

template <int D, int P, bool HILO, int W>
__global__ __launch_bounds__(64 * W) __attribute__((amdgpu_waves_per_eu(kWavesPerEU<D>)))
void split_mfma_kernel(SplitArgs a)
{
    constexpr int NG = D / kGroup, NA = D / 64, NCB = D / 16;
    extern __shared__ float lds[];  // per-wave tile stages; then the merge

    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar loop control
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
    const int start = split * a.chunk;
    // first token of the block's tile it (its pieces interleave with the
    // other splits' at piece_stride; one piece: start + 32 it)
    const int pshift = a.piece_shift;
    auto tile_tok = [&](int it) {
        return start + (it >> pshift) * a.piece_stride + (it & ((1 << pshift) - 1)) * kTile;
    };
    const int n16 = lane & 15, r = lane >> 4, slot = lane & 3;
    const bool col_valid = n16 < PG;
    const int jl = col_valid ? n16 / G : P - 1;  // KV head of this lane's column

    using St = Stage<D, P>;
    constexpr int NST = kStages<D, P, W>;
    constexpr bool ROWS = kScaleRows<D, P, HILO>;
    static_assert((NST - 1) * St::COPIES <= 63, "vmcnt holds at most 63");
    const size_t head0 = (size_t)b * a.H + hk0;
    // the wave's LDS stages, contiguous per wave: stage s of wave w at
    // (w NST + s) * BYTES; after its last tile a wave's stages hold its
    // share of the merge
    auto stage_of = [&](int st) { return reinterpret_cast<char*>(lds) + (wave * NST + st) * St::BYTES; };

    // sequence length first, as a scalar load: nothing has been written yet
    // lens clamped to [0, max_len] first, as the combine does, then the
    // fused append's token (lens_offset = 1) left to the combine
    const int raw_len = a.lens[b];
    const int len = max(min(max(raw_len, 0), a.max_len) - a.lens_offset, 0);
    if (tid == 0 && split == 0 && hk0 == 0 && (raw_len < 0 || raw_len > a.max_len)) report_error(a.err, kErrLens);

    // ---- q straight into registers, before any tile copy is queued: lane
    //      (n16, r) needs, per scale group g, channels 32 g + 8 r + 0..7 of
    //      query head n16 (one 16-byte load), and the same signs when rotated
    //      and channel scales when K has them; lanes of unused columns load
    //      head 0 of the block and drop it
    const bool rot = a.signs != nullptr, scaled = a.lam != nullptr;  // HILO when either holds
    uint4 qraw[NG];
    float4 sgn[HILO ? NG : 1][2], lmv[HILO ? NG : 1][2];
    {
        const uint16_t* qsrc =
            static_cast<const uint16_t*>(a.q) + ((size_t)b * a.Hq + hk0 * G + (col_valid ? n16 : 0)) * D;
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            qraw[g] = *reinterpret_cast<const uint4*>(qsrc + 32 * g + 8 * r);
            if constexpr (HILO) {
                if (rot) {
                    sgn[g][0] = *reinterpret_cast<const float4*>(a.signs + 32 * g + 8 * r);
                    sgn[g][1] = *reinterpret_cast<const float4*>(a.signs + 32 * g + 8 * r + 4);
                }
                if (kLamEarly<D> && scaled) {
                    lmv[g][0] = *reinterpret_cast<const float4*>(a.lam + 32 * g + 8 * r);
                    lmv[g][1] = *reinterpret_cast<const float4*>(a.lam + 32 * g + 8 * r + 4);
                }
            }
        }
    }

    // Buffer resources of the block's P heads (K codes, V tiles, K and V
    // scales); each spans exactly those heads, so no copy can leave them.
    const v4i_t rs_k = make_rsrc(a.kc + head0 * a.cap * (D / 2), P * a.cap * (D / 2));
    const v4i_t rs_v = make_rsrc(a.vc + head0 * a.cap * (D / 2), P * a.cap * (D / 2));
    const v4i_t rs_ks = make_rsrc(a.ks + head0 * a.cap * NG, P * a.cap * NG * 4);
    static_assert(St::SPAD == 1024, "one 1 KB piece per scale array");
    const v4i_t rs_vs = make_rsrc(reinterpret_cast<const char*>(a.vs + head0 * a.cap * NG) - 1024,
                                  P * a.cap * NG * 4 + 1024);
    // per-lane byte offsets of each copy instruction (tile-independent; the
    // tile enters as the scalar offset tok0 * D/2, or tok0 * D/8 for scales).
    // Piece i of one head and array lies 1024 i bytes after piece 0 both in
    // memory and in LDS (k_unslot keeps the rotation of a row when its token
    // moves by 16 or 8), which the copy runs rely on.
    int vo_k[P][D / 64], vo_v[P][D / 64], vo_s;
#pragma unroll
    for (int j = 0; j < P; ++j)
#pragma unroll
        for (int i = 0; i < D / 64; ++i) {
            int t, c;
            k_unslot<D>(64 * i + lane, t, c);
            vo_k[j][i] = j * a.cap * (D / 2) + t * (D / 2) + 16 * c;
            vo_v[j][i] = j * a.cap * (D / 2) + 1024 * i + 16 * lane;
        }
    {
        const int o = (16 * lane) % St::SRAW;  // lanes past the scale bytes repeat them
        vo_s = (o / (4 * D)) * a.cap * NG * 4 + o % (4 * D);
    }

    // issue the St::COPIES direct-to-LDS copies of tile it into stage st
    // (no registers held)
    int vk0[P], vv0[P];
#pragma unroll
    for (int j = 0; j < P; ++j) { vk0[j] = vo_k[j][0]; vv0[j] = vo_v[j][0]; }
    auto dma_tile = [&](int it, int st) {
        const int tok0 = tile_tok(it);
        const int so_code = tok0 * (D / 2), so_scale = tok0 * NG * 4;
        const uint32_t base = lds_address(stage_of(st));
        uint32_t mk[P], mv[P];
#pragma unroll
        for (int j = 0; j < P; ++j) { mk[j] = base + St::koff(j); mv[j] = base + St::voff(j); }
        dma_tile_asm<D / 64, P>(rs_k, rs_v, rs_ks, rs_vs, vk0, vv0, vo_s, so_code, so_scale, mk, mv,
                                base + St::KSOFF);
    };

    // The first tile of every wave streams in without waiting for lens[b] to
    // arrive, if it lies inside the cache (capacity is a multiple of 32, so a
    // tile starting below it is whole); tokens past lens[b] are masked later,
    // or the block leaves.
    if (tile_tok(wave) < a.cap) dma_tile(wave, 0);
    if (start >= len) {  // block-uniform: no partial for an empty split
        __builtin_amdgcn_s_waitcnt(kWaitVm0);  // no copy may land after the block is gone
        return;
    }
    // tiles of the split: with one piece, those of [start, min(start + chunk,
    // len)); with interleaved pieces, whole rounds of S pieces and the part
    // of the last round that falls to this split
    int ntiles;
    {
        const int nt = (len + kTile - 1) / kTile;  // tiles of the sequence
        if (pshift >= 30) {
            ntiles = (min(start + a.chunk, len) - start + kTile - 1) / kTile;
        } else {
            const int tpp = 1 << pshift, round = a.num_splits << pshift;
            const int full = nt / round, rest = nt - full * round;
            ntiles = full * tpp + min(max(rest - split * tpp, 0), tpp);
        }
    }
    const int end = len;  // only the sequence's last tile can be partial

    // ---- q prologue, registers only: widen, rotate like K when the cache
    //      is (channel c = 32 g + 8 r + e: the butterflies over bits 0-2 and
    //      5.. stay in the lane, bits 3 and 4 pair lanes 16 and 32 apart; the
    //      stages of a Walsh-Hadamard transform commute), then divide by K's
    //      channel scales when it has them
    float qx[NG][8];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const uint32_t w4[4] = {qraw[g].x, qraw[g].y, qraw[g].z, qraw[g].w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const uint16_t h16 = (uint16_t)(w4[e / 2] >> (16 * (e % 2)));
            qx[g][e] = col_valid ? widen(h16, a.dtype) : 0.0f;
        }
    }
    if (HILO && rot && a.rot_kind) {
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const float sg[8] = {sgn[g][0].x, sgn[g][0].y, sgn[g][0].z, sgn[g][0].w,
                                 sgn[g][1].x, sgn[g][1].y, sgn[g][1].z, sgn[g][1].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) qx[g][e] *= sg[e];
        }
        srft_query<NG>(qx, r);
    } else if (HILO && rot) {
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const float sg[8] = {sgn[g][0].x, sgn[g][0].y, sgn[g][0].z, sgn[g][0].w,
                                 sgn[g][1].x, sgn[g][1].y, sgn[g][1].z, sgn[g][1].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) qx[g][e] *= sg[e];
        }
        fwht_query<NG>(qx, r);
    }
    if (HILO && scaled) {
        if constexpr (!kLamEarly<D>) {
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                lmv[g][0] = *reinterpret_cast<const float4*>(a.lam + 32 * g + 8 * r);
                lmv[g][1] = *reinterpret_cast<const float4*>(a.lam + 32 * g + 8 * r + 4);
            }
        }
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            const float lm[8] = {lmv[g][0].x, lmv[g][0].y, lmv[g][0].z, lmv[g][0].w,
                                 lmv[g][1].x, lmv[g][1].y, lmv[g][1].z, lmv[g][1].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) qx[g][e] = qx[g][e] / lm[e];
        }
    }
    // Each query head's row is scaled by a power of two 2^qk that puts its
    // largest |element| in [2^14, 2^15): any bf16 row then fits fp16's range,
    // and a row of small values keeps its bits instead of turning subnormal.
    // The factor is exact and is undone in qmul.  The row's channels are
    // spread over the lanes of column n16 (r = lane / 16).
    int qk = 0;
    {
        float qa = 0.0f;
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) qa = fmaxf(qa, fabsf(qx[g][e]));
        qa = max_xor32(max_xor16(qa));
        qk = qa > 0.0f ? 15 - __builtin_amdgcn_frexp_expf(qa) : 0;  // qa = f 2^e, f in [0.5, 1)
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int e = 0; e < 8; ++e) qx[g][e] = __builtin_ldexpf(qx[g][e], qk);
    }
    // B operands of the score MFMAs, one per KV head: column n16 holds q of
    // query head n16 in the set of head jl and zeros in the others; k slot e
    // = channel 32 g + 8 r + kSlot[e].
    half8_t qb[P][NG], qb_lo[HILO ? P : 1][HILO ? NG : 1];
    floatx4_t qinit4[kQinitInAcc<D, HILO> ? NG : 1];
    float qinit1[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        half8_t hv, lv;
        float tq = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = qx[g][kSlot[e]];
            const _Float16 h16 = (_Float16)x;
            const _Float16 l16 = (_Float16)(x - (float)h16);
            // cancel the code's 2^kShift (a power of two)
            const float down = kShift[e] ? 0.0625f : 1.0f, up = kShift[e] ? 16.0f : 1.0f;
            hv[e] = (_Float16)((float)h16 * down);
            tq += (float)hv[e] * up;
            if (HILO) {
                lv[e] = (_Float16)((float)l16 * down);
                tq += (float)lv[e] * up;
            }
        }
        // the score accumulator starts at -8 * 2^-24 * sum(q over the group)
        const float qi = -8.0f * 0x1p-24f * sum_xor32(sum_xor16(tq));
        if constexpr (kQinitInAcc<D, HILO>) qinit4[g] = floatx4_t{qi, qi, qi, qi};
        qinit1[g] = qi;
#pragma unroll
        for (int j = 0; j < P; ++j) {
            const bool mine = col_valid && j == jl;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                qb[j][g][e] = mine ? hv[e] : (_Float16)0.0f;
                if (HILO) qb_lo[j][g][e] = mine ? lv[e] : (_Float16)0.0f;
            }
        }
    }
    const float qmul = __builtin_ldexpf((HILO && rot ? a.qscale * a.rot_norm : a.qscale) * 0x1p24f, -qk);

    float m_run = kNegInf;  // softmax reference M of column n16 (>= its running max)
    int e_v = 0;            // E (wave-uniform): the value operand carries 2^E
    float v_lim = 0.0f;     // V scales above this move E (0 until the first nonzero one)
    float l_lane = 0.0f;    // sum of this lane's probabilities (column n16)
    // acc[j]: sum p s_v c V rows of KV head j (p with its 2^E)
    floatx4_t acc[P][NCB];
#pragma unroll
    for (int j = 0; j < P; ++j)
#pragma unroll
        for (int cb = 0; cb < NCB; ++cb) acc[j][cb] = floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};

    // this lane's operands of the staged tile, into registers
    auto read_stage = [&](TileLoads<D, P, ROWS>& t, const char* stage) {
#pragma unroll
        for (int j = 0; j < P; ++j) {
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int tr = 16 * s + n16;  // quarter r of row tr: word g = channels 32 g + 8 r + 0..7
                if constexpr (D == 64) {
                    const uint2 w = *reinterpret_cast<const uint2*>(
                        stage + St::koff(j) + 16 * k_slot<D>(tr, r >> 1) + 8 * (r & 1));
                    t.kw[j][s][0] = w.x; t.kw[j][s][1] = w.y;
                } else {
#pragma unroll
                    for (int q = 0; q < NG / 4; ++q) {
                        const uint4 w = *reinterpret_cast<const uint4*>(
                            stage + St::koff(j) + 16 * k_slot<D>(tr, (NG / 4) * r + q));
                        t.kw[j][s][4 * q + 0] = w.x; t.kw[j][s][4 * q + 1] = w.y;
                        t.kw[j][s][4 * q + 2] = w.z; t.kw[j][s][4 * q + 3] = w.w;
                    }
                }
            }
#pragma unroll
            for (int av = 0; av < NA; ++av)
                t.vw[j][av] = *reinterpret_cast<const uint4*>(stage + St::voff(j) + 1024 * av + 16 * lane);
        }
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int tt = 16 * s + 4 * r + slot;
            if constexpr (ROWS) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    load_scales<NG>(t.sk[s][i], reinterpret_cast<const float*>(stage + St::KSOFF) +
                                                    (jl * 32 + 16 * s + 4 * r + i) * NG);
            } else {
                load_scales<NG>(t.sk[s][0], reinterpret_cast<const float*>(stage + St::KSOFF) +
                                                (jl * 32 + tt) * NG);
            }
            load_scales<NG>(t.sv[s], reinterpret_cast<const float*>(stage + St::VSOFF) + (jl * 32 + tt) * NG);
        }
    };

    auto compute_tile = [&](TileLoads<D, P, ROWS>& t, int it) {
        const int tok0 = tile_tok(it);
        // ---- scores, as T = S / qmul (qmul > 0 is applied inside exp2)
        float T[2][4];
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            floatx4_t tot = {0.0f, 0.0f, 0.0f, 0.0f};
            static_for<NG>([&](auto gI) {
                constexpr int g = decltype(gI)::value;
                floatx4_t d = kQinitInAcc<D, HILO> ? qinit4[g] : floatx4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int j = 0; j < P; ++j) {
                    const half8_t A = unpack_codes_sub(t.kw[j][s][g]);
                    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qb[j][g], d, 0, 0, 0);
                    if constexpr (HILO) d = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, qb_lo[j][g], d, 0, 0, 0);
                }
                static_for<4>([&](auto iI) {
                    constexpr int i = decltype(iI)::value;
                    float term;
                    const float di = kQinitInAcc<D, HILO> ? d[i] : d[i] + qinit1[g];
                    if constexpr (ROWS) term = t.sk[s][i % (ROWS ? 4 : 1)][g] * di;
                    else term = quad_bcast<i>(t.sk[s][0][g]) * di;  // folds into v_mul_f32_dpp
                    tot[i] = (g == 0) ? term : tot[i] + term;
                });
            });
#pragma unroll
            for (int i = 0; i < 4; ++i) T[s][i] = tot[i];
        }
        if (tok0 + kTile > end) {  // wave-uniform: the sequence's last, partial tile
#pragma unroll
            for (int s = 0; s < 2; ++s) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    if (tok0 + 16 * s + 4 * r + i >= end) T[s][i] = kNegInf;
                // the V scales of tokens past the end (whatever bits the cache
                // holds there) must not reach the value products, where 0 * Inf
                // or 0 * NaN would poison the row
                if (tok0 + 16 * s + 4 * r + slot >= end) {
#pragma unroll
                    for (int g = 0; g < NG; ++g) t.sv[s][g] = 0.0f;
                }
            }
        }

        // ---- online softmax for column n16 over the tile's 32 tokens (base-2
        //      exponents).  The reference m_run only moves when a score passes
        //      it, and then to kHeadroom above that score, so that most tiles
        //      keep it and skip the rescale; every p stays <= 1.
        float mt = kNegInf;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) mt = fmaxf(mt, T[s][i]);
        mt = max_xor32(max_xor16(mt)) * qmul;  // finite: the tile has a valid token
        // the largest V scale of the lane's tokens (0 past the end)
        float svm = t.sv[0][0];
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int g = 0; g < NG; ++g) svm = fmaxf(svm, t.sv[s][g]);
        const bool vmove = __any(svm > v_lim);
        // decided for the whole wave, so that the cross-lane moves of the
        // rescale see every lane
        if (__any(mt > m_run) || vmove) {
            const float m_new = (mt > m_run) ? mt + kHeadroom : m_run;
            int e_new = e_v;
            if (vmove) {  // wave-uniform: E from the wave's largest V scale
                const int ve = __builtin_amdgcn_frexp_expf(group_max<64>(svm));
                const int en = min(max(kVTarget - ve, kEMin), kEMax);
                e_new = en;
                v_lim = __builtin_ldexpf(1.0f, kVLimit - en);
            }
            // 0 on the first tile, 1 if unmoved
            const float alpha = exp2_approx(m_run - m_new);
            // the accumulators also take 2^(E' - E) (exact)
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
            for (int g = 0; g < NG; ++g) t.sv[s][g] = __builtin_ldexpf(t.sv[s][g], e_v);
        // p of the tile's tokens.  Odd i hold the bit-4 nibbles of the V words
        // (see below), whose 2^4 is cancelled here: p / 16 comes straight from
        // the exponent, and l takes 16 (p / 16).
        float p[2][4];
        const float m_odd = m_run + 4.0f;
#pragma unroll
        for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                p[s][i] = exp2_approx(__builtin_fmaf(T[s][i], qmul, -((i & 1) ? m_odd : m_run)));
                l_lane = (i & 1) ? __builtin_fmaf(p[s][i], 16.0f, l_lane) : l_lane + p[s][i];
            }

        // ---- values, one scale group (two 16-channel blocks) at a time:
        //      A_g = p * s_v[token][g] as fp16 hi + lo, B = V_j codes.  k slots
        //      (2 m, 2 m + 1) are token m of the quad in sub-tiles 0 and 1; DPP
        //      quad broadcasts hand out the s_v of token m.
        static_for<NG>([&](auto gI) {
            constexpr int g = decltype(gI)::value;
            v4u_t ha, la;
            static_for<4>([&](auto mI) {
                // one product per element, consumed by both halves, so the
                // broadcast folds into v_mul_f32_dpp
#pragma clang fp contract(off)
                constexpr int m = decltype(mI)::value;
                const float x0 = p[0][m] * quad_bcast<m>(t.sv[0][g]);
                const float x1 = p[1][m] * quad_bcast<m>(t.sv[1][g]);
                ha[m] = __builtin_bit_cast(uint32_t, half2_t{(_Float16)x0, (_Float16)x1});
                la[m] = lo_pair<m == 3>(x0, x1, ha[m]);
            });
            const half8_t pa = __builtin_bit_cast(half8_t, ha), pl = __builtin_bit_cast(half8_t, la);
#pragma unroll
            for (int j = 0; j < P; ++j) {
                static_for<2>([&](auto hI) {
                    constexpr int cb = 2 * g + decltype(hI)::value;
                    constexpr int av = cb / 4, bv = cb % 4;
                    const uint32_t word = bv == 0 ? t.vw[j][av].x : bv == 1 ? t.vw[j][av].y
                                        : bv == 2 ? t.vw[j][av].z : t.vw[j][av].w;
                    const half8_t B = unpack_codes_signed(word);
                    acc[j][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pa, B, acc[j][cb], 0, 0, 0);
                    acc[j][cb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(pl, B, acc[j][cb], 0, 0, 0);
                });
            }
        });
    };

    // NST LDS stages per wave, used in turn: tile it + (NST - 1) W streams
    // in while tile it is computed.  Before reading a stage the wave waits
    // until at most the copies issued after that stage's (the other stages'
    // tiles still to come) are in flight; the vector-memory counter retires
    // in issue order.
#pragma unroll
    for (int k = 1; k < NST; ++k)
        if (wave + k * W < ntiles) dma_tile(wave + k * W, k);
    if (wave >= ntiles) __builtin_amdgcn_s_waitcnt(kWaitVm0);  // its tile is unused
    int st = 0;
    for (int it = wave; it < ntiles; it += W) {
        // tiles it + W .. it + (NST - 1) W, as far as they exist, were issued
        // after this one and may stay in flight
        const int n_after = min(NST - 1, (ntiles - 1 - it) / W);
        static_for<NST>([&](auto kI) {
            constexpr int k = decltype(kI)::value;
            if (n_after == k) __builtin_amdgcn_s_waitcnt(wait_vm(k * St::COPIES));
        });
        asm volatile("" ::: "memory");  // the stage's reads stay after the wait
        TileLoads<D, P, ROWS> t;
        read_stage(t, stage_of(st));
        compute_tile(t, it);
        // The stage just read is refilled only once the tile's products are
        // done, so that about one tile per wave is in flight while a wave
        // computes.  Refilling earlier (after the scores, or before them) puts
        // about twice the bytes in flight over the whole chip, beyond what the
        // memory system serves best: measured slower on every workload (the
        // 70B layer at 128K: split 32.6 against 32.2 us).  The copies
        // overwrite the stage, whose reads have long finished.
        if (it + NST * W < ntiles) {
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
            dma_tile(it + NST * W, st);
        }
        st = (st + 1 == NST) ? 0 : st + 1;
    }

    // ---- merge: l over the 4 rows of each column (m and O are already
    //      wave-wide), then the W waves.  Each wave leaves its (m, l) and its
    //      O rows in its own stages, which no copy targets any more (every
    //      copy it issued has been waited for), so it need not wait for the
    //      other waves first; rows are padded by 4 floats so that the 4 rows
    //      of a store fall in distinct banks.
    constexpr int RS = D + 4;
    static_assert(16 * RS * 4 + 16 * 8 <= NST * St::BYTES, "a wave's merge share fits its stages");
    auto merge_o = [&](int w) { return reinterpret_cast<float*>(lds) + w * (NST * St::BYTES / 4); };
    auto merge_ml = [&](int w) { return reinterpret_cast<float2*>(merge_o(w) + 16 * RS); };
    const float L = sum_xor32(sum_xor16(l_lane));
    // acc carries 2^E.  With F = floor(E / 2), (M - F, l 2^F, acc 2^(F - E))
    // is the partial (M, l, acc 2^-E), with both sums inside fp32's range for
    // every E the V scales can give
    const int f_e = e_v >> 1;
    if (lane < 16) merge_ml(wave)[lane] = make_float2(m_run - (float)f_e, __builtin_ldexpf(L, f_e));
    // rows 4 r .. 4 r + 3 of O lie in one KV head (two heads only if G >= 4):
    // keep that head's set
    const int jr = min(4 * r / G, P - 1);
    float* own = merge_o(wave);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int h = 4 * r + i;
        if (h < PG) {
#pragma unroll
            for (int cb = 0; cb < NCB; ++cb) {
                float v = acc[0][cb][i];
#pragma unroll
                for (int j = 1; j < P; ++j) v = (jr == j) ? acc[j][cb][i] : v;
                own[h * RS + 16 * cb + n16] = __builtin_ldexpf(v, f_e - e_v);
            }
        }
    }
    __syncthreads();
    // one thread per (head, 4 channels); the iterations are unrolled so
    // that their LDS reads are in flight together
    constexpr int kMergeIters = (16 * (D / 4) + 64 * W - 1) / (64 * W);
#pragma unroll
    for (int k = 0; k < kMergeIters; ++k) {
        const int i = tid + k * 64 * W;
        if (i >= PG * (D / 4)) break;
        const int h = i / (D / 4), c = 4 * (i % (D / 4));
        float2 ml[W];
        float Mb = kNegInf;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            ml[w] = merge_ml(w)[h];
            Mb = fmaxf(Mb, ml[w].x);
        }
        float4 o = {0.0f, 0.0f, 0.0f, 0.0f};
        float Ls = 0.0f;
#pragma unroll
        for (int w = 0; w < W; ++w) {
            const float f = (ml[w].x == kNegInf) ? 0.0f : exp2_approx(ml[w].x - Mb);
            const float4 x = *reinterpret_cast<const float4*>(merge_o(w) + h * RS + c);
            o.x += f * x.x; o.y += f * x.y; o.z += f * x.z; o.w += f * x.w;
            Ls += f * ml[w].y;
        }
        const size_t prow = ((size_t)b * a.Hq + hk0 * G + h) * a.num_splits + split;
        *reinterpret_cast<float4*>(a.part_o + prow * D + c) = o;
        if (c == 0) a.part_ml[prow] = make_float2(Mb, Ls);
    }
}


// Waves per block: 4, one per SIMD, each with two LDS stages (80 KB per
// block at head_dim 128).  Measured against 8 waves with one stage: equal on
// one long sequence, faster on many ragged ones, where a second block fits
// the CU beside the first.
template <int D>
constexpr int kBlockWaves = 4;

template <int D, int P, bool HILO>
hipError_t launch(const SplitArgs& a, hipStream_t stream)
{
    constexpr int W = kBlockWaves<D>;
    // the merge lives in the stages (checked in the kernel)
    const size_t lds = (size_t)kStages<D, P, W> * W * Stage<D, P>::BYTES;
    dim3 grid(a.num_splits, a.H / P, a.B), block(64 * W);
    static const hipError_t attr = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&split_mfma_kernel<D, P, HILO, W>),
        hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (attr != hipSuccess) return attr;
    split_mfma_kernel<D, P, HILO, W><<<grid, block, lds, stream>>>(a);
    return hipGetLastError();
}

template <int D>
hipError_t dispatch(const SplitArgs& a, hipStream_t stream)
{
    const bool hilo = a.signs != nullptr || a.lam != nullptr;  // q not exact in fp16
    if constexpr (D != 256) {  // head_dim 256 serves one KV head per wave
        if (split_mfma_heads_per_wave(a.D, a.Hq / a.H, a.H) == 2)
            return hilo ? launch<D, 2, true>(a, stream) : launch<D, 2, false>(a, stream);
    }
    return hilo ? launch<D, 1, true>(a, stream) : launch<D, 1, false>(a, stream);
}

}  // namespace

// KV heads per wave: two (filling 16 MFMA columns at G = 8) when G >= 4
// (every quad of columns inside one head), the head count allows it and the
// registers suffice, else one.
int split_mfma_heads_per_wave(int D, int G, int H)
{
    return (D != 256 && G >= 4 && G <= 8 && H % 2 == 0) ? 2 : 1;
}

int split_mfma_block_waves(int D)
{
    return D == 256 ? kBlockWaves<256> : D == 64 ? kBlockWaves<64> : kBlockWaves<128>;
}

bool split_mfma_supports(int D, int G)
{
    return (D == 64 || D == 128 || D == 256) && G >= 1 && G <= 16;
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
