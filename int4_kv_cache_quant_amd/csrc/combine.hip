// combine.hip - merge the split partials of decode attention, optionally with
// the step's new token appended.
//
// Each split s of a (sequence, query head) row carries (m_s, l_s, o_s): its
// softmax reference (log2 domain; any value the split pass chose to keep l_s
// and o_s in fp32's range), its sum of 2^(S_t - m_s), and its unnormalised
// value sum with the same weights.  The exact
// softmax over the union of splits is
//   M = max_s m_s,  L = sum_s l_s 2^(m_s - M),  out = sum_s 2^(m_s - M) o_s / L
// evaluated in fp32 (the high-precision accumulation the zingnex
// Open-TQ-Metal page asks for in its section on numerical stability).
// A row with lens == 0 has no splits and gets zeros.
//
// With the append, the split pass covered [0, lens - 1) and this kernel
// quantises the token at lens - 1 as it is produced (Open-TQ-Metal abstract;
// zingnex page, section on on-the-fly quantisation), writes it into the
// cache, and merges it as one more term (m = its score, l = 1, o = its
// dequantised V).
#include "bits_layout.hpp"
#include "common.hpp"
#include "kernels.hpp"
#include "quant_lane.hpp"
#include "srft.hpp"

namespace otq {

namespace {

constexpr int kThreads = 256;
constexpr int kCh = 32;  // channels per block of the slice form
constexpr float kNegInf = -__builtin_huge_valf();

// Sum over the lanes of a wave that share lane % CQ (CQ = 8, 16, 32 or 64
// threads per split: lanes 8, 16 and 32 apart; a row's rotation by 8 is lane
// i ^ 8).
template <int CQ>
__device__ __forceinline__ float sum_split_lanes(float v)
{
    static_assert(CQ == 8 || CQ == 16 || CQ == 32 || CQ == 64, "threads per split");
    if constexpr (CQ <= 8) v = v + dpp_mov<kDppRor8>(v);
    if constexpr (CQ <= 16) v = sum_xor16(v);
    if constexpr (CQ <= 32) v = sum_xor32(v);
    return v;
}

// In-place Walsh-Hadamard butterflies over one element per thread (threads
// 0..D-1), stages in ascending stride: the lower element of a pair becomes
// lower + upper, the upper one lower - upper.  Strides below 64 stay in the
// wave; wider ones go through LDS.
template <int D>
__device__ __forceinline__ float fwht_thread(float y, float* xch)
{
#pragma clang fp contract(off)
    const int t = threadIdx.x;
#pragma unroll
    for (int h = 1; h < D; h <<= 1) {
        float o;
        if (h < 64) {
            o = shfl_xor(y, h);
        } else {  // threads past D hold no channel and stay out of xch
            __syncthreads();
            if (t < D) xch[t] = y;
            __syncthreads();
            o = t < D ? xch[t ^ h] : y;
        }
        y = (t & h) ? (o - y) : (y + o);
    }
    return y;
}

// The V fields of token pos (codes[c], c < D) in its b-bit tile: word x of
// the VBitsTile<D, BITS>::TOKEN_WORDS words that hold them (x past them:
// nothing).  The other fields of the word are other tokens', so this token's
// bits are cleared and set with two atomics (no read to wait for; one
// thread's two operations on a word take effect in order).
template <int D, int BITS>
__device__ __forceinline__ void put_v_bits(uint8_t* vc, size_t head, int cap, int pos, int x, const int8_t* codes)
{
    if (x >= VBitsTile<D, BITS>::TOKEN_WORDS) return;
    const int u = pos % kTile;
    const int W = vtile_token_word<D, BITS>(u, x);
    uint32_t val = 0, mask = 0;
    vtile_fields<D, BITS>(W, [&](int fu, int c, int bpos, int width, int shift) {
        if (fu == u) {
            const uint32_t fm = (1u << width) - 1u;
            val |= (((uint32_t)(int)codes[c] >> shift) & fm) << bpos;
            mask |= fm << bpos;
        }
    });
    unsigned* w = reinterpret_cast<unsigned*>(vc + (head * (cap / kTile) + pos / kTile) * (size_t)(kTile * D * BITS / 8)) + W;
    __hip_atomic_fetch_and(w, ~mask, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_fetch_or(w, val, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Block (row, c0): row = b * Hq + h, channels [CH c0, CH c0 + CH), CH = 32
// (slices) or the whole head_dim (ROWS).  Thread t reads channels
// CH c0 + 4 (t % CQ) .. + 3 of the splits s = t / CQ (mod LS), CQ = CH / 4,
// LS = 256 / CQ, so LS splits stream in side by side; each thread folds its
// splits into a running (m, l, o) (the same merge rule as above), then the
// block merges the threads' triples: one pass over the partials.  DT =
// head_dim, or 0 where it is read at run time (slices without the append).
// Whole rows serve a rotated V, whose output the block brings back by the
// inverse rotation, and a rotated K with the append, whose in-block
// transforms then run once per row instead of once per slice.
template <int DT, bool APPEND, bool ROWS, bool ROT, bool LAM, bool VROT>
__global__ __launch_bounds__(kThreads) void lse_combine_kernel(CombineArgs a)
{
    static_assert(DT > 0 || (!APPEND && !ROWS), "compile-time head_dim");
    static_assert(!VROT || ROWS, "a rotated V needs whole rows");
    constexpr int CH = ROWS ? DT : kCh;
    constexpr int CQ = CH / 4;          // threads sharing one split (a float4 each)
    constexpr int LS = kThreads / CQ;   // splits read side by side
    // splits in flight per thread: whole rows read LS = 4..16 splits side by
    // side, so each thread holds more of them
    constexpr int NF = ROWS ? (LS >= 16 ? 4 : 8) : 2;
    constexpr int DA = DT;
    __shared__ float red_m[kThreads / 64];
    __shared__ float4 red_o[kThreads / 64][CQ];
    __shared__ float red_l[kThreads / 64];
    __shared__ float red_s[kThreads / 64];
    __shared__ float xch[DT > 0 ? DT : 1];   // butterflies, then the new token's V
    __shared__ float orow[VROT ? DT : 1];    // the output row before the inverse rotation
    __shared__ int8_t bcodes[2][APPEND ? DT : 1];  // a b-bit token's K and V codes, before packing
    // every argument the loads below need, fetched together: otherwise the
    // fields arrive one scalar round trip after another, each gating the next
    // address
    asm volatile("" ::"s"(a.part_o), "s"(a.part_ml), "s"(a.lens), "s"(a.S), "s"(a.Hq), "s"(a.D),
                 "s"(a.k_new), "s"(a.v_new), "s"(a.q), "s"(a.H), "s"(a.signs));
    const int D = DT > 0 ? DT : a.D;
    const int row = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = row / a.Hq;
    const int q = tid % CQ, g = tid / CQ;
    const int c = CH * blockIdx.y + 4 * q;
    // the new token's K, V and this row's q (one channel per thread; threads
    // past D work on channel D - 1 and write nothing), loaded before lens[b]
    // like the first splits below
    [[maybe_unused]] uint16_t kx = 0, vx = 0, qx = 0;
    [[maybe_unused]] float sg = 1.0f, lm = 1.0f, vsg = 1.0f;
    [[maybe_unused]] int kvh = 0, pos = 0, ch = 0;
    [[maybe_unused]] bool writer = false;
    // the FFT rotation's twiddles (radix 2; head_dim 192 takes the
    // mixed-radix stages through LDS, srft_mixed_block, in their place)
    constexpr bool kMixed = DA == 192;
    [[maybe_unused]] SrftThreadTw<(DA > 0 && !kMixed ? DA : 64)> stw;
    if constexpr ((ROT || VROT) && !kMixed) {
        if (a.rot_kind) stw.load(tid);
    }
    if constexpr (APPEND) {
        const int G = a.Hq / a.H, h = row % a.Hq;
        kvh = h / G;
        ch = min(tid, DA - 1);
        const size_t src = ((size_t)b * a.H + kvh) * DA + ch;
        kx = a.k_new[src];
        vx = a.v_new[src];
        qx = static_cast<const uint16_t*>(a.q)[(size_t)row * DA + ch];
        if (ROT) sg = a.signs[ch];
        if (LAM) lm = a.lam[ch];  // K's channel scale
        if (VROT) vsg = a.vsigns[ch];
        // one block per KV head writes the token: the first query head's,
        // first channel slice
        writer = h % G == 0 && blockIdx.y == 0 && tid < DA;
    }

    // The first NF splits of each thread (g, g + LS, ...) are loaded before
    // lens[b] is known, as far as the workspace holds them (the plan's split
    // count), and folded below only if the split pass wrote them: these
    // loads do not wait for the length's round trip.
    const float2* ml = a.part_ml + (size_t)row * a.S;
    const float* po = a.part_o + (size_t)row * a.S * D + c;
    float2 vf[NF];
    float4 xf[NF];
#pragma unroll
    for (int k = 0; k < NF; ++k) {
        vf[k] = make_float2(0.0f, 0.0f);
        xf[k] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    }
#pragma unroll
    for (int k = 0; k < NF; ++k) {
        const int sk = g + k * LS;
        if (sk < a.S) {
            vf[k] = ml[sk];
            xf[k] = *reinterpret_cast<const float4*>(po + (size_t)sk * D);
        }
    }
    const int raw_len = a.lens[b];
    const int len = min(max(raw_len, 0), a.max_len);
    if (tid == 0 && blockIdx.y == 0 && row % a.Hq == 0 && (raw_len < 0 || raw_len > a.max_len))
        report_error(a.err, kErrLens);
    const int nsplit_tok = APPEND ? max(len - 1, 0) : len;  // tokens the split pass covered
    // splits holding a partial: those whose first piece starts below the
    // covered length (each split's later pieces follow S chunk further on)
    const int ns = min((nsplit_tok + a.chunk - 1) / a.chunk, a.S);
    if constexpr (APPEND) pos = len - 1;
    float4* dst = reinterpret_cast<float4*>(a.out + (size_t)row * D + c);
    if (len == 0) {  // block-uniform: nothing attended, nothing appended
        if (tid < CQ) *dst = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        return;
    }

    // ---- the splits
    float m = kNegInf, l = 0.0f;
    float4 o = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
    auto fold = [&](float2 v, float4 x) {  // every written partial has a finite m
        const float mn = fmaxf(m, v.x);
        const float al = exp2_approx(m - mn), w = exp2_approx(v.x - mn);
        o = make_float4(o.x * al + x.x * w, o.y * al + x.y * w, o.z * al + x.z * w, o.w * al + x.w * w);
        l = l * al + v.y * w;
        m = mn;
    };
#pragma unroll
    for (int k = 0; k < NF; ++k)
        if (g + k * LS < ns) fold(vf[k], xf[k]);
    for (int s = g + NF * LS; s < ns; s += NF * LS) {  // NF splits in flight per thread
#pragma unroll
        for (int k = 0; k < NF; ++k) {
            const int sk = s + k * LS;
            if (sk < ns) {
                vf[k] = ml[sk];
                xf[k] = *reinterpret_cast<const float4*>(po + (size_t)sk * D);
            }
        }
#pragma unroll
        for (int k = 0; k < NF; ++k)
            if (s + k * LS < ns) fold(vf[k], xf[k]);
    }

    // ---- the new token: quantise K and V to the same bytes as the append kernels
    //      (the small-append kernel's operations in its order), write them, score it
    [[maybe_unused]] float s_new = kNegInf;
    if constexpr (APPEND) {
        float x = widen(kx, a.dtype);
        if (ROT) {
            x = x * sg;
            if constexpr (kMixed) x = srft_mixed_block<DA>(x, xch);  // the FFT kind only at 192
            else x = a.rot_kind ? srft_thread<DA>(x, xch, stw) : fwht_thread<DA>(x, xch);
            x = x * a.rot_norm;
        }
        if (LAM) x = x * lm;  // after the rotation
        float xk[1] = {x};
        int ck[1];
        // one channel per lane: the lane layout of a 64-channel vector, whose
        // 32-lane groups are this vector's 32-channel groups
        const int bits = a.bits;  // block-uniform: 4, or 2 / 3
        const float sk = bits == 4 ? quantize_lane<64>(xk, ck, lane) : quantize_lane_bits(xk[0], ck[0], bits);
        float xv[1] = {widen(vx, a.dtype)};
        if constexpr (VROT) {  // V rotated as K is, with its own signs
            xv[0] = xv[0] * vsg;
            xv[0] = a.rot_kind ? srft_thread<DA>(xv[0], xch, stw) : fwht_thread<DA>(xv[0], xch);
            xv[0] = xv[0] * a.rot_norm;
        }
        int cv[1];
        const float sv = bits == 4 ? quantize_lane<64>(xv, cv, lane) : quantize_lane_bits(xv[0], cv[0], bits);
        if (bits != 4) {  // block-uniform: b-bit codes, staged in LDS, then packed
            const size_t head = (size_t)b * a.H + kvh, krow = head * a.cap + pos;
            if (writer) {
                bcodes[0][ch] = (int8_t)ck[0];
                bcodes[1][ch] = (int8_t)cv[0];
                if (ch % kGroup == 0) {
                    a.ks[krow * (DA / kGroup) + ch / kGroup] = sk;
                    a.vs[krow * (DA / kGroup) + ch / kGroup] = sv;
                }
            }
            __syncthreads();
            const int nword = DA * bits / 32;  // words per K row
            if (writer && tid < nword) {       // the K row, written whole
                uint32_t word = 0;
                const int i0 = (32 * tid) / bits, i1 = min((32 * tid + 31) / bits, DA - 1);
                for (int i = i0; i <= i1; ++i) {
                    const uint32_t u = (uint32_t)bcodes[0][i] & ((1u << bits) - 1u);
                    const int off = i * bits - 32 * tid;  // negative for a code that starts in the word before
                    word |= off >= 0 ? u << off : u >> -off;
                }
                reinterpret_cast<uint32_t*>(a.kc + krow * (size_t)(DA * bits / 8))[tid] = word;
            } else if (writer) {  // this token's V fields, word by word of its tile
                if (bits == 2) put_v_bits<DA, 2>(a.vc, head, a.cap, pos, tid - nword, bcodes[1]);
                else put_v_bits<DA, 3>(a.vc, head, a.cap, pos, tid - nword, bcodes[1]);
            }
        } else if (writer) {
            const size_t head = (size_t)b * a.H + kvh, krow = head * a.cap + pos;
            const int cnext = __shfl_xor(ck[0], 1, 64);
            if ((ch & 1) == 0)
                a.kc[krow * (DA / 2) + k_row_byte<DA>(ch)] = (uint8_t)((ck[0] & 0xF) | ((cnext & 0xF) << 4));
            // the V byte is shared with token pos ^ 1: replace only this
            // token's nibble, by clearing and setting it with two atomics on
            // the containing word (no read to wait for; the other nibbles of
            // the word are other channels' and other tokens', and the same
            // thread's two operations on one word take effect in order)
            const size_t vbyte = (head * (a.cap / kTile) + pos / kTile) * (size_t)(16 * DA) +
                                 v_tile_byte<DA>(ch, (pos % kTile) & ~1);
            const int shift = 8 * (int)(vbyte & 3) + 4 * (pos & 1);
            unsigned* vword = reinterpret_cast<unsigned*>(a.vc + (vbyte & ~(size_t)3));
            __hip_atomic_fetch_and(vword, ~(0xFu << shift), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_or(vword, ((unsigned)cv[0] & 0xFu) << shift, __ATOMIC_RELAXED,
                                  __HIP_MEMORY_SCOPE_AGENT);
            if (ch % kGroup == 0) {
                a.ks[krow * (DA / kGroup) + ch / kGroup] = sk;
                a.vs[krow * (DA / kGroup) + ch / kGroup] = sv;
            }
        }
        // score: q' . k^ (q rotated like K, then divided by K's channel
        // scale), in log2 units
        float y = widen(qx, a.dtype);
        if (ROT) {
            y = y * sg;
            if constexpr (kMixed) y = srft_mixed_block<DA>(y, xch);
            else y = a.rot_kind ? srft_thread<DA>(y, xch, stw) : fwht_thread<DA>(y, xch);
            y = y * a.rot_norm;
        }
        if (LAM) y = y / lm;
        const float kd = (float)ck[0] * sk;
        s_new = group_sum<64>(tid < DA ? y * kd : 0.0f);  // this wave's part of q' . k^
        if ((ROT || VROT) && DA > 64) __syncthreads();  // the butterflies' last reads of xch are done
        if (tid < DA) xch[tid] = (float)cv[0] * sv;
        if (lane == 0) red_s[wave] = s_new;
    }

    // block maximum of the threads' references (and the new token's score:
    // one LDS round for both)
    float M = group_max<64>(m);
    if (lane == 0) red_m[wave] = M;
    __syncthreads();
    M = red_m[0];
#pragma unroll
    for (int w = 1; w < kThreads / 64; ++w) M = fmaxf(M, red_m[w]);
    if constexpr (APPEND) {
        s_new = red_s[0];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) s_new += red_s[w];
        s_new *= a.qscale;  // log2 units
    }
    const float f = (m == kNegInf) ? 0.0f : exp2_approx(m - M);
    o = make_float4(o.x * f, o.y * f, o.z * f, o.w * f);
    l = (q == 0) ? l * f : 0.0f;  // the CQ threads of a split group hold the same l
    // sum over the threads of one channel quad: within the wave, then waves
    o = make_float4(sum_split_lanes<CQ>(o.x), sum_split_lanes<CQ>(o.y), sum_split_lanes<CQ>(o.z),
                    sum_split_lanes<CQ>(o.w));
    l = sum_split_lanes<CQ>(l);  // lane 0 (q == 0): the wave's split lanes
    if (lane < CQ) red_o[wave][lane] = o;
    if (lane == 0) red_l[wave] = l;
    __syncthreads();
    if (tid < CQ) {
        float4 r = red_o[0][tid];
        float L = red_l[0];
#pragma unroll
        for (int w = 1; w < kThreads / 64; ++w) {
            const float4 x = red_o[w][tid];
            r.x += x.x; r.y += x.y; r.z += x.z; r.w += x.w;
            L += red_l[w];
        }
        if constexpr (APPEND) {  // one more term: m = s_new, l = 1, o = V^ of the token
            const float Mn = fmaxf(M, s_new);
            const float a1 = (M == kNegInf) ? 0.0f : exp2_approx(M - Mn), a2 = exp2_approx(s_new - Mn);
            const float* vh = xch + CH * blockIdx.y + 4 * tid;
            r = make_float4(r.x * a1 + vh[0] * a2, r.y * a1 + vh[1] * a2, r.z * a1 + vh[2] * a2,
                            r.w * a1 + vh[3] * a2);
            L = L * a1 + a2;
        }
        if constexpr (VROT) {
            *reinterpret_cast<float4*>(orow + 4 * tid) = make_float4(r.x / L, r.y / L, r.z / L, r.w / L);
        } else {
            *dst = make_float4(r.x / L, r.y / L, r.z / L, r.w / L);
        }
    }
    if constexpr (VROT) {  // back to the original basis: s_v (.) (rot_norm * inverse(row))
        __syncthreads();
        float y = tid < DT ? orow[tid] : 0.0f;
        y = a.rot_kind ? isrft_thread<DT>(y, xch, stw) : fwht_thread<DT>(y, xch);
        if (tid < DT) a.out[(size_t)row * DT + tid] = y * a.rot_norm * a.vsigns[tid];
    }
}

}  // namespace

hipError_t launch_lse_combine(const CombineArgs& a, hipStream_t stream)
{
    if (a.D % kCh != 0) return hipErrorInvalidValue;
    const bool append = a.k_new != nullptr, rot = a.signs != nullptr, lam = a.lam != nullptr,
               vrot = a.vsigns != nullptr;
    // whole rows for a rotated V, for the append with a rotated K, and for a
    // plain combine whose slices would take more than one round of resident
    // blocks (2048); at head_dim 192 (no whole-row form: its split groups
    // would not divide the block) the slices, each block transforming the
    // new token's K itself when it is rotated
    const bool pow2 = a.D == 64 || a.D == 128 || a.D == 256;  // the whole-row forms' widths
    const bool big = !append && pow2 && (long)a.B * a.Hq * (a.D / kCh) > 2048;
    const bool rows = pow2 && (vrot || (append && rot) || big);
    if (!pow2 && (a.D != 192 || vrot)) return hipErrorInvalidValue;
    dim3 grid(a.B * a.Hq, rows ? 1 : a.D / kCh), block(kThreads);
    if (!append && !rows) {
        lse_combine_kernel<0, false, false, false, false, false><<<grid, block, 0, stream>>>(a);
        return hipGetLastError();
    }
    using K = void (*)(CombineArgs);
    auto pick = [&](auto d) -> K {
        constexpr int DT = decltype(d)::value;
        if (!append) return vrot ? lse_combine_kernel<DT, false, true, false, false, true>
                                 : lse_combine_kernel<DT, false, true, false, false, false>;
        if (!rows) return lam ? lse_combine_kernel<DT, true, false, false, true, false>
                              : lse_combine_kernel<DT, true, false, false, false, false>;
        switch ((rot ? 1 : 0) + (lam ? 2 : 0) + (vrot ? 4 : 0)) {
        case 0: return lse_combine_kernel<DT, true, true, false, false, false>;
        case 1: return lse_combine_kernel<DT, true, true, true, false, false>;
        case 2: return lse_combine_kernel<DT, true, true, false, true, false>;
        case 3: return lse_combine_kernel<DT, true, true, true, true, false>;
        case 4: return lse_combine_kernel<DT, true, true, false, false, true>;
        case 5: return lse_combine_kernel<DT, true, true, true, false, true>;
        case 6: return lse_combine_kernel<DT, true, true, false, true, true>;
        default: return lse_combine_kernel<DT, true, true, true, true, true>;
        }
    };
    K kern = nullptr;
    switch (a.D) {
    case 192:  // the slice form with the token (rotation and scale as compile-time choices)
        switch ((rot ? 1 : 0) + (lam ? 2 : 0)) {
        case 0: kern = lse_combine_kernel<192, true, false, false, false, false>; break;
        case 1: kern = lse_combine_kernel<192, true, false, true, false, false>; break;
        case 2: kern = lse_combine_kernel<192, true, false, false, true, false>; break;
        default: kern = lse_combine_kernel<192, true, false, true, true, false>; break;
        }
        break;
    case 64: kern = pick(std::integral_constant<int, 64>{}); break;
    case 128: kern = pick(std::integral_constant<int, 128>{}); break;
    case 256: kern = pick(std::integral_constant<int, 256>{}); break;
    default: return hipErrorInvalidValue;
    }
    kern<<<grid, block, 0, stream>>>(a);
    return hipGetLastError();
}

}  // namespace otq
