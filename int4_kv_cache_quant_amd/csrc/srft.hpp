// srft.hpp - the sign-randomised FFT rotation (SRFT) of K and of the query
// ("SRFT + int4 KV-cache", core method: a sign-randomised FFT may take the
// place of the Hadamard rotation, at the same quality).
//
// A vector of D reals is D/2 complex numbers z_j = (y_2j, y_2j+1).  After
// the signs, the radix-2 decimation-in-frequency FFT runs in place: stages
// of half-size h = N/2, N/4, ..., 1 (N = D/2) replace each pair (a, b) =
// (z_j, z_j+h) with (a + b, (a - b) W^t), W = exp(-2 pi i / N), t = (j mod
// h) N / (2h), which leaves the DFT coefficient of index bitrev(k) at
// position k.  The result is multiplied by rot_norm = fp32(1/sqrt(N)); the
// map is orthogonal, so a query rotated the same way keeps q . k.
//
// Every step is one IEEE fp32 operation (the bodies forbid contraction), the
// complex product being (dr wr - di wi, dr wi + di wr) with each product
// rounded before the sum, and the twiddles are the correctly rounded fp32
// values of cos and -sin: the rotated values, and the codes quantised from
// them, are the same bits in every kernel and in any other evaluation of the
// same steps.
#pragma once

#include "common.hpp"

namespace otq {
namespace srft_detail {

constexpr double kPi = 3.14159265358979323846;

// cos and sin of x in [0, pi/4] by their Taylor series, in double: a few
// ulps of double, far inside the distance of every twiddle below from an
// fp32 rounding midpoint, so the fp32 roundings are the correct ones.
constexpr void cos_sin(double x, double& c, double& s)
{
    double tc = 1.0, ts = x;
    c = 0.0;
    s = 0.0;
    for (int n = 0; n < 30; ++n) {
        c += tc;
        s += ts;
        tc = -tc * x * x / ((2.0 * n + 1.0) * (2.0 * n + 2.0));
        ts = -ts * x * x / ((2.0 * n + 2.0) * (2.0 * n + 3.0));
    }
}

// W_128^u = (cos, -sin)(2 pi u / 128), u < 64; a stage of half-size h of
// any N <= 128 reads entry (j mod h) * 64 / h.  Angles are reduced to the
// first octant, so the quarter-turn values are exact.
struct Twiddles {
    float re[64];
    float im[64];
};

constexpr Twiddles make_twiddles()
{
    Twiddles t{};
    for (int u = 0; u < 64; ++u) {
        const int oct = u / 16, rem = u % 16;           // angle (pi/4) (oct + rem/16)
        const int m = (oct & 1) ? 16 - rem : rem;       // odd octants: the complement
        double c1 = 1.0, s1 = 0.0;
        if (m != 0) cos_sin(kPi / 4.0 * m / 16.0, c1, s1);
        double c = 0.0, s = 0.0;
        switch (oct) {
        case 0: c = c1; s = s1; break;      // a
        case 1: c = s1; s = c1; break;      // pi/2 - b
        case 2: c = -s1; s = c1; break;     // pi/2 + a
        default: c = -c1; s = s1; break;    // pi - b
        }
        t.re[u] = static_cast<float>(c) + 0.0f;  // zeros are +0
        t.im[u] = static_cast<float>(-s) + 0.0f;
    }
    return t;
}

static __constant__ Twiddles kTw = make_twiddles();

// The twiddles of a stage of half-size h in lane order: entry h + v holds
// W_128^(v 64 / h) for v < h (h = 1, 2, ..., 64; entry 0 unused), so the
// twiddles of consecutive complex numbers are adjacent and a lane reads its
// share of a stage with 16-byte loads.
struct Cf {
    float re, im;
};
struct alignas(16) StageTwiddles {
    Cf w[128];
};

constexpr StageTwiddles make_stage_twiddles()
{
    const Twiddles t = make_twiddles();
    StageTwiddles s{};
    for (int h = 1; h <= 64; h *= 2)
        for (int v = 0; v < h; ++v) s.w[h + v] = Cf{t.re[v * (64 / h)], t.im[v * (64 / h)]};
    return s;
}

static __constant__ StageTwiddles kTwS = make_stage_twiddles();

// n consecutive entries from entry i (i a multiple of 2 when n >= 2)
template <int n>
__device__ __forceinline__ void load_tw(Cf* dst, int i)
{
    if constexpr (n == 1) {
        dst[0] = kTwS.w[i];
    } else {
#pragma unroll
        for (int k = 0; k < n; k += 2) {
            const float4 v = *reinterpret_cast<const float4*>(&kTwS.w[i + k]);
            dst[k] = Cf{v.x, v.y};
            dst[k + 1] = Cf{v.z, v.w};
        }
    }
}


// The mixed-radix form at head_dim 192 (N = 96 = 3 * 32): the radix-3
// stage's constant and the 96-point twiddles.
constexpr float kC3 = 0x1.bb67aep-1f;  // fp32(sqrt(3) / 2), correctly rounded

// W_96^t = (cos, -sin)(2 pi t / 96) for t < 96, rounded once from a double
// Taylor series of the angle reduced to the first octant (quarter turns
// exact).
struct Twiddles96 {
    float re[96];
    float im[96];
};

constexpr Twiddles96 make_twiddles96()
{
    Twiddles96 t{};
    for (int u = 0; u < 96; ++u) {
        const int oct = u / 12, rem = u % 12;       // angle (pi/4) (oct + rem / 12)
        const int m = (oct & 1) ? 12 - rem : rem;   // odd octants: the complement
        double c1 = 1.0, s1 = 0.0;
        if (m != 0) cos_sin(kPi / 4.0 * m / 12.0, c1, s1);
        double c = 0.0, s = 0.0;
        switch (oct) {
        case 0: c = c1; s = s1; break;       // a
        case 1: c = s1; s = c1; break;       // pi/2 - b
        case 2: c = -s1; s = c1; break;      // pi/2 + a
        case 3: c = -c1; s = s1; break;      // pi - b
        case 4: c = -c1; s = -s1; break;     // pi + a
        case 5: c = -s1; s = -c1; break;     // 3 pi/2 - b
        case 6: c = s1; s = -c1; break;      // 3 pi/2 + a
        default: c = c1; s = -s1; break;     // 2 pi - b
        }
        t.re[u] = static_cast<float>(c) + 0.0f;  // zeros are +0
        t.im[u] = static_cast<float>(-s) + 0.0f;
    }
    return t;
}

static __constant__ Twiddles96 kTw96 = make_twiddles96();

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

}  // namespace srft_detail

// The lane-dependent twiddles of a vector of D reals spread over D / E
// lanes, E reals per lane: for every stage whose pairs lie in different
// lanes, those of the lane's complex numbers (E >= 2), or of the lane's
// element's complex number (E = 1).  Loaded once, used for every vector the
// lane rotates at the same position.
template <int D, int E>
struct SrftLaneTw {
    static constexpr int N = D / 2;
    static constexpr int CE = E >= 2 ? E / 2 : 1;
    // stages of half-size N/2 ... CE (E >= 2) or N/2 ... 1 (E = 1)
    static constexpr int S = srft_detail::ilog2(N) - (E >= 2 ? srft_detail::ilog2(CE) : 0);
    srft_detail::Cf w[S][CE];

    __device__ __forceinline__ void load(int lane)
    {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int h = (N / 2) >> s;
            if constexpr (E == 1)
                srft_detail::load_tw<1>(w[s], h + ((lane >> 1) & (h - 1)));
            else  // the lane's complex numbers lane CE + c, c < CE: (lane mod h / CE) CE + c
                srft_detail::load_tw<CE>(w[s], h + ((lane & (h / CE - 1)) * CE));
        }
    }
};

// y <- rot_norm * FFT(y) (y already multiplied by the signs): a vector of D
// reals spread over D / E consecutive lanes of an aligned lane group, E
// consecutive reals per lane (E = 1 needs D <= 64); `lane` is the lane's
// index within its group and tw its loaded twiddles.
template <int D, int E>
__device__ __forceinline__ void srft_signed(float (&y)[E], float rot_norm, int lane,
                                            const SrftLaneTw<D, E>& tw)
{
#pragma clang fp contract(off)
    constexpr int N = D / 2;
    if constexpr (E == 1) {
        static_assert(D <= 64, "one real per lane: one wave");
        const int j = lane >> 1;
        const bool im = (lane & 1) != 0;
#pragma unroll
        for (int s = 0; s < SrftLaneTw<D, E>::S; ++s) {
            const int h = (N / 2) >> s;
            const float o = shfl_xor(y[0], 2 * h);
            const float d = o - y[0];          // a - b, used by upper elements
            const float dd = shfl_xor(d, 1);   // the other component of the pair
            const float wr = tw.w[s][0].re, wi = tw.w[s][0].im;
            const float up = im ? dd * wi + d * wr : d * wr - dd * wi;
            y[0] = (j & h) ? up : y[0] + o;
        }
    } else {
        constexpr int CE = E / 2;  // complex numbers per lane
        constexpr int NS = srft_detail::ilog2(N);  // stages; the first S pair lanes
#pragma unroll
        for (int s = 0; s < NS; ++s) {
            const int h = (N / 2) >> s;
            if (h >= CE) {  // pairs in lanes h / CE apart
                const int m = h / CE;
                const bool upper = (lane & m) != 0;
#pragma unroll
                for (int c = 0; c < CE; ++c) {
                    const float ore = shfl_xor(y[2 * c], m), oim = shfl_xor(y[2 * c + 1], m);
                    const float wr = tw.w[s][c].re, wi = tw.w[s][c].im;
                    const float dr = ore - y[2 * c], di = oim - y[2 * c + 1];
                    const float ur = dr * wr - di * wi, ui = dr * wi + di * wr;
                    y[2 * c] = upper ? ur : y[2 * c] + ore;
                    y[2 * c + 1] = upper ? ui : y[2 * c + 1] + oim;
                }
            } else {  // pairs inside the lane: (lane CE + c) mod h = c mod h
#pragma unroll
                for (int c = 0; c < CE; ++c) {
                    if ((c & h) == 0) {
                        const int u = (c & (h - 1)) * (64 / h);
                        const float wr = srft_detail::kTw.re[u], wi = srft_detail::kTw.im[u];
                        const float ar = y[2 * c], ai = y[2 * c + 1];
                        const float br = y[2 * (c + h)], bi = y[2 * (c + h) + 1];
                        const float dr = ar - br, di = ai - bi;
                        y[2 * c] = ar + br;
                        y[2 * c + 1] = ai + bi;
                        y[2 * (c + h)] = dr * wr - di * wi;
                        y[2 * (c + h) + 1] = dr * wi + di * wr;
                    }
                }
            }
        }
    }
#pragma unroll
    for (int e = 0; e < E; ++e) y[e] = y[e] * rot_norm;
}

// The twiddles of one real per thread: one per stage, for the thread's
// complex number j = t / 2.
template <int D>
struct SrftThreadTw {
    static constexpr int S = srft_detail::ilog2(D / 2);
    srft_detail::Cf w[S];

    __device__ __forceinline__ void load(int t)
    {
#pragma unroll
        for (int s = 0; s < S; ++s) {
            const int h = (D / 4) >> s;
            srft_detail::load_tw<1>(&w[s], h + ((t >> 1) & (h - 1)));
        }
    }
};

// The same transform over one real per thread (threads 0..D-1 of the block;
// threads past D hold no element and stay out of xch), without the final
// rot_norm: pairs up to 64 reals apart meet by lane exchange, wider ones
// through LDS.
template <int D>
__device__ __forceinline__ float srft_thread(float y, float* xch, const SrftThreadTw<D>& tw)
{
#pragma clang fp contract(off)
    constexpr int N = D / 2;
    const int t = threadIdx.x, j = t >> 1;
    const bool im = (t & 1) != 0;
#pragma unroll
    for (int s = 0; s < SrftThreadTw<D>::S; ++s) {
        const int h = (N / 2) >> s;
        float o;
        if (2 * h < 64) {
            o = shfl_xor(y, 2 * h);
        } else {
            __syncthreads();
            if (t < D) xch[t] = y;
            __syncthreads();
            o = t < D ? xch[t ^ (2 * h)] : y;
        }
        const float d = o - y;
        const float dd = shfl_xor(d, 1);
        const float wr = tw.w[s].re, wi = tw.w[s].im;
        const float up = im ? dd * wi + d * wr : d * wr - dd * wi;
        y = (j & h) ? up : y + o;
    }
    return y;
}

// The inverse transform over one real per thread, without the final
// rot_norm and signs: the stages undone in reverse order (half-size 1, 2,
// ..., N/2), a pair (a', b') becoming (a' + b' conj(W), a' - b' conj(W)).
// The upper element forms b' conj(W) and hands it to the lower one, which
// hands back a'.
template <int D>
__device__ __forceinline__ float isrft_thread(float y, float* xch, const SrftThreadTw<D>& tw)
{
#pragma clang fp contract(off)
    constexpr int N = D / 2;
    const int t = threadIdx.x, j = t >> 1;
    const bool im = (t & 1) != 0;
#pragma unroll
    for (int s = SrftThreadTw<D>::S - 1; s >= 0; --s) {
        const int h = (N / 2) >> s;
        const bool upper = (j & h) != 0;
        const float yd = shfl_xor(y, 1);  // the other component of the element's number
        const float wr = tw.w[s].re, wi = tw.w[s].im;
        const float prod = im ? y * wr - yd * wi : y * wr + yd * wi;
        const float send = upper ? prod : y;
        float o;
        if (2 * h < 64) {
            o = shfl_xor(send, 2 * h);
        } else {
            __syncthreads();
            if (t < D) xch[t] = send;
            __syncthreads();
            o = t < D ? xch[t ^ (2 * h)] : send;
        }
        y = upper ? o - prod : y + o;
    }
    return y;
}

// The complex product (dr wr - di wi, dr wi + di wr), products rounded
// before the sum; the real part when part == 0, else the imaginary part.
__device__ __forceinline__ float cmul_part(float dr, float di, float wr, float wi, int part)
{
#pragma clang fp contract(off)
    if (part == 0) {
        const float p1 = dr * wr, p2 = di * wi;
        return p1 - p2;
    }
    const float p3 = dr * wi, p4 = di * wr;
    return p3 + p4;
}

// The transform (without rot_norm) of a vector of D reals held one per
// thread (thread i < D holds real i, i.e. part i % 2 of complex i / 2),
// through LDS xch[D]; returns thread i's real of the result.  Threads past D
// take part in the barriers only.
template <int D>
__device__ __forceinline__ float srft_mixed_block(float y, float* xch)
{
#pragma clang fp contract(off)
    constexpr int N = D / 2, M = N / 3;
    static_assert(N % 3 == 0 && (M & (M - 1)) == 0, "N = 3 * 2^k");
    const int i = threadIdx.x, P = i >> 1, part = i & 1;
    const bool mine = i < D;
    __syncthreads();
    if (mine) xch[i] = y;
    __syncthreads();
    if (mine) {  // the radix-3 stage: output position P = m M + j
        const int m = P / M, j = P % M;
        const float a0r = xch[2 * j], a0i = xch[2 * j + 1];
        const float a1r = xch[2 * (j + M)], a1i = xch[2 * (j + M) + 1];
        const float a2r = xch[2 * (j + 2 * M)], a2i = xch[2 * (j + 2 * M) + 1];
        const float sr = a1r + a2r, si = a1i + a2i;
        const float dr = a1r - a2r, di = a1i - a2i;
        const float hr = 0.5f * sr, hi = 0.5f * si;
        const float mr = a0r - hr, mi = a0i - hi;
        const float tr = srft_detail::kC3 * dr, ti = srft_detail::kC3 * di;
        if (m == 0) {
            y = part ? a0i + si : a0r + sr;
        } else if (m == 1) {  // (m - i t) W^j
            const float br = mr + ti, bi = mi - tr;
            y = cmul_part(br, bi, srft_detail::kTw96.re[j], srft_detail::kTw96.im[j], part);
        } else {  // (m + i t) W^2j
            const float br = mr - ti, bi = mi + tr;
            y = cmul_part(br, bi, srft_detail::kTw96.re[2 * j], srft_detail::kTw96.im[2 * j], part);
        }
    }
#pragma unroll
    for (int h = M / 2; h >= 1; h >>= 1) {  // radix-2 stages inside each block of M
        __syncthreads();
        if (mine) xch[i] = y;
        __syncthreads();
        if (mine) {
            const int q = P % M, w = q & (2 * h - 1);  // position inside the 2h-block
            if (w < h) {
                y = xch[2 * P + part] + xch[2 * (P + h) + part];
            } else {
                const int lo = P - h;
                const float dr = xch[2 * lo] - xch[2 * P], di = xch[2 * lo + 1] - xch[2 * P + 1];
                const int t = (w - h) * (N / (2 * h));
                y = cmul_part(dr, di, srft_detail::kTw96.re[t], srft_detail::kTw96.im[t], part);
            }
        }
    }
    return y;
}

}  // namespace otq
