/*
 * oracle.c - plain, slow CPU reference for int4 KV-cache quantisation and
 * decode attention computed on the quantised cache.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this file: only the test suite, the smoke check and the
 * bench's CPU-baseline leg use it.  It shares no code, header, table or
 * constant with the GPU library.
 *
 * What it computes, and where that comes from:
 *
 *  - "Open-TQ-Metal: Fused Compressed-Domain Attention for Long-Context LLM
 *    Inference on Apple Silicon" (arXiv 2604.16957, abstract): the KV cache
 *    is quantised to int4 as it is produced, and attention is evaluated on
 *    the compressed form with no dequantised intermediate.  Skipping the
 *    intermediate does not change the mathematics, so the oracle simply
 *    dequantises (exactly, in fp64) and runs textbook softmax attention.
 *
 *  - "SRFT + int4 KV-cache" (agents-report page, section on the core method):
 *    every group gets its own abs-max, then symmetric int4 quantisation and
 *    nibble packing; rotation happens before quantisation, all in one pass.
 *
 *  - "AdapTQ" (zingnex page, section on Fast Hadamard Rotation): an
 *    O(d log d) in-place Hadamard rotation applied before quantisation to
 *    spread outliers.  The sign-randomised form (SRHT) is named on the
 *    agents-report page as the reference rotation.
 *
 * Readings where the pages are silent (each one listed in the design notes):
 * group = 32 contiguous channels; scale = abs-max / 7 in IEEE fp32;
 * code = round-half-to-even(x / scale) clamped to [-8, 7]; scale == 0 gives
 * all-zero codes; byte j holds element 2j in its low nibble and element
 * 2j+1 in its high nibble; rotation y = c * H_D * (s (.) x) with H_D the
 * Sylvester Hadamard matrix, butterflies in ascending stride order, and the
 * normalisation c applied last as one fp32 multiply; no fused multiply-add
 * anywhere in the fp32 quantiser (this file is built with
 * -ffp-contract=off).
 *
 * Rotated V (the same page's rotate-then-quantise applied to V as well,
 * with the output brought back by the inverse rotation): V rows may be
 * quantised with signs of their own, y = c * H_D * (s_v (.) v) exactly as K
 * is; attention then dequantises every V row back to the original basis in
 * fp64, v^ = s_v (.) (c * H_D * (code * scale)), since (c H_D S)^-1 =
 * S H_D c for c = 1/sqrt(D) and S = diag(s_v) of +-1.
 *
 * SRFT ("SRFT + int4 KV-cache", core-method section: a sign-randomised FFT
 * may take the place of the Hadamard rotation, with the same quality).
 * Reading: the D reals of a vector are D/2 complex numbers z_j = x_2j +
 * i x_2j+1 (after the signs), transformed by the radix-2 decimation-in-
 * frequency FFT in place (stages of half-size N/2, N/4, ..., 1 for N = D/2;
 * a stage replaces (a, b) with (a + b, (a - b) W^t), W = exp(-2 pi i / N),
 * t = (j mod h) N / (2h) for the pair's lower index j), which leaves the
 * DFT coefficient of index bitrev(k) at position k, and the result is
 * multiplied by c = 1/sqrt(N).  That map is orthogonal on R^D, so a query
 * rotated the same way keeps every dot product.  V may be rotated by the
 * same kind (its own signs), and attention then brings every dequantised V
 * row back by the inverse map in fp64.  In fp32 every step is one
 * IEEE operation: the complex product is (d_re w_re - d_im w_im, d_re w_im
 * + d_im w_re), each product rounded, then the sum; twiddles are the
 * correctly rounded fp32 values of cos and -sin of 2 pi t / N.
 *
 * Mixed radix ("SRFT + int4 KV-cache", core-method section and the
 * comparison of methods: the FFT's advantage over the Hadamard form is that
 * it is not tied to powers of two).  Reading: for N = 3 * 2^k complex
 * numbers, the decimation-in-frequency FFT takes one radix-3 stage first,
 * over the triples (a0, a1, a2) = (z_j, z_j+M, z_j+2M), M = N / 3, j < M:
 * the 3-point DFT with omega = exp(-2 pi i / 3), evaluated as s = a1 + a2,
 * d = a1 - a2, m = a0 - s / 2, t = c3 d (c3 = sqrt(3) / 2),
 * b0 = a0 + s, b1 = m - i t, b2 = m + i t, then z_j = b0,
 * z_j+M = b1 W_N^j, z_j+2M = b2 W_N^2j; then the radix-2 stages above run
 * inside each block of M.  Position M m + p then holds the DFT coefficient
 * of index 3 bitrev(p) + m, and c = 1/sqrt(N) as before.  In fp32 each of
 * those steps is one IEEE operation (s / 2 is the product by 0.5, and c3 is
 * the correctly rounded fp32 value).  The inverse undoes the radix-2
 * stages, then the radix-3 one: the twiddles are divided out (times their
 * conjugates) and the 3-point DFT with the conjugate root is applied.
 *
 * Other code widths (the AdapTQ page lists 2-bit and 3-bit quantisation
 * beside 4-bit; int2 is named as later work elsewhere).  Reading: b-bit
 * codes follow the same steps with the symmetric range of b bits, s = a /
 * (2^(b-1) - 1) and codes clamped to [-2^(b-1), 2^(b-1) - 1], and element i
 * of a row occupies bits [b i, b i + b) of the row's little-endian bit
 * stream, two's complement (for b = 4: the nibble order above).
 *
 * Per-channel scale ("SRFT + int4 KV-cache", core-method section: a
 * per-coordinate scale lambda is applied after the rotation and before the
 * group abs-max).  Reading: when a scale vector is given, the quantised
 * vector is z = lambda (.) y (one fp32 multiply per element, after the
 * rotation if there is one), and the cache then stands for y = z / lambda:
 * attention dequantises K^_i = code_i * s_g / lambda_i in fp64.
 *
 * Parity pins for every function here live in the CPU test suite.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_GROUP 32
#define ORACLE_PI 3.14159265358979323846

/* ---------------------------------------------------------------- widening */

/* IEEE binary16 -> binary32, from the format's definition:
 * normal  (e in 1..30): (1024 + m) * 2^(e - 25)
 * subnormal (e == 0)  :  m * 2^-24
 * e == 31             :  inf / nan                                       */
float oracle_f16_to_f32(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(m + 1024), e - 25);
    return (float)(sign ? -v : v);
}

/* bfloat16 is the upper half of a binary32 word. */
float oracle_bf16_to_f32(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

static float widen(uint16_t bits, int dtype)
{
    return dtype == 0 ? oracle_f16_to_f32(bits) : oracle_bf16_to_f32(bits);
}

/* ---------------------------------------------------------------- rotation */

/* y <- c * H_D * (s (.) y) in fp32, H_D Sylvester-ordered (H_1 = [1],
 * H_2n = [[H_n, H_n], [H_n, -H_n]]).  Stage h pairs element j with j + h
 * inside each block of 2h and replaces them with (a + b, a - b). */
void oracle_srht_f32(float *y, const float *signs, int D, float c)
{
    for (int i = 0; i < D; ++i)
        y[i] = y[i] * signs[i];
    for (int h = 1; h < D; h *= 2)
        for (int blk = 0; blk < D; blk += 2 * h)
            for (int j = blk; j < blk + h; ++j) {
                float a = y[j], b = y[j + h];
                y[j] = a + b;
                y[j + h] = a - b;
            }
    for (int i = 0; i < D; ++i)
        y[i] = y[i] * c;
}

/* The same rotation in fp64, used on the query so that q'.k' = q.k. */
void oracle_srht_f64(double *y, const float *signs, int D, double c)
{
    for (int i = 0; i < D; ++i)
        y[i] = y[i] * (double)signs[i];
    for (int h = 1; h < D; h *= 2)
        for (int blk = 0; blk < D; blk += 2 * h)
            for (int j = blk; j < blk + h; ++j) {
                double a = y[j], b = y[j + h];
                y[j] = a + b;
                y[j + h] = a - b;
            }
    for (int i = 0; i < D; ++i)
        y[i] = y[i] * c;
}

/* The inverse rotation in fp64: y <- s (.) (c * H_D * y). */
void oracle_unrotate_f64(double *y, const float *signs, int D, double c)
{
    for (int h = 1; h < D; h *= 2)
        for (int blk = 0; blk < D; blk += 2 * h)
            for (int j = blk; j < blk + h; ++j) {
                double a = y[j], b = y[j + h];
                y[j] = a + b;
                y[j + h] = a - b;
            }
    for (int i = 0; i < D; ++i)
        y[i] = y[i] * c * (double)signs[i];
}

/* Twiddle W_N^t = (cos(2 pi t / N), -sin(2 pi t / N)) for N a power of two
 * up to 2^20 and 0 <= t < N, evaluated through the symmetries of the first
 * octant, so that the quarter-turn values are exact and every other value
 * comes from cos or sin of an angle in (0, pi/4], where the library's
 * double results are accurate to an ulp. */
static void twiddle(int t, int N, double *wr, double *wi)
{
    /* angle = 2 pi t / N = (pi / 4) * u / Q with u = 8 t, Q = N */
    long u = 8L * t, Q = N;
    int oct = (int)(u / Q);     /* octant 0..7 */
    long rem = u - oct * Q;     /* angle inside the octant: (pi/4) rem / Q */
    double c, s;
    /* cos and sin of (pi/4) * m / Q for 0 <= m <= Q */
#define CS_Q(m, cc, ss)                                                   \
    do {                                                                  \
        if ((m) == 0) { cc = 1.0; ss = 0.0; }                             \
        else { double a_ = (ORACLE_PI / 4.0) * (double)(m) / (double)Q;        \
               cc = cos(a_); ss = sin(a_); }                              \
    } while (0)
    double c1, s1;
    switch (oct) {
    case 0: CS_Q(rem, c1, s1); c = c1; s = s1; break;                    /* a        */
    case 1: CS_Q(Q - rem, c1, s1); c = s1; s = c1; break;                /* pi/2 - b */
    case 2: CS_Q(rem, c1, s1); c = -s1; s = c1; break;                   /* pi/2 + a */
    case 3: CS_Q(Q - rem, c1, s1); c = -c1; s = s1; break;               /* pi - b   */
    case 4: CS_Q(rem, c1, s1); c = -c1; s = -s1; break;                  /* pi + a   */
    case 5: CS_Q(Q - rem, c1, s1); c = -s1; s = -c1; break;              /* 3pi/2 - b */
    case 6: CS_Q(rem, c1, s1); c = s1; s = -c1; break;                   /* 3pi/2 + a */
    default: CS_Q(Q - rem, c1, s1); c = c1; s = -s1; break;              /* 2pi - b  */
    }
#undef CS_Q
    /* zeros are +0 */
    *wr = c + 0.0;
    *wi = -s + 0.0;
}

/* fp32 twiddle: the double value rounded once to fp32. */
void oracle_twiddle_f32(int t, int N, float *wr, float *wi)
{
    double r, i;
    twiddle(t, N, &r, &i);
    *wr = (float)r;
    *wi = (float)i;
}

/* N complex numbers for the FFT rotation: a power of two, or three times
 * one (mixed radix); 0 for other N. */
static int fft_size_ok(int N)
{
    if (N < 1)
        return 0;
    if (N % 3 == 0)
        N /= 3;
    return (N & (N - 1)) == 0;
}

/* The radix-2 decimation-in-frequency stages over complex numbers
 * [base, base + n) of y (n a power of two), as part of an N-point
 * transform: the pair's twiddle exponent is (j mod h) n / (2h) of W_n, that
 * is (j mod h) N / (2h) of W_N. */
static void radix2_stages_f32(float *y, int base, int n, int N)
{
    for (int h = n / 2; h >= 1; h /= 2)
        for (int blk = base; blk < base + n; blk += 2 * h)
            for (int j = blk; j < blk + h; ++j) {
                float ar = y[2 * j], ai = y[2 * j + 1];
                float br = y[2 * (j + h)], bi = y[2 * (j + h) + 1];
                float wr, wi;
                oracle_twiddle_f32((j - blk) * (N / (2 * h)), N, &wr, &wi);
                float dr = ar - br, di = ai - bi;
                y[2 * j] = ar + br;
                y[2 * j + 1] = ai + bi;
                float p1 = dr * wr, p2 = di * wi, p3 = dr * wi, p4 = di * wr;
                y[2 * (j + h)] = p1 - p2;
                y[2 * (j + h) + 1] = p3 + p4;
            }
}

static void radix2_stages_f64(double *y, int base, int n, int N)
{
    for (int h = n / 2; h >= 1; h /= 2)
        for (int blk = base; blk < base + n; blk += 2 * h)
            for (int j = blk; j < blk + h; ++j) {
                double ar = y[2 * j], ai = y[2 * j + 1];
                double br = y[2 * (j + h)], bi = y[2 * (j + h) + 1];
                double wr, wi;
                twiddle((j - blk) * (N / (2 * h)), N, &wr, &wi);
                double dr = ar - br, di = ai - bi;
                y[2 * j] = ar + br;
                y[2 * j + 1] = ai + bi;
                y[2 * (j + h)] = dr * wr - di * wi;
                y[2 * (j + h) + 1] = dr * wi + di * wr;
            }
}

/* The radix-2 stages undone in reverse order (half-size 1, 2, ..., n/2),
 * without the factor 1/2 per stage: 2a = a' + b' conj(W), 2b = a' - b'
 * conj(W). */
static void unradix2_stages_f64(double *y, int base, int n, int N)
{
    for (int h = 1; h < n; h *= 2)
        for (int blk = base; blk < base + n; blk += 2 * h)
            for (int j = blk; j < blk + h; ++j) {
                double xr = y[2 * j], xi = y[2 * j + 1];
                double br = y[2 * (j + h)], bi = y[2 * (j + h) + 1];
                double wr, wi;
                twiddle((j - blk) * (N / (2 * h)), N, &wr, &wi);
                /* t = b' conj(W) */
                double tr = br * wr + bi * wi, ti = bi * wr - br * wi;
                y[2 * j] = xr + tr;
                y[2 * j + 1] = xi + ti;
                y[2 * (j + h)] = xr - tr;
                y[2 * (j + h) + 1] = xi - ti;
            }
}

/* sqrt(3) / 2, correctly rounded to fp32 and in double. */
static float c3_f32(void) { return (float)(sqrt(3.0) / 2.0); }

/* The radix-3 stage of an N-point transform (N = 3 M) in fp32, in the
 * order of operations given at the top. */
static void radix3_stage_f32(float *y, int N)
{
    const int M = N / 3;
    const float c3 = c3_f32();
    for (int j = 0; j < M; ++j) {
        float a0r = y[2 * j], a0i = y[2 * j + 1];
        float a1r = y[2 * (j + M)], a1i = y[2 * (j + M) + 1];
        float a2r = y[2 * (j + 2 * M)], a2i = y[2 * (j + 2 * M) + 1];
        float sr = a1r + a2r, si = a1i + a2i;
        float dr = a1r - a2r, di = a1i - a2i;
        float hr = 0.5f * sr, hi = 0.5f * si;
        float mr = a0r - hr, mi = a0i - hi;
        float tr = c3 * dr, ti = c3 * di;
        float b1r = mr + ti, b1i = mi - tr;   /* m - i t */
        float b2r = mr - ti, b2i = mi + tr;   /* m + i t */
        y[2 * j] = a0r + sr;
        y[2 * j + 1] = a0i + si;
        float wr, wi;
        oracle_twiddle_f32(j, N, &wr, &wi);
        float p1 = b1r * wr, p2 = b1i * wi, p3 = b1r * wi, p4 = b1i * wr;
        y[2 * (j + M)] = p1 - p2;
        y[2 * (j + M) + 1] = p3 + p4;
        oracle_twiddle_f32(2 * j, N, &wr, &wi);
        p1 = b2r * wr; p2 = b2i * wi; p3 = b2r * wi; p4 = b2i * wr;
        y[2 * (j + 2 * M)] = p1 - p2;
        y[2 * (j + 2 * M) + 1] = p3 + p4;
    }
}

static void radix3_stage_f64(double *y, int N)
{
    const int M = N / 3;
    const double c3 = sqrt(3.0) / 2.0;
    for (int j = 0; j < M; ++j) {
        double a0r = y[2 * j], a0i = y[2 * j + 1];
        double a1r = y[2 * (j + M)], a1i = y[2 * (j + M) + 1];
        double a2r = y[2 * (j + 2 * M)], a2i = y[2 * (j + 2 * M) + 1];
        double sr = a1r + a2r, si = a1i + a2i;
        double dr = a1r - a2r, di = a1i - a2i;
        double mr = a0r - 0.5 * sr, mi = a0i - 0.5 * si;
        double tr = c3 * dr, ti = c3 * di;
        double b1r = mr + ti, b1i = mi - tr, b2r = mr - ti, b2i = mi + tr;
        y[2 * j] = a0r + sr;
        y[2 * j + 1] = a0i + si;
        double wr, wi;
        twiddle(j, N, &wr, &wi);
        y[2 * (j + M)] = b1r * wr - b1i * wi;
        y[2 * (j + M) + 1] = b1r * wi + b1i * wr;
        twiddle(2 * j, N, &wr, &wi);
        y[2 * (j + 2 * M)] = b2r * wr - b2i * wi;
        y[2 * (j + 2 * M) + 1] = b2r * wi + b2i * wr;
    }
}

/* The radix-3 stage undone without its factor 1/3: the twiddles divided
 * out, then the 3-point DFT with the conjugate root. */
static void unradix3_stage_f64(double *y, int N)
{
    const int M = N / 3;
    const double c3 = sqrt(3.0) / 2.0;
    for (int j = 0; j < M; ++j) {
        double wr, wi;
        double b0r = y[2 * j], b0i = y[2 * j + 1];
        double zr = y[2 * (j + M)], zi = y[2 * (j + M) + 1];
        twiddle(j, N, &wr, &wi);
        double b1r = zr * wr + zi * wi, b1i = zi * wr - zr * wi;   /* z conj(W^j) */
        zr = y[2 * (j + 2 * M)]; zi = y[2 * (j + 2 * M) + 1];
        twiddle(2 * j, N, &wr, &wi);
        double b2r = zr * wr + zi * wi, b2i = zi * wr - zr * wi;
        double sr = b1r + b2r, si = b1i + b2i, dr = b1r - b2r, di = b1i - b2i;
        double mr = b0r - 0.5 * sr, mi = b0i - 0.5 * si;
        double tr = c3 * dr, ti = c3 * di;
        y[2 * j] = b0r + sr;
        y[2 * j + 1] = b0i + si;
        y[2 * (j + M)] = mr - ti;          /* m + i t: the conjugate root */
        y[2 * (j + M) + 1] = mi + tr;
        y[2 * (j + 2 * M)] = mr + ti;      /* m - i t */
        y[2 * (j + 2 * M) + 1] = mi - tr;
    }
}

/* y <- c * FFT_{D/2}(s (.) y) in fp32: the in-place decimation-in-frequency
 * FFT over z_j = (y[2j], y[2j+1]) described at the top (a radix-3 stage
 * first when D/2 is three times a power of two). */
void oracle_srft_f32(float *y, const float *signs, int D, float c)
{
    const int N = D / 2;
    for (int i = 0; i < D; ++i)
        y[i] = y[i] * signs[i];
    if (N % 3 == 0) {
        radix3_stage_f32(y, N);
        for (int b = 0; b < 3; ++b)
            radix2_stages_f32(y, b * (N / 3), N / 3, N);
    } else {
        radix2_stages_f32(y, 0, N, N);
    }
    for (int i = 0; i < D; ++i)
        y[i] = y[i] * c;
}

/* The same transform in fp64 (twiddles in double), used on the query. */
void oracle_srft_f64(double *y, const float *signs, int D, double c)
{
    const int N = D / 2;
    for (int i = 0; i < D; ++i)
        y[i] = y[i] * (double)signs[i];
    if (N % 3 == 0) {
        radix3_stage_f64(y, N);
        for (int b = 0; b < 3; ++b)
            radix2_stages_f64(y, b * (N / 3), N / 3, N);
    } else {
        radix2_stages_f64(y, 0, N, N);
    }
    for (int i = 0; i < D; ++i)
        y[i] = y[i] * c;
}

/* The inverse of oracle_srft_f64 in fp64: y <- s (.) (c * U(y)), where U
 * undoes the stages in reverse order without their factors 1/2 and 1/3:
 * together those factors are N, which with the forward c = 1/sqrt(N) makes
 * the final factor c again. */
void oracle_unsrft_f64(double *y, const float *signs, int D, double c)
{
    const int N = D / 2;
    if (N % 3 == 0) {
        for (int b = 0; b < 3; ++b)
            unradix2_stages_f64(y, b * (N / 3), N / 3, N);
        unradix3_stage_f64(y, N);
    } else {
        unradix2_stages_f64(y, 0, N, N);
    }
    for (int i = 0; i < D; ++i)
        y[i] = y[i] * c * (double)signs[i];
}

/* Whether a head width admits rotation kind `kind` (0 = SRHT: a power of
 * two; 1 = SRFT: D/2 a power of two or three times one). */
static int rotation_ok(int D, int kind)
{
    return kind == 1 ? (D % 2 == 0 && fft_size_ok(D / 2)) : (D & (D - 1)) == 0;
}

/* K's rotation by kind: 0 = SRHT, 1 = SRFT. */
static void rotate_f32(float *y, const float *signs, int D, float c, int kind)
{
    if (kind == 1)
        oracle_srft_f32(y, signs, D, c);
    else
        oracle_srht_f32(y, signs, D, c);
}

static void rotate_f64(double *y, const float *signs, int D, double c, int kind)
{
    if (kind == 1)
        oracle_srft_f64(y, signs, D, c);
    else
        oracle_srht_f64(y, signs, D, c);
}

static void unrotate_f64(double *y, const float *signs, int D, double c, int kind)
{
    if (kind == 1)
        oracle_unsrft_f64(y, signs, D, c);
    else
        oracle_unrotate_f64(y, signs, D, c);
}

/* ---------------------------------------------------------------- quantise */

/* One vector x[D] (already widened to fp32, already rotated if rotation is
 * on) -> codes[D/2] packed nibbles and scales[D/32]. */
void oracle_quantize_vector(const float *x, int D, uint8_t *codes, float *scales)
{
    int8_t c[1024];
    for (int g = 0; g < D / ORACLE_GROUP; ++g) {
        const float *xg = x + g * ORACLE_GROUP;
        float a = 0.0f;
        for (int i = 0; i < ORACLE_GROUP; ++i) {
            float v = fabsf(xg[i]);
            if (v > a)
                a = v;
        }
        float s = a / 7.0f;
        scales[g] = s;
        for (int i = 0; i < ORACLE_GROUP; ++i) {
            int8_t code = 0;
            if (s != 0.0f) {
                float r = rintf(xg[i] / s); /* default rounding: half to even */
                if (r != r)
                    r = 0.0f; /* non-finite input: unspecified, kept defined */
                if (r > 7.0f)
                    r = 7.0f;
                if (r < -8.0f)
                    r = -8.0f;
                code = (int8_t)r;
            }
            c[g * ORACLE_GROUP + i] = code;
        }
    }
    for (int j = 0; j < D / 2; ++j)
        codes[j] = (uint8_t)((c[2 * j] & 0xF) | ((c[2 * j + 1] & 0xF) << 4));
}

/* One vector x[D] -> b-bit codes (b = 2, 3 or 4) packed into D b / 8 bytes
 * (element i at bits [b i, b i + b) of the little-endian bit stream) and
 * scales[D/32], s = abs-max / (2^(b-1) - 1) in IEEE fp32. */
void oracle_quantize_vector_bits(const float *x, int D, int bits, uint8_t *codes, float *scales)
{
    const float qmax = (float)((1 << (bits - 1)) - 1);
    const float qmin = -(float)(1 << (bits - 1));
    memset(codes, 0, (size_t)D * bits / 8);
    for (int g = 0; g < D / ORACLE_GROUP; ++g) {
        const float *xg = x + g * ORACLE_GROUP;
        float a = 0.0f;
        for (int i = 0; i < ORACLE_GROUP; ++i) {
            float v = fabsf(xg[i]);
            if (v > a)
                a = v;
        }
        float s = a / qmax;
        scales[g] = s;
        for (int i = 0; i < ORACLE_GROUP; ++i) {
            int code = 0;
            if (s != 0.0f) {
                float r = rintf(xg[i] / s);
                if (r != r)
                    r = 0.0f;
                if (r > qmax)
                    r = qmax;
                if (r < qmin)
                    r = qmin;
                code = (int)r;
            }
            const unsigned u = (unsigned)code & ((1u << bits) - 1u);
            const long pos = (long)(g * ORACLE_GROUP + i) * bits;
            for (int k = 0; k < bits; ++k)
                if ((u >> k) & 1u)
                    codes[(pos + k) >> 3] |= (uint8_t)(1u << ((pos + k) & 7));
        }
    }
}

/* Signed value of the b-bit code of element i of a packed row. */
static int code_at(const uint8_t *row, int i, int bits)
{
    const long pos = (long)i * bits;
    unsigned u = 0;
    for (int k = 0; k < bits; ++k)
        u |= (unsigned)((row[(pos + k) >> 3] >> ((pos + k) & 7)) & 1) << k;
    return u >= (1u << (bits - 1)) ? (int)u - (1 << bits) : (int)u;
}

struct qrows_job {
    const uint16_t *src;
    int dtype;
    long n0, n1;
    int D;
    const float *signs;
    float rot_norm;
    int rot_kind;
    const float *chan_scale;
    int bits;
    uint8_t *codes;
    float *scales;
};

static void *qrows_worker(void *arg)
{
    struct qrows_job *j = (struct qrows_job *)arg;
    float x[1024];
    for (long n = j->n0; n < j->n1; ++n) {
        for (int i = 0; i < j->D; ++i)
            x[i] = widen(j->src[n * j->D + i], j->dtype);
        if (j->signs)
            rotate_f32(x, j->signs, j->D, j->rot_norm, j->rot_kind);
        if (j->chan_scale)
            for (int i = 0; i < j->D; ++i)
                x[i] = x[i] * j->chan_scale[i];
        oracle_quantize_vector_bits(x, j->D, j->bits, j->codes + n * (j->D * j->bits / 8),
                                    j->scales + n * (j->D / ORACLE_GROUP));
    }
    return NULL;
}

/* N rows of D 16-bit values (dtype 0 = fp16, 1 = bf16) -> N rows of codes
 * and scales.  signs == NULL means no rotation (else rot_kind 0 = SRHT,
 * 1 = SRFT), chan_scale == NULL no per-channel scale.  Rows are independent, so spreading them over threads
 * does not change any result. */
int oracle_quantize_rows(const uint16_t *src, int dtype, long N, int D,
                         const float *signs, float rot_norm, int rot_kind,
                         const float *chan_scale, int bits, uint8_t *codes, float *scales,
                         int nthreads)
{
    if (D <= 0 || D > 1024 || D % ORACLE_GROUP != 0 || N < 0 || dtype < 0 || dtype > 1 ||
        rot_kind < 0 || rot_kind > 1 || bits < 2 || bits > 4)
        return -1;
    if (signs && !rotation_ok(D, rot_kind))
        return -1;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    pthread_t th[256];
    struct qrows_job jobs[256];
    long per = (N + nthreads - 1) / nthreads;
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        long n0 = t * per, n1 = n0 + per > N ? N : n0 + per;
        if (n0 >= n1)
            break;
        jobs[t] = (struct qrows_job){src, dtype, n0, n1, D, signs, rot_norm, rot_kind,
                                     chan_scale, bits, codes, scales};
        if (nthreads == 1) {
            qrows_worker(&jobs[t]);
        } else {
            pthread_create(&th[t], NULL, qrows_worker, &jobs[t]);
            ++started;
        }
    }
    for (int t = 0; t < started; ++t)
        pthread_join(th[t], NULL);
    return 0;
}

/* ---------------------------------------------------------------- attend */

/* One query row against one head's cache rows t < T:
 *   K^[t][i] = code * scale  (exact in fp64), divided by lambda_i when a
 *              per-channel scale is given
 *   S_t      = scale_attn * sum_i q'_i K^[t][i]
 *   w_t      = exp(S_t - max_u S_u)
 *   V^[t][i] = code * scale, brought back to the original basis (the
 *              inverse rotation of kind rot_kind) when v_signs != NULL
 *   out      = sum_t w_t V^[t] / sum_t w_t
 * T == 0 gives out = 0.  q' is q rotated in fp64 when signs != NULL (rot_kind
 * 0 = SRHT, 1 = SRFT; the same kind serves V).
 * work must hold T doubles. */
void oracle_attend_row(const uint16_t *q, int dtype, int D,
                       const uint8_t *kc, const float *ks,
                       const uint8_t *vc, const float *vs, long T,
                       double scale, const float *signs, float rot_norm, int rot_kind,
                       const float *chan_scale, const float *v_signs, int bits, double *work,
                       double *out)
{
    double qd[1024], kd[1024], vd[1024];
    int ng = D / ORACLE_GROUP;
    for (int i = 0; i < D; ++i)
        qd[i] = (double)widen(q[i], dtype);
    if (signs)
        rotate_f64(qd, signs, D, (double)rot_norm, rot_kind);
    for (int i = 0; i < D; ++i)
        out[i] = 0.0;
    if (T <= 0)
        return;

    double m = -INFINITY;
    for (long t = 0; t < T; ++t) {
        const uint8_t *row = kc + t * (D * bits / 8);
        const float *srow = ks + t * ng;
        for (int i = 0; i < D; ++i) {
            kd[i] = (double)code_at(row, i, bits) * (double)srow[i / ORACLE_GROUP];
            if (chan_scale)
                kd[i] /= (double)chan_scale[i];
        }
        double dot = 0.0;
        for (int i = 0; i < D; ++i)
            dot += qd[i] * kd[i];
        work[t] = scale * dot;
        if (work[t] > m)
            m = work[t];
    }
    double l = 0.0;
    for (long t = 0; t < T; ++t) {
        double w = exp(work[t] - m);
        l += w;
        const uint8_t *row = vc + t * (D * bits / 8);
        const float *srow = vs + t * ng;
        for (int i = 0; i < D; ++i)
            vd[i] = (double)code_at(row, i, bits) * (double)srow[i / ORACLE_GROUP];
        if (v_signs)
            unrotate_f64(vd, v_signs, D, (double)rot_norm, rot_kind);
        for (int i = 0; i < D; ++i)
            out[i] += w * vd[i];
    }
    for (int i = 0; i < D; ++i)
        out[i] /= l;
}

struct attn_job {
    const uint16_t *q;
    int dtype, B, Hq, Hkv, D;
    long cap;
    const uint8_t *kc, *vc;
    const float *ks, *vs;
    const int32_t *lens;
    double scale;
    const float *signs;
    float rot_norm;
    int rot_kind;
    const float *chan_scale;
    const float *v_signs;
    int bits;
    double *out;
    const int32_t *rows;
    long r0, r1;
};

static void *attn_worker(void *arg)
{
    struct attn_job *j = (struct attn_job *)arg;
    double *work = (double *)malloc(sizeof(double) * (size_t)(j->cap > 0 ? j->cap : 1));
    if (!work)
        return NULL;
    int G = j->Hq / j->Hkv;
    for (long r = j->r0; r < j->r1; ++r) {
        long row = j->rows ? j->rows[r] : r; /* row = b * Hq + h */
        int b = (int)(row / j->Hq), h = (int)(row % j->Hq), hk = h / G;
        long T = j->lens[b];
        if (T > j->cap)
            T = j->cap;
        size_t head = (size_t)b * j->Hkv + hk;
        const size_t rb = (size_t)j->D * j->bits / 8;  /* code bytes per row */
        oracle_attend_row(j->q + (size_t)row * j->D, j->dtype, j->D,
                          j->kc + head * j->cap * rb, j->ks + head * j->cap * (j->D / ORACLE_GROUP),
                          j->vc + head * j->cap * rb, j->vs + head * j->cap * (j->D / ORACLE_GROUP),
                          T, j->scale, j->signs, j->rot_norm, j->rot_kind, j->chan_scale,
                          j->v_signs, j->bits, work,
                          j->out + (size_t)r * j->D);
    }
    free(work);
    return NULL;
}

/* Decode attention for a batch.  q: [B][Hq][D] 16-bit; cache in the plain
 * layout codes [B][Hkv][cap][D/2], scales [B][Hkv][cap][D/32]; lens [B].
 * Query head h reads KV head h / (Hq / Hkv).  If rows != NULL only the
 * listed rows (b * Hq + h) are computed and out is [nrows][D]; otherwise
 * out is [B * Hq][D].  Threads split rows; results do not depend on them. */
int oracle_sdpa(const uint16_t *q, int dtype, int B, int Hq, int Hkv, int D, long cap,
                const uint8_t *kc, const float *ks, const uint8_t *vc, const float *vs,
                const int32_t *lens, double scale, const float *signs, float rot_norm,
                int rot_kind, const float *chan_scale, const float *v_signs, int bits,
                const int32_t *rows, long nrows, double *out, int nthreads)
{
    if (B < 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv != 0 || D <= 0 || D > 1024 ||
        D % ORACLE_GROUP != 0 || cap < 0 || dtype < 0 || dtype > 1 || rot_kind < 0 ||
        rot_kind > 1 || bits < 2 || bits > 4)
        return -1;
    if ((signs || v_signs) && !rotation_ok(D, rot_kind))
        return -1;
    long R = rows ? nrows : (long)B * Hq;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > 256)
        nthreads = 256;
    pthread_t th[256];
    struct attn_job jobs[256];
    long per = (R + nthreads - 1) / nthreads;
    int started = 0;
    for (int t = 0; t < nthreads; ++t) {
        long r0 = t * per, r1 = r0 + per > R ? R : r0 + per;
        if (r0 >= r1)
            break;
        jobs[t] = (struct attn_job){q, dtype, B, Hq, Hkv, D, cap, kc, vc, ks, vs, lens,
                                    scale, signs, rot_norm, rot_kind, chan_scale, v_signs, bits,
                                    out, rows, r0, r1};
        if (nthreads == 1) {
            attn_worker(&jobs[t]);
        } else {
            pthread_create(&th[t], NULL, attn_worker, &jobs[t]);
            ++started;
        }
    }
    for (int t = 0; t < started; ++t)
        pthread_join(th[t], NULL);
    return 0;
}
