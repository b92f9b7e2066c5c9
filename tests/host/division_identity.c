/* Host check of the arithmetic identities the bulk quantiser relies on: the
 * Markstein-corrected quotients equal the IEEE fp32 quotients, and the
 * rounding-constant packing equals the clamp(rint(.)) codes.
 *
 *   ./division_identity exhaustive   a / 7 for every a of six binades of
 *                                    [2^-80, 2^100] and for 2^100
 *   ./division_identity random N     N draws of (x, s = RN(a / 7)): x / s and
 *                                    the 8-code word
 *   ./division_identity bits N       N draws each for qmax = 1 and 3 (the 2-
 *                                    and 3-bit quantiser): x / s and the codes
 *
 * Built with -ffp-contract=off; fmaf is the C library's correctly rounded
 * fused multiply-add.  Exit status 0 when no draw differs. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float fu(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t uf(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static const float kRecip7 = 1.0f / 7.0f; /* RN(1/7), 0x3E124925 */

static float div7(float a)
{
    float s = a * kRecip7;
    s = fmaf(fmaf(-s, 7.0f, a), kRecip7, s);
    return fmaf(fmaf(-s, 7.0f, a), kRecip7, s);
}

static float quot(float x, float s, float y)
{
    float q = x * y;
    q = fmaf(fmaf(-q, s, x), y, q);
    return fmaf(fmaf(-q, s, x), y, q);
}

/* splitmix64 */
static uint64_t rs = 0x9E3779B97F4A7C15ull;
static uint64_t next(void)
{
    uint64_t z = (rs += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

int main(int argc, char** argv)
{
    if (uf(kRecip7) != 0x3E124925u) {
        printf("RN(1/7) constant wrong\n");
        return 2;
    }
    if (argc >= 2 && strcmp(argv[1], "exhaustive") == 0) {
        /* Away from underflow and overflow every step scales exactly with a
         * power of two of a, so a binade's mantissas decide all binades; the
         * two lowest and highest binades of the range and two in its middle
         * are covered completely, with the range's end 2^100. */
        static const int binades[] = {-80, -79, -1, 0, 98, 99};
        uint64_t bad = 0, n = 0;
        for (int i = 0; i < 6; ++i) {
            const uint32_t lo = uf(ldexpf(1.0f, binades[i]));
            for (uint32_t u = lo; u < lo + (1u << 23); ++u, ++n)
                if (uf(div7(fu(u))) != uf(fu(u) / 7.0f)) ++bad;
        }
        if (uf(div7(0x1p100f)) != uf(0x1p100f / 7.0f)) ++bad;
        ++n;
        printf("a/7: %llu values, %llu differ\n", (unsigned long long)n, (unsigned long long)bad);
        return bad != 0;
    }
    if (argc >= 3 && strcmp(argv[1], "random") == 0) {
        const long n = atol(argv[2]);
        uint64_t badq = 0, badc = 0;
        for (long i = 0; i < n; ++i) {
            const uint64_t r = next(), r2 = next();
            const int ea = (int)(r % 181) - 80; /* a in [2^-80, 2^101) */
            float a = ldexpf(1.0f + (float)((r >> 8) & 0x7fffff) * 0x1p-23f, ea);
            if (a > 0x1p100f) a = 0x1p100f;
            const float s = a / 7.0f, y = 1.0f / s;
            uint32_t word_ref = 0, acc = 0;
            for (int e = 0; e < 8; ++e) {
                const uint64_t rr = next();
                float x;
                switch ((r2 >> (2 * e)) & 3) {
                case 0: /* uniform in [-a, a] */
                    x = a * ((float)(rr & 0xffffff) * 0x1p-23f - 1.0f);
                    break;
                case 1: { /* a few ulps around (k + 1/2) s */
                    const float t = ((float)((int)(rr % 15) - 7) + 0.5f) * s;
                    x = fu(uf(t) + (uint32_t)((int)((rr >> 8) % 9) - 4));
                    break;
                }
                case 2: /* a bf16 value below a */
                    x = fu(uf(a * (float)((rr & 0xffff) + 1) * 0x1p-16f) & 0xffff0000u);
                    if (rr & 0x10000) x = -x;
                    break;
                default: /* the group maximum itself */
                    x = (rr & 1) ? -a : a;
                }
                if (!(fabsf(x) <= a)) x = a;
                const float ref = x / s;
                const float q = quot(x, s, y);
                if (fabsf(ref) >= 0x1p-13f && uf(q) != uf(ref)) ++badq;
                float c = rintf(ref);
                c = fminf(fmaxf(c, -8.0f), 7.0f);
                word_ref |= ((uint32_t)(int)c & 0xFu) << (4 * e);
                acc += uf(q + (0x1.8p23f + 8.0f)) << (4 * e);
            }
            uint32_t cancel = 0;
            for (int e = 0; e < 8; ++e) cancel += 0x4B400000u << (4 * e);
            const uint32_t word = (acc - cancel) ^ 0x88888888u;
            if (word != word_ref) ++badc;
        }
        printf("x/s: %ld groups of 8, %llu quotients differ (|q| >= 2^-13), %llu words differ\n", n,
               (unsigned long long)badq, (unsigned long long)badc);
        return badq != 0 || badc != 0;
    }
    if (argc >= 3 && strcmp(argv[1], "bits") == 0) {
        /* the 2- and 3-bit quantiser: s = RN(a / qmax) by IEEE division for
         * qmax = 1 and 3, quotients as above, codes clamp(rint(q), -qmax - 1,
         * qmax) against those of the IEEE quotient, for every draw */
        const long n = atol(argv[2]);
        uint64_t badq = 0, badc = 0;
        for (int qm = 1; qm <= 3; qm += 2) {
            const float qmax = (float)qm, qmin = -(float)(qm + 1);
            for (long i = 0; i < n; ++i) {
                const uint64_t r = next(), r2 = next();
                const int ea = (int)(r % 181) - 80;
                float a = ldexpf(1.0f + (float)((r >> 8) & 0x7fffff) * 0x1p-23f, ea);
                if (a > 0x1p100f) a = 0x1p100f;
                const float s = a / qmax, y = 1.0f / s;
                for (int e = 0; e < 8; ++e) {
                    const uint64_t rr = next();
                    float x;
                    switch ((r2 >> (2 * e)) & 3) {
                    case 0:
                        x = a * ((float)(rr & 0xffffff) * 0x1p-23f - 1.0f);
                        break;
                    case 1: { /* a few ulps around (k + 1/2) s, k in [-qmax - 1, qmax] */
                        const float t = ((float)((int)(rr % (2 * qm + 2)) - qm - 1) + 0.5f) * s;
                        x = fu(uf(t) + (uint32_t)((int)((rr >> 8) % 9) - 4));
                        break;
                    }
                    case 2:
                        x = fu(uf(a * (float)((rr & 0xffff) + 1) * 0x1p-16f) & 0xffff0000u);
                        if (rr & 0x10000) x = -x;
                        break;
                    default:
                        x = (rr & 1) ? -a : a;
                    }
                    if (!(fabsf(x) <= a)) x = a;
                    const float ref = x / s;
                    const float q = quot(x, s, y);
                    if (fabsf(ref) >= 0x1p-13f && uf(q) != uf(ref)) ++badq;
                    const float c_ref = fminf(fmaxf(rintf(ref), qmin), qmax);
                    const float c = fminf(fmaxf(rintf(q), qmin), qmax);
                    if (c != c_ref) ++badc;
                }
            }
        }
        printf("b-bit x/s: 2 x %ld groups of 8, %llu quotients differ (|q| >= 2^-13), %llu codes differ\n", n,
               (unsigned long long)badq, (unsigned long long)badc);
        return badq != 0 || badc != 0;
    }
    fprintf(stderr, "usage: %s exhaustive | random N | bits N\n", argv[0]);
    return 2;
}
