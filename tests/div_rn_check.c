/* div_rn_check.c -- host check of the corrected division the quantizer kernels use for their
 * block scales (q = RN(a r_b), residual fma(-q, b, a), result fma(residual, r_b, q) with
 * r_b = RN(1 / b); Markstein's correction), against the correctly rounded IEEE division of
 * the host.  Built and run by tests/test_div_rn_cpu.py (gcc -O2 -ffp-contract=off -fopenmp).
 *
 *   exhaustive   every positive finite binary32 a, for b = 6 and b = 4: the results must be
 *                equal wherever the quotient is normal (the kernels take no decision on
 *                subnormal quotients: the block-scale code is 0 either way); those are
 *                counted and reported
 *   random       n pairs from a seeded generator: b with an exponent in [-92, 127), a = RN(q0 b)
 *                for q0 with an exponent in [-12, 10), kept when a is normal
 * Output: one line "div6 <bad> <subnormal-diff> div4 <bad> <subnormal-diff> random <bad> <n>". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float bits_f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

static float div_corrected(float a, float b, float rb)
{
    float q = a * rb;
    float r = fmaf(-q, b, a);
    return fmaf(r, rb, q);
}

static uint64_t mix64(uint64_t z)   /* splitmix64 finaliser */
{
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

static void fixed(float b, long long* bad, long long* sub)
{
    const float rb = 1.0f / b;
    long long nb = 0, ns = 0;
    #pragma omp parallel for schedule(static) reduction(+:nb, ns)
    for (int64_t u = 1; u < 0x7F800000; ++u) {
        const float a = bits_f((uint32_t)u);
        const float want = a / b, got = div_corrected(a, b, rb);
        if (want != got) {
            if (want >= 0x1p-126f) ++nb; else ++ns;
        }
    }
    *bad = nb;
    *sub = ns;
}

int main(int argc, char** argv)
{
    const int64_t n = argc > 1 ? atoll(argv[1]) : 100000000;
    long long b6, s6, b4, s4, br = 0;
    fixed(6.0f, &b6, &s6);
    fixed(4.0f, &b4, &s4);
    #pragma omp parallel for schedule(static) reduction(+:br)
    for (int64_t i = 0; i < n; ++i) {
        const uint64_t r = mix64((uint64_t)i + 0x5EEDull);
        const uint32_t eb = (uint32_t)((r >> 32) % 219u) + 35u;
        const uint32_t eq = (uint32_t)((r >> 24) % 22u) + 115u;
        const float b = bits_f((eb << 23) | (uint32_t)(r & 0x7FFFFFu));
        const float q0 = bits_f((eq << 23) | (uint32_t)((r >> 40) & 0x7FFFFFu));
        const float a = q0 * b;
        if (!(a >= 0x1p-126f) || !isfinite(a)) continue;
        if (a / b != div_corrected(a, b, 1.0f / b)) ++br;
    }
    printf("div6 %lld %lld div4 %lld %lld random %lld %lld\n", b6, s6, b4, s4, br, (long long)n);
    return 0;
}
