/*
 * nvfp4_oracle.c -- plain scalar CPU reference of the NVFP4 quantized linear
 * path.  TEST INFRASTRUCTURE ONLY (tests, the package smoke check and the
 * benchmark's CPU-baseline leg); the GPU library never links or calls it and
 * shares no code with it.  Source passages are cited per function with the page
 * tags explained in nvfp4_oracle.h.
 *
 * Build: gcc -O2 -std=c11 -ffp-contract=off -fopenmp -fPIC -shared.
 * Nothing here is blocked, fused or reordered beyond what each definition
 * states; loops over independent rows carry an OpenMP pragma and nothing else.
 */
#include "nvfp4_oracle.h"
#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* ------------------------------------------------------------------------- */
/* E2M1 element format.                                                       */
/* [FS4] sec. 2: NVFP4 elements are E2M1 (1 sign, 2 exponent, 1 mantissa bit). */
/* [OPT] enumerates the positive grid with exponent bias 1: e = 0 is          */
/* subnormal (0 and 0.5), e = 1..3 are normal (1, 1.5, 2, 3, 4, 6).           */
/* Bit order taken: code = sign<<3 | exponent<<1 | mantissa (the field order  */
/* of the enumeration); code 8 decodes to -0.                                 */
/* ------------------------------------------------------------------------- */
double or_e2m1_value(int code)
{
    int s = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int m = code & 1;
    double mag;
    if (e == 0)
        mag = 0.5 * m;                                  /* 2^(1-bias) * 0.m */
    else
        mag = ldexp(1.0 + 0.5 * m, e - 1);              /* 2^(e-bias) * 1.m */
    return s ? -mag : mag;
}

/* Nearest grid magnitude, ties to the even code, saturating at 6.
 * [NVP] sec. 4: weights and activations use round-to-nearest-even; [FS4] sec. 2
 * calls the deterministic mode RTN and Appendix 7 lists the saturation cell
 * [5, inf).  Reading: ties go to the even code (the RNE of [NVP]); the
 * half-open bins printed in Appendix 7 describe an input-averaged analysis in
 * which ties have measure zero. */
int or_e2m1_rne(float u)
{
    if (!(u <= 6.0f))
        return 7;                                       /* saturation (and +inf) */
    int best = 0;
    double bestd = fabs((double)u - or_e2m1_value(0));
    for (int c = 1; c < 8; ++c) {
        double d = fabs((double)u - or_e2m1_value(c));  /* exact in binary64 */
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bestd = d;
        }
    }
    return best;
}

/* Stochastic rounding: [FS4] Appendix 7, "Stochastic rounding": for u in bin
 * [c_k, c_{k+1}] with d = u - c_k, round up to c_{k+1} with probability
 * d / Delta_k.  Reading for the random draw: 16 uniform bits r per element and
 * "round up iff d/Delta_k + r/2^16 >= 1", i.e. add the random fraction below the
 * kept precision and truncate; P(up) = floor(2^16 d/Delta_k) / 2^16, within
 * 2^-16 of d/Delta_k.  Magnitudes at or above 6 stay 6 (saturation cell). */
int or_e2m1_sr(float u, uint32_t r16)
{
    if (!(u < 6.0f))
        return 7;
    int k = 0;                                          /* largest c with value(c) <= u */
    for (int c = 1; c < 8; ++c)
        if (or_e2m1_value(c) <= (double)u)
            k = c;
    double lo = or_e2m1_value(k), hi = or_e2m1_value(k + 1);
    double frac = ((double)u - lo) / (hi - lo);         /* exact: Delta is 0.5, 1 or 2 */
    double need = 1.0 - (double)(r16 & 0xFFFFu) / 65536.0;
    return frac >= need ? k + 1 : k;
}

/* ------------------------------------------------------------------------- */
/* E4M3 block scale.  [FS4] sec. 2 and [NVP] sec. 2 name FP8 E4M3 scales.     */
/* Reading: the OCP FP8 E4M3 ("fn") encoding -- bias 7, subnormal step 2^-9,  */
/* largest finite 448 (code 0x7E), 0x7F is NaN, no infinity.  Scales are       */
/* non-negative so the sign bit is always 0.                                  */
/* ------------------------------------------------------------------------- */
double or_e4m3_value(uint8_t code)
{
    int e = (code >> 3) & 15;
    int m = code & 7;
    double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return (code & 0x80) ? -mag : mag;
}

uint8_t or_e4m3_encode(float v)
{
    if (v >= 448.0f)
        return 0x7E;                                    /* saturate */
    int best = 0;
    double bestd = fabs((double)v);
    for (int c = 1; c <= 0x7E; ++c) {
        double d = fabs((double)v - or_e4m3_value((uint8_t)c));
        if (d < bestd || (d == bestd && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            bestd = d;
        }
    }
    return (uint8_t)best;
}

/* bfloat16 nearest-even: [GST] sec. 2.2 and [FS4] sec. 3.3 store the tile mean
 * in BF16; the conversion is the IEEE nearest-even one. */
float or_bf16_value(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

uint16_t or_bf16_rne(float v)
{
    uint32_t u;
    memcpy(&u, &v, 4);
    uint16_t lo = (uint16_t)(u >> 16);                  /* truncation toward zero */
    uint16_t hi = (uint16_t)(lo + 1);                   /* next magnitude up */
    double dl = fabs((double)v - (double)or_bf16_value(lo));
    double dh = fabs((double)v - (double)or_bf16_value(hi));
    if (dl < dh) return lo;
    if (dh < dl) return hi;
    return (lo & 1) ? hi : lo;
}

/* ------------------------------------------------------------------------- */
/* Philox4x32-10, the counter-based generator of Salmon et al. (SC'11):       */
/* each round multiplies words 0 and 2 by the two published multipliers,      */
/* and the output is (hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0); the key is     */
/* bumped by the two Weyl constants between rounds.                            */
/* ------------------------------------------------------------------------- */
void or_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4])
{
    uint32_t c0 = ctr[0], c1 = ctr[1], c2 = ctr[2], c3 = ctr[3];
    uint32_t k0 = key[0], k1 = key[1];
    for (int round = 0; round < 10; ++round) {
        uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* Counter layout (a convention; the pages name no generator):
 *   key = (seed low 32 bits, seed high 32 bits)
 *   SR draw for element j of a copy: counter (lo32(j/8), hi32(j/8), copy_id, "SR16"),
 *        16 bits = half (j mod 2) of word ((j/2) mod 4)
 *   RHT signs: counter (0, 0, 0, "RHT1"), bit i of word 0 set means D_ii = -1. */
#define OR_TAG_SR16 0x53523136u
#define OR_TAG_RHT1 0x52485431u

uint32_t or_sr_bits(uint64_t seed, uint32_t copy_id, uint64_t j)
{
    uint64_t group = j >> 3;
    uint32_t ctr[4] = {(uint32_t)group, (uint32_t)(group >> 32), copy_id, OR_TAG_SR16};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    or_philox4x32_10(ctr, key, out);
    uint32_t w = out[(j >> 1) & 3];
    return (j & 1) ? (w >> 16) : (w & 0xFFFFu);
}

void or_rht_signs(uint64_t seed, float sgn[16])
{
    uint32_t ctr[4] = {0u, 0u, 0u, OR_TAG_RHT1};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    or_philox4x32_10(ctr, key, out);
    for (int i = 0; i < 16; ++i)
        sgn[i] = ((out[0] >> i) & 1u) ? -1.0f : 1.0f;
}

/* ------------------------------------------------------------------------- */
/* Hadamard transform.  [OPT]: H_1 = [1], H_2k = [[H_k, H_k], [H_k, -H_k]];    */
/* the random transform multiplies by (1/sqrt(N)) H D with D a random sign     */
/* diagonal.  [NVP] B.4: rotate before quantizing, compute the scale in the    */
/* rotated space; orthogonal factors cancel across the two GEMM operands.     */
/* [FS4] sec. 3.2: one 16x16 random Hadamard matrix per backward pass;         */
/* sec. 3.3: O(16 log 16) fast transform.                                     */
/* Butterfly convention: stages h = 1, 2, 4, 8; pair (i, i+h) with bit h of i  */
/* clear becomes (a + b, a - b).  This computes H16 * v in Sylvester order.    */
/* ------------------------------------------------------------------------- */
void or_wht16(float v[16])
{
    for (int h = 1; h < 16; h <<= 1)
        for (int i = 0; i < 16; ++i)
            if ((i & h) == 0) {
                float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
}

void or_rht16_forward(float v[16], const float sgn[16])
{
    for (int i = 0; i < 16; ++i) v[i] = v[i] * sgn[i];
    or_wht16(v);
    for (int i = 0; i < 16; ++i) v[i] = v[i] * 0.25f;
}

void or_rht16_inverse(float v[16], const float sgn[16])
{
    or_wht16(v);
    for (int i = 0; i < 16; ++i) v[i] = v[i] * 0.25f;
    for (int i = 0; i < 16; ++i) v[i] = v[i] * sgn[i];
}

/* ------------------------------------------------------------------------- */
/* Quantization of one copy along its rows.                                    */
/* [FS4] sec. 2: x_hat = x_E2M1 * s * s_g, one E4M3 s per 1x16 or 16x16 block  */
/* and one FP32 s_g per tensor.  [NVP] sec. 2: each block's absolute maximum   */
/* maps to the FP4 maximum; the FP32 tensor scale keeps block scales inside    */
/* E4M3.  [FS4] App. 10.1: s_b = max|x| / 6.                                   */
/* Readings: s_g = fl(amax_t / (6*448)) so the block holding the tensor amax   */
/* gets s = 448; s_g = 1 if that is 0 (all-zero tensor); s = E4M3(fl(fl(amax_b */
/* / 6) / s_g)); elements are scaled by the reciprocal r = fl(1 / fl(s*s_g)),  */
/* u = fl(|x| * r); a zero scale gives magnitude 0.  The sign of x is kept in  */
/* the code (a negative value that rounds to 0 gives code 8).                  */
/* ------------------------------------------------------------------------- */
static int all_finite(const float* x, int64_t count)
{
    for (int64_t i = 0; i < count; ++i)
        if (!isfinite(x[i])) return 0;
    return 1;
}

/* Element scaling u = |x| / (s s_g) ([FS4] sec. 2: x_hat = x_E2M1 s s_g).  Reading
 * ([NVP] sec. 2, "reciprocal scale"): one correctly rounded reciprocal R of d = fl(s s_g) per
 * block, kept at binary32 precision, and u = fl(|x| R).  Where R's exponent leaves binary32's
 * range (d below about 2^-128, which needs a tensor maximum below about 2^-107), R is held
 * as R 2^-64 = fl(1 / (d 2^64)): scaling d up by 2^64 is exact, and both that reciprocal
 * (at most 2^85, as d >= 2^-149) and |x| R 2^-64 (at least 2^-85 for x != 0) are normal, so
 * fl(|x| (R 2^-64)) 2^64 = fl(|x| R). */
static float scale_element(float x, float d)
{
    float rcp = 1.0f / d;
    if (!isinf(rcp))
        return fabsf(x) * rcp;
    return (fabsf(x) * (1.0f / (d * 0x1p64f))) * 0x1p64f;
}

/* 4/6 adaptive block scaling.  [FS4] sec. 3 (and the introduction's list of
 * primitives) applies "4/6 scaling" to every NVFP4 quantization and the related-work
 * paragraph describes it as MSE-optimal adaptive block scaling; the rule itself is not
 * given.  Reading: each 1x16 block has two candidate E4M3 scales,
 * the usual one mapping the block amax to 6 and one mapping it to 4, both formed by the
 * same nearest-even saturating encode with the tensor scale unchanged; the block keeps
 * the candidate whose nearest-even quantization has the smaller squared error, 6 on a
 * tie.  The squared error is taken in binary32 in a fixed order: per element
 * e = fma(-(v s), s_g, y) with v the signed decoded code, accumulated as
 * (fma chain over elements 0..7) + (fma chain over elements 8..15).  With stochastic
 * rounding the choice is the same (made on nearest-even errors) and the elements are
 * then rounded stochastically with the chosen scale. */
static float block_sse_rne(const float* y, uint8_t scode, float sg)
{
    float part[2] = {0.0f, 0.0f};
    float s = (float)or_e4m3_value(scode);
    for (int i = 0; i < 16; ++i) {
        int mag = scode ? or_e2m1_rne(scale_element(y[i], s * sg)) : 0;
        float v = (float)or_e2m1_value(mag);
        if (signbit(y[i])) v = -v;
        float e = fmaf(-(v * s), sg, y[i]);
        part[i / 8] = fmaf(e, e, part[i / 8]);
    }
    return part[0] + part[1];
}

/* Measurement, not part of the method: the same squared error in binary64 (each error
 * y - v s s_g exact, its square and the sum rounded to 53 bits), to count how often the
 * binary32 evaluation order above decides a 4/6 choice differently. */
static double block_sse_f64(const float* y, uint8_t scode, float sg)
{
    double acc = 0.0;
    float s = (float)or_e4m3_value(scode);
    for (int i = 0; i < 16; ++i) {
        int mag = scode ? or_e2m1_rne(scale_element(y[i], s * sg)) : 0;
        double v = or_e2m1_value(mag);
        if (signbit(y[i])) v = -v;
        double e = (double)y[i] - v * (double)s * (double)sg;
        acc += e * e;
    }
    return acc;
}

/* Quantize already-transformed values y[n][k]. */
static void quantize_core(const float* y, int64_t n, int64_t k, int block2d, int rounding,
                          int scale46, uint64_t seed, uint32_t copy_id,
                          uint8_t* codes, uint8_t* scales, float* sg_out)
{
    float amax_t = 0.0f;
    for (int64_t i = 0; i < n * k; ++i) {
        float a = fabsf(y[i]);
        if (a > amax_t) amax_t = a;
    }
    float sg = amax_t / 2688.0f;                        /* 2688 = 6 * 448 */
    if (sg == 0.0f) sg = 1.0f;
    *sg_out = sg;

    int64_t kb = k / 16;
    /* block scales */
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t b = 0; b < kb; ++b) {
            float amax_b = 0.0f;
            int64_t r0 = block2d ? (r / 16) * 16 : r;
            int64_t r1 = block2d ? r0 + 16 : r + 1;
            for (int64_t rr = r0; rr < r1; ++rr)
                for (int64_t c = b * 16; c < b * 16 + 16; ++c) {
                    float a = fabsf(y[rr * k + c]);
                    if (a > amax_b) amax_b = a;
                }
            uint8_t scode = or_e4m3_encode((amax_b / 6.0f) / sg);
            if (scale46 && !block2d) {
                uint8_t scode4 = or_e4m3_encode((amax_b / 4.0f) / sg);
                const float* blk = &y[r * k + b * 16];
                if (block_sse_rne(blk, scode4, sg) < block_sse_rne(blk, scode, sg))
                    scode = scode4;
            }
            scales[r * kb + b] = scode;
        }
    }
    /* elements */
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t c = 0; c < k; ++c) {
            uint8_t scode = scales[r * kb + c / 16];
            float x = y[r * k + c];
            int mag;
            if (scode == 0) {
                mag = 0;
            } else {
                float u = scale_element(x, (float)or_e4m3_value(scode) * sg);
                if (rounding == 1)
                    mag = or_e2m1_sr(u, or_sr_bits(seed, copy_id, (uint64_t)(r * k + c)));
                else
                    mag = or_e2m1_rne(u);
            }
            int code = (signbit(x) ? 8 : 0) | mag;
            uint8_t* p = &codes[r * (k / 2) + c / 2];
            if ((c & 1) == 0)
                *p = (uint8_t)((*p & 0xF0) | code);
            else
                *p = (uint8_t)((*p & 0x0F) | (code << 4));
        }
    }
}

int or_quantize_rows(const float* x, int64_t n, int64_t k, int block2d, int rounding,
                     int rht, int scale46, uint64_t seed, uint32_t copy_id,
                     uint8_t* codes, uint8_t* scales, float* sg)
{
    if (n < 0 || k < 0 || k % 16 != 0 || (block2d && n % 16 != 0)) return -2;
    if (rounding != 0 && rounding != 1) return -5;
    if (scale46 && block2d) return -5;              /* 4/6 is defined for 1D blocks */
    if (!all_finite(x, n * k)) return -8;
    float* y = (float*)malloc(sizeof(float) * (size_t)(n * k > 0 ? n * k : 1));
    if (!y) return -9;
    memcpy(y, x, sizeof(float) * (size_t)(n * k));
    if (rht) {
        float sgn[16];
        or_rht_signs(seed, sgn);
        for (int64_t r = 0; r < n; ++r)
            for (int64_t c = 0; c < k; c += 16)
                or_rht16_forward(&y[r * k + c], sgn);
    }
    memset(codes, 0, (size_t)(n * (k / 2)));
    quantize_core(y, n, k, block2d, rounding, scale46, seed, copy_id, codes, scales, sg);
    free(y);
    return 0;
}

/* For the rows of x (rotated first when rht), the number of 1x16 blocks whose 4/6 choice
 * differs between the binary32 evaluation of the squared errors (the method's) and their
 * binary64 evaluation, and the number of blocks whose binary64 errors tie exactly. */
int or_scale46_disagreements(const float* x, int64_t n, int64_t k, int rht, uint64_t seed,
                             int64_t* differ, int64_t* ties64, double* max_gap)
{
    if (n < 0 || k < 0 || k % 16 != 0) return -2;
    if (!all_finite(x, n * k)) return -8;
    float* y = (float*)malloc(sizeof(float) * (size_t)(n * k > 0 ? n * k : 1));
    if (!y) return -9;
    memcpy(y, x, sizeof(float) * (size_t)(n * k));
    if (rht) {
        float sgn[16];
        or_rht_signs(seed, sgn);
        for (int64_t r = 0; r < n; ++r)
            for (int64_t c = 0; c < k; c += 16)
                or_rht16_forward(&y[r * k + c], sgn);
    }
    float amax_t = 0.0f;
    for (int64_t i = 0; i < n * k; ++i)
        if (fabsf(y[i]) > amax_t) amax_t = fabsf(y[i]);
    float sg = amax_t / 2688.0f;
    if (sg == 0.0f) sg = 1.0f;
    int64_t nd = 0, nt = 0;
    double gap = 0.0;   /* largest |e4 - e6| / max(e4, e6) (binary64) where the choices differ */
    #pragma omp parallel for schedule(static) reduction(+:nd, nt) reduction(max:gap)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t b = 0; b < k / 16; ++b) {
            const float* blk = &y[r * k + b * 16];
            float amax_b = 0.0f;
            for (int i = 0; i < 16; ++i)
                if (fabsf(blk[i]) > amax_b) amax_b = fabsf(blk[i]);
            uint8_t s6 = or_e4m3_encode((amax_b / 6.0f) / sg);
            uint8_t s4 = or_e4m3_encode((amax_b / 4.0f) / sg);
            int use4_32 = block_sse_rne(blk, s4, sg) < block_sse_rne(blk, s6, sg);
            double e6 = block_sse_f64(blk, s6, sg), e4 = block_sse_f64(blk, s4, sg);
            int use4_64 = e4 < e6;
            if (use4_32 != use4_64) {
                ++nd;
                double g = fabs(e4 - e6) / (e4 > e6 ? e4 : e6);
                if (g > gap) gap = g;
            }
            if (e4 == e6 && s4 != s6) ++nt;
        }
    free(y);
    *differ = nd;
    *ties64 = nt;
    *max_gap = gap;
    return 0;
}

/* [FS4] sec. 2: x_hat = x_E2M1 * s * s_g.  The first product is exact
 * (2-bit times 4-bit significand); the second is one binary32 rounding. */
int or_dequantize(const uint8_t* codes, const uint8_t* scales, float sg,
                  int64_t n, int64_t k, float* out)
{
    if (n < 0 || k < 0 || k % 16 != 0) return -2;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t c = 0; c < k; ++c) {
            uint8_t byte = codes[r * (k / 2) + c / 2];
            int code = (c & 1) ? (byte >> 4) : (byte & 15);
            double vs = or_e2m1_value(code) * or_e4m3_value(scales[r * (k / 16) + c / 16]);
            float p = (float)vs;
            if ((double)p != vs) return -10;            /* cannot happen: exactness check */
            out[r * k + c] = p * sg;
        }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* GEMM reference.  [FS4] sec. 2 and eq. (1)-(2): the linear layer's three      */
/* GEMMs multiply NVFP4 operands; [NVP] sec. 4: FP4 inputs, FP32/BF16 outputs.  */
/* The plain definition is the dot product of the dequantized operands; it is  */
/* evaluated in binary64 with each operand value v*s*s_g exact in binary64.     */
/* ------------------------------------------------------------------------- */
static double deq64(const uint8_t* codes, const uint8_t* scales, float sg, int64_t K,
                    int64_t row, int64_t k)
{
    uint8_t byte = codes[row * (K / 2) + k / 2];
    int code = (k & 1) ? (byte >> 4) : (byte & 15);
    return or_e2m1_value(code) * or_e4m3_value(scales[row * (K / 16) + k / 16]) * (double)sg;
}

int or_gemm_f64(const uint8_t* codesA, const uint8_t* scalesA, float sgA,
                const uint8_t* codesB, const uint8_t* scalesB, float sgB,
                int64_t M, int64_t N, int64_t K, double* C, double* absdot)
{
    if (M < 0 || N < 0 || K < 0 || K % 16 != 0) return -2;
    double* A = (double*)malloc(sizeof(double) * (size_t)(M * K > 0 ? M * K : 1));
    double* B = (double*)malloc(sizeof(double) * (size_t)(N * K > 0 ? N * K : 1));
    if (!A || !B) { free(A); free(B); return -9; }
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) A[m * K + k] = deq64(codesA, scalesA, sgA, K, m, k);
    #pragma omp parallel for schedule(static)
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) B[n * K + k] = deq64(codesB, scalesB, sgB, K, n, k);
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0, aacc = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = A[m * K + k] * B[n * K + k];
                acc += p;
                aacc += fabs(p);
            }
            C[m * N + n] = acc;
            if (absdot) absdot[m * N + n] = aacc;
        }
    free(A);
    free(B);
    return 0;
}

int or_gemm_f64_entries(const uint8_t* codesA, const uint8_t* scalesA, float sgA,
                        const uint8_t* codesB, const uint8_t* scalesB, float sgB,
                        int64_t M, int64_t N, int64_t K,
                        const int64_t* em, const int64_t* en, int64_t count,
                        double* out, double* absdot)
{
    if (M < 0 || N < 0 || K < 0 || K % 16 != 0) return -2;
    for (int64_t i = 0; i < count; ++i)
        if (em[i] < 0 || em[i] >= M || en[i] < 0 || en[i] >= N) return -2;
    #pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; ++i) {
        double acc = 0.0, aacc = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double p = deq64(codesA, scalesA, sgA, K, em[i], k) *
                       deq64(codesB, scalesB, sgB, K, en[i], k);
            acc += p;
            aacc += fabs(p);
        }
        out[i] = acc;
        if (absdot) absdot[i] = aacc;
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Low-rank branch of the LoRA-SVD linear.  [FS4] sec. 3.2 eq. (1): Y is the     */
/* NVFP4 product Q(X) Q(W_res)^T plus beta (X L1^T) L2^T computed in BF16, and   */
/* Appendix 9 fuses the down-projection X L1^T with the quantizer (same input)   */
/* and the up-projection with the GEMM (same output).  Readings: the rank r and  */
/* beta are parameters (the pages give neither); the down-projection output is   */
/* one BF16 tensor T = BF16(beta X L1^T) (beta applied before that rounding, so  */
/* the up-projection adds T L2^T); both factors are BF16.  The reference forms   */
/* beta * sum_k x a in binary64 and rounds it once to BF16; the up-projection    */
/* term is binary64 over the BF16 T and L2.                                      */
/* ------------------------------------------------------------------------- */

/* Nearest BF16 (8 significant bits, binary32 exponent range, ties to even) of a
 * binary64 value, rounded once. */
static uint16_t bf16_rne_f64(double v)
{
    if (v == 0.0) return signbit(v) ? 0x8000u : 0u;
    const double a = fabs(v);
    int e;
    frexp(a, &e);                      /* a = f 2^e, f in [0.5, 1) */
    int q = e - 8;                     /* weight of the last kept bit */
    if (q < -133) q = -133;            /* BF16 subnormal spacing */
    const double units = ldexp(a, -q); /* exact: a power-of-two scaling */
    const double fl = floor(units), fr = units - fl;
    double n = fl;
    if (fr > 0.5 || (fr == 0.5 && fmod(fl, 2.0) != 0.0)) n = fl + 1.0;
    const float f = (float)ldexp(n, q); /* at most 8 significant bits (or a power of two) */
    uint32_t u;
    memcpy(&u, &f, 4);
    const uint16_t b = (uint16_t)(u >> 16);
    return v < 0 ? (uint16_t)(b | 0x8000u) : b;
}

int or_lora_down(const float* x, int64_t M, int64_t K, const uint16_t* a, int64_t r, float beta,
                 uint16_t* t, double* t64, double* tabs)
{
    if (M < 0 || K < 0 || r < 0) return -2;
    for (int64_t i = 0; i < M * K; ++i)
        if (!isfinite(x[i])) return -3;
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t j = 0; j < r; ++j) {
            double s = 0.0, sa = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                const double p = (double)x[m * K + k] * (double)or_bf16_value(a[j * K + k]);
                s += p;
                sa += fabs(p);
            }
            const double v = (double)beta * s;
            t[m * r + j] = bf16_rne_f64(v);
            if (t64) t64[m * r + j] = v;
            if (tabs) tabs[m * r + j] = fabs((double)beta) * sa;
        }
    return 0;
}

/* The low-rank term sum_j T[m][j] B[n][j] (binary64; the BF16 products are exact). */
static double lora_term(const uint16_t* t, const uint16_t* b, int64_t r, int64_t m, int64_t n,
                        double* abs_out)
{
    double s = 0.0, sa = 0.0;
    for (int64_t j = 0; j < r; ++j) {
        const double p = (double)or_bf16_value(t[m * r + j]) * (double)or_bf16_value(b[n * r + j]);
        s += p;
        sa += fabs(p);
    }
    *abs_out = sa;
    return s;
}

int or_gemm_lora_f64(const uint8_t* codesA, const uint8_t* scalesA, float sgA,
                     const uint8_t* codesB, const uint8_t* scalesB, float sgB,
                     int64_t M, int64_t N, int64_t K, const uint16_t* t, const uint16_t* b,
                     int64_t r, double* C, double* absdot)
{
    if (r < 0) return -2;
    int rc = or_gemm_f64(codesA, scalesA, sgA, codesB, scalesB, sgB, M, N, K, C, absdot);
    if (rc) return rc;
    #pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double sa;
            C[m * N + n] += lora_term(t, b, r, m, n, &sa);
            if (absdot) absdot[m * N + n] += sa;
        }
    return 0;
}

int or_gemm_lora_f64_entries(const uint8_t* codesA, const uint8_t* scalesA, float sgA,
                             const uint8_t* codesB, const uint8_t* scalesB, float sgB,
                             int64_t M, int64_t N, int64_t K, const uint16_t* t,
                             const uint16_t* b, int64_t r, const int64_t* em, const int64_t* en,
                             int64_t count, double* out, double* absdot)
{
    if (r < 0) return -2;
    int rc = or_gemm_f64_entries(codesA, scalesA, sgA, codesB, scalesB, sgB, M, N, K, em, en,
                                 count, out, absdot);
    if (rc) return rc;
    for (int64_t i = 0; i < count; ++i) {
        double sa;
        out[i] += lora_term(t, b, r, em[i], en[i], &sa);
        if (absdot) absdot[i] += sa;
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Quantized-state AdamW second moment.  [FS4] sec. 3.3: (1) square root,      */
/* (2) subtract the tile-wise mean, (3) fast Hadamard transform of the         */
/* residual (times H16), (4) NVFP4 quantization; reconstruction                */
/* v ~ ((s_g s v_hat) H16 + mu)^2.  [GST] sec. 2.2: the tile mean is stored    */
/* in BF16.  Readings: tiles are 16x16 and NVFP4 blocks 1x16 along rows; the   */
/* Hadamard is the random one of sec. 3.2 (signs optional, use_signs = 0 gives */
/* the plain normalised H16); the residual is taken against the stored BF16    */
/* mean so decoding inverts exactly what was stored; the tile sum uses a fixed */
/* pairwise tree (adjacent pairs within each row of 16, then the same tree      */
/* over the 16 row sums) and the mean is that sum times 2^-8.                  */
/* ------------------------------------------------------------------------- */
static float tree16(const float a[16])
{
    float t[16];
    memcpy(t, a, sizeof(t));
    for (int width = 16; width > 1; width /= 2)
        for (int i = 0; i < width / 2; ++i)
            t[i] = t[2 * i] + t[2 * i + 1];
    return t[0];
}

int or_qadamw_v_encode(const float* v, int64_t R, int64_t C, uint64_t seed, int use_signs,
                       uint16_t* mu, uint8_t* codes, uint8_t* scales, float* sg)
{
    if (R < 0 || C < 0 || R % 16 != 0 || C % 16 != 0) return -2;
    for (int64_t i = 0; i < R * C; ++i)
        if (!isfinite(v[i]) || v[i] < 0.0f) return -8;
    float* y = (float*)malloc(sizeof(float) * (size_t)(R * C > 0 ? R * C : 1));
    if (!y) return -9;
    for (int64_t i = 0; i < R * C; ++i) y[i] = sqrtf(v[i]);          /* step 1 */
    int64_t tc = C / 16;
    for (int64_t ti = 0; ti < R / 16; ++ti)                          /* step 2 */
        for (int64_t tj = 0; tj < tc; ++tj) {
            float rows[16];
            for (int rr = 0; rr < 16; ++rr)
                rows[rr] = tree16(&y[(ti * 16 + rr) * C + tj * 16]);
            float mean = tree16(rows) * 0.00390625f;                 /* 2^-8, exact */
            uint16_t m = or_bf16_rne(mean);
            mu[ti * tc + tj] = m;
            float mf = or_bf16_value(m);
            for (int rr = 0; rr < 16; ++rr)
                for (int cc = 0; cc < 16; ++cc) {
                    float* p = &y[(ti * 16 + rr) * C + tj * 16 + cc];
                    *p = *p - mf;
                }
        }
    float sgn[16];                                                   /* step 3 */
    if (use_signs) or_rht_signs(seed, sgn);
    else for (int i = 0; i < 16; ++i) sgn[i] = 1.0f;
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < C; c += 16)
            or_rht16_forward(&y[r * C + c], sgn);
    memset(codes, 0, (size_t)(R * (C / 2)));                          /* step 4 */
    quantize_core(y, R, C, 0, 0, 0, seed, 0, codes, scales, sg);
    free(y);
    return 0;
}

int or_qadamw_v_decode(const uint16_t* mu, const uint8_t* codes, const uint8_t* scales,
                       float sg, int64_t R, int64_t C, uint64_t seed, int use_signs,
                       float* v_out)
{
    if (R < 0 || C < 0 || R % 16 != 0 || C % 16 != 0) return -2;
    int rc = or_dequantize(codes, scales, sg, R, C, v_out);
    if (rc) return rc;
    float sgn[16];
    if (use_signs) or_rht_signs(seed, sgn);
    else for (int i = 0; i < 16; ++i) sgn[i] = 1.0f;
    int64_t tc = C / 16;
    for (int64_t r = 0; r < R; ++r)
        for (int64_t c = 0; c < C; c += 16) {
            float* w = &v_out[r * C + c];
            or_rht16_inverse(w, sgn);
            float mf = or_bf16_value(mu[(r / 16) * tc + c / 16]);
            for (int i = 0; i < 16; ++i) {
                float z = w[i] + mf;
                w[i] = z * z;
            }
        }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* Quantized-state AdamW step.  [FS4] sec. 2 (preliminaries) gives the moments  */
/* m_t = beta1 m_{t-1} + g_t and v_t = beta2 v_{t-1} + (1 - beta2) g_t^2; sec.   */
/* 3.3 stores m_t through a Hadamard rotation, stochastic rounding and 4/6       */
/* scaling, and v_t through the sqrt / tile-mean / Hadamard / NVFP4 pipeline.   */
/* The update itself is not printed.  Readings: the gradient                    */
/* coefficient of m is a parameter (1 in the pages' form, 1 - beta1 in the      */
/* common one); the update is decoupled AdamW with caller-supplied bias          */
/* multipliers, w <- w - lr (bias1 m / (sqrt(bias2 v) + eps) + wd w); the m      */
/* rotation uses random signs from a seed that stays with the state, and the    */
/* stochastic rounding a fresh seed per step.  Every elementwise operation is   */
/* one binary32 rounding in the order written below.                           */
/* hp = {lr, beta1, beta2, eps, weight_decay, grad_coef, bias1, bias2}.          */
/* ------------------------------------------------------------------------- */
int or_qadamw_step(float* w, const float* g, int64_t R, int64_t C,
                   const uint8_t* m_codes, const uint8_t* m_scales, float m_sg,
                   const uint16_t* mu, const uint8_t* v_codes, const uint8_t* v_scales, float v_sg,
                   const float* hp, uint64_t m_rht_seed, uint64_t m_sr_seed, uint64_t v_seed,
                   int v_use_signs,
                   uint8_t* m_codes_out, uint8_t* m_scales_out, float* m_sg_out,
                   uint16_t* mu_out, uint8_t* v_codes_out, uint8_t* v_scales_out, float* v_sg_out,
                   float* m_new_out, float* v_new_out)
{
    if (R < 0 || C < 0 || R % 16 != 0 || C % 16 != 0) return -2;
    size_t n = (size_t)(R * C > 0 ? R * C : 1);
    float* mp = (float*)malloc(sizeof(float) * n);
    float* vp = (float*)malloc(sizeof(float) * n);
    float* y = (float*)malloc(sizeof(float) * n);
    if (!mp || !vp || !y) { free(mp); free(vp); free(y); return -9; }
    int rc = or_dequantize(m_codes, m_scales, m_sg, R, C, mp);
    if (!rc) rc = or_qadamw_v_decode(mu, v_codes, v_scales, v_sg, R, C, v_seed, v_use_signs, vp);
    if (rc) { free(mp); free(vp); free(y); return rc; }
    float sgn[16];
    or_rht_signs(m_rht_seed, sgn);
    for (int64_t i = 0; i < R * C; i += 16) or_rht16_inverse(&mp[i], sgn);

    const float lr = hp[0], b1 = hp[1], b2 = hp[2], eps = hp[3], wd = hp[4], cg = hp[5];
    const float bias1 = hp[6], bias2 = hp[7];
    const float omb2 = 1.0f - b2;
    for (int64_t i = 0; i < R * C; ++i) {
        const float gi = g[i];
        const float m = b1 * mp[i] + cg * gi;
        const float v = b2 * vp[i] + omb2 * (gi * gi);
        const float den = sqrtf(bias2 * v) + eps;
        const float upd = (bias1 * m) / den + wd * w[i];
        w[i] = w[i] - lr * upd;
        mp[i] = m;
        vp[i] = v;
    }
    if (m_new_out) memcpy(m_new_out, mp, sizeof(float) * (size_t)(R * C));
    if (v_new_out) memcpy(v_new_out, vp, sizeof(float) * (size_t)(R * C));
    /* m: rotate each 1x16 chunk, then NVFP4 1x16 with 4/6 scaling and stochastic rounding */
    memcpy(y, mp, sizeof(float) * (size_t)(R * C));
    for (int64_t i = 0; i < R * C; i += 16) or_rht16_forward(&y[i], sgn);
    memset(m_codes_out, 0, (size_t)(R * (C / 2)));
    quantize_core(y, R, C, 0, 1, 1, m_sr_seed, 0, m_codes_out, m_scales_out, m_sg_out);
    /* v: the Q-AdamW second-moment pipeline */
    rc = or_qadamw_v_encode(vp, R, C, v_seed, v_use_signs, mu_out, v_codes_out, v_scales_out,
                            v_sg_out);
    free(mp);
    free(vp);
    free(y);
    return rc;
}

int or_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Thread count of the OpenMP row loops (timing only; results do not depend on it). */
void or_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
