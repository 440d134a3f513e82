/*
 * nvfp4_oracle.h -- plain, slow, scalar CPU reference for the NVFP4 quantized
 * linear path.  TEST INFRASTRUCTURE ONLY: the only code allowed to load this
 * library is the test suite, the package smoke check and the CPU-baseline leg
 * of the benchmark.  The GPU library shares no code, header, table or
 * constant with this file, and the product path never calls it.
 *
 * Every function follows a passage of the pages it was written from:
 *   [FS4]   Full-Stack FP4 (academ.us article 2607.04422): sec. 2 "Preliminaries",
 *           sec. 3.2 eq. (1)-(2), sec. 3.3 "Quantized-State AdamW", Appendix 7,
 *           Appendix 10.1.
 *   [NVP]   "Pretraining Large Language Models with NVFP4" (paperlayer.ai summary of
 *           arXiv 2509.25149v2): sec. 2 "NVFP4 Format", sec. 4 "Training
 *           Methodology", A.2, B.4, E.2.
 *   [OPT]   OptiTrain-FP4 README (github mirror): E2M1 enumeration, RHT worked
 *           example, Walsh-Hadamard recursion.
 *   [GST]   gist.science summary of 2607.04422, sec. 2.2 (Q-AdamW v_t).
 * Where the pages leave a step open, the reading taken is stated at the function.
 *
 * Floating point: every operation documented as "fl(.)" is one IEEE binary32
 * operation with round-to-nearest-even; the file is compiled with
 * -ffp-contract=off and without fast-math so no fused or reassociated form
 * appears.  Integer decisions (codes, scales) are taken in binary32, the
 * precision of the format's tensor scale.  GEMM references are binary64.
 *
 * All arrays are host memory owned by the caller.  Functions return 0 on
 * success, a negative value on invalid arguments (non-multiple-of-16 sizes,
 * non-finite input, negative second moment).
 */
#ifndef NVFP4_ORACLE_H
#define NVFP4_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* E2M1 element: value of a 4-bit code (sign | 2 exponent bits | 1 mantissa bit). */
double or_e2m1_value(int code);
/* Round-to-nearest-even of a non-negative binary32 magnitude onto the E2M1 grid,
 * saturating at 6.  Returns the 3-bit magnitude code. */
int or_e2m1_rne(float u);
/* Stochastic rounding of a non-negative magnitude with 16 random bits r. */
int or_e2m1_sr(float u, uint32_t r16);

/* E4M3 (OCP "fn" variant) block scale: nearest finite non-negative value, ties to
 * even code, saturating at 448.  v must be >= 0 and not NaN. */
uint8_t or_e4m3_encode(float v);
double or_e4m3_value(uint8_t code);

/* bfloat16 nearest-even of a binary32 value (finite input). */
uint16_t or_bf16_rne(float v);
float or_bf16_value(uint16_t b);

/* Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, SC'11). */
void or_philox4x32_10(const uint32_t ctr[4], const uint32_t key[2], uint32_t out[4]);
/* 16 random bits for element j of output copy copy_id under seed. */
uint32_t or_sr_bits(uint64_t seed, uint32_t copy_id, uint64_t j);
/* The 16 signs of the random Hadamard diagonal drawn from seed (+1.0f / -1.0f). */
void or_rht_signs(uint64_t seed, float sgn[16]);

/* In-place unnormalised Walsh-Hadamard transform of 16 binary32 values (Sylvester
 * order); returns H16 * v with one fl() per butterfly output. */
void or_wht16(float v[16]);
/* Random Hadamard transform of one 16-chunk: v <- 0.25 * H16 * (D .* v). */
void or_rht16_forward(float v[16], const float sgn[16]);
/* Its inverse: v <- D .* (0.25 * H16 * v). */
void or_rht16_inverse(float v[16], const float sgn[16]);

/* Quantize x[n][k] (row-major binary32) along its rows: every 16 consecutive
 * elements of a row form a block (block2d = 0), or every 16x16 tile (block2d = 1).
 * rounding: 0 = nearest-even, 1 = stochastic.  rht: 0/1 random Hadamard transform
 * of each 16-chunk along the rows before scaling.  copy_id enters the stochastic
 * rounding counter (0 = rowwise copy, 1 = columnwise copy).
 * Outputs: codes[n][k/2] (element 2i in the low nibble), scales[n][k/16] (E4M3
 * codes; 16x16 tiles stored expanded, one byte per row of the tile), *sg. */
int or_quantize_rows(const float* x, int64_t n, int64_t k, int block2d, int rounding,
                     int rht, int scale46, uint64_t seed, uint32_t copy_id,
                     uint8_t* codes, uint8_t* scales, float* sg);

/* Decode codes[n][k/2], scales[n][k/16], sg into binary32 out[n][k]:
 * out = fl(fl(value(code) * value(scale)) * sg). */
int or_dequantize(const uint8_t* codes, const uint8_t* scales, float sg,
                  int64_t n, int64_t k, float* out);

/* C[M][N] = sum_k A[m][k] * B[n][k] in binary64 over the exact dequantized
 * operands value(code) * value(scale) * sg.  absdot (optional) receives
 * sum_k |A[m][k] * B[n][k]|. */
int or_gemm_f64(const uint8_t* codesA, const uint8_t* scalesA, float sgA,
                const uint8_t* codesB, const uint8_t* scalesB, float sgB,
                int64_t M, int64_t N, int64_t K, double* C, double* absdot);
/* The same for a list of (m, n) entries only. */
int or_gemm_f64_entries(const uint8_t* codesA, const uint8_t* scalesA, float sgA,
                        const uint8_t* codesB, const uint8_t* scalesB, float sgB,
                        int64_t M, int64_t N, int64_t K,
                        const int64_t* em, const int64_t* en, int64_t count,
                        double* out, double* absdot);

/* Quantized-state AdamW second moment, sec. 3.3: v[R][C] >= 0 ->
 * mu[R/16][C/16] (bf16 bits), codes[R][C/2], scales[R][C/16], *sg. */
int or_qadamw_v_encode(const float* v, int64_t R, int64_t C, uint64_t seed, int use_signs,
                       uint16_t* mu, uint8_t* codes, uint8_t* scales, float* sg);
int or_qadamw_v_decode(const uint16_t* mu, const uint8_t* codes, const uint8_t* scales,
                       float sg, int64_t R, int64_t C, uint64_t seed, int use_signs,
                       float* v_out);

/* Low-rank branch of the LoRA-SVD linear ([FS4] sec. 3.2 eq. (1), Appendix 9; reading in
 * nvfp4_oracle.c).  Down-projection: t[M][r] = BF16(beta * x[M][K] a[r][K]^T), a in BF16
 * bits; t64 (may be NULL) the binary64 value before rounding, tabs (may be NULL)
 * |beta| sum_k |x a|. */
int or_lora_down(const float* x, int64_t M, int64_t K, const uint16_t* a, int64_t r, float beta,
                 uint16_t* t, double* t64, double* tabs);
/* GEMM plus the up-projection: C = A B^T (dequantized, as or_gemm_f64) + t[M][r] b[N][r]^T
 * (BF16 bits); absdot adds sum_j |t b|. */
int or_gemm_lora_f64(const uint8_t* codesA, const uint8_t* scalesA, float sgA,
                     const uint8_t* codesB, const uint8_t* scalesB, float sgB,
                     int64_t M, int64_t N, int64_t K, const uint16_t* t, const uint16_t* b,
                     int64_t r, double* C, double* absdot);
int or_gemm_lora_f64_entries(const uint8_t* codesA, const uint8_t* scalesA, float sgA,
                             const uint8_t* codesB, const uint8_t* scalesB, float sgB,
                             int64_t M, int64_t N, int64_t K, const uint16_t* t,
                             const uint16_t* b, int64_t r, const int64_t* em, const int64_t* en,
                             int64_t count, double* out, double* absdot);

/* Number of OpenMP threads the oracle runs with (1 without OpenMP). */
/* Quantized-state AdamW step (reading in nvfp4_oracle.c): decodes m (NVFP4 1x16 of the
 * Hadamard-rotated moment) and v (second-moment pipeline), updates the moments and the
 * FP32 weights w in place, re-encodes m (rotation, 4/6, stochastic rounding with
 * m_sr_seed) and v.  hp = {lr, beta1, beta2, eps, weight_decay, grad_coef, bias1, bias2}.
 * m_new_out / v_new_out (may be NULL) receive the updated moments before encoding. */
int or_qadamw_step(float* w, const float* g, int64_t R, int64_t C,
                   const uint8_t* m_codes, const uint8_t* m_scales, float m_sg,
                   const uint16_t* mu, const uint8_t* v_codes, const uint8_t* v_scales, float v_sg,
                   const float* hp, uint64_t m_rht_seed, uint64_t m_sr_seed, uint64_t v_seed,
                   int v_use_signs,
                   uint8_t* m_codes_out, uint8_t* m_scales_out, float* m_sg_out,
                   uint16_t* mu_out, uint8_t* v_codes_out, uint8_t* v_scales_out, float* v_sg_out,
                   float* m_new_out, float* v_new_out);

/* Measurement (not part of the method): blocks whose 4/6 choice differs between the binary32
 * and the binary64 evaluation of the squared errors; exact binary64 ties; the largest relative
 * gap between the two binary64 errors among the differing blocks. */
int or_scale46_disagreements(const float* x, int64_t n, int64_t k, int rht, uint64_t seed,
                             int64_t* differ, int64_t* ties64, double* max_gap);
int or_num_threads(void);
void or_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
