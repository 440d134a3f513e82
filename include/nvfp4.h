/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 quantized-linear library.
 *
 * The library implements the data-parallel hot path of NVFP4 training as the
 * pages describe it:
 *   - Full-Stack FP4 (academ.us 2607.04422), sec. 2 "Preliminaries": NVFP4 =
 *     E2M1 elements, one E4M3 scale per 1x16 or 16x16 block, one FP32 tensor
 *     scale; x_hat = x_E2M1 * s * s_g.  Sec. 3.2 eq. (1)-(2): the three GEMMs of
 *     a linear layer take Q_1x16 / Q_16x1 / Q_16x16 operands, with a fresh
 *     16x16 random Hadamard transform in the weight-gradient GEMM.  Sec. 3.3:
 *     the quantized-state AdamW second-moment pipeline.
 *   - "Pretraining Large Language Models with NVFP4" (paperlayer.ai summary of
 *     arXiv 2509.25149v2), sec. 2 "NVFP4 Format" (amax of each block maps to the
 *     FP4 maximum; FP32 tensor scale keeps block scales in E4M3), sec. 4
 *     "Training Methodology" (RNE for weights/activations, stochastic rounding
 *     for gradients, 2D weight blocks, RHT on Wgrad inputs), B.4 (scale computed
 *     in the rotated space), A.2 (decode scales stored for the GEMM).
 *
 * Conventions shared by every call
 *   - Every data pointer is DEVICE memory allocated and owned by the caller;
 *     struct arguments themselves are host memory read during the call only.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).  Calls
 *     validate their arguments on the host, enqueue kernels on `stream` and
 *     return; they never allocate, free or synchronise the device.
 *   - Status: NVFP4_OK or a negative NVFP4_ERR_* code.  Argument errors are
 *     returned before anything is enqueued.  A failed kernel launch returns
 *     NVFP4_ERR_HIP (from hipGetLastError); faults inside a kernel surface at
 *     the caller's next synchronisation.
 *   - Matrices are row-major.  Block dimensions must be multiples of 16 (the
 *     pages give no padding rule); every other extent may be any size >= 0.
 *   - Input values must be finite; any finite values are quantized as described, down
 *     to tensors of subnormal values.  Elements are scaled by the correctly rounded
 *     reciprocal of fl(s s_g), kept at binary32 precision; where its exponent exceeds
 *     binary32's range (fl(s s_g) < about 2^-128, only for tensor maxima below about
 *     2^-107) it is carried as R 2^-64 with the 2^64 restored in the E2M1 conversion.
 *     The GEMM's stated accuracy assumes s_gA s_gB is a normal binary32.
 *   - Calls on one stream are ordered.  The library holds no state apart from the
 *     scratch array of nvfp4_quantize_noalloc and the hand-off flags of nvfp4_gemm's
 *     balanced schedule (one 64-bit word per workgroup and device, tagged per launch), so
 *     calls on different streams may run concurrently on distinct buffers (except two
 *     nvfp4_quantize_noalloc calls on one device; concurrent GEMMs stay correct).
 *
 * Quantized tensor layout (one "copy"): an n x k matrix quantized along its
 * rows has
 *   codes  uint8 [n][k/2]   element 2i in the low nibble, 2i+1 in the high
 *                           nibble; a nibble is sign<<3 | exponent<<1 | mantissa
 *   scales uint8 [n][k/16]  E4M3 (OCP "fn") code of the block scale; 16x16
 *                           blocks are stored expanded (each of the 16 rows of a
 *                           tile repeats its scale)
 *   gscale float [1]        the FP32 tensor scale s_g
 * The rowwise copy of an R x C tensor X is X quantized along its rows (n = R,
 * k = C); the columnwise copy is X^T quantized along its rows (n = C, k = R).
 */
#ifndef NVFP4_H
#define NVFP4_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NVFP4_ABI_VERSION 6

enum nvfp4_status {
    NVFP4_OK = 0,
    NVFP4_ERR_NULL = -1,      /* a required pointer is NULL */
    NVFP4_ERR_SHAPE = -2,     /* negative extent, or a block dimension not a multiple of 16 */
    NVFP4_ERR_ALIGN = -3,     /* pointer or leading dimension not aligned as documented */
    NVFP4_ERR_DTYPE = -4,     /* unknown dtype enum */
    NVFP4_ERR_MODE = -5,      /* unknown or unsupported combination of options */
    NVFP4_ERR_WORKSPACE = -6, /* workspace missing or smaller than required */
    NVFP4_ERR_HIP = -7        /* kernel launch failed */
};

enum nvfp4_dtype { NVFP4_F32 = 0, NVFP4_BF16 = 1 };
enum nvfp4_rounding { NVFP4_RNE = 0, NVFP4_SR = 1 };
enum nvfp4_block { NVFP4_BLOCK_1D = 0, NVFP4_BLOCK_2D = 1 };

/* Options of one nvfp4_quantize call.
 *   rowwise, colwise   produce the rowwise and/or the columnwise copy (at least one)
 *   block              NVFP4_BLOCK_1D: 1x16 blocks along each copy's rows (Q_1x16 for
 *                      the rowwise copy, Q_16x1 for the columnwise one);
 *                      NVFP4_BLOCK_2D: 16x16 tiles shared by both copies (Q_16x16), so
 *                      the columnwise copy is bit-identical to the transposed rowwise
 *                      copy (NVFP4 report sec. 4).  2D requires RNE and no RHT.
 *   round_row/col      NVFP4_RNE or NVFP4_SR per copy (the report: RNE for weights and
 *                      activations, SR for gradients)
 *   rht_row/col        0/1: apply the random Hadamard transform T(v) = 1/4 H16 (D v) to
 *                      every 16-chunk along the copy's rows before scaling; D is one
 *                      random sign vector per call derived from `seed` (Full-Stack FP4
 *                      sec. 3.2: one random 16x16 Hadamard matrix per backward pass; both
 *                      Wgrad operands must use the same seed so the transforms cancel)
 *   scale46            0/1: 4/6 adaptive block scaling (Full-Stack FP4 sec. 3 and its
 *                      introduction name it for every NVFP4 quantization; the related-work
 *                      paragraph calls it MSE-optimal adaptive block scaling).  Each 1x16
 *                      block keeps, of the two E4M3 scales mapping its amax to 6 and to 4,
 *                      the one whose nearest-even quantization has the smaller squared
 *                      error (binary32: e = fma(-(v s), s_g, x), summed as two fma chains
 *                      over elements 0..7 and 8..15, then added); 6 on a tie.  Stochastic
 *                      rounding uses the scale so chosen.  Not defined for 16x16 blocks.
 *   seed               key of the Philox4x32-10 generator behind D and the SR draws */
typedef struct {
    int32_t rowwise, colwise;
    int32_t block;
    int32_t round_row, round_col;
    int32_t rht_row, rht_col;
    int32_t scale46;
    uint64_t seed;
} nvfp4_quant_params;

/* One quantized copy (pointers to device memory; see the layout above). */
typedef struct {
    uint8_t* codes;
    uint8_t* scales;
    float* gscale;
} nvfp4_qtensor;

/* Device workspace (bytes) nvfp4_quantize needs for a rows x cols input. */
size_t nvfp4_quantize_workspace_bytes(int64_t rows, int64_t cols, const nvfp4_quant_params* p);

/* Quantize X[rows][cols] (row pitch ld_x elements, ld_x >= cols) to NVFP4.
 * Passages: Full-Stack FP4 sec. 2 (format, x_hat = x_E2M1 s s_g), sec. 3.2 eq. (1)-(2)
 * (Q_1x16, Q_16x1, Q_16x16, H16^r); NVFP4 report sec. 2 (amax -> FP4 max, FP32 tensor
 * scale), sec. 4 and E.2 (RNE, SR on gradients, 2D weights, RHT on Wgrad inputs), B.4
 * (scale computed after the rotation).  Per copy: s_g = amax/(6*448) over the
 * (rotated) values (1 if that is 0); block scale s = E4M3_rne_sat((amax_b/6)/s_g);
 * elements u = x * 1/(s*s_g) rounded to E2M1 (nearest-even saturating at 6, or
 * stochastic: up iff frac + r/2^16 >= 1 with 16 Philox bits r per element).
 *   x       bf16 or f32 per `dtype`, 16-byte aligned, ld_x * element size a multiple of 16
 *   row_out rowwise copy ([rows][cols/2] codes, [rows][cols/16] scales, 1 float); may be
 *           NULL when p->rowwise == 0
 *   col_out columnwise copy ([cols][rows/2], [cols][rows/16], 1 float); may be NULL when
 *           p->colwise == 0
 *   ws      device workspace of at least nvfp4_quantize_workspace_bytes() bytes,
 *           16-byte aligned; its contents need no initialisation
 * rows and cols must be multiples of 16; codes arrays 8-byte aligned. */
int nvfp4_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld_x,
                   const nvfp4_quant_params* p, const nvfp4_qtensor* row_out,
                   const nvfp4_qtensor* col_out, void* ws, size_t ws_bytes, void* stream);

/* nvfp4_quantize with the tensor amax taken from caller-supplied partial maxima instead of a
 * first pass over x, so that x is read once.  The amax is the largest of amax_parts[0 ..
 * n_parts), the same for both copies; with amax_parts holding the maxima of |x| over any
 * cover of x (for instance nvfp4_gemm_bf16's tile maxima of the x it wrote), the copies are
 * bit for bit those of nvfp4_quantize.  Passages: NVFP4 report sec. 2 (per-tensor amax ->
 * FP32 tensor scale) and sec. 4 (mixed precision: BF16 GEMM outputs are the next layer's
 * inputs).
 *   amax_parts  device array of n_parts >= 1 floats (4-byte aligned), not written
 * Copies with a Hadamard rotation (p->rht_row, p->rht_col) need the amax of the rotated
 * values and are refused (NVFP4_ERR_MODE).  No workspace.  Other arguments and errors as in
 * nvfp4_quantize. */
int nvfp4_quantize_amax(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld_x,
                        const nvfp4_quant_params* p, const nvfp4_qtensor* row_out,
                        const nvfp4_qtensor* col_out, const float* amax_parts, int64_t n_parts,
                        void* stream);

/* nvfp4_quantize without a workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Arguments, results and errors are those of nvfp4_quantize with the same x, p and copies.
 * The per-workgroup partial maxima go to a file-scope device array of
 * NVFP4_NOALLOC_SCRATCH_BYTES (6 KiB) instead of `ws`; each device holds its own copy from
 * the first call on it until the process ends.  Every shape fits (the first pass never has
 * more than 768 workgroups); a larger need would give NVFP4_ERR_WORKSPACE.  The call uses
 * the array of the current device (hipGetDevice), so `stream` must belong to it.  The call
 * allocates nothing: the array's address is looked up once per device on the first call.
 * Calls that overlap in time on one device share that array and race: order them on one
 * stream (or synchronise between streams).  nvfp4_quantize with its own workspace has no
 * such restriction. */
#define NVFP4_NOALLOC_SCRATCH_BYTES 6144
int nvfp4_quantize_noalloc(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld_x,
                           const nvfp4_quant_params* p, const nvfp4_qtensor* row_out,
                           const nvfp4_qtensor* col_out, void* stream);

/* nvfp4_quantize with the LoRA-SVD down-projection fused into its first pass:
 *   lora_t[rows][rank] = BF16(beta * x lora_a^T)   (nearest-even from the FP32 sum)
 * besides the copies nvfp4_quantize writes (identical to its output for the same p).
 * Passage: Full-Stack FP4 sec. 3.2 eq. (1) (the BF16 branch beta (X L1^T) L2^T next to the
 * NVFP4 GEMM; for dX, (dY L2) L1) and Appendix 9 (the down-projection reuses the
 * quantizer's read of X).  lora_a [rank][cols]: device BF16, row-major, 16-byte aligned
 * (L1 for X, L2^T for dY).  beta: the branch factor, applied before the BF16 rounding (the
 * up-projection then adds lora_t times the up factor; see nvfp4_gemm_lora).  The sum over
 * cols is FP32 (BF16 matrix-core products), in a fixed order: parts of the columns summed
 * separately, then the parts in order.
 * Limits: dtype NVFP4_BF16 (else NVFP4_ERR_DTYPE); rank a multiple of 16 up to 64, cols
 * a multiple of 128, and ld_x and cols below 2^24 (the first pass addresses 64 rows of x
 * and all of lora_a with 32-bit byte offsets) (else NVFP4_ERR_SHAPE); ws of
 * nvfp4_quantize_lora_workspace_bytes. */
size_t nvfp4_quantize_lora_workspace_bytes(int64_t rows, int64_t cols, int64_t rank);
int nvfp4_quantize_lora(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld_x,
                        const nvfp4_quant_params* p, const nvfp4_qtensor* row_out,
                        const nvfp4_qtensor* col_out, const uint16_t* lora_a, int64_t rank,
                        float beta, uint16_t* lora_t, void* ws, size_t ws_bytes, void* stream);

/* The columnwise copy of a rowwise copy's decoded values: Full-Stack FP4 eq. (2) takes the
 * Wgrad operand Q_16x1(H^T Q_1x16(X)), the columnwise (16x1, optionally rotated)
 * quantization of the already quantized activation.  row_in is a rowwise copy of a
 * rows x cols tensor (as nvfp4_quantize writes it); its values fl(fl(v s) s_g) are
 * quantized as nvfp4_quantize would quantize them with p, into col_out [cols][rows/2],
 * [cols][rows/16].  p must ask for the columnwise copy only (rowwise 0, colwise 1, 1x16
 * blocks, no row Hadamard; round_col, rht_col, seed, scale46 as in nvfp4_quantize), else
 * NVFP4_ERR_MODE.  Reads 0.5625 bytes per element instead of the input's 2 or 4.
 * ws of nvfp4_requantize_cols_workspace_bytes; rows, cols multiples of 16. */
size_t nvfp4_requantize_cols_workspace_bytes(int64_t rows, int64_t cols);
int nvfp4_requantize_cols(const nvfp4_qtensor* row_in, int64_t rows, int64_t cols,
                          const nvfp4_quant_params* p, const nvfp4_qtensor* col_out, void* ws,
                          size_t ws_bytes, void* stream);

/* Decode one copy: out[n][k] = (value(code) * s) * s_g, rounded once to binary32
 * (Full-Stack FP4 sec. 2), then to bfloat16 nearest-even if out_dtype is NVFP4_BF16.
 * Rotated copies decode to the rotated values.  out has row pitch ld_out elements
 * (ld_out >= k); k must be a multiple of 16; codes 8-byte aligned. */
int nvfp4_dequantize(const nvfp4_qtensor* q, int64_t n, int64_t k, int out_dtype, void* out,
                     int64_t ld_out, void* stream);

/* W4A4 GEMM: C[M][N] = s_gA s_gB * sum_k (v(qA[m,k]) sA[m,k/16]) (v(qB[n,k]) sB[n,k/16]),
 * both operands K-major copies (A: M x K, B: N x K, as produced by nvfp4_quantize), FP32
 * accumulation, FP32 output with row pitch ldc >= N.
 * Passages: Full-Stack FP4 sec. 2 and eq. (1)-(2) (Fprop Y = X W^T, Dgrad, Wgrad on
 * NVFP4 operands); NVFP4 report sec. 4 (FP4 inputs, FP32 output) and A.2 (decode scales
 * stored for the GEMM).  Every product of a decoded element and its block scale is
 * exact in binary16, so the only rounding is the FP32 accumulation.
 * K must be a multiple of 16; M and N any size >= 0; codes 16-byte aligned (row pitch K/2
 * bytes; when K % 32 == 16 the rows are read 8 bytes at a time), C 4-byte aligned.
 * Schedule: 256 x 256 output tiles, one workgroup per compute unit at a time.  When the
 * last round of tiles would keep at most half the units busy, it runs either as twice as
 * many 256 x 128 tiles, each over the whole K range (every element is then the sum one
 * workgroup per tile forms), or, when the whole rounds are long (rounds x ceil(K/128) >= 64),
 * with each of its tiles split into two K halves computed by two workgroups and summed as
 * fl(head + tail) of the two FP32 partial accumulations; the tail half is parked in the
 * tile's own region of C meanwhile.  Results are bitwise reproducible on a given device
 * (they depend on its compute-unit count through that choice and split). */
int nvfp4_gemm(const nvfp4_qtensor* a, const nvfp4_qtensor* b, int64_t M, int64_t N,
               int64_t K, float* c, int64_t ldc, void* stream);

/* Number of 256 x 256 output tiles of an M x N product (0 if either is <= 0). */
int64_t nvfp4_gemm_tiles(int64_t M, int64_t N);

/* nvfp4_gemm with C rounded once to bfloat16 (nearest-even) and each output tile's maximum
 * of |C|.  Passages: NVFP4 report sec. 4 (GEMMs on FP4 inputs produce BF16 or FP32 outputs)
 * and sec. 2 (the next quantize needs the tensor amax of this output).
 *   c          bf16 [M][ldc], ldc >= N, 2-byte aligned
 *   tile_amax  NULL, or nvfp4_gemm_tiles(M, N) floats (4-byte aligned): tile (i, j), rows
 *              256 i .. and columns 256 j .., at index i * ceil(N/256) + j, gets the largest
 *              |C| over its elements (a bf16 value; NaN elements are not counted)
 * Every element is bf16_rne of the FP32 value nvfp4_gemm stores when it takes one workgroup
 * per tile.  When whole rounds of tiles (one per compute unit, rounded down to a multiple of
 * 8) leave a last round at most half full, that round runs as twice as many 256 x 128 tiles,
 * each over the whole K range with the MFMA order of a 256 x 256 tile; the first launch
 * zeroes those tiles' maxima and the second combines its two halves' maxima with an atomic
 * maximum (NVFP4_GEMM_SK=0 keeps one workgroup per tile).  Other arguments and errors as in
 * nvfp4_gemm. */
int nvfp4_gemm_bf16(const nvfp4_qtensor* a, const nvfp4_qtensor* b, int64_t M, int64_t N,
                    int64_t K, uint16_t* c, int64_t ldc, float* tile_amax, void* stream);

/* The W4A4 GEMM with the LoRA-SVD low-rank term fused into its epilogue:
 *   C[M][N] = (nvfp4_gemm's product) + sum_j T[m][j] L[n][j].
 * Passage: Full-Stack FP4 sec. 3.2 eq. (1) (Y = Q(X) Q(W_res)^T + beta (X L1^T) L2^T, the
 * branch in BF16; dX likewise with (dY L2) L1) and Appendix 9 (the up-projection shares
 * the GEMM's output).  T is the down-projection with beta already applied (as written by
 * nvfp4_quantize_lora), L the up factor: L2 [N][rank] for Y, L1^T [N][rank] for dX.
 * lora_t [M][rank] and lora_b [N][rank]: device BF16, row-major, 16-byte aligned, read
 * only.  rank must be a multiple of 16 (rank 0 gives nvfp4_gemm); the term is formed by
 * BF16 matrix-core products with FP32 accumulation onto fl(s_gA s_gB acc).  Other
 * arguments and errors as nvfp4_gemm; a rank that is not a multiple of 16 gives
 * NVFP4_ERR_SHAPE, a null factor with rank > 0 NVFP4_ERR_NULL. */
int nvfp4_gemm_lora(const nvfp4_qtensor* a, const nvfp4_qtensor* b, int64_t M, int64_t N,
                    int64_t K, float* c, int64_t ldc, const uint16_t* lora_t,
                    const uint16_t* lora_b, int64_t rank, void* stream);

/* The W4A4 GEMM with a linear epilogue: C = alpha * (nvfp4_gemm's product) + beta * D,
 * each element stored as fma(fl(alpha s_gA s_gB), acc, fl(beta d)).  D [M][N] FP32 with
 * row pitch ldd >= N, 4-byte aligned; D may be C itself (same pitch): each element of D is
 * read by the thread that writes the same element of C.  Passage: Full-Stack FP4 sec. 3.4
 * (the quantized Newton-Schulz updates B = b A + c qA qA' and X = a X + qB qX').  Other
 * arguments and errors as nvfp4_gemm; a null D gives NVFP4_ERR_NULL. */
int nvfp4_gemm_axpby(const nvfp4_qtensor* a, const nvfp4_qtensor* b, int64_t M, int64_t N,
                     int64_t K, float alpha, const float* d, int64_t ldd, float beta, float* c,
                     int64_t ldc, void* stream);

/* One quantized Newton-Schulz iteration of NVFP4 Root (Full-Stack FP4 sec. 3.4; the
 * iteration X = a X + b X (X^T X) + c X (X^T X)^2 of sec. 2 in the wide orientation):
 *   qX = Q_1x16(X H), qX' = Q_16x1(H^T X), A = qX qX^T,
 *   qA = Q_1x16(A H), qA' = Q_16x1(H^T A), B = b A + c qA qA',
 *   qB = Q_1x16(B H), X <- a X + qB qX'.
 * x [m][n] FP32 row-major, 16-byte aligned, updated in place.  Every quantization is
 * nearest-even with 1x16 / 16x1 blocks, 4/6 scaling when scale46 = 1 (the pages'), and the
 * random Hadamard of seed (one per iteration; use a fresh seed per iteration).  a, b, c:
 * the caller's coefficients (the pages take shape-specialised ones from Root and print
 * none).  A and B are FP32 m x m.  m and n must be multiples of 32 (else
 * NVFP4_ERR_SHAPE); ws: nvfp4_ns_step_workspace_bytes(m, n) bytes, 256-byte aligned.
 * The call enqueues three quantizes and three GEMMs.  When m is a multiple of 256, A (which
 * is symmetric) is formed on its upper-triangle tiles with K split into parts, then summed
 * in part order and mirrored; the workspace then also holds those partial products
 * (58.5 MB for m = 3072, n = 9216).
 * After the call (once the stream reaches it) the workspace holds the iteration's
 * intermediates, each starting at the previous one's end rounded up to 256 bytes, from
 * offset 0: qX (codes [m][n/2], scales [m][n/16], s_g float), qX' ([n][m/2], [n][m/16],
 * s_g), A (FP32 [m][m]), qA, qA' (each [m][m/2], [m][m/16], s_g), B (FP32 [m][m]), qB
 * ([m][m/2], [m][m/16], s_g); the rest is scratch. */
size_t nvfp4_ns_step_workspace_bytes(int64_t m, int64_t n);
int nvfp4_ns_step(float* x, int64_t m, int64_t n, float a, float b, float c, uint64_t seed,
                  int32_t scale46, void* ws, size_t ws_bytes, void* stream);

/* Device workspace (bytes) qadamw_v_encode needs. */
size_t qadamw_v_workspace_bytes(int64_t rows, int64_t cols);

/* Quantized-state AdamW second moment (Full-Stack FP4 sec. 3.3; gist.science summary
 * sec. 2.2): y = sqrt(v); mu = per-16x16-tile mean of y stored as bfloat16; residual
 * y - mu; random Hadamard transform of each 1x16 chunk along the rows (signs from
 * `seed` when use_signs != 0, plain normalised H16 otherwise); NVFP4 1x16
 * nearest-even quantization of the residual.
 *   v       f32 [rows][cols], non-negative, 16-byte aligned
 *   mu      bf16 bits [rows/16][cols/16]
 *   q       one copy: codes [rows][cols/2], scales [rows][cols/16], gscale
 *   ws      workspace of at least qadamw_v_workspace_bytes() bytes
 * rows and cols must be multiples of 16. */
int qadamw_v_encode(const float* v, int64_t rows, int64_t cols, uint64_t seed, int32_t use_signs,
                    uint16_t* mu, const nvfp4_qtensor* q, void* ws, size_t ws_bytes,
                    void* stream);

/* Inverse pipeline: v_out = (D (1/4 H16 x_hat) + mu)^2 with x_hat the dequantized
 * residual (reconstruction formula of Full-Stack FP4 sec. 3.3).  Same layouts; seed and
 * use_signs must match the encode call. */
int qadamw_v_decode(const uint16_t* mu, const nvfp4_qtensor* q, int64_t rows, int64_t cols,
                    uint64_t seed, int32_t use_signs, float* v_out, void* stream);

/* Quantized-state AdamW step (Full-Stack FP4 sec. 2: m = beta1 m + c g,
 * v = beta2 v + (1 - beta2) g^2; sec. 3.3: m stored through a Hadamard rotation, 4/6
 * scaling and stochastic rounding, v through the qadamw_v pipeline; the update, not printed
 * there, is read as decoupled AdamW):
 *   m = beta1 m_old + grad_coef g;  v = beta2 v_old + (1 - beta2) g^2;
 *   w = w - lr (bias1 m / (sqrt(bias2 v) + eps) + weight_decay w)
 * each operation one binary32 rounding in this order (the division correctly rounded).
 *   grad_coef      1 in the pages' form of m, 1 - beta1 in the common one
 *   bias1, bias2   bias-correction multipliers, e.g. 1/(1 - beta^t), or 1
 *   m_rht_seed     signs of m's 1x16 Hadamard rotation; fixed for the life of the state
 *   m_sr_seed      stochastic rounding of the new m; fresh each step
 *   v_seed, v_use_signs   as qadamw_v_encode; fixed for the life of the state */
typedef struct {
    float lr, beta1, beta2, eps, weight_decay, grad_coef, bias1, bias2;
    uint64_t m_rht_seed, m_sr_seed, v_seed;
    int32_t v_use_signs;
} qadamw_step_params;

/* Device workspace (bytes) qadamw_step needs. */
size_t qadamw_step_workspace_bytes(int64_t rows, int64_t cols);

/* One step on a rows x cols parameter (multiples of 16).
 *   w        f32 [rows][cols] master weights, updated in place, 16-byte aligned
 *   g        gradient, f32 or bf16 per g_dtype, [rows][cols], 16-byte aligned
 *   m_in     first-moment state: NVFP4 1x16 copy of the rotated m (codes, scales, s_g)
 *   m_out    the new first-moment state (same layout); must not overlap m_in
 *   mu_in, v_in    second-moment state as written by qadamw_v_encode
 *   mu_out, v_out  the new second-moment state; must not overlap mu_in, v_in
 *   ws       workspace of at least qadamw_step_workspace_bytes() bytes, 16-byte aligned
 * A zero state (all codes and scales 0, tile means 0, any s_g) decodes to m = v = 0. */
int qadamw_step(float* w, const void* g, int g_dtype, int64_t rows, int64_t cols,
                const nvfp4_qtensor* m_in, const nvfp4_qtensor* m_out,
                const uint16_t* mu_in, const nvfp4_qtensor* v_in, uint16_t* mu_out,
                const nvfp4_qtensor* v_out, const qadamw_step_params* p, void* ws,
                size_t ws_bytes, void* stream);

/* Static string naming a status code. */
const char* nvfp4_status_string(int status);
/* NVFP4_ABI_VERSION of the loaded library. */
int nvfp4_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif
