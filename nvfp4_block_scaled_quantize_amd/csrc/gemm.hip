// gemm.hip -- W4A4 NVFP4 GEMM for gfx950: C = s_gA s_gB * A_hat B_hat^T, FP32 accumulate.
//
// Method: Full-Stack FP4 sec. 2 and eq. (1)-(2) (the three GEMMs of a linear layer on
// NVFP4 operands); NVFP4 report sec. 4 (FP4 inputs, FP32 output) and A.2 (decode
// scales stored for the matrix multiplication).
//
// Exactness.  A decoded element times its E4M3 block scale, v * s, has at most a
// 6-bit significand and lies in [2^-10, 2688], so it is exact in binary16; the f16
// matrix cores multiply such values exactly and accumulate in FP32.  The only rounding
// is therefore the FP32 accumulation (plus the final multiply by s_gA s_gB).  gfx950's
// block-scaled FP4 MFMA takes power-of-two scales per 32 elements and cannot carry
// E4M3 scales per 16 elements exactly, so it is not used.
//
// Work decomposition.  One workgroup (4 waves) computes a 256x256 tile of C; wave
// (wm, wn) owns a 128x128 sub-tile as 4x4 MFMA 32x32x16 accumulators.  Packed codes and
// scale bytes (not decoded values) are staged through LDS, 128 K-elements (64 bytes per
// row) per stage: on gfx950 LDS writes run at about a third of the read rate, so
// staging 4-bit codes instead of 16-bit values keeps LDS off the critical path.  Each
// wave decodes its own MFMA operands right before use: the hardware fp4 -> f16
// conversion (exact; it issues at a quarter of the VALU rate) asked for v * 256 through
// its power-of-two scale operand, and one packed f16 multiply by s / 256, which is the
// E4M3 scale byte shifted into the binary16 fields.  Conversions and multiplies are
// interleaved between the MFMAs of the previous slot so that the VALU work runs under
// the matrix cores.
//
// Staging.  Two paths fill the LDS tiles.
//  * Direct (K % 64 == 0, scale rows 4-byte aligned, each operand under 2 GiB): buffer
//    loads with the LDS flag write global bytes straight into LDS, lane l of a load to
//    LDS address base + 16 l (or 4 l), so neither VGPRs nor LDS store instructions are
//    spent, and four stages are in flight.  A lane whose 16-byte chunk lies outside the
//    operand (row past M or N, k past K) gets an offset past the end of its buffer, and
//    the buffer range check turns its load into zeros.  The choice of which global
//    chunk each lane fetches lays the tile out in the swizzled order below.
//  * Generic (any K % 16 == 0): each thread loads its chunks into registers with bounds
//    checks and stores them to LDS; two stages.
//
// K ordering.  An MFMA sums over 16 k-slots; lanes 0-31 supply slots 0-7 and lanes
// 32-63 slots 8-15.  Lane (i, h) of both operands reads the 64 contiguous k of half h
// of the stage and feeds nibbles 8t..8t+7 to the t-th MFMA, so slot k of A always meets
// slot k of B and every k of the stage is summed exactly once.
#include "nvfp4.h"
#include "device_common.h"

#include <atomic>
#include <cstdlib>

namespace nvfp4 {

constexpr int GBM = 256, GBN = 256, GBK = 128;  // GBK in elements: 64 bytes of codes per row
constexpr int GThreads = 256;
constexpr int kStageCodeBytes = GBM * 64;       // per operand
constexpr int kStageScaleBytes = GBM * 8;       // per operand
constexpr int kStageBytes = 2 * kStageCodeBytes + 2 * kStageScaleBytes;
// Stage buffers in LDS: two for the register-staged path, four (144 KiB) for the direct
// path, whose loads then run three stages ahead (three stages measured 1-3% slower).
constexpr int kRegStages = 2, kDmaStages = 4;
constexpr int kGemmLds = kRegStages * kStageBytes;
constexpr int kGemmDmaLds = kDmaStages * kStageBytes;
// direct loads per wave and stage: 4 + 4 code chunks, 2 + 2 scale words
constexpr int kDmaLoadsPerStage = 12;
// MFMAs per direct load in the stage's second half: the loads of the four waves, issued at
// once, queue in the texture-address unit and hold up the waves behind them; one load per
// two MFMAs measured best against one per MFMA or per four.
constexpr int kDmaSpread = 2;

struct GArgs {
    const uint8_t* ac;
    const uint8_t* as;
    const float* asg;
    const uint8_t* bc;
    const uint8_t* bs;
    const float* bsg;
    int64_t M, N, K;
    float* c;
    int64_t ldc;
    int tiles_m, tiles_n;
    const uint16_t* lt;   // low-rank term: T [M][lr] and L [N][lr] (BF16), or null
    const uint16_t* lb;
    int64_t lr;
    const float* d;       // C = alpha * product + beta * D (the EpiAxpby kernels)
    int64_t ldd;
    float alpha, beta;
    float* part;          // EpiPart: [kparts][triangle tiles][256][256] raw accumulators
    int kparts;
    // balanced schedule, k_gemm_sk: whole rounds, remaining tiles (each split in two K
    // halves), K stages per tile; launch epoch tagging the hand-off flags; longest wait for a
    // hand-off (wall-clock ticks); sk_test != 0 makes every tail half skip its hand-off (so
    // that the head computes it itself; for tests)
    int sk_rounds, sk_rem;
    int sk_nst;
    uint64_t sk_epoch;
    uint64_t sk_spin;
    int sk_test;
    // EpiBf16: C as bfloat16 (row pitch ldc) and each tile's maximum of |C| (or null)
    uint16_t* c16;
    float* tmax;
    // a product whose last round runs as half-width tiles (k_gemm_half): sk_g workgroups per
    // round, sk_rounds whole rounds, sk_rem remaining tiles; 0 when there is none
    int sk_g;
};

// Epilogue variants: plain product; plus the LoRA-SVD low-rank term; alpha * product +
// beta * D (the Newton-Schulz updates).
// EpiPart: the raw accumulators of one K-part of an upper-triangle tile of A A^T go to a
// partial buffer (k_syrk_reduce sums the parts and mirrors the result).
// EpiBf16: the plain product rounded to bfloat16, with each tile's maximum of |C|.
enum { EpiPlain = 0, EpiLora = 1, EpiAxpby = 2, EpiPart = 3, EpiBf16 = 4 };

// Packed tile layout: row r holds 64 bytes as four 16-byte chunks; chunk q sits at slot
// q ^ (r/4 mod 4), which keeps both the staging stores (four lanes per row) and the
// fragment reads (one chunk of sixteen consecutive rows per 16 lanes) on distinct banks.
// Scale bytes: row r's eight bytes of the stage at offset 8 r of the operand's scale area.
__device__ __forceinline__ int code_off(int row, int chunk) {
    return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4);
}

// ---------------------------------------------------------------- one stage of MMA

// {s/256, s/256} as a binary16 pair from byte B of w, an E4M3 scale code with the sign
// bit clear: the code shifted left by 7 lands its exponent and mantissa in the binary16
// fields, which reads as the scale / 256 for normal and subnormal codes alike.
template <int B>
__device__ __forceinline__ half2v scale_pair(uint32_t w) {
    constexpr uint32_t sel = 0x000C000Cu | (B << 8) | (B << 24);   // bytes {0, b, 0, b}
    return __builtin_bit_cast(half2v, __builtin_amdgcn_perm(0u, w, sel) >> 1);
}

// 8 codes -> 8 binary16 values (v * 256) * (s / 256) = v * s (exact), in the order
// (n0, n1), (n2, n3), (n4, n5), (n6, n7) of the word's nibbles.  The conversion reads
// one VGPR per output pair; bit-manipulation decodes (byte-table v_perm and the like)
// need fewer issue cycles but several VGPR operands per pair, and measured slower here
// because the MFMAs running beside them compete for the same register-file ports.
__device__ __forceinline__ half8v decode8(uint32_t w, half2v s2) {
    const half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 0) * s2;
    const half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 1) * s2;
    const half2v p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2) * s2;
    const half2v p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 3) * s2;
    half8v o = {p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
    return o;
}

__device__ __forceinline__ uint32_t dword_of(const uint4& v, int i) {
    return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// Sched-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedVALU = 0x002, kSchedMFMA = 0x008;

// This wave's packed operands of one stage: 32 code bytes and 4 scale bytes per sub-tile.
struct Frags {
    uint4 fa[4][2], fb[4][2];
    uint32_t wsa[4], wsb[4];
};

__device__ __forceinline__ void read_frags(const uint8_t* cur, int wm, int wn, int h, int li,
                                           Frags& f) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        const int ra = wm * 128 + x * 32 + li, rb = wn * 128 + x * 32 + li;
#pragma unroll
        for (int c2 = 0; c2 < 2; ++c2) {
            f.fa[x][c2] = *(const uint4*)(cur + code_off(ra, 2 * h + c2));
            f.fb[x][c2] = *(const uint4*)(cur + kStageCodeBytes + code_off(rb, 2 * h + c2));
        }
        f.wsa[x] = *(const uint32_t*)(cur + 2 * kStageCodeBytes + ra * 8 + 4 * h);
        f.wsb[x] = *(const uint32_t*)(cur + 2 * kStageCodeBytes + kStageScaleBytes + rb * 8 + 4 * h);
    }
}

__device__ __forceinline__ void mma_stage(const Frags& f, float16v (&acc)[4][4]) {
    // scales of this lane's four blocks per sub-tile as binary16 pairs
    half2v psa[4][4], psb[4][4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        psa[x][0] = scale_pair<0>(f.wsa[x]); psa[x][1] = scale_pair<1>(f.wsa[x]);
        psa[x][2] = scale_pair<2>(f.wsa[x]); psa[x][3] = scale_pair<3>(f.wsa[x]);
        psb[x][0] = scale_pair<0>(f.wsb[x]); psb[x][1] = scale_pair<1>(f.wsb[x]);
        psb[x][2] = scale_pair<2>(f.wsb[x]); psb[x][3] = scale_pair<3>(f.wsb[x]);
    }
    half8v av[4], bv[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        av[x] = decode8(f.fa[x][0].x, psa[x][0]);
        bv[x] = decode8(f.fb[x][0].x, psb[x][0]);
    }
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
        half8v an[4], bn[4];
        if (tt < 7) {
#pragma unroll
            for (int x = 0; x < 4; ++x) {
                an[x] = decode8(dword_of(f.fa[x][(tt + 1) >> 2], (tt + 1) & 3), psa[x][(tt + 1) >> 1]);
                bn[x] = decode8(dword_of(f.fb[x][(tt + 1) >> 2], (tt + 1) & 3), psb[x][(tt + 1) >> 1]);
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
        // each MFMA followed by four decode instructions of the next slot
#pragma unroll
        for (int k = 0; k < 16; ++k) {
            __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
            __builtin_amdgcn_sched_group_barrier(kSchedVALU, 4, 0);
        }
        if (tt < 7) {
#pragma unroll
            for (int x = 0; x < 4; ++x) { av[x] = an[x]; bv[x] = bn[x]; }
        }
    }
}

// D register r of lane l is row 8(r/4) + 4(l/32) + r%4, column l%32 of its 32x32 block.
// Rows are written whole before the next: for each row the four 128-byte pieces of its
// 512-byte span come from consecutive stores, which keeps DRAM pages open.  The stores are
// non-temporal: C is written once and not read back here, and letting it stream past
// the caches cut the FFN-up GEMM from 508 to 433 us on this part.  One block row
// (32 rows) at a time, with a scheduling fence between block rows, so the compiler does
// not pull all 256 accumulators into VGPRs at once.
// MODE: StPlain stores acc * scale; StAdd first adds the raw partial sum that the same
// position of C holds (the other K half of a tile split by the balanced schedule),
// fl(acc + p) * scale; StAxpby stores fma(scale, acc, fl(beta d)) with d from D (which may be
// C: each element of D is read by the lane that writes the same element of C, before it);
// StPark stores acc * scale with ordinary stores: a parked K half is read back by the other
// workgroup of its tile on the same XCD, which then finds it in the caches (balanced
// FFN-down 369.6 -> 364.7 us against non-temporal parking).
// A block row's 64 loads are issued before any of its stores: a load issued after stores can
// only be waited for together with them.  FULL: the tile lies inside C, so no element needs a
// bounds test (a test per element becomes a branch, and the compiler waits for every
// outstanding store at each branch's end).
enum { StPlain = 0, StAdd = 1, StAxpby = 2, StPark = 3 };
template <int MODE, bool FULL>
__device__ __forceinline__ void store_rows(const GArgs& g, const float16v (&acc)[4][4], int64_t m0,
                                           int64_t n0, int wm, int wn, int h, int li, float scale) {
    const int64_t rbase = m0 + wm * 128 + 4 * h, cbase = n0 + wn * 128 + li;
    constexpr int RB = MODE == StAxpby ? 8 : 16;  // accumulator rows per batch of loads
#pragma unroll
    for (int b = 0; b < 64; b += RB) {
        const int i = b >> 4;
        float pv[RB][4];
        if constexpr (MODE == StAdd || MODE == StAxpby) {
#pragma unroll
            for (int r = b & 15; r < (b & 15) + RB; ++r) {
                const int64_t row = rbase + i * 32 + 8 * (r >> 2) + (r & 3);
                const float* src = MODE == StAdd ? g.c + row * g.ldc + cbase : g.d + row * g.ldd + cbase;
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    pv[r - (b & 15)][j] = (FULL || (row < g.M && cbase + j * 32 < g.N)) ? src[j * 32] : 0.0f;
            }
        }
#pragma unroll
        for (int r = b & 15; r < (b & 15) + RB; ++r) {
            const int64_t row = rbase + i * 32 + 8 * (r >> 2) + (r & 3);
            float* rowp = g.c + row * g.ldc + cbase;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (FULL || (row < g.M && cbase + j * 32 < g.N)) {
                    if constexpr (MODE == StAxpby) {
                        rowp[j * 32] = __builtin_fmaf(scale, acc[i][j][r], g.beta * pv[r - (b & 15)][j]);
                    } else {
                        float x = acc[i][j][r];
                        if constexpr (MODE == StAdd) x = x + pv[r - (b & 15)][j];
                        if constexpr (MODE == StPark) rowp[j * 32] = x * scale;
                        else __builtin_nontemporal_store(x * scale, rowp + j * 32);
                    }
                }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

template <int MODE = StPlain>
__device__ __forceinline__ void store_tile(const GArgs& g, const float16v (&acc)[4][4], int64_t m0,
                                           int64_t n0, int wm, int wn, int h, int li, float scale) {
    if (m0 + GBM <= g.M && n0 + GBN <= g.N) store_rows<MODE, true>(g, acc, m0, n0, wm, wn, h, li, scale);
    else store_rows<MODE, false>(g, acc, m0, n0, wm, wn, h, li, scale);
}

// bfloat16 output: C = bf16_rne(fl(acc s)), one block row at a time as in store_rows.
// Returns this lane's maximum of fl(|acc| s) over the elements it stores (NaN ignored);
// rounding is monotone, so the largest |C| is that maximum rounded to bf16.  Ordinary stores,
// unlike the FP32 output's non-temporal ones: a bf16 C of FFN-up size (151 MB) then stays in
// the 256 MB last-level cache for the kernel that reads it next (its quantize), at no cost
// to this kernel.
template <bool FULL>
__device__ __forceinline__ float store_rows_bf16(const GArgs& g, const float16v (&acc)[4][4],
                                                 int64_t m0, int64_t n0, int wm, int wn, int h,
                                                 int li, float scale) {
    const int64_t rbase = m0 + wm * 128 + 4 * h, cbase = n0 + wn * 128 + li;
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t row = rbase + i * 32 + 8 * (r >> 2) + (r & 3);
            uint16_t* rowp = g.c16 + row * g.ldc + cbase;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (FULL || (row < g.M && cbase + j * 32 < g.N)) {
                    const float y = acc[i][j][r] * scale;
                    mx = fmaxf(mx, fabsf(y));
                    rowp[j * 32] = __builtin_bit_cast(uint16_t, (__bf16)y);
                }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    return mx;
}

// The tile's maximum of |C| into tmax[tile row * tiles_n + tile column], as the bf16 value
// (widened to FP32): a wave reduction, then the four waves' values through LDS (free after
// the main loop).
__device__ __forceinline__ void tile_max_out(const GArgs& g, uint8_t* lds, float mx, int64_t m0,
                                             int64_t n0) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    float* red = (float*)lds;
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = mx;
    __syncthreads();
    if (threadIdx.x == 0) {
        const float m = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
        g.tmax[(m0 / GBM) * g.tiles_n + n0 / GBN] = (float)(__bf16)m;
    }
}

// The raw accumulators of the tile into its 256 x 256 slot of the partial buffer (row-major),
// in the row order of store_tile.
__device__ __forceinline__ void store_part(float* slot, const float16v (&acc)[4][4], int wm, int wn,
                                           int h, int li) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            float* rowp = slot + (wm * 128 + 4 * h + i * 32 + 8 * (r >> 2) + (r & 3)) * GBN +
                          wn * 128 + li;
#pragma unroll
            for (int j = 0; j < 4; ++j) rowp[j * 32] = acc[i][j][r];
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// Upper-triangle tile t (row-major over tm <= tn) of a T x T tile grid.
__device__ __forceinline__ void tri_tile(int t, int T, int& tm, int& tn) {
    int r = 0, rem = t;
    while (rem >= T - r) {
        rem -= T - r;
        ++r;
    }
    tm = r;
    tn = r + rem;
}

// ---------------------------------------------------------------- low-rank epilogue

// LoRA-SVD up-projection in the epilogue (Full-Stack FP4 sec. 3.2 eq. (1), Appendix 9: the
// low-rank branch shares the GEMM's output tile).  After the main loop the stage buffers are
// free: the workgroup copies its 256 rows of T and of L, 64 rank entries at a time, into
// LDS (one round trip instead of one per MFMA operand).  The accumulators are scaled by
// s_gA s_gB in place, and per 16 rank entries each wave reads its 4 T and 4 L fragments
// and issues its 16 BF16 MFMAs 32x32x16 (FP32 accumulate) on them.  LDS rows hold 8 chunks
// of 16 bytes, chunk c at c ^ (row mod 8),
// so the fragment reads (16 bytes of 32 consecutive rows per half-wave) spread over the
// banks.  Lane (li, h) supplies row li of the block and rank entries 8h..8h+7 of a step.
typedef __bf16 bf16x8v __attribute__((ext_vector_type(8)));
constexpr int kLoraChunk = 64;                    // rank entries staged per round
constexpr int kLoraLdsRow = kLoraChunk * 2;       // bytes per staged row

__device__ __forceinline__ void stage_lora(const GArgs& g, uint8_t* lds, int64_t m0, int64_t n0,
                                           int64_t k0, int kc) {
    // kc rank entries (a multiple of 16) from k0, rows of T then rows of L
    if (kc == kLoraChunk && (uint64_t)g.M * g.lr * 2 < kOutOfRange &&
        (uint64_t)g.N * g.lr * 2 < kOutOfRange) {
        // A full chunk by direct loads: 64 KB in 64 loads of 1 KB, 16 per wave, all in
        // flight at once.  Load S fills LDS bytes [1024 S, +1024): 8 rows of one matrix,
        // lane l taking the global chunk whose swizzled position is l mod 8.  Rows past M or
        // N read zeros (offset past the buffer's end).
        const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
        const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
        const int4v rt = make_rsrc(g.lt, (uint32_t)(g.M * g.lr * 2));
        const int4v rl = make_rsrc(g.lb, (uint32_t)(g.N * g.lr * 2));
#pragma unroll
        for (int i = 0; i < 2 * GBM * kLoraLdsRow / 1024 / 4; ++i) {
            const int S = i * 4 + wid, which = S / (GBM * kLoraLdsRow / 1024);
            const int row = (S % (GBM * kLoraLdsRow / 1024)) * 8 + (lane >> 3);
            const int ch = (lane & 7) ^ (row & 7);
            const int64_t grow = (which ? n0 : m0) + row;
            const uint32_t off = grow < (which ? g.N : g.M)
                                     ? (uint32_t)((grow * g.lr + k0 + ch * 8) * 2) : kOutOfRange;
            dma16(which ? rl : rt, lds0 + (uint32_t)S * 1024, off);
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        return;
    }
    const int chunks = kc / 8;                    // 16-byte chunks per row
    for (int q = threadIdx.x; q < 2 * GBM * chunks; q += GThreads) {
        const int which = q / (GBM * chunks), rem = q % (GBM * chunks);
        const int row = rem / chunks, ch = rem % chunks;
        const int64_t grow = (which ? n0 : m0) + row;
        const int64_t rows = which ? g.N : g.M;
        const uint16_t* src = which ? g.lb : g.lt;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (grow < rows) v = *(const uint4*)(src + grow * g.lr + k0 + ch * 8);
        *(uint4*)(lds + which * GBM * kLoraLdsRow + row * kLoraLdsRow + ((ch ^ (row & 7)) << 4)) = v;
    }
}

__device__ __forceinline__ bf16x8v lds_frag(const uint8_t* lds, int which, int row, int ch) {
    return __builtin_bit_cast(bf16x8v, *(const uint4*)(lds + which * GBM * kLoraLdsRow +
                                                        row * kLoraLdsRow + ((ch ^ (row & 7)) << 4)));
}

// add: as for store_tile, the partial held in C is added before the scaling.
__device__ __forceinline__ void lora_epilogue(const GArgs& g, uint8_t* lds, float16v (&acc)[4][4],
                                              int64_t m0, int64_t n0, int wm, int wn, int h, int li,
                                              bool add = false) {
    const float scale = *g.asg * *g.bsg;
    const int ra = wm * 128 + li, rb = wn * 128 + li;
    for (int64_t k0 = 0; k0 < g.lr; k0 += kLoraChunk) {
        const int kc = g.lr - k0 < kLoraChunk ? (int)(g.lr - k0) : kLoraChunk;
        __syncthreads();   // every wave is done with the stage buffers (or the previous chunk)
        stage_lora(g, lds, m0, n0, k0, kc);
        __syncthreads();
        if (k0 == 0) {
            const int64_t rbase = m0 + wm * 128 + 4 * h, cbase = n0 + wn * 128 + li;
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int r = 0; r < 16; ++r) {
                        float x = acc[i][j][r];
                        if (add) {
                            const int64_t row = rbase + i * 32 + 8 * (r >> 2) + (r & 3);
                            const int64_t col = cbase + j * 32;
                            if (row < g.M && col < g.N) x = x + g.c[row * g.ldc + col];
                        }
                        acc[i][j][r] = x * scale;
                    }
        }
        // per 16 rank entries: the wave's 4 A and 4 B fragments, then its 16 products
        for (int s = 0; s < kc; s += 16) {
            bf16x8v a[4], b[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = lds_frag(lds, 0, ra + 32 * i, s / 8 + h);
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = lds_frag(lds, 1, rb + 32 * j, s / 8 + h);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
        }
    }
}

// The epilogue variant is a compile-time switch so that the plain kernels keep their
// register allocation.  mode (the balanced schedule's; every other caller takes 1):
// 0 the raw accumulators into C (a K half parked for the other half's workgroup), 1 the
// tile's result, 2 the result of the accumulators plus the half parked in C, 3 NaN (the
// parked half was lost).
enum { FinPark = 0, FinResult = 1, FinAdd = 2, FinNan = 3 };
template <int EPI>
__device__ __forceinline__ void finish_tile(const GArgs& g, uint8_t* lds, float16v (&acc)[4][4],
                                            int64_t m0, int64_t n0, int wm, int wn, int h, int li,
                                            int mode = FinResult) {
    const float nan = __builtin_nanf("");
    if constexpr (EPI == EpiLora) {
        if (mode == FinResult || mode == FinAdd)
            lora_epilogue(g, lds, acc, m0, n0, wm, wn, h, li, mode == FinAdd);
        store_tile(g, acc, m0, n0, wm, wn, h, li, mode == FinNan ? nan : 1.0f);
    } else if constexpr (EPI == EpiAxpby) {
        // alpha * product + beta * D, stored as fma(fl(alpha s_gA s_gB), acc, fl(beta d))
        store_tile<StAxpby>(g, acc, m0, n0, wm, wn, h, li, (*g.asg * *g.bsg) * g.alpha);
    } else if constexpr (EPI == EpiPart) {
        store_part(g.part + ((int64_t)blockIdx.x << 16), acc, wm, wn, h, li);
    } else if constexpr (EPI == EpiBf16) {   // one workgroup per tile: mode is FinResult
        const float scale = *g.asg * *g.bsg;
        const float mx = m0 + GBM <= g.M && n0 + GBN <= g.N
                             ? store_rows_bf16<true>(g, acc, m0, n0, wm, wn, h, li, scale)
                             : store_rows_bf16<false>(g, acc, m0, n0, wm, wn, h, li, scale);
        if (g.tmax) tile_max_out(g, lds, mx, m0, n0);
    } else {
        const float scale = mode == FinPark ? 1.0f : (mode == FinNan ? nan : *g.asg * *g.bsg);
        if (mode == FinAdd) store_tile<StAdd>(g, acc, m0, n0, wm, wn, h, li, scale);
        else if (mode == FinPark) store_tile<StPark>(g, acc, m0, n0, wm, wn, h, li, scale);
        else store_tile(g, acc, m0, n0, wm, wn, h, li, scale);
    }
}

// Tile of workgroup `bid`.  Workgroups are dealt to the eight XCDs round-robin (bid mod 8)
// and each XCD has its own L2, so XCD x is given the contiguous range of tile ids
// [x T/8, (x+1) T/8) (remainder spread over the first XCDs), and tile ids walk down
// groups of 8 tile rows column by column: the 32 workgroups an XCD runs at once then share
// A rows of 8 tile rows and B rows of about 4 tile columns in that XCD's L2.
constexpr int kXcds = 8, kGroupRows = 8;
__device__ __forceinline__ void tile_of(int bid, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int total = tiles_m * tiles_n;
    const int q = total / kXcds, r = total % kXcds;
    const int x = bid % kXcds, k = bid / kXcds;
    const int id = x * q + (x < r ? x : r) + k;
    const int group = id / (kGroupRows * tiles_n);
    const int first = group * kGroupRows;
    const int rows = tiles_m - first < kGroupRows ? tiles_m - first : kGroupRows;
    const int in = id - group * kGroupRows * tiles_n;
    tm = first + in % rows;
    tn = in / rows;
}

// Workgroup number of blockIdx b in a grid of G (G % 8 == 0) whose blocks go to the 8 XCDs in
// turn: XCD x gets the contiguous numbers [x G/8, (x+1) G/8).
__device__ __forceinline__ int sk_virtual(int b, int G) {
    return (b & 7) * (G >> 3) + (b >> 3);
}

// Tile id -> (tm, tn): groups of kGroupRows tile rows, column by column within a group.
__device__ __forceinline__ void grouped_tile(int id, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int group = id / (kGroupRows * tiles_n);
    const int first = group * kGroupRows;
    const int rows = tiles_m - first < kGroupRows ? tiles_m - first : kGroupRows;
    const int in = id - group * kGroupRows * tiles_n;
    tm = first + in % rows;
    tn = in / rows;
}

__device__ __forceinline__ void zero_acc(float16v (&acc)[4][4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;
}

// ---------------------------------------------------------------- generic staging path

struct StageRegs {
    uint4 a[4], b[4];
    uint2 sa, sb;
};

__device__ __forceinline__ uint2 load_scales8(const uint8_t* base, int64_t row, int64_t rows,
                                              int64_t kb0, int64_t kblocks) {
    if (row >= rows) return make_uint2(0u, 0u);
    const uint8_t* p = base + row * kblocks + kb0;
    const int64_t left = kblocks - kb0;
    if (left >= 8 && ((uintptr_t)p & 7) == 0) return *(const uint2*)p;
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i)
        if (i < left) w[i >> 2] |= (uint32_t)p[i] << (8 * (i & 3));
    return make_uint2(w[0], w[1]);
}

// 16 code bytes at p, the last 8 zero when only 8 are left in the row: rows of K % 32 == 16
// codes are 8-byte aligned and end in a half chunk.
__device__ __forceinline__ uint4 load_chunk8(const uint8_t* p, int64_t left) {
    const uint2 lo = *(const uint2*)p;
    const uint2 hi = left >= 16 ? *(const uint2*)(p + 8) : make_uint2(0u, 0u);
    return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

__device__ __forceinline__ void load_stage(const GArgs& g, int64_t m0, int64_t n0, int s,
                                           StageRegs& r) {
    const int t = threadIdx.x;
    const int64_t kbytes = g.K / 2, k0b = (int64_t)s * 64;
    const bool whole = (kbytes & 15) == 0;   // K % 32 == 0: 16-byte aligned whole chunks
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = t + GThreads * i, row = q >> 2, ch = q & 3;
        const int64_t off = k0b + ch * 16;
        const int64_t gm = m0 + row, gn = n0 + row;
        const uint4 z = make_uint4(0u, 0u, 0u, 0u);
        if (whole) {
            r.a[i] = (gm < g.M && off < kbytes) ? *(const uint4*)(g.ac + gm * kbytes + off) : z;
            r.b[i] = (gn < g.N && off < kbytes) ? *(const uint4*)(g.bc + gn * kbytes + off) : z;
        } else {
            r.a[i] = (gm < g.M && off < kbytes) ? load_chunk8(g.ac + gm * kbytes + off, kbytes - off) : z;
            r.b[i] = (gn < g.N && off < kbytes) ? load_chunk8(g.bc + gn * kbytes + off, kbytes - off) : z;
        }
    }
    const int64_t kblocks = g.K / 16, kb0 = (int64_t)s * 8;
    r.sa = load_scales8(g.as, m0 + t, g.M, kb0, kblocks);
    r.sb = load_scales8(g.bs, n0 + t, g.N, kb0, kblocks);
}

__device__ __forceinline__ void store_stage(uint8_t* buf, const StageRegs& r) {
    const int t = threadIdx.x;
    uint8_t* ac = buf;
    uint8_t* bc = buf + kStageCodeBytes;
    uint8_t* as = buf + 2 * kStageCodeBytes;
    uint8_t* bs = as + kStageScaleBytes;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = t + GThreads * i, row = q >> 2, ch = q & 3;
        *(uint4*)(ac + code_off(row, ch)) = r.a[i];
        *(uint4*)(bc + code_off(row, ch)) = r.b[i];
    }
    *(uint2*)(as + t * 8) = r.sa;
    *(uint2*)(bs + t * 8) = r.sb;
}

template <int EPI>
__global__ __launch_bounds__(GThreads, 1) void k_gemm(GArgs g) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6, wm = wid >> 1, wn = wid & 1;
    int tm, tn;
    tile_of(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
    const int64_t m0 = (int64_t)tm * GBM, n0 = (int64_t)tn * GBN;
    const int h = lane >> 5, li = lane & 31;

    float16v acc[4][4];
    zero_acc(acc);
    const int nst = (int)((g.K + GBK - 1) / GBK);
    StageRegs regs;
    if (nst > 0) {
        load_stage(g, m0, n0, 0, regs);
        store_stage(lds, regs);
    }
    __syncthreads();
    for (int s = 0; s < nst; ++s) {
        const uint8_t* cur = lds + (s & 1) * kStageBytes;
        if (s + 1 < nst) load_stage(g, m0, n0, s + 1, regs);
        Frags f;
        read_frags(cur, wm, wn, h, li, f);
        mma_stage(f, acc);
        if (s + 1 < nst) store_stage(lds + ((s + 1) & 1) * kStageBytes, regs);
        __syncthreads();
    }
    finish_tile<EPI>(g, lds, acc, m0, n0, wm, wn, h, li);
}

// ---------------------------------------------------------------- direct staging path

struct Rsrc4 {
    int4v ac, as, bc, bs;
};

// This wave's 12 direct loads of one K stage: the global offsets of its four code chunks
// per operand (16 bytes per lane) and two scale words per operand (4 bytes per lane), and
// the LDS stage they fill.  Load i of the codes covers LDS slots [256 i + 64 wid, +64) of
// the operand's tile; slot p = row * 4 + q receives global chunk q ^ (row/4 mod 4) of the
// row, which is the layout code_off describes.  A stage outside [c.s0, c.s0 + c.nst) gets
// offsets past the end of every operand: its loads read nothing and write zeros into buf.
struct StageLoads {
    uint32_t ca[4], cb[4], sa[2], sb[2];
    uint32_t buf;
};

template <int K>
__device__ __forceinline__ void issue_load(const Rsrc4& rs, const StageLoads& L, int wid) {
    if constexpr (K < 8) {
        const uint32_t dst = L.buf + (uint32_t)((K >> 1) * 256 + wid * 64) * 16;
        if constexpr (K & 1) dma16(rs.bc, dst + kStageCodeBytes, L.cb[K >> 1]);
        else dma16(rs.ac, dst, L.ca[K >> 1]);
    } else {
        constexpr int i = (K - 8) >> 1;
        const uint32_t dst = L.buf + 2 * kStageCodeBytes + (uint32_t)(i * 256 + wid * 64) * 4;
        if constexpr (K & 1) dma4(rs.bs, dst + kStageScaleBytes, L.sb[i]);
        else dma4(rs.as, dst, L.sa[i]);
    }
}

// Wait until at most N of this wave's direct loads are outstanding (they complete in
// issue order), then meet the other waves: after it every wave's loads of the awaited
// stage are in LDS and every wave has finished reading the buffer about to be refilled.
template <int N>
__device__ __forceinline__ void dma_wait_barrier() {
    if constexpr (N == 0)
        asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)\n\ts_barrier" ::: "memory");
    else
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N) : "memory");
}

// Software-pipelined stage of the direct path.  A wave's packed operands of a stage are
// held as two halves: `lo` (code words of slots 0..3) and `hi` (slots 4..7), plus the four
// scale words per operand.  Once slot 4 is decoded `lo` is dead, so the next stage's `lo`
// and scale words are read into it mid-stage (after that stage's barrier); once slot 7 is
// decoded `hi` is dead and the next `hi` is read.  Slot 7's MFMAs then cover the decode of
// the next stage's slot 0, so the matrix cores do not idle across the stage boundary.
struct HalfFrags {
    uint4 a[4], b[4];
};
struct Pairs {
    half2v a[4], b[4];
};

__device__ __forceinline__ void read_half(const uint8_t* cur, int c2, int wm, int wn, int h, int li,
                                          HalfFrags& f) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        const int ra = wm * 128 + x * 32 + li, rb = wn * 128 + x * 32 + li;
        f.a[x] = *(const uint4*)(cur + code_off(ra, 2 * h + c2));
        f.b[x] = *(const uint4*)(cur + kStageCodeBytes + code_off(rb, 2 * h + c2));
    }
}

__device__ __forceinline__ void read_scales(const uint8_t* cur, int wm, int wn, int h, int li,
                                            uint32_t (&sa)[4], uint32_t (&sb)[4]) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        const int ra = wm * 128 + x * 32 + li, rb = wn * 128 + x * 32 + li;
        sa[x] = *(const uint32_t*)(cur + 2 * kStageCodeBytes + ra * 8 + 4 * h);
        sb[x] = *(const uint32_t*)(cur + 2 * kStageCodeBytes + kStageScaleBytes + rb * 8 + 4 * h);
    }
}

template <int B>
__device__ __forceinline__ void make_pairs(const uint32_t (&sa)[4], const uint32_t (&sb)[4], Pairs& p) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        p.a[x] = scale_pair<B>(sa[x]);
        p.b[x] = scale_pair<B>(sb[x]);
    }
}

template <int T>
__device__ __forceinline__ void decode_slot(const HalfFrags& f, const Pairs& p, half8v (&av)[4],
                                            half8v (&bv)[4]) {
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        av[x] = decode8(dword_of(f.a[x], T & 3), p.a[x]);
        bv[x] = decode8(dword_of(f.b[x], T & 3), p.b[x]);
    }
}

__device__ __forceinline__ void mma_slot(const half8v (&av)[4], const half8v (&bv)[4],
                                         float16v (&acc)[4][4]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
}

// Each MFMA of a slot followed by K VALU instructions.
template <int K>
__device__ __forceinline__ void pace() {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
        __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedVALU, K, 0);
    }
}

struct DmaCtx {
    GArgs g;
    Rsrc4 rs;
    uint32_t lds0;
    const uint8_t* lds;
    int64_t m0, n0;
    int t, wid, wm, wn, h, li, nst;
    int s0;   // first K stage of this workgroup (EpiPart: its K-part)
    uint32_t kbytes, kblocks;
};

__device__ __forceinline__ void stage_loads(const DmaCtx& c, int s, uint32_t buf, StageLoads& L) {
    const bool live = s < c.s0 + c.nst;
    const uint32_t k0b = (uint32_t)s * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = i * 256 + c.t, row = p >> 2, q = p & 3;
        const uint32_t off = k0b + (uint32_t)((q ^ ((row >> 2) & 3)) << 4);
        const bool kin = live && off < c.kbytes;
        L.ca[i] = (kin && c.m0 + row < c.g.M) ? (uint32_t)(c.m0 + row) * c.kbytes + off : kOutOfRange;
        L.cb[i] = (kin && c.n0 + row < c.g.N) ? (uint32_t)(c.n0 + row) * c.kbytes + off : kOutOfRange;
    }
    const uint32_t kb0 = (uint32_t)s * 8;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int j = i * 256 + c.t, row = j >> 1;
        const uint32_t kb = kb0 + 4 * (j & 1);
        const bool kin = live && kb < c.kblocks;
        L.sa[i] = (kin && c.m0 + row < c.g.M) ? (uint32_t)(c.m0 + row) * c.kblocks + kb : kOutOfRange;
        L.sb[i] = (kin && c.n0 + row < c.g.N) ? (uint32_t)(c.n0 + row) * c.kblocks + kb : kOutOfRange;
    }
    L.buf = buf;
}

// All 12 loads of a stage at once (the prologue).
__device__ __forceinline__ void dma_stage(const DmaCtx& c, int s, uint32_t buf) {
    StageLoads L;
    stage_loads(c, s, buf, L);
    static_for<0, 12>([&](auto K) { issue_load<K>(c.rs, L, c.wid); });
}

// Two halves of decode8: code pairs 2Q and 2Q + 1 of w into elements 4Q .. 4Q + 3 of o.
template <int Q>
__device__ __forceinline__ void decode4(uint32_t w, half2v s2, half8v& o) {
    const half2v p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2 * Q) * s2;
    const half2v p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 256.0f, 2 * Q + 1) * s2;
    o[4 * Q] = p0.x; o[4 * Q + 1] = p0.y; o[4 * Q + 2] = p1.x; o[4 * Q + 3] = p1.y;
}

// A slot's 16 MFMAs on (av, bv), each followed by a quarter of one operand's decode of slot
// T into (an, bn) and by X(k), in a scheduling region of its own: memory instructions
// placed in X are spread over the slot instead of issued as a burst.
template <int T, class Fx>
__device__ __forceinline__ void mma_slot_steps(const half8v (&av)[4], const half8v (&bv)[4],
                                               float16v (&acc)[4][4], const HalfFrags& f,
                                               const Pairs& p, half8v (&an)[4], half8v (&bn)[4],
                                               Fx&& X) {
    static_for<0, 16>([&](auto K) {
        constexpr int k = K, d = k >> 1, q = k & 1;
        acc[k >> 2][k & 3] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[k >> 2], bv[k & 3],
                                                                    acc[k >> 2][k & 3], 0, 0, 0);
        if constexpr (d < 4) decode4<q>(dword_of(f.a[d], T & 3), p.a[d], an[d]);
        else decode4<q>(dword_of(f.b[d - 4], T & 3), p.b[d - 4], bn[d - 4]);
        X(K);
        __builtin_amdgcn_sched_barrier(0);
    });
}

// Stage s.  On entry lo, hi, sa, sb hold stage s, p the scale pairs of its block 0 and
// (av, bv) its decoded slot 0; on return they hold the same for stage s + 1 (stale LDS
// data after the last stage, never used).
__device__ __forceinline__ void piped_stage(const DmaCtx& c, int s, HalfFrags& lo, HalfFrags& hi,
                                            uint32_t (&sa)[4], uint32_t (&sb)[4], Pairs& p,
                                            half8v (&av)[4], half8v (&bv)[4], float16v (&acc)[4][4]) {
    half8v an[4], bn[4];
    decode_slot<1>(lo, p, an, bn);
    mma_slot(av, bv, acc);
    pace<4>();
    make_pairs<1>(sa, sb, p);
    decode_slot<2>(lo, p, av, bv);
    mma_slot(an, bn, acc);
    pace<5>();
    decode_slot<3>(lo, p, an, bn);
    mma_slot(av, bv, acc);
    pace<4>();
    make_pairs<2>(sa, sb, p);
    decode_slot<4>(hi, p, av, bv);
    mma_slot(an, bn, acc);
    pace<5>();
    // Slot 4's operands must be formed here, under slot 3's MFMAs: without this the compiler
    // sinks their decode past the branch below, into the half of the stage that already
    // carries the next stage's slot 0, and that half becomes VALU-bound.
#pragma unroll
    for (int x = 0; x < 4; ++x) asm volatile("" : "+v"(av[x]), "+v"(bv[x]));
    // Stage s + kDmaStages refills this stage's buffer (out of range past the segment's last
    // stage).
    StageLoads L;
    stage_loads(c, c.s0 + s + kDmaStages, c.lds0 + (s % kDmaStages) * kStageBytes, L);
    // lo is dead: stage s + 1 must be in LDS (the loads of the stages after it may be in
    // flight), and every wave is done with this stage's buffer
    dma_wait_barrier<(kDmaStages - 2) * kDmaLoadsPerStage>();
    const uint8_t* nxt = c.lds + ((s + 1) % kDmaStages) * kStageBytes;
    uint32_t nsa[4], nsb[4];
    // Slots 4 to 6: each MFMA with a quarter of the next slot's decode; the 12 loads of stage
    // s + kDmaStages go one per kDmaSpread MFMAs from slot 4's first MFMA on, and the reads of the
    // next stage's lo and scale words two per MFMA over the second half of slot 4.
    const auto extra = [&](auto J, auto K) {
        constexpr int g = J * 16 + K;
        if constexpr (g % kDmaSpread == 0 && g / kDmaSpread < kDmaLoadsPerStage)
            issue_load<g / kDmaSpread>(c.rs, L, c.wid);
        if constexpr (J == 0 && K >= 8) {
            constexpr int x = (K - 8) & 3;
            const int ra = c.wm * 128 + x * 32 + c.li, rb = c.wn * 128 + x * 32 + c.li;
            if constexpr (K < 12) {
                lo.a[x] = *(const uint4*)(nxt + code_off(ra, 2 * c.h));
                lo.b[x] = *(const uint4*)(nxt + kStageCodeBytes + code_off(rb, 2 * c.h));
            } else {
                nsa[x] = *(const uint32_t*)(nxt + 2 * kStageCodeBytes + ra * 8 + 4 * c.h);
                nsb[x] = *(const uint32_t*)(nxt + 2 * kStageCodeBytes + kStageScaleBytes + rb * 8 + 4 * c.h);
            }
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    mma_slot_steps<5>(av, bv, acc, hi, p, an, bn, [&](auto K) { extra(I0{}, K); });
    make_pairs<3>(sa, sb, p);
    mma_slot_steps<6>(an, bn, acc, hi, p, av, bv, [&](auto K) { extra(I1{}, K); });
    mma_slot_steps<7>(av, bv, acc, hi, p, an, bn, [&](auto K) { extra(I2{}, K); });
    // hi is dead
    read_half(nxt, 1, c.wm, c.wn, c.h, c.li, hi);
    make_pairs<0>(nsa, nsb, p);
    decode_slot<0>(lo, p, av, bv);
    mma_slot(an, bn, acc);
    pace<5>();
#pragma unroll
    for (int x = 0; x < 4; ++x) { sa[x] = nsa[x]; sb[x] = nsb[x]; }
}

// Stages [c.s0, c.s0 + c.nst) of the tile at (c.m0, c.n0), c.nst >= 1, added onto acc: the
// first kDmaStages stages' direct loads, then the pipelined stages.  On return every direct load
// has landed and every wave has passed the last stage's barrier; LDS holds nothing needed.
__device__ __forceinline__ void run_stages(const DmaCtx& c, float16v (&acc)[4][4]) {
    for (int j = 0; j < kDmaStages; ++j) dma_stage(c, c.s0 + j, c.lds0 + j * kStageBytes);
    dma_wait_barrier<(kDmaStages - 1) * kDmaLoadsPerStage>();
    HalfFrags lo, hi;
    uint32_t sa[4], sb[4];
    Pairs p;
    half8v av[4], bv[4];
    read_half(c.lds, 0, c.wm, c.wn, c.h, c.li, lo);
    read_half(c.lds, 1, c.wm, c.wn, c.h, c.li, hi);
    read_scales(c.lds, c.wm, c.wn, c.h, c.li, sa, sb);
    make_pairs<0>(sa, sb, p);
    decode_slot<0>(lo, p, av, bv);
    for (int s = 0; s < c.nst; ++s) piped_stage(c, s, lo, hi, sa, sb, p, av, bv, acc);
    // the loads of the (empty) stages past the segment land before LDS is used again
    dma_wait_barrier<0>();
}

// The thread's lane coordinates from its index t.
__device__ __forceinline__ void set_lanes(DmaCtx& c, int t) {
    c.t = t;
    const int lane = t & 63;
    c.wid = __builtin_amdgcn_readfirstlane(t >> 6);
    c.wm = c.wid >> 1;
    c.wn = c.wid & 1;
    c.h = lane >> 5;
    c.li = lane & 31;
}

// The per-workgroup constants of the direct path (tile and K range set by the caller).
__device__ __forceinline__ void init_ctx(DmaCtx& c, const GArgs& g, uint8_t* lds) {
    c.g = g;
    set_lanes(c, threadIdx.x);
    c.kbytes = (uint32_t)(g.K / 2);
    c.kblocks = (uint32_t)(g.K / 16);
    c.rs.ac = make_rsrc(g.ac, (uint32_t)(g.M * c.kbytes));
    c.rs.bc = make_rsrc(g.bc, (uint32_t)(g.N * c.kbytes));
    c.rs.as = make_rsrc(g.as, (uint32_t)(g.M * c.kblocks));
    c.rs.bs = make_rsrc(g.bs, (uint32_t)(g.N * c.kblocks));
    c.lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;
    c.lds = lds;
}

template <int EPI>
__global__ __launch_bounds__(GThreads, 1) void k_gemm_dma(GArgs g) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    DmaCtx c;
    init_ctx(c, g, lds);
    int tm, tn;
    const int nst_all = (int)((g.K + GBK - 1) / GBK);
    c.s0 = 0;
    c.nst = nst_all;
    if constexpr (EPI == EpiPart) {
        // workgroup = K-part kp of upper-triangle tile t: blockIdx = kp * ntri + t
        const int ntri = g.tiles_m * (g.tiles_m + 1) / 2;
        const int kp = blockIdx.x / ntri;
        tri_tile(blockIdx.x - kp * ntri, g.tiles_m, tm, tn);
        c.s0 = (int)((int64_t)kp * nst_all / g.kparts);
        c.nst = (int)((int64_t)(kp + 1) * nst_all / g.kparts) - c.s0;
    } else if ((EPI == EpiBf16 || EPI == EpiPlain) && g.sk_g > 0) {
        // whole rounds before a round of half-width tiles: block b takes tile id
        // (b / G) G + sk_virtual(b mod G) (as the balanced FP32 kernel's whole rounds), and
        // block 0 zeroes the remaining tiles' maxima, which k_gemm_half then combines
        const int b = blockIdx.x, G = g.sk_g;
        grouped_tile((b / G) * G + sk_virtual(b % G, G), g.tiles_m, g.tiles_n, tm, tn);
        if (b == 0 && g.tmax)
            for (int i = c.t; i < g.sk_rem; i += GThreads) {
                int rm, rn;
                grouped_tile(g.sk_rounds * G + i, g.tiles_m, g.tiles_n, rm, rn);
                g.tmax[rm * g.tiles_n + rn] = 0.0f;
            }
    } else {
        tile_of(blockIdx.x, g.tiles_m, g.tiles_n, tm, tn);
    }
    c.m0 = (int64_t)tm * GBM;
    c.n0 = (int64_t)tn * GBN;

    float16v acc[4][4];
    zero_acc(acc);
    run_stages(c, acc);
    finish_tile<EPI>(g, lds, acc, c.m0, c.n0, c.wm, c.wn, c.h, c.li);
}

// ---------------------------------------------------------------- half-width tiles
// A 256 x 128 tile per workgroup, on the direct path's stages and LDS layout (B rows 0..127
// of each stage used): wave (wm, wn) owns a 128 x 64 sub-tile as 4 x 2 MFMA 32x32x16
// accumulators.  Every element of C sees the same MFMAs in the same order as in a 256 x 256
// tile, so the two agree bit for bit.  Used for a last round at most half full (bf16 output
// always, FP32 output where the balanced K split does not pay): its tiles then run as twice
// as many half-width tiles, each over the whole K range, so no partial sums are handed
// between workgroups.  A wave issues 9 direct loads per stage: 4 + 2 code chunks, 2 + 1
// scale words (A, then B).
constexpr int kNrLoadsPerStage = 9;

struct NrLoads {
    uint32_t ca[4], sa[2], cb[2], sb;
    uint32_t buf;
};
struct NrHalf {
    uint4 a[4], b[2];
};
struct NrPairs {
    half2v a[4], b[2];
};

__device__ __forceinline__ void nr_stage_loads(const DmaCtx& c, int s, uint32_t buf, NrLoads& L) {
    const bool live = s < c.s0 + c.nst;
    const uint32_t k0b = (uint32_t)s * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int p = i * 256 + c.t, row = p >> 2, q = p & 3;
        const uint32_t off = k0b + (uint32_t)((q ^ ((row >> 2) & 3)) << 4);
        const bool kin = live && off < c.kbytes;
        L.ca[i] = (kin && c.m0 + row < c.g.M) ? (uint32_t)(c.m0 + row) * c.kbytes + off : kOutOfRange;
        if (i < 2)
            L.cb[i] = (kin && c.n0 + row < c.g.N) ? (uint32_t)(c.n0 + row) * c.kbytes + off : kOutOfRange;
    }
    const uint32_t kb0 = (uint32_t)s * 8;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int j = i * 256 + c.t, row = j >> 1;
        const uint32_t kb = kb0 + 4 * (j & 1);
        const bool kin = live && kb < c.kblocks;
        L.sa[i] = (kin && c.m0 + row < c.g.M) ? (uint32_t)(c.m0 + row) * c.kblocks + kb : kOutOfRange;
        if (i == 0)
            L.sb = (kin && c.n0 + row < c.g.N) ? (uint32_t)(c.n0 + row) * c.kblocks + kb : kOutOfRange;
    }
    L.buf = buf;
}

// Load K of a stage: code chunks of A (0..3) and B (4, 5), scale words of A (6, 7) and B (8).
template <int K>
__device__ __forceinline__ void nr_issue(const Rsrc4& rs, const NrLoads& L, int wid) {
    if constexpr (K < 4) {
        dma16(rs.ac, L.buf + (uint32_t)(K * 256 + wid * 64) * 16, L.ca[K]);
    } else if constexpr (K < 6) {
        dma16(rs.bc, L.buf + kStageCodeBytes + (uint32_t)((K - 4) * 256 + wid * 64) * 16, L.cb[K - 4]);
    } else if constexpr (K < 8) {
        dma4(rs.as, L.buf + 2 * kStageCodeBytes + (uint32_t)((K - 6) * 256 + wid * 64) * 4, L.sa[K - 6]);
    } else {
        dma4(rs.bs, L.buf + 2 * kStageCodeBytes + kStageScaleBytes + (uint32_t)(wid * 64) * 4, L.sb);
    }
}

__device__ __forceinline__ void nr_dma_stage(const DmaCtx& c, int s, uint32_t buf) {
    NrLoads L;
    nr_stage_loads(c, s, buf, L);
    static_for<0, kNrLoadsPerStage>([&](auto K) { nr_issue<K>(c.rs, L, c.wid); });
}

__device__ __forceinline__ void nr_read_half(const uint8_t* cur, int c2, const DmaCtx& c, NrHalf& f) {
#pragma unroll
    for (int x = 0; x < 4; ++x)
        f.a[x] = *(const uint4*)(cur + code_off(c.wm * 128 + x * 32 + c.li, 2 * c.h + c2));
#pragma unroll
    for (int y = 0; y < 2; ++y)
        f.b[y] = *(const uint4*)(cur + kStageCodeBytes + code_off(c.wn * 64 + y * 32 + c.li, 2 * c.h + c2));
}

__device__ __forceinline__ void nr_read_scales(const uint8_t* cur, const DmaCtx& c, uint32_t (&sa)[4],
                                               uint32_t (&sb)[2]) {
#pragma unroll
    for (int x = 0; x < 4; ++x)
        sa[x] = *(const uint32_t*)(cur + 2 * kStageCodeBytes + (c.wm * 128 + x * 32 + c.li) * 8 + 4 * c.h);
#pragma unroll
    for (int y = 0; y < 2; ++y)
        sb[y] = *(const uint32_t*)(cur + 2 * kStageCodeBytes + kStageScaleBytes +
                                   (c.wn * 64 + y * 32 + c.li) * 8 + 4 * c.h);
}

template <int B>
__device__ __forceinline__ void nr_make_pairs(const uint32_t (&sa)[4], const uint32_t (&sb)[2], NrPairs& p) {
#pragma unroll
    for (int x = 0; x < 4; ++x) p.a[x] = scale_pair<B>(sa[x]);
#pragma unroll
    for (int y = 0; y < 2; ++y) p.b[y] = scale_pair<B>(sb[y]);
}

template <int T>
__device__ __forceinline__ void nr_decode_slot(const NrHalf& f, const NrPairs& p, half8v (&av)[4],
                                               half8v (&bv)[2]) {
#pragma unroll
    for (int x = 0; x < 4; ++x) av[x] = decode8(dword_of(f.a[x], T & 3), p.a[x]);
#pragma unroll
    for (int y = 0; y < 2; ++y) bv[y] = decode8(dword_of(f.b[y], T & 3), p.b[y]);
}

__device__ __forceinline__ void nr_mma(const half8v (&av)[4], const half8v (&bv)[2], float16v (&acc)[4][2]) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[i], bv[j], acc[i][j], 0, 0, 0);
}

// Each of a slot's 8 MFMAs followed by K VALU instructions.
template <int K>
__device__ __forceinline__ void nr_pace() {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        __builtin_amdgcn_sched_group_barrier(kSchedMFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(kSchedVALU, K, 0);
    }
}

// A slot's 8 MFMAs on (av, bv), the next slot T's decode (12 half-operand steps) spread over
// them, and X(k) after MFMA k, each in a scheduling region of its own.
template <int T, class Fx>
__device__ __forceinline__ void nr_slot_steps(const half8v (&av)[4], const half8v (&bv)[2],
                                              float16v (&acc)[4][2], const NrHalf& f,
                                              const NrPairs& p, half8v (&an)[4], half8v (&bn)[2],
                                              Fx&& X) {
    static_for<0, 8>([&](auto K) {
        constexpr int k = K;
        acc[k >> 1][k & 1] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[k >> 1], bv[k & 1],
                                                                    acc[k >> 1][k & 1], 0, 0, 0);
        static_for<(12 * k) / 8, (12 * (k + 1)) / 8>([&](auto D) {
            constexpr int d = D, o = d >> 1, q = d & 1;
            if constexpr (o < 4) decode4<q>(dword_of(f.a[o], T & 3), p.a[o], an[o]);
            else decode4<q>(dword_of(f.b[o - 4], T & 3), p.b[o - 4], bn[o - 4]);
        });
        X(K);
        __builtin_amdgcn_sched_barrier(0);
    });
}

// Stage s, pipelined as piped_stage: on entry lo, hi, sa, sb hold stage s, p the scale pairs
// of its block 0 and (av, bv) its decoded slot 0; on return the same for stage s + 1.
__device__ __forceinline__ void nr_piped_stage(const DmaCtx& c, int s, NrHalf& lo, NrHalf& hi,
                                               uint32_t (&sa)[4], uint32_t (&sb)[2], NrPairs& p,
                                               half8v (&av)[4], half8v (&bv)[2],
                                               float16v (&acc)[4][2]) {
    half8v an[4], bn[2];
    nr_decode_slot<1>(lo, p, an, bn);
    nr_mma(av, bv, acc);
    nr_pace<6>();
    nr_make_pairs<1>(sa, sb, p);
    nr_decode_slot<2>(lo, p, av, bv);
    nr_mma(an, bn, acc);
    nr_pace<7>();
    nr_decode_slot<3>(lo, p, an, bn);
    nr_mma(av, bv, acc);
    nr_pace<6>();
    nr_make_pairs<2>(sa, sb, p);
    nr_decode_slot<4>(hi, p, av, bv);
    nr_mma(an, bn, acc);
    nr_pace<7>();
#pragma unroll
    for (int x = 0; x < 4; ++x) asm volatile("" : "+v"(av[x]));
#pragma unroll
    for (int y = 0; y < 2; ++y) asm volatile("" : "+v"(bv[y]));
    NrLoads L;
    nr_stage_loads(c, c.s0 + s + kDmaStages, c.lds0 + (s % kDmaStages) * kStageBytes, L);
    // stage s + 1 is in LDS, every wave is done with stage s's buffer
    dma_wait_barrier<(kDmaStages - 2) * kNrLoadsPerStage>();
    const uint8_t* nxt = c.lds + ((s + 1) % kDmaStages) * kStageBytes;
    uint32_t nsa[4], nsb[2];
    // slots 5 to 7: the 9 loads of stage s + kDmaStages, one per kDmaSpread MFMAs; slot 5
    // also reads the next stage's lo and scale words, two per MFMA from its third MFMA on
    const auto extra = [&](auto J, auto K) {
        constexpr int g = J * 8 + K;
        if constexpr (g % kDmaSpread == 0 && g / kDmaSpread < kNrLoadsPerStage)
            nr_issue<g / kDmaSpread>(c.rs, L, c.wid);
        if constexpr (J == 0 && K >= 2) {
            constexpr int e0 = 2 * (K - 2);
            static_for<e0, e0 + 2>([&](auto E) {
                constexpr int e = E;
                if constexpr (e < 4) {
                    lo.a[e] = *(const uint4*)(nxt + code_off(c.wm * 128 + e * 32 + c.li, 2 * c.h));
                } else if constexpr (e < 6) {
                    lo.b[e - 4] = *(const uint4*)(nxt + kStageCodeBytes +
                                                  code_off(c.wn * 64 + (e - 4) * 32 + c.li, 2 * c.h));
                } else if constexpr (e < 10) {
                    nsa[e - 6] = *(const uint32_t*)(nxt + 2 * kStageCodeBytes +
                                                    (c.wm * 128 + (e - 6) * 32 + c.li) * 8 + 4 * c.h);
                } else {
                    nsb[e - 10] = *(const uint32_t*)(nxt + 2 * kStageCodeBytes + kStageScaleBytes +
                                                     (c.wn * 64 + (e - 10) * 32 + c.li) * 8 + 4 * c.h);
                }
            });
        }
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    nr_slot_steps<5>(av, bv, acc, hi, p, an, bn, [&](auto K) { extra(I0{}, K); });
    nr_make_pairs<3>(sa, sb, p);
    nr_slot_steps<6>(an, bn, acc, hi, p, av, bv, [&](auto K) { extra(I1{}, K); });
    nr_slot_steps<7>(av, bv, acc, hi, p, an, bn, [&](auto K) { extra(I2{}, K); });
    nr_read_half(nxt, 1, c, hi);
    nr_make_pairs<0>(nsa, nsb, p);
    nr_decode_slot<0>(lo, p, av, bv);
    nr_mma(an, bn, acc);
    nr_pace<7>();
#pragma unroll
    for (int x = 0; x < 4; ++x) sa[x] = nsa[x];
#pragma unroll
    for (int y = 0; y < 2; ++y) sb[y] = nsb[y];
}

// bf16 output of a half-width tile, as store_rows_bf16 with a 128 x 64 sub-tile per wave.
template <bool FULL>
__device__ __forceinline__ float nr_store_bf16(const GArgs& g, const float16v (&acc)[4][2], const DmaCtx& c,
                                               float scale) {
    const int64_t rbase = c.m0 + c.wm * 128 + 4 * c.h, cbase = c.n0 + c.wn * 64 + c.li;
    float mx = 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t row = rbase + i * 32 + 8 * (r >> 2) + (r & 3);
            uint16_t* rowp = g.c16 + row * g.ldc + cbase;
#pragma unroll
            for (int j = 0; j < 2; ++j)
                if (FULL || (row < g.M && cbase + j * 32 < g.N)) {
                    const float y = acc[i][j][r] * scale;
                    mx = fmaxf(mx, fabsf(y));
                    rowp[j * 32] = __builtin_bit_cast(uint16_t, (__bf16)y);
                }
        }
        __builtin_amdgcn_sched_barrier(0);
    }
    return mx;
}

// FP32 output of a half-width tile (non-temporal, as store_rows).
template <bool FULL>
__device__ __forceinline__ void nr_store_f32(const GArgs& g, const float16v (&acc)[4][2], const DmaCtx& c,
                                             float scale) {
    const int64_t rbase = c.m0 + c.wm * 128 + 4 * c.h, cbase = c.n0 + c.wn * 64 + c.li;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const int64_t row = rbase + i * 32 + 8 * (r >> 2) + (r & 3);
            float* rowp = g.c + row * g.ldc + cbase;
#pragma unroll
            for (int j = 0; j < 2; ++j)
                if (FULL || (row < g.M && cbase + j * 32 < g.N))
                    __builtin_nontemporal_store(acc[i][j][r] * scale, rowp + j * 32);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
}

// The last round of a product as half-width tiles: block u takes column half `half` of
// tile id base + i (base = sk_rounds sk_g, grouped_tile order), both halves of a tile on one
// XCD when sk_rem % 8 == 0 (blocks 16 k + x and 16 k + 8 + x take tile 8 k + x), else on
// blocks 2 i and 2 i + 1.  The tile's maximum of |C| is the larger of its halves' maxima,
// combined by an atomic maximum on the binary32 bits (non-negative values order like their
// bits) into an entry that k_gemm_dma<EpiBf16> zeroed before this launch.  EPI: EpiBf16 or
// EpiPlain (FP32 C).
template <int EPI>
__global__ __launch_bounds__(GThreads, 1) void k_gemm_half(GArgs g) {
    static_assert(EPI == EpiBf16 || EPI == EpiPlain, "bf16 and FP32 epilogues");
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    DmaCtx c;
    init_ctx(c, g, lds);
    const int u = blockIdx.x, base = g.sk_rounds * g.sk_g;
    const bool xcd = (g.sk_rem & 7) == 0;
    const int i = xcd ? (u >> 4) * 8 + (u & 7) : u >> 1;
    const int half = xcd ? (u >> 3) & 1 : u & 1;
    int tm, tn;
    grouped_tile(base + i, g.tiles_m, g.tiles_n, tm, tn);
    c.m0 = (int64_t)tm * GBM;
    c.n0 = (int64_t)tn * GBN + half * (GBN / 2);
    if (c.n0 >= g.N) return;   // a right half wholly past the last column (uniform)
    c.s0 = 0;
    c.nst = (int)((g.K + GBK - 1) / GBK);

    float16v acc[4][2];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.0f;
    for (int j = 0; j < kDmaStages; ++j) nr_dma_stage(c, j, c.lds0 + j * kStageBytes);
    dma_wait_barrier<(kDmaStages - 1) * kNrLoadsPerStage>();
    NrHalf lo, hi;
    uint32_t sa[4], sb[2];
    NrPairs p;
    half8v av[4], bv[2];
    nr_read_half(c.lds, 0, c, lo);
    nr_read_half(c.lds, 1, c, hi);
    nr_read_scales(c.lds, c, sa, sb);
    nr_make_pairs<0>(sa, sb, p);
    nr_decode_slot<0>(lo, p, av, bv);
    for (int s = 0; s < c.nst; ++s) nr_piped_stage(c, s, lo, hi, sa, sb, p, av, bv, acc);
    dma_wait_barrier<0>();

    const float scale = *g.asg * *g.bsg;
    const bool full = c.m0 + GBM <= g.M && c.n0 + GBN / 2 <= g.N;
    if constexpr (EPI == EpiPlain) {
        if (full) nr_store_f32<true>(g, acc, c, scale);
        else nr_store_f32<false>(g, acc, c, scale);
        return;
    }
    float mx = full ? nr_store_bf16<true>(g, acc, c, scale) : nr_store_bf16<false>(g, acc, c, scale);
    if (g.tmax) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        float* red = (float*)lds;
        if ((c.t & 63) == 0) red[c.wid] = mx;
        __syncthreads();
        if (c.t == 0) {
            const float m = (float)(__bf16)fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
            __hip_atomic_fetch_max((uint32_t*)&g.tmax[tm * g.tiles_n + tn], __float_as_uint(m),
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// ---------------------------------------------------------------- balanced schedule
// With T = q G + r tiles (0 < r <= G/2) and G resident workgroups (one per CU; the direct
// path's LDS allows no second), a grid of one workgroup per tile ends with a round in which
// at most half the CUs work (384 tiles on 256 CUs: two rounds for 1.5 of work), and every CU
// writes its tile of C at the same moment.  k_gemm_sk runs the q whole rounds as before
// (workgroup v takes tile j G + v in round j, so each XCD's L2 serves a compact block of
// neighbouring tiles) and splits each of the r remaining tiles into two K halves: workgroup
// 2i+1 computes the tail stages [h, nst) of tile q G + i first thing, workgroup 2i its head
// stages [0, h) last thing.  (Workgroups numbered 2r and up have no half.)  The tail's raw
// accumulators go into the tile's own region of C and a flag marks them ready; the head adds
// them to its accumulators (one binary32 addition per element) and runs the epilogue,
// overwriting them.  Workgroup v is numbered XCD-major from blockIdx (workgroups go to the 8
// XCDs in turn), so both halves of a tile and each round's 32 tiles per XCD share an L2.
//
// Hand-off flags: one 64-bit word per workgroup number in g_sk_flag, tagged with the
// launch's epoch E (distinct per launch on a device): 4E+3 the tail is writing its part,
// 4E+1 the part is in C, 4E+2 the head has claimed the tile.  The tail reserves (compare and
// swap from anything but 4E+2) before it writes; the head waits for 4E+1 at most
// g.sk_spin wall-clock ticks, then claims (compare and swap from anything but 4E+3) and
// computes the tail stages itself, after parking its own part in C.  Either way C gets
// fl(head + tail) of the same two partial sums, bit for bit.  A tail that finds the tile
// claimed writes nothing.  Concurrent launches on one device may overwrite each other's
// flags; that only sends a head to the fallback.  Every wait is bounded.  The last user of a
// flag in a launch clears it (the head once it has seen the part, the tail once it has seen
// the claim), so replays of one captured launch, which share its epoch, start from neutral
// flags; a launch whose hand-off timed out (kSkWriteTicks) may leave one set.
constexpr int kSkMaxGroups = 1024;
__device__ uint64_t g_sk_flag[kSkMaxGroups];
constexpr uint64_t kSkWriteTicks = 100000000ull;   // 1 s at 100 MHz: a reserved tail must publish


// Tail side: reserve the hand-off (1) unless the head has claimed the tile (0).  The caller
// then writes the part and publishes it.
__device__ __forceinline__ int sk_reserve(const DmaCtx& c, int v, int* bcast) {
    const uint64_t E = c.g.sk_epoch;
    if (c.t == 0) {
        int ok = 0;
        if (!c.g.sk_test) {
            uint64_t cur = __hip_atomic_load(&g_sk_flag[v], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            for (int tries = 0; tries < 64 && cur != 4 * E + 2; ++tries)
                if (__hip_atomic_compare_exchange_strong(&g_sk_flag[v], &cur, 4 * E + 3, __ATOMIC_RELAXED,
                                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
                    ok = 1;
                    break;
                }
            // claimed: the head is done with the flag, and this is its last use in the launch
            if (!ok && cur == 4 * E + 2)
                __hip_atomic_store(&g_sk_flag[v], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        *bcast = ok;
    }
    __syncthreads();
    const int ok = *bcast;
    __syncthreads();
    return ok;
}

// Head side: 1 the tail's part is in C, 2 the tile is claimed (compute the tail here), 0 the
// tail reserved the tile and did not publish within kSkWriteTicks (cannot happen while the
// workgroups are resident; the tile is then left as NaN).
__device__ __forceinline__ int sk_await(const DmaCtx& c, int w, int* bcast) {
    const uint64_t E = c.g.sk_epoch;
    if (c.t == 0) {
        int res = 0;
        const uint64_t t0 = (uint64_t)wall_clock64();
        for (;;) {
            uint64_t cur = __hip_atomic_load(&g_sk_flag[w], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (cur == 4 * E + 1) {
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");   // pairs with the tail's release
                // the tail is done with the flag: clear it, so that a replay of this launch
                // (same epoch, as in a captured graph) starts from a neutral flag
                __hip_atomic_store(&g_sk_flag[w], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                res = 1;
                break;
            }
            const uint64_t dt = (uint64_t)wall_clock64() - t0;
            if (dt > c.g.sk_spin) {
                if (cur != 4 * E + 3) {
                    if (__hip_atomic_compare_exchange_strong(&g_sk_flag[w], &cur, 4 * E + 2, __ATOMIC_RELAXED,
                                                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
                        res = 2;
                        break;
                    }
                    continue;
                }
                if (dt > c.g.sk_spin + kSkWriteTicks) break;
            }
            __builtin_amdgcn_s_sleep(4);
        }
        *bcast = res;
    }
    __syncthreads();
    const int res = *bcast;
    __syncthreads();
    return res;
}

// One segment per pass of the loop below, so that the pipelined stages, the transfers and
// the epilogue appear once in the code (a second copy of the stages pushes the accumulators
// out of registers).  Roles: a whole tile; a tail half (published); a head half (waits for
// the tail); the tail stages computed by a head that claimed the tile (after which the
// parked head half is added).
enum { SkWhole = 0, SkTail = 1, SkHead = 2, SkFallback = 3 };

// Segment `idx` of workgroup v: false past the last.
__device__ __forceinline__ bool sk_segment(const GArgs& g, int v, int G, int idx, int& tile, int& k0,
                                           int& k1, int& role) {
    const int q = g.sk_rounds, r = g.sk_rem, nst = g.sk_nst, h = nst / 2;
    const bool half = v < 2 * r, tail = half && (v & 1), head = half && !(v & 1);
    if (tail) {
        if (idx == 0) { tile = q * G + (v >> 1); k0 = h; k1 = nst; role = SkTail; return true; }
        --idx;
    }
    if (idx < q) { tile = idx * G + v; k0 = 0; k1 = nst; role = SkWhole; return true; }
    if (head && idx == q) { tile = q * G + (v >> 1); k0 = 0; k1 = h; role = SkHead; return true; }
    return false;
}

template <int EPI>
__global__ __launch_bounds__(GThreads, 1) void k_gemm_sk(GArgs g) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    __shared__ int bcast;
    DmaCtx c;
    init_ctx(c, g, lds);
    const int G = gridDim.x, v = sk_virtual(blockIdx.x, G), nst = g.sk_nst;
    int idx = 0, role = -1, tile = 0, k0 = 0, k1 = 0;
    for (;;) {
        if (role != SkFallback) {
            if (!sk_segment(g, v, G, idx++, tile, k0, k1, role)) break;
            int tm, tn;
            grouped_tile(tile, g.tiles_m, g.tiles_n, tm, tn);
            c.m0 = (int64_t)tm * GBM;
            c.n0 = (int64_t)tn * GBN;
            c.s0 = k0;
            c.nst = k1 - k0;
        } else {
            c.s0 = k1;
            c.nst = nst - k1;
        }
        __syncthreads();   // the previous segment's epilogue is done with LDS
        // Per-thread values are derived afresh for each segment: hoisted out of this loop,
        // the stages' address arithmetic stays live through the epilogue, where it spills,
        // and each spill reload waits for all of the tile's outstanding C stores.
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        set_lanes(c, tid);
        float16v acc[4][4];
        zero_acc(acc);
        run_stages(c, acc);
        // the accumulators are touched only by finish_tile, as in k_gemm_dma: any other
        // vector arithmetic on them splits them between register files and spills
        int mode = FinResult, next = -1, publish = 0;
        if (role == SkTail) {
            publish = sk_reserve(c, v, &bcast);
            mode = publish ? FinPark : -1;
        } else if (role == SkHead) {
            const int res = sk_await(c, v + 1, &bcast);
            if (res == 1) mode = FinAdd;
            else if (res == 2) { mode = FinPark; next = SkFallback; }
            else mode = FinNan;
        } else if (role == SkFallback) {
            mode = FinAdd;
        }
        if (mode >= 0) finish_tile<EPI>(g, lds, acc, c.m0, c.n0, c.wm, c.wn, c.h, c.li, mode);
        if (mode == FinPark) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // this wave's part has landed
            __syncthreads();
            if (publish && c.t == 0)
                __hip_atomic_store(&g_sk_flag[v], 4 * g.sk_epoch + 1, __ATOMIC_RELEASE,
                                   __HIP_MEMORY_SCOPE_AGENT);
        }
        role = next;
    }
}

// C = s_gA s_gB (P_0 + P_1 + ...) over the K-parts, in part order, for the upper-triangle
// tiles of A A^T, and the same values mirrored into the tiles below the diagonal.  A
// workgroup takes one 64 x 64 sub-block of one triangle tile: thread t sums four consecutive
// columns of rows t/16 + 16q; an off-diagonal sub-block is transposed through LDS so the
// mirrored rows are written whole.
__global__ __launch_bounds__(256) void k_syrk_reduce(const float* part, int ntri, int kparts, int T,
                                                     const float* asg, const float* bsg, float* c,
                                                     int64_t ldc) {
    __shared__ float tr[64][65];
    const int t = threadIdx.x, tile = blockIdx.x >> 4, sb = blockIdx.x & 15;
    int tm, tn;
    tri_tile(tile, T, tm, tn);
    const int br = (sb >> 2) * 64, bc = (sb & 3) * 64, cl = (t & 15) * 4;
    const float scale = *asg * *bsg;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int rl = (t >> 4) + 16 * q;
        const int64_t off = (int64_t)(br + rl) * GBN + bc + cl;
        float4 sum = *(const float4*)(part + ((int64_t)tile << 16) + off);
        for (int kp = 1; kp < kparts; ++kp) {
            const float4 p = *(const float4*)(part + ((int64_t)(kp * ntri + tile) << 16) + off);
            sum.x = sum.x + p.x; sum.y = sum.y + p.y; sum.z = sum.z + p.z; sum.w = sum.w + p.w;
        }
        sum.x = sum.x * scale; sum.y = sum.y * scale; sum.z = sum.z * scale; sum.w = sum.w * scale;
        *(float4*)(c + ((int64_t)tm * GBM + br + rl) * ldc + (int64_t)tn * GBN + bc + cl) = sum;
        tr[rl][cl] = sum.x; tr[rl][cl + 1] = sum.y; tr[rl][cl + 2] = sum.z; tr[rl][cl + 3] = sum.w;
    }
    if (tm == tn) return;   // uniform: the diagonal tiles hold both halves already
    __syncthreads();
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int xr = (t >> 4) + 16 * q;   // row of the mirrored sub-block = column here
        const float4 m = make_float4(tr[cl][xr], tr[cl + 1][xr], tr[cl + 2][xr], tr[cl + 3][xr]);
        *(float4*)(c + ((int64_t)tn * GBN + bc + xr) * ldc + (int64_t)tm * GBM + br + cl) = m;
    }
}

// K-parts for A A^T with m a multiple of 256: as many as fill one round of the 256 CUs with
// the triangle's tiles, each K-part at least four stages; 1 means no gain over the plain GEMM.
static int syrk_kparts(int64_t m, int64_t k) {
    if (m <= 0 || m % GBM || k <= 0 || k % 64) return 1;
    const int64_t T = m / GBM, ntri = T * (T + 1) / 2, nst = (k + GBK - 1) / GBK;
    int64_t kp = 256 / ntri;
    if (kp > nst / 4) kp = nst / 4;
    return kp > 1 ? (int)kp : 1;
}

size_t syrk_part_bytes(int64_t m, int64_t k) {
    const int kp = syrk_kparts(m, k);
    if (kp <= 1) return 0;
    const int64_t T = m / GBM;
    return (size_t)kp * (size_t)(T * (T + 1) / 2) * GBM * GBN * sizeof(float);
}

// C = s_gA^2 A A^T (m x m, FP32) for one NVFP4 copy a of an m x k matrix: the upper-triangle
// tiles with K split into parts on the direct path, then k_syrk_reduce.  Returns
// NVFP4_ERR_MODE when the shape or alignment does not allow it (the caller then takes the
// plain GEMM).  part: syrk_part_bytes(m, k) bytes, 16-byte aligned.
int syrk_splitk(const nvfp4_qtensor* a, int64_t m, int64_t k, float* c, int64_t ldc, float* part,
                size_t part_bytes, hipStream_t st) {
    const int kparts = syrk_kparts(m, k);
    if (kparts <= 1 || !part || part_bytes < syrk_part_bytes(m, k)) return NVFP4_ERR_MODE;
    if (((uintptr_t)a->codes & 15) || ((uintptr_t)a->scales & 3) || ((uintptr_t)c & 15) ||
        ((uintptr_t)part & 15) || ldc % 4 || ldc < m || m * (k / 2) >= (int64_t)kOutOfRange)
        return NVFP4_ERR_MODE;
    GArgs g;
    g.ac = a->codes; g.as = a->scales; g.asg = a->gscale;
    g.bc = a->codes; g.bs = a->scales; g.bsg = a->gscale;
    g.M = m; g.N = m; g.K = k; g.c = c; g.ldc = ldc;
    g.lt = nullptr; g.lb = nullptr; g.lr = 0;
    g.d = nullptr; g.ldd = 0; g.alpha = 1.0f; g.beta = 0.0f;
    g.part = part;
    g.kparts = kparts;
    g.sk_rounds = 0;
    g.sk_rem = 0;
    g.sk_nst = 0;
    g.sk_epoch = 0;
    g.sk_spin = 0;
    g.sk_test = 0;
    g.c16 = nullptr;
    g.tmax = nullptr;
    const int T = (int)(m / GBM), ntri = T * (T + 1) / 2;
    g.tiles_m = T;
    g.tiles_n = T;
    if (hipFuncSetAttribute((const void*)k_gemm_dma<EpiPart>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            kGemmDmaLds) != hipSuccess)
        return NVFP4_ERR_HIP;
    k_gemm_dma<EpiPart><<<(unsigned)(kparts * ntri), GThreads, kGemmDmaLds, st>>>(g);
    k_syrk_reduce<<<(unsigned)(ntri * 16), 256, 0, st>>>(part, ntri, kparts, T, a->gscale, a->gscale,
                                                        c, ldc);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

}  // namespace nvfp4

using namespace nvfp4;

// Schedule settings, for tests and measurements: NVFP4_GEMM_SK=0 keeps one workgroup per
// tile, 1 (the default) chooses as below, 2 takes the balanced K split and 3 the half-width
// tiles whenever the last round qualifies; NVFP4_GEMM_SK_SPIN sets the balanced schedule's
// wait for a tail part (wall-clock ticks, 100 MHz; default 20 ms); NVFP4_GEMM_SK_TEST=1 makes
// every tail skip its hand-off so that every split tile takes the head's fallback.
static int env_int(const char* name, int dflt) {
    const char* e = getenv(name);
    return e && *e ? atoi(e) : dflt;
}

// Workgroups of the balanced schedule on the current device: its compute units rounded down
// to a multiple of 8 (the XCD-major numbering needs whole rounds of 8), 0 if unknown.
static int sk_groups(int* dev_out) {
    constexpr int kMaxDev = 64;
    static std::atomic<int> cache[kMaxDev];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDev) return 0;
    *dev_out = dev;
    int g = cache[dev].load();
    if (g == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
        g = cus & ~7;
        if (g > kSkMaxGroups) g = kSkMaxGroups;
        cache[dev].store(g > 0 ? g : -1);
    }
    return g > 0 ? g : 0;
}

static uint64_t next_epoch(int dev) {
    static std::atomic<uint64_t> epoch[64];
    return epoch[dev & 63].fetch_add(1) + 1;
}

// c16: bf16 output instead of c, with the tile maxima in tmax (may be null).
static int gemm_launch(const nvfp4_qtensor* a, const nvfp4_qtensor* b, int64_t M, int64_t N,
                       int64_t K, float* c, int64_t ldc, const uint16_t* lt, const uint16_t* lb,
                       int64_t lr, const float* d, int64_t ldd, float alpha, float beta,
                       void* stream, uint16_t* c16 = nullptr, float* tmax = nullptr) {
    if (!a || !b || !a->gscale || !b->gscale) return NVFP4_ERR_NULL;
    if (M < 0 || N < 0 || K < 0 || K % 16 || ldc < N) return NVFP4_ERR_SHAPE;
    if (lr < 0 || lr % 16) return NVFP4_ERR_SHAPE;
    if (M == 0 || N == 0) return NVFP4_OK;
    if (!c && !c16) return NVFP4_ERR_NULL;
    if (((uintptr_t)c16 & 1) || ((uintptr_t)tmax & 3)) return NVFP4_ERR_ALIGN;
    if (K > 0 && (!a->codes || !a->scales || !b->codes || !b->scales)) return NVFP4_ERR_NULL;
    if (lr > 0 && (!lt || !lb)) return NVFP4_ERR_NULL;
    if (d && ldd < N) return NVFP4_ERR_SHAPE;
    if (d && ((uintptr_t)d & 3)) return NVFP4_ERR_ALIGN;
    if (((uintptr_t)a->codes & 15) || ((uintptr_t)b->codes & 15) || ((uintptr_t)c & 3) ||
        ((uintptr_t)a->gscale & 3) || ((uintptr_t)b->gscale & 3) || ((uintptr_t)lt & 15) ||
        ((uintptr_t)lb & 15))
        return NVFP4_ERR_ALIGN;
    GArgs g;
    g.ac = a->codes; g.as = a->scales; g.asg = a->gscale;
    g.bc = b->codes; g.bs = b->scales; g.bsg = b->gscale;
    g.M = M; g.N = N; g.K = K; g.c = c; g.ldc = ldc;
    g.lt = lr > 0 ? lt : nullptr;
    g.lb = lr > 0 ? lb : nullptr;
    g.lr = lr;
    g.d = d;
    g.ldd = d ? ldd : 0;
    g.alpha = alpha;
    g.beta = beta;
    g.part = nullptr;
    g.kparts = 1;
    g.sk_rounds = 0;
    g.sk_rem = 0;
    g.sk_nst = 0;
    g.sk_epoch = 0;
    g.sk_spin = 0;
    g.sk_test = 0;
    g.c16 = c16;
    g.tmax = tmax;
    g.sk_g = 0;
    const int epi = c16 ? EpiBf16 : d ? EpiAxpby : (lr > 0 ? EpiLora : EpiPlain);
    const int64_t tiles_m = (M + GBM - 1) / GBM, tiles_n = (N + GBN - 1) / GBN;
    g.tiles_m = (int)tiles_m;
    g.tiles_n = (int)tiles_n;
    const unsigned grid = (unsigned)(tiles_m * tiles_n);
    static_assert(kGemmDmaLds <= 160 * 1024 && kGemmLds <= 160 * 1024, "LDS budget");
    static_assert(2 * GBM * kLoraLdsRow <= kGemmLds, "low-rank staging fits the stage buffers");
    // direct path: whole 4-byte scale words per row and stage, 32-bit buffer offsets
    const int64_t kbytes = K / 2, limit = (int64_t)kOutOfRange;
    const bool direct = K > 0 && K % 64 == 0 && ((uintptr_t)a->scales & 3) == 0 &&
                        ((uintptr_t)b->scales & 3) == 0 && M * kbytes < limit && N * kbytes < limit;
    const void* fns[2][5] = {{(const void*)k_gemm<EpiPlain>, (const void*)k_gemm<EpiLora>,
                              (const void*)k_gemm<EpiAxpby>, nullptr, (const void*)k_gemm<EpiBf16>},
                             {(const void*)k_gemm_dma<EpiPlain>, (const void*)k_gemm_dma<EpiLora>,
                              (const void*)k_gemm_dma<EpiAxpby>, nullptr,
                              (const void*)k_gemm_dma<EpiBf16>}};
    const void* fn = fns[direct ? 1 : 0][epi];
    if (hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                            direct ? kGemmDmaLds : kGemmLds) != hipSuccess)
        return NVFP4_ERR_HIP;
    hipStream_t st = (hipStream_t)stream;
    // A last round of tiles at most half full (plain and bf16 epilogues, direct path) runs
    // either as twice as many half-width tiles over the whole K range (the per-tile sums), or,
    // for FP32 output, with each of its tiles split into two K halves on two workgroups (the
    // balanced schedule, fl(head + tail)).  The split pays where a workgroup's whole rounds
    // are long (rounds x K stages >= 64: FFN-down 1 x 72, FP32 FFN-up 4 x 24, 3-4% ahead);
    // below that its hand-off costs more than it saves (2000 x 4000 x 192: 58 us against
    // 19 us), and bf16 has no room for the parked half.  The axpby epilogue keeps one
    // workgroup per tile (D may be C), and so does the low-rank one (its epilogue spills in
    // the balanced loop and runs slower than the rounds it saves).
    int dev = 0;
    const int sk_mode = env_int("NVFP4_GEMM_SK", 1);
    const int G = direct && (epi == EpiPlain || epi == EpiBf16) && sk_mode ? sk_groups(&dev) : 0;
    const int sk_nst = (int)((K + GBK - 1) / GBK), sk_rem = G > 0 ? (int)(grid % G) : 0;
    const int sk_q = G > 0 ? (int)(grid / G) : 0;
    const bool tail = sk_rem > 0 && 2 * sk_rem <= G;
    const bool balanced = epi == EpiPlain && tail && sk_nst >= 2 && sk_mode != 3 &&
                          (sk_mode == 2 || sk_q * sk_nst >= 64);
    if (epi == EpiBf16 && tail && sk_q > 0) {
        // bf16: the whole rounds, then the remaining tiles as twice as many half-width tiles
        // (k_gemm_half), each over the whole K range: the same sums as one workgroup per tile
        if (hipFuncSetAttribute((const void*)k_gemm_half<EpiBf16>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                kGemmDmaLds) != hipSuccess)
            return NVFP4_ERR_HIP;
        g.sk_g = G;
        g.sk_rounds = (int)(grid / G);
        g.sk_rem = sk_rem;
        k_gemm_dma<EpiBf16><<<g.sk_rounds * G, GThreads, kGemmDmaLds, st>>>(g);
        k_gemm_half<EpiBf16><<<2 * sk_rem, GThreads, kGemmDmaLds, st>>>(g);
        return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
    }
    if (epi == EpiPlain && tail && !balanced) {
        if (hipFuncSetAttribute((const void*)k_gemm_half<EpiPlain>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                kGemmDmaLds) != hipSuccess)
            return NVFP4_ERR_HIP;
        g.sk_g = G;
        g.sk_rounds = (int)(grid / G);
        g.sk_rem = sk_rem;
        if (g.sk_rounds > 0) k_gemm_dma<EpiPlain><<<g.sk_rounds * G, GThreads, kGemmDmaLds, st>>>(g);
        k_gemm_half<EpiPlain><<<2 * sk_rem, GThreads, kGemmDmaLds, st>>>(g);
        return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
    }
    if (balanced) {
        if (hipFuncSetAttribute((const void*)k_gemm_sk<EpiPlain>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                kGemmDmaLds) != hipSuccess)
            return NVFP4_ERR_HIP;
        g.sk_nst = sk_nst;
        g.sk_rounds = (int)(grid / G);
        g.sk_rem = sk_rem;
        g.sk_epoch = next_epoch(dev);
        g.sk_spin = (uint64_t)env_int("NVFP4_GEMM_SK_SPIN", 2000000);
        g.sk_test = env_int("NVFP4_GEMM_SK_TEST", 0);
        k_gemm_sk<EpiPlain><<<G, GThreads, kGemmDmaLds, st>>>(g);
        return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
    }
    if (direct) {
        if (epi == EpiAxpby) k_gemm_dma<EpiAxpby><<<grid, GThreads, kGemmDmaLds, st>>>(g);
        else if (epi == EpiLora) k_gemm_dma<EpiLora><<<grid, GThreads, kGemmDmaLds, st>>>(g);
        else if (epi == EpiBf16) k_gemm_dma<EpiBf16><<<grid, GThreads, kGemmDmaLds, st>>>(g);
        else k_gemm_dma<EpiPlain><<<grid, GThreads, kGemmDmaLds, st>>>(g);
    } else {
        if (epi == EpiAxpby) k_gemm<EpiAxpby><<<grid, GThreads, kGemmLds, st>>>(g);
        else if (epi == EpiLora) k_gemm<EpiLora><<<grid, GThreads, kGemmLds, st>>>(g);
        else if (epi == EpiBf16) k_gemm<EpiBf16><<<grid, GThreads, kGemmLds, st>>>(g);
        else k_gemm<EpiPlain><<<grid, GThreads, kGemmLds, st>>>(g);
    }
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

extern "C" int nvfp4_gemm(const nvfp4_qtensor* a, const nvfp4_qtensor* b, int64_t M, int64_t N,
                          int64_t K, float* c, int64_t ldc, void* stream) {
    return gemm_launch(a, b, M, N, K, c, ldc, nullptr, nullptr, 0, nullptr, 0, 1.0f, 0.0f, stream);
}

extern "C" int64_t nvfp4_gemm_tiles(int64_t M, int64_t N) {
    if (M <= 0 || N <= 0) return 0;
    return ((M + GBM - 1) / GBM) * ((N + GBN - 1) / GBN);
}

extern "C" int nvfp4_gemm_bf16(const nvfp4_qtensor* a, const nvfp4_qtensor* b, int64_t M,
                               int64_t N, int64_t K, uint16_t* c, int64_t ldc, float* tile_amax,
                               void* stream) {
    if (M > 0 && N > 0 && !c) return NVFP4_ERR_NULL;
    return gemm_launch(a, b, M, N, K, nullptr, ldc, nullptr, nullptr, 0, nullptr, 0, 1.0f, 0.0f,
                       stream, c, tile_amax);
}

extern "C" int nvfp4_gemm_lora(const nvfp4_qtensor* a, const nvfp4_qtensor* b, int64_t M,
                               int64_t N, int64_t K, float* c, int64_t ldc, const uint16_t* lora_t,
                               const uint16_t* lora_b, int64_t rank, void* stream) {
    return gemm_launch(a, b, M, N, K, c, ldc, lora_t, lora_b, rank, nullptr, 0, 1.0f, 0.0f, stream);
}

extern "C" int nvfp4_gemm_axpby(const nvfp4_qtensor* a, const nvfp4_qtensor* b, int64_t M,
                                int64_t N, int64_t K, float alpha, const float* d, int64_t ldd,
                                float beta, float* c, int64_t ldc, void* stream) {
    if (!d) return NVFP4_ERR_NULL;
    return gemm_launch(a, b, M, N, K, c, ldc, nullptr, nullptr, 0, d, ldd, alpha, beta, stream);
}
