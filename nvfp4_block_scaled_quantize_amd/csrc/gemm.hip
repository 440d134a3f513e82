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
// row) per stage, double buffered: on gfx950 LDS writes run at about a third of the
// read rate, so staging 4-bit codes instead of 16-bit values keeps LDS off the critical
// path.  Each wave decodes its own MFMA operands right before use: the hardware
// fp4 -> f16 conversion (exact; it issues at a quarter of the VALU rate) and a packed f16
// multiply by the block scale.  Conversions and multiplies are interleaved between the
// MFMAs of the previous slot so that the VALU work runs under the matrix cores.
//
// K ordering.  An MFMA sums over 16 k-slots; lanes 0-31 supply slots 0-7 and lanes
// 32-63 slots 8-15.  Lane (i, h) of both operands reads the 64 contiguous k of half h
// of the stage and feeds nibbles 8t..8t+7 to the t-th MFMA, so slot k of A always meets
// slot k of B and every k of the stage is summed exactly once.
#include "nvfp4.h"
#include "device_common.h"

namespace nvfp4 {

constexpr int GBM = 256, GBN = 256, GBK = 128;  // GBK in elements: 64 bytes of codes per row
constexpr int GThreads = 256;
constexpr int kStageCodeBytes = GBM * 64;       // per operand
constexpr int kStageScaleBytes = GBM * 8;       // per operand
constexpr int kStageBytes = 2 * kStageCodeBytes + 2 * kStageScaleBytes;
constexpr int kGemmLds = 2 * kStageBytes;

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
    int tiles_n;
};

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

__device__ __forceinline__ void load_stage(const GArgs& g, int64_t m0, int64_t n0, int s,
                                           StageRegs& r) {
    const int t = threadIdx.x;
    const int64_t kbytes = g.K / 2, k0b = (int64_t)s * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int q = t + GThreads * i, row = q >> 2, ch = q & 3;
        const int64_t off = k0b + ch * 16;
        const int64_t gm = m0 + row, gn = n0 + row;
        r.a[i] = (gm < g.M && off < kbytes) ? *(const uint4*)(g.ac + gm * kbytes + off)
                                             : make_uint4(0u, 0u, 0u, 0u);
        r.b[i] = (gn < g.N && off < kbytes) ? *(const uint4*)(g.bc + gn * kbytes + off)
                                             : make_uint4(0u, 0u, 0u, 0u);
    }
    const int64_t kblocks = g.K / 16, kb0 = (int64_t)s * 8;
    r.sa = load_scales8(g.as, m0 + t, g.M, kb0, kblocks);
    r.sb = load_scales8(g.bs, n0 + t, g.N, kb0, kblocks);
}

// Packed tile layout: row r holds 64 bytes as four 16-byte chunks; chunk q sits at slot
// q ^ (r/4 mod 4), which keeps both the staging stores (four lanes per row) and the
// fragment reads (one chunk of sixteen consecutive rows per 16 lanes) on distinct banks.
__device__ __forceinline__ int code_off(int row, int chunk) {
    return row * 64 + ((chunk ^ ((row >> 2) & 3)) << 4);
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

// E4M3 code -> binary16 without branches: the E4M3 bits shifted into the binary16
// exponent/mantissa fields give value / 256 (both formats put their subnormals at the
// same offset), so one exact multiply by 256 restores it.
__device__ __forceinline__ _Float16 scale_f16(uint32_t code) {
    const uint16_t bits = (uint16_t)((code & 0x7Fu) << 7);
    return __builtin_bit_cast(_Float16, bits) * (_Float16)256.0f;
}

__device__ __forceinline__ uint32_t dword_of(const uint4& v, int i) {
    return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

// 8 codes -> 8 binary16 values v * s (exact).
__device__ __forceinline__ half8v decode8(uint32_t w, half2v s2) {
    const half2v p0 = fp4x2_to_f16<0>(w) * s2;
    const half2v p1 = fp4x2_to_f16<1>(w) * s2;
    const half2v p2 = fp4x2_to_f16<2>(w) * s2;
    const half2v p3 = fp4x2_to_f16<3>(w) * s2;
    half8v o = {p0.x, p0.y, p1.x, p1.y, p2.x, p2.y, p3.x, p3.y};
    return o;
}

// Sched-group masks of __builtin_amdgcn_sched_group_barrier.
constexpr int kSchedVALU = 0x002, kSchedMFMA = 0x008;

__global__ __launch_bounds__(GThreads, 1) void k_gemm(GArgs g) {
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6, wm = wid >> 1, wn = wid & 1;
    const int tm = blockIdx.x / g.tiles_n, tn = blockIdx.x % g.tiles_n;
    const int64_t m0 = (int64_t)tm * GBM, n0 = (int64_t)tn * GBN;
    const int h = lane >> 5, li = lane & 31;
    const float scale = *g.asg * *g.bsg;
    uint8_t* stages = lds;

    float16v acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    const int nst = (int)((g.K + GBK - 1) / GBK);
    StageRegs regs;
    if (nst > 0) {
        load_stage(g, m0, n0, 0, regs);
        store_stage(stages, regs);
    }
    __syncthreads();

    for (int s = 0; s < nst; ++s) {
        const uint8_t* cur = stages + (s & 1) * kStageBytes;
        if (s + 1 < nst) load_stage(g, m0, n0, s + 1, regs);

        // this wave's packed fragments: 32 bytes of codes and 4 scale bytes per sub-tile
        uint4 fa[4][2], fb[4][2];
        uint32_t wsa[4], wsb[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int ra = wm * 128 + x * 32 + li, rb = wn * 128 + x * 32 + li;
#pragma unroll
            for (int c2 = 0; c2 < 2; ++c2) {
                fa[x][c2] = *(const uint4*)(cur + code_off(ra, 2 * h + c2));
                fb[x][c2] = *(const uint4*)(cur + kStageCodeBytes + code_off(rb, 2 * h + c2));
            }
            wsa[x] = *(const uint32_t*)(cur + 2 * kStageCodeBytes + ra * 8 + 4 * h);
            wsb[x] = *(const uint32_t*)(cur + 2 * kStageCodeBytes + kStageScaleBytes + rb * 8 + 4 * h);
        }
        // scales of this lane's four blocks per sub-tile as binary16 pairs
        half2v psa[4][4], psb[4][4];
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const _Float16 sa = scale_f16((wsa[x] >> (8 * b)) & 0xFFu);
                const _Float16 sb = scale_f16((wsb[x] >> (8 * b)) & 0xFFu);
                psa[x][b] = half2v{sa, sa};
                psb[x][b] = half2v{sb, sb};
            }
        half8v av[4], bv[4];
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            av[x] = decode8(fa[x][0].x, psa[x][0]);
            bv[x] = decode8(fb[x][0].x, psb[x][0]);
        }
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
            half8v an[4], bn[4];
            if (tt < 7) {
#pragma unroll
                for (int x = 0; x < 4; ++x) {
                    an[x] = decode8(dword_of(fa[x][(tt + 1) >> 2], (tt + 1) & 3), psa[x][(tt + 1) >> 1]);
                    bn[x] = decode8(dword_of(fb[x][(tt + 1) >> 2], (tt + 1) & 3), psb[x][(tt + 1) >> 1]);
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
        if (s + 1 < nst) store_stage(stages + ((s + 1) & 1) * kStageBytes, regs);
        __syncthreads();
    }

    // epilogue: D register r of lane l is row 8(r/4) + 4(l/32) + r%4, column l%32
    const int64_t rbase = m0 + wm * 128 + 4 * h, cbase = n0 + wn * 128 + li;
    if (m0 + GBM <= g.M && n0 + GBN <= g.N) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                float* rowp = g.c + (rbase + i * 32 + 8 * (r >> 2) + (r & 3)) * g.ldc + cbase;
#pragma unroll
                for (int j = 0; j < 4; ++j) rowp[j * 32] = acc[i][j][r] * scale;
            }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int64_t row = rbase + i * 32 + 8 * (r >> 2) + (r & 3);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int64_t col = cbase + j * 32;
                    if (row < g.M && col < g.N) g.c[row * g.ldc + col] = acc[i][j][r] * scale;
                }
            }
    }
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" int nvfp4_gemm(const nvfp4_qtensor* a, const nvfp4_qtensor* b, int64_t M, int64_t N,
                          int64_t K, float* c, int64_t ldc, void* stream) {
    if (!a || !b || !a->gscale || !b->gscale) return NVFP4_ERR_NULL;
    if (M < 0 || N < 0 || K < 0 || K % 32 || ldc < N) return NVFP4_ERR_SHAPE;
    if (M == 0 || N == 0) return NVFP4_OK;
    if (!c) return NVFP4_ERR_NULL;
    if (K > 0 && (!a->codes || !a->scales || !b->codes || !b->scales)) return NVFP4_ERR_NULL;
    if (((uintptr_t)a->codes & 15) || ((uintptr_t)b->codes & 15) || ((uintptr_t)c & 3) ||
        ((uintptr_t)a->gscale & 3) || ((uintptr_t)b->gscale & 3))
        return NVFP4_ERR_ALIGN;
    GArgs g;
    g.ac = a->codes; g.as = a->scales; g.asg = a->gscale;
    g.bc = b->codes; g.bs = b->scales; g.bsg = b->gscale;
    g.M = M; g.N = N; g.K = K; g.c = c; g.ldc = ldc;
    const int64_t tiles_m = (M + GBM - 1) / GBM, tiles_n = (N + GBN - 1) / GBN;
    g.tiles_n = (int)tiles_n;
    static_assert(kGemmLds <= 160 * 1024, "LDS budget");
    if (hipFuncSetAttribute((const void*)k_gemm, hipFuncAttributeMaxDynamicSharedMemorySize,
                            kGemmLds) != hipSuccess)
        return NVFP4_ERR_HIP;
    k_gemm<<<(unsigned)(tiles_m * tiles_n), GThreads, kGemmLds, (hipStream_t)stream>>>(g);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}
