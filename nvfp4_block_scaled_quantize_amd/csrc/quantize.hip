// quantize.hip -- NVFP4 quantizer (rowwise + columnwise copies from one read) and
// dequantizer for gfx950.
//
// Method (Full-Stack FP4 sec. 2 and sec. 3.2 eq. (1)-(2); NVFP4 report sec. 2, sec. 4,
// B.4): per copy, an optional random Hadamard transform of each 16-chunk along the
// copy's rows, the FP32 tensor scale s_g = amax / (6*448), E4M3 block scales
// s = E4M3((amax_b / 6) / s_g) over 1x16 or 16x16 blocks, E2M1 codes of x / (s s_g)
// (nearest-even or stochastic), two codes per byte.
//
// Work decomposition.  A workgroup of 256 threads owns a 256-row x 128-column tile of
// X; each thread owns a 16-row x 8-column register patch (16 coalesced 16-byte row
// loads for bfloat16).  Columnwise 16x1 blocks (and the columnwise Hadamard) are
// complete inside one thread; rowwise 1x16 blocks span the thread and its lane
// neighbour (lane ^ 1), which exchange one value per stage through cross-lane moves.
// Columnwise codes are transposed through LDS so each column's 128 bytes leave the
// workgroup as contiguous stores.  The tensor amax needs a pass over all of X before
// any block can be scaled, so the quantizer is two kernels: k_amax writes one partial
// maximum per tile and copy; k_encode reduces them (in every workgroup, no atomics)
// and encodes.
#include "nvfp4.h"
#include "device_common.h"

namespace nvfp4 {

constexpr int kTileRows = 256;
constexpr int kTileCols = 128;
constexpr int kThreads = 256;

struct QArgs {
    const void* x;
    int64_t rows, cols, ld;
    int is_bf16;
    int rowwise, colwise, block2d;
    int sr_row, sr_col, rht_row, rht_col;
    uint32_t k0, k1;
    uint8_t* rcodes;
    uint8_t* rscales;
    float* rsg;
    uint8_t* ccodes;
    uint8_t* cscales;
    float* csg;
    float* partial;  // [2][ntiles]: rowwise-copy and columnwise-copy amax per tile
    int tiles_c;
    int ntiles;
};

template <bool BF16>
__device__ __forceinline__ void load_patch(const QArgs& a, int64_t r0, int64_t c0, bool valid,
                                           float v[16][8]) {
    if (!valid) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) v[i][e] = 0.0f;
        return;
    }
    if (BF16) {
        const uint16_t* p = (const uint16_t*)a.x + r0 * a.ld + c0;
        uint4 q[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) q[i] = *(const uint4*)(p + (int64_t)i * a.ld);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            uint32_t w[4] = {q[i].x, q[i].y, q[i].z, q[i].w};
#pragma unroll
            for (int h = 0; h < 4; ++h) {
                v[i][2 * h] = __uint_as_float(w[h] << 16);
                v[i][2 * h + 1] = __uint_as_float(w[h] & 0xFFFF0000u);
            }
        }
    } else {
        const float* p = (const float*)a.x + r0 * a.ld + c0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float4 q0 = *(const float4*)(p + (int64_t)i * a.ld);
            float4 q1 = *(const float4*)(p + (int64_t)i * a.ld + 4);
            v[i][0] = q0.x; v[i][1] = q0.y; v[i][2] = q0.z; v[i][3] = q0.w;
            v[i][4] = q1.x; v[i][5] = q1.y; v[i][6] = q1.z; v[i][7] = q1.w;
        }
    }
}

// Random Hadamard transform of one 16-chunk held as 8 values per lane in a lane pair
// (lane with half = 0 holds positions 0..7, its neighbour positions 8..15).  Stages 1,
// 2, 4 are in-register; stage 8 exchanges with lane ^ 1.
__device__ __forceinline__ void rht_pair8(float w[8], uint32_t signs, int half) {
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = apply_sign(w[e], signs, half * 8 + e);
#pragma unroll
    for (int h = 1; h < 8; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if ((i & h) == 0) {
                float a = w[i], b = w[i + h];
                w[i] = a + b;
                w[i + h] = a - b;
            }
        }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        float p = __shfl_xor(w[e], 1, 64);
        w[e] = half ? (p - w[e]) : (w[e] + p);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) w[e] = w[e] * 0.25f;
}

__device__ __forceinline__ void rht_col16(float w[16], uint32_t signs) {
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = apply_sign(w[i], signs, i);
    wht16(w);
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = w[i] * 0.25f;
}

// Workgroup max of two values; every thread gets the results.
__device__ __forceinline__ void block_max2(float& a, float& b, float* red) {
    a = wave_max(a);
    b = wave_max(b);
    int wid = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) { red[wid] = a; red[4 + wid] = b; }
    __syncthreads();
    a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    b = fmaxf(fmaxf(red[4], red[5]), fmaxf(red[6], red[7]));
}

// Specialised on the input dtype and the Hadamard flags (bit 0: rowwise copy, bit 1:
// columnwise copy) so that each variant keeps its 16x8 patch in registers.
template <bool BF16, int H>
__global__ __launch_bounds__(kThreads) void k_amax(QArgs a) {
    constexpr bool RHT_ROW = H & 1, RHT_COL = (H >> 1) & 1;
    __shared__ float red[8];
    const int t = threadIdx.x, pc = t & 15, pr = t >> 4;
    const int tile_r = blockIdx.x / a.tiles_c, tile_c = blockIdx.x % a.tiles_c;
    const int64_t r0 = (int64_t)tile_r * kTileRows + pr * 16;
    const int64_t c0 = (int64_t)tile_c * kTileCols + pc * 8;
    const bool valid = r0 < a.rows && c0 < a.cols;
    float v[16][8];
    load_patch<BF16>(a, r0, c0, valid, v);
    const uint32_t signs = (RHT_ROW || RHT_COL) ? rht_sign_bits(a.k0, a.k1) : 0u;

    float plain = 0.0f, arow = 0.0f, acol = 0.0f;
    if ((a.rowwise && !RHT_ROW) || (a.colwise && !RHT_COL)) {
#pragma unroll
        for (int i = 0; i < 16; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) plain = fmaxf(plain, fabsf(v[i][e]));
    }
    if (RHT_ROW) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float w[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) w[e] = v[i][e];
            rht_pair8(w, signs, pc & 1);
#pragma unroll
            for (int e = 0; e < 8; ++e) arow = fmaxf(arow, fabsf(w[e]));
        }
    }
    if (RHT_COL) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float w[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) w[i] = v[i][j];
            rht_col16(w, signs);
#pragma unroll
            for (int i = 0; i < 16; ++i) acol = fmaxf(acol, fabsf(w[i]));
        }
    }
    float mr = RHT_ROW ? arow : plain;
    float mc = RHT_COL ? acol : plain;
    block_max2(mr, mc, red);
    if (t == 0) {
        a.partial[blockIdx.x] = mr;
        a.partial[a.ntiles + blockIdx.x] = mc;
    }
}

// Codes for 8 values (one dword), nearest-even.
__device__ __forceinline__ uint32_t encode8_rne(const float w[8], float rcp) {
    uint32_t r = 0;
    r = cvt_fp4x2<0>(r, w[0] * rcp, w[1] * rcp);
    r = cvt_fp4x2<1>(r, w[2] * rcp, w[3] * rcp);
    r = cvt_fp4x2<2>(r, w[4] * rcp, w[5] * rcp);
    r = cvt_fp4x2<3>(r, w[6] * rcp, w[7] * rcp);
    return r;
}

// Codes for 8 values (one dword), stochastic, with the 4 Philox words of their group.
__device__ __forceinline__ uint32_t encode8_sr(const float w[8], float rcp, const U4& rw) {
    uint32_t r = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        uint32_t word = word_of(rw, e >> 1);
        uint32_t r16 = (e & 1) ? (word >> 16) : (word & 0xFFFFu);
        r |= sr_code(w[e], rcp, r16) << (4 * e);
    }
    return r;
}

__device__ __forceinline__ float sg_from_amax(float amax) {
    float sg = __fdiv_rn(amax, 2688.0f);
    return sg == 0.0f ? 1.0f : sg;
}

// Specialised on the input dtype and on F: bit 0 rowwise SR, bit 1 columnwise SR,
// bit 2 rowwise Hadamard, bit 3 columnwise Hadamard.
template <bool BF16, int F>
__global__ __launch_bounds__(kThreads) void k_encode(QArgs a) {
    constexpr bool SR_ROW = F & 1, SR_COL = (F >> 1) & 1;
    constexpr bool RHT_ROW = (F >> 2) & 1, RHT_COL = (F >> 3) & 1;
    __shared__ uint2 ccodes_lds[kTileCols][16];           // [column][16-row slot], slot ^ (column/8)
    __shared__ uint8_t cscales_lds[kTileCols * 17];       // [column][slot], stride 17
    __shared__ float red[8];
    const int t = threadIdx.x, pc = t & 15, pr = t >> 4;
    const int tile_r = blockIdx.x / a.tiles_c, tile_c = blockIdx.x % a.tiles_c;
    const int64_t r0 = (int64_t)tile_r * kTileRows + pr * 16;
    const int64_t c0 = (int64_t)tile_c * kTileCols + pc * 8;
    const bool valid = r0 < a.rows && c0 < a.cols;

    // tensor scales from the per-tile partial maxima
    float mr = 0.0f, mc = 0.0f;
    for (int i = t; i < a.ntiles; i += kThreads) {
        mr = fmaxf(mr, a.partial[i]);
        mc = fmaxf(mc, a.partial[a.ntiles + i]);
    }
    block_max2(mr, mc, red);
    const float sg_r = sg_from_amax(mr), sg_c = sg_from_amax(mc);
    if (blockIdx.x == 0 && t == 0) {
        if (a.rowwise) *a.rsg = sg_r;
        if (a.colwise) *a.csg = sg_c;
    }

    float v[16][8];
    load_patch<BF16>(a, r0, c0, valid, v);
    const uint32_t signs = (RHT_ROW || RHT_COL) ? rht_sign_bits(a.k0, a.k1) : 0u;

    uint32_t scode2d = 0;
    if (a.block2d) {  // one scale per 16x16 tile = this patch and its neighbour's
        float am = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(v[i][e]));
        am = fmaxf(am, __shfl_xor(am, 1, 64));
        scode2d = e4m3_encode(__fdiv_rn(__fdiv_rn(am, 6.0f), sg_r));
    }

    if (a.colwise) {
        static_for<0, 8>([&](auto J) {
            constexpr int j = decltype(J)::value;
            float w[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) w[i] = v[i][j];
            if (RHT_COL) rht_col16(w, signs);
            uint32_t scode;
            if (a.block2d) {
                scode = scode2d;
            } else {
                float am = 0.0f;
#pragma unroll
                for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(w[i]));
                scode = e4m3_encode(__fdiv_rn(__fdiv_rn(am, 6.0f), sg_c));
            }
            const float d = e4m3_value(scode) * sg_c;
            const float rcp = scode ? __fdiv_rn(1.0f, d) : 0.0f;
            uint32_t lo, hi;
            if (!SR_COL) {
                lo = encode8_rne(&w[0], rcp);
                hi = encode8_rne(&w[8], rcp);
            } else {
                const uint64_t g = ((uint64_t)(c0 + j) * (uint64_t)a.rows + (uint64_t)r0) >> 3;
                lo = encode8_sr(&w[0], rcp, sr_words(g, 1u, a.k0, a.k1));
                hi = encode8_sr(&w[8], rcp, sr_words(g + 1, 1u, a.k0, a.k1));
            }
            const int cl = pc * 8 + j;
            ccodes_lds[cl][pr ^ pc] = make_uint2(lo, hi);
            cscales_lds[cl * 17 + pr] = (uint8_t)scode;
        });
    }

    if (a.rowwise) {
        const int64_t rpitch = a.cols / 2, spitch = a.cols / 16;
        static_for<0, 16>([&](auto I) {
            constexpr int i = decltype(I)::value;
            float w[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) w[e] = v[i][e];
            if (RHT_ROW) rht_pair8(w, signs, pc & 1);
            uint32_t scode;
            if (a.block2d) {
                scode = scode2d;
            } else {
                float am = 0.0f;
#pragma unroll
                for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(w[e]));
                am = fmaxf(am, __shfl_xor(am, 1, 64));
                scode = e4m3_encode(__fdiv_rn(__fdiv_rn(am, 6.0f), sg_r));
            }
            const float d = e4m3_value(scode) * sg_r;
            const float rcp = scode ? __fdiv_rn(1.0f, d) : 0.0f;
            uint32_t codes;
            if (!SR_ROW) {
                codes = encode8_rne(w, rcp);
            } else {
                const uint64_t g = ((uint64_t)(r0 + i) * (uint64_t)a.cols + (uint64_t)c0) >> 3;
                codes = encode8_sr(w, rcp, sr_words(g, 0u, a.k0, a.k1));
            }
            if (valid) {
                *(uint32_t*)(a.rcodes + (r0 + i) * rpitch + c0 / 2) = codes;
                if ((pc & 1) == 0) a.rscales[(r0 + i) * spitch + c0 / 16] = (uint8_t)scode;
            }
        });
    }

    if (a.colwise) {
        __syncthreads();
        const int64_t cpitch = a.rows / 2, spitch = a.rows / 16;
        const int64_t gc0 = (int64_t)tile_c * kTileCols, gr0 = (int64_t)tile_r * kTileRows;
        for (int q = t; q < kTileCols * 16; q += kThreads) {
            const int cl = q >> 4, s = q & 15;
            const int64_t gc = gc0 + cl, gr = gr0 + s * 16;
            if (gc < a.cols && gr < a.rows) {
                *(uint2*)(a.ccodes + gc * cpitch + gr / 2) = ccodes_lds[cl][s ^ (cl >> 3)];
                a.cscales[gc * spitch + gr / 16] = cscales_lds[cl * 17 + s];
            }
        }
    }
}

__global__ void k_fill_scale_one(float* a, float* b) {
    if (threadIdx.x == 0) {
        if (a) *a = 1.0f;
        if (b) *b = 1.0f;
    }
}

// ---------------------------------------------------------------- dequantize
// One thread decodes one 16-element block: out = fl(fl(v * s) * s_g).
__global__ __launch_bounds__(256) void k_dequant(const uint8_t* codes, const uint8_t* scales,
                                                 const float* gscale, int64_t n, int64_t k,
                                                 int out_bf16, void* out, int64_t ld_out) {
    const int64_t kb = k / 16;
    const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (blk >= n * kb) return;
    const int64_t r = blk / kb, b = blk % kb;
    const uint2 cw = *(const uint2*)(codes + r * (k / 2) + b * 8);
    const float s = e4m3_value(scales[r * kb + b]);
    const float sg = *gscale;
    float o[16];
    uint32_t w2[2] = {cw.x, cw.y};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float2v p0 = fp4x2_to_f32<0>(w2[h]);
        float2v p1 = fp4x2_to_f32<1>(w2[h]);
        float2v p2 = fp4x2_to_f32<2>(w2[h]);
        float2v p3 = fp4x2_to_f32<3>(w2[h]);
        o[8 * h + 0] = p0.x; o[8 * h + 1] = p0.y; o[8 * h + 2] = p1.x; o[8 * h + 3] = p1.y;
        o[8 * h + 4] = p2.x; o[8 * h + 5] = p2.y; o[8 * h + 6] = p3.x; o[8 * h + 7] = p3.y;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) o[e] = (o[e] * s) * sg;
    if (!out_bf16) {
        float4* p = (float4*)((float*)out + r * ld_out + b * 16);
#pragma unroll
        for (int q = 0; q < 4; ++q) p[q] = make_float4(o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]);
    } else {
        uint32_t pk[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) pk[q] = f32_to_bf16_rne(o[2 * q]) | (f32_to_bf16_rne(o[2 * q + 1]) << 16);
        uint4* p = (uint4*)((uint16_t*)out + r * ld_out + b * 16);
        p[0] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
        p[1] = make_uint4(pk[4], pk[5], pk[6], pk[7]);
    }
}

}  // namespace nvfp4

using namespace nvfp4;

static inline bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

static int64_t quant_tiles(int64_t rows, int64_t cols, int* tiles_c) {
    int64_t tr = (rows + kTileRows - 1) / kTileRows, tc = (cols + kTileCols - 1) / kTileCols;
    if (tiles_c) *tiles_c = (int)tc;
    return tr * tc;
}

template <bool BF16, int F>
static void launch_quant(const QArgs& a, hipStream_t st) {
    k_amax<BF16, (F >> 2)><<<a.ntiles, kThreads, 0, st>>>(a);
    k_encode<BF16, F><<<a.ntiles, kThreads, 0, st>>>(a);
}

template <bool BF16>
static void launch_quant_f(int f, const QArgs& a, hipStream_t st) {
    switch (f) {
#define NVFP4_CASE(F) case F: launch_quant<BF16, F>(a, st); break;
    NVFP4_CASE(0) NVFP4_CASE(1) NVFP4_CASE(2) NVFP4_CASE(3)
    NVFP4_CASE(4) NVFP4_CASE(5) NVFP4_CASE(6) NVFP4_CASE(7)
    NVFP4_CASE(8) NVFP4_CASE(9) NVFP4_CASE(10) NVFP4_CASE(11)
    NVFP4_CASE(12) NVFP4_CASE(13) NVFP4_CASE(14) NVFP4_CASE(15)
#undef NVFP4_CASE
    }
}

extern "C" size_t nvfp4_quantize_workspace_bytes(int64_t rows, int64_t cols,
                                                 const nvfp4_quant_params* p) {
    (void)p;
    if (rows <= 0 || cols <= 0) return 0;
    return (size_t)quant_tiles(rows, cols, nullptr) * 2 * sizeof(float);
}

static int check_qtensor(const nvfp4_qtensor* q) {
    if (!q || !q->codes || !q->scales || !q->gscale) return NVFP4_ERR_NULL;
    if (!aligned(q->codes, 8) || !aligned(q->gscale, 4)) return NVFP4_ERR_ALIGN;
    return NVFP4_OK;
}

extern "C" int nvfp4_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld_x,
                              const nvfp4_quant_params* p, const nvfp4_qtensor* row_out,
                              const nvfp4_qtensor* col_out, void* ws, size_t ws_bytes,
                              void* stream) {
    if (!p) return NVFP4_ERR_NULL;
    if (dtype != NVFP4_F32 && dtype != NVFP4_BF16) return NVFP4_ERR_DTYPE;
    if (rows < 0 || cols < 0 || rows % 16 || cols % 16 || ld_x < cols) return NVFP4_ERR_SHAPE;
    if (!p->rowwise && !p->colwise) return NVFP4_ERR_MODE;
    if (p->block != NVFP4_BLOCK_1D && p->block != NVFP4_BLOCK_2D) return NVFP4_ERR_MODE;
    if ((p->round_row != NVFP4_RNE && p->round_row != NVFP4_SR) ||
        (p->round_col != NVFP4_RNE && p->round_col != NVFP4_SR))
        return NVFP4_ERR_MODE;
    if (p->block == NVFP4_BLOCK_2D &&
        ((p->rowwise && (p->round_row != NVFP4_RNE || p->rht_row)) ||
         (p->colwise && (p->round_col != NVFP4_RNE || p->rht_col))))
        return NVFP4_ERR_MODE;
    hipStream_t st = (hipStream_t)stream;
    if (rows == 0 || cols == 0) {  // nothing to encode; the tensor scale is 1
        if ((p->rowwise && (!row_out || !row_out->gscale)) ||
            (p->colwise && (!col_out || !col_out->gscale)))
            return NVFP4_ERR_NULL;
        k_fill_scale_one<<<1, 64, 0, st>>>(p->rowwise ? row_out->gscale : nullptr,
                                           p->colwise ? col_out->gscale : nullptr);
        return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
    }
    int rc;
    if (p->rowwise && (rc = check_qtensor(row_out)) != NVFP4_OK) return rc;
    if (p->colwise && (rc = check_qtensor(col_out)) != NVFP4_OK) return rc;
    if (!x) return NVFP4_ERR_NULL;
    const int64_t esize = dtype == NVFP4_BF16 ? 2 : 4;
    if (!aligned(x, 16) || (ld_x * esize) % 16) return NVFP4_ERR_ALIGN;
    const size_t need = nvfp4_quantize_workspace_bytes(rows, cols, p);
    if (!ws || ws_bytes < need) return NVFP4_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return NVFP4_ERR_ALIGN;

    QArgs a;
    a.x = x;
    a.rows = rows;
    a.cols = cols;
    a.ld = ld_x;
    a.is_bf16 = dtype == NVFP4_BF16;
    a.rowwise = p->rowwise != 0;
    a.colwise = p->colwise != 0;
    a.block2d = p->block == NVFP4_BLOCK_2D;
    a.sr_row = a.rowwise && p->round_row == NVFP4_SR;
    a.sr_col = a.colwise && p->round_col == NVFP4_SR;
    a.rht_row = a.rowwise && p->rht_row != 0;
    a.rht_col = a.colwise && p->rht_col != 0;
    a.k0 = (uint32_t)p->seed;
    a.k1 = (uint32_t)(p->seed >> 32);
    a.rcodes = a.rowwise ? row_out->codes : nullptr;
    a.rscales = a.rowwise ? row_out->scales : nullptr;
    a.rsg = a.rowwise ? row_out->gscale : nullptr;
    a.ccodes = a.colwise ? col_out->codes : nullptr;
    a.cscales = a.colwise ? col_out->scales : nullptr;
    a.csg = a.colwise ? col_out->gscale : nullptr;
    a.partial = (float*)ws;
    a.ntiles = (int)quant_tiles(rows, cols, &a.tiles_c);
    const int f = a.sr_row | (a.sr_col << 1) | (a.rht_row << 2) | (a.rht_col << 3);
    if (a.is_bf16)
        launch_quant_f<true>(f, a, st);
    else
        launch_quant_f<false>(f, a, st);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

extern "C" int nvfp4_dequantize(const nvfp4_qtensor* q, int64_t n, int64_t k, int out_dtype,
                                void* out, int64_t ld_out, void* stream) {
    if (!q) return NVFP4_ERR_NULL;
    if (out_dtype != NVFP4_F32 && out_dtype != NVFP4_BF16) return NVFP4_ERR_DTYPE;
    if (n < 0 || k < 0 || k % 16 || ld_out < k) return NVFP4_ERR_SHAPE;
    if (n == 0 || k == 0) return NVFP4_OK;
    int rc = check_qtensor(q);
    if (rc != NVFP4_OK) return rc;
    if (!out) return NVFP4_ERR_NULL;
    const int64_t esize = out_dtype == NVFP4_BF16 ? 2 : 4;
    if (!aligned(out, 16) || (ld_out * esize) % 16) return NVFP4_ERR_ALIGN;
    const int64_t blocks = n * (k / 16);
    const int64_t grid = (blocks + 255) / 256;
    k_dequant<<<(unsigned)grid, 256, 0, (hipStream_t)stream>>>(q->codes, q->scales, q->gscale, n, k,
                                                             out_dtype == NVFP4_BF16, out, ld_out);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}
