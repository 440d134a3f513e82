// quantize.hip -- C ABI entry points of the NVFP4 quantizer and the dequantizer kernel.
// The quantizer kernels live in quantize_kernels.h (see there for the method and the
// work decomposition); their specialisations are compiled in quantize_launch_*.hip.
#include "quantize_kernels.h"

#include <mutex>

namespace nvfp4 {

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

// The same for k a multiple of 1024, laid out for whole-wave stores: a wave takes 1024
// consecutive elements of one row in four slices of 256, and in slice q lane l decodes the
// four elements at 256 q + 4 l (two code bytes of block 16 q + l / 4).  Each store
// instruction of the wave then writes 1 KB (f32) or 512 B (bf16) of contiguous output,
// where one block per lane writes 16 bytes every 64.
__global__ __launch_bounds__(256) void k_dequant_w(const uint8_t* codes, const uint8_t* scales,
                                                   const float* gscale, int64_t nwaves, int64_t k,
                                                   int out_bf16, void* out, int64_t ld_out) {
    const int64_t w = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (w >= nwaves) return;
    const int lane = threadIdx.x & 63;
    const int64_t spans = k >> 10;
    const int64_t r = w / spans, c0 = (w - r * spans) << 10;
    const float sg = *gscale;
    const uint8_t* crow = codes + r * (k / 2);
    const uint8_t* srow = scales + r * (k / 16);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int64_t c = c0 + q * 256 + 4 * lane;
        const uint32_t cw = *(const uint16_t*)(crow + c / 2);
        const float s = e4m3_value(srow[c / 16]);
        const float2v p0 = fp4x2_to_f32<0>(cw), p1 = fp4x2_to_f32<1>(cw);
        const float o0 = (p0.x * s) * sg, o1 = (p0.y * s) * sg;
        const float o2 = (p1.x * s) * sg, o3 = (p1.y * s) * sg;
        if (!out_bf16) {
            *(float4*)((float*)out + r * ld_out + c) = make_float4(o0, o1, o2, o3);
        } else {
            *(uint2*)((uint16_t*)out + r * ld_out + c) =
                make_uint2(f32_to_bf16_rne(o0) | (f32_to_bf16_rne(o1) << 16),
                           f32_to_bf16_rne(o2) | (f32_to_bf16_rne(o3) << 16));
        }
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

// Workgroups of the k_amax pass: one wave per 16 x 512 wave tile, four per workgroup, at most
// about one round of resident workgroups (each then loops), never more than the encode's
// tiles.  Each writes one partial maximum per copy.
constexpr int64_t kMaxAmaxParts = 768;
static int64_t amax_parts(int64_t rows, int64_t cols) {
    const int64_t wtiles = (rows / 16) * ((cols + kAmaxWaveCols - 1) / kAmaxWaveCols);
    int64_t np = (wtiles + 3) / 4;
    if (np > kMaxAmaxParts) np = kMaxAmaxParts;
    const int64_t nt = quant_tiles(rows, cols, nullptr);
    if (np > nt) np = nt;
    return np > 0 ? np : 1;
}

extern "C" size_t nvfp4_quantize_workspace_bytes(int64_t rows, int64_t cols,
                                                 const nvfp4_quant_params* p) {
    (void)p;
    if (rows <= 0 || cols <= 0) return 0;
    return (size_t)amax_parts(rows, cols) * 2 * sizeof(float);
}

static int check_qtensor(const nvfp4_qtensor* q) {
    if (!q || !q->codes || !q->scales || !q->gscale) return NVFP4_ERR_NULL;
    if (!aligned(q->codes, 8) || !aligned(q->gscale, 4)) return NVFP4_ERR_ALIGN;
    return NVFP4_OK;
}

// LoRA first pass: 64-row blocks times K-parts of kp columns (a multiple of 128), with about
// 512 workgroups in all (its two LDS stages fit two workgroups per CU).
struct LoraSplit {
    int64_t row_blocks, parts, kp;
};
static LoraSplit lora_split(int64_t rows, int64_t cols) {
    LoraSplit s;
    s.row_blocks = (rows + kLoraRowsWG - 1) / kLoraRowsWG;
    const int64_t steps = (cols + kLoraStep - 1) / kLoraStep;
    int64_t target = (512 + s.row_blocks - 1) / (s.row_blocks > 0 ? s.row_blocks : 1);
    if (target < 1) target = 1;
    const int64_t steps_per_part = (steps + target - 1) / target;
    s.kp = (steps_per_part > 0 ? steps_per_part : 1) * kLoraStep;
    s.parts = (cols + s.kp - 1) / s.kp;
    return s;
}

static size_t align256(size_t n) { return (n + 255) & ~(size_t)255; }

extern "C" size_t nvfp4_quantize_lora_workspace_bytes(int64_t rows, int64_t cols, int64_t rank) {
    if (rows <= 0 || cols <= 0 || rank <= 0) return 0;
    const LoraSplit sp = lora_split(rows, cols);
    return align256((size_t)(sp.row_blocks * sp.parts) * 2 * sizeof(float)) +
           (size_t)(sp.parts * rows * rank) * sizeof(float);
}

// ---------------------------------------------------------------- allocation-free variant
// The partial maxima of nvfp4_quantize_noalloc go to this file-scope device array instead of
// a caller workspace.  Every device holds its own copy until the process ends.  In host code
// the name is only a host-side stand-in: the device address of the current device's copy is
// taken once per device with hipGetSymbolAddress and kept in g_scratch_ptr.  Nothing in it
// needs clearing: k_amax writes every partial that k_encode reads.
static __device__ __align__(256) float scratch[2 * kMaxAmaxParts];
static_assert(sizeof(scratch) == NVFP4_NOALLOC_SCRATCH_BYTES, "scratch size of the header");
constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices];

static int scratch_of_current_device(void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return NVFP4_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
            return NVFP4_ERR_HIP;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return NVFP4_OK;
}

// use_scratch: the partial maxima go to the current device's copy of `scratch` (ws and
// ws_bytes are ignored).  given (n_given of them): the caller's partial maxima of |x|, which
// replace the first pass for both copies (no workspace is used).
static int quantize_impl(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld_x,
                         const nvfp4_quant_params* p, const nvfp4_qtensor* row_out,
                         const nvfp4_qtensor* col_out, const uint16_t* lora_a, int64_t rank,
                         float beta, uint16_t* lora_t, void* ws, size_t ws_bytes, void* stream,
                         bool use_scratch = false, const float* given = nullptr,
                         int64_t n_given = 0) {
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
    if ((p->scale46 != 0 && p->scale46 != 1) || (p->scale46 && p->block == NVFP4_BLOCK_2D))
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
    if (given) {
        // the maxima are of the unrotated values: a copy with a Hadamard rotation needs its own
        if (lora_t || (p->rowwise && p->rht_row) || (p->colwise && p->rht_col)) return NVFP4_ERR_MODE;
        if (n_given < 1 || n_given > (1 << 30)) return NVFP4_ERR_SHAPE;
        if (!aligned(given, 4)) return NVFP4_ERR_ALIGN;
    }
    const size_t need = given ? 0
                      : lora_t ? nvfp4_quantize_lora_workspace_bytes(rows, cols, rank)
                               : nvfp4_quantize_workspace_bytes(rows, cols, p);
    if (use_scratch && !given) {
        if (lora_t || need > sizeof(scratch)) return NVFP4_ERR_WORKSPACE;
        if ((rc = scratch_of_current_device(&ws)) != NVFP4_OK) return rc;
        ws_bytes = sizeof(scratch);
    }
    if (!given && (!ws || ws_bytes < need)) return NVFP4_ERR_WORKSPACE;
    if (!given && !aligned(ws, 16)) return NVFP4_ERR_ALIGN;

    QArgs a;
    a.in_codes = nullptr;
    a.in_scales = nullptr;
    a.in_sg = nullptr;
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
    a.scale46 = p->scale46 != 0;
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
    a.lora_a = nullptr;
    a.lora_t = nullptr;
    a.lora_part = nullptr;
    a.lora_r = 0;
    a.lora_parts = 0;
    a.lora_kp = 0;
    a.lora_beta = 0.0f;
    if (lora_t) {   // the first pass is k_amax_lora: one workgroup per 64 rows and K-part
        const LoraSplit sp = lora_split(rows, cols);
        a.npart = (int)(sp.row_blocks * sp.parts);
        a.lora_a = lora_a;
        a.lora_t = lora_t;
        a.lora_part = (float*)((uint8_t*)ws + align256((size_t)a.npart * 2 * sizeof(float)));
        a.lora_r = (int)rank;
        a.lora_parts = (int)sp.parts;
        a.lora_kp = sp.kp;
        a.lora_beta = beta;
    } else if (given) {
        a.partial = const_cast<float*>(given);   // read only: no first pass writes it
        a.npart = (int)n_given;
    } else {
        a.npart = (int)amax_parts(rows, cols);
    }
    a.cpart = given ? 0 : a.npart;
    a.amax_given = given != nullptr;
    const int f = a.sr_row | (a.sr_col << 1) | (a.rht_row << 2) | (a.rht_col << 3);
    if (a.is_bf16)
        (f < 8 ? launch_quant_bf16_lo : launch_quant_bf16_hi)(f, a, st);
    else
        (f < 8 ? launch_quant_f32_lo : launch_quant_f32_hi)(f, a, st);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

extern "C" int nvfp4_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld_x,
                              const nvfp4_quant_params* p, const nvfp4_qtensor* row_out,
                              const nvfp4_qtensor* col_out, void* ws, size_t ws_bytes,
                              void* stream) {
    return quantize_impl(x, dtype, rows, cols, ld_x, p, row_out, col_out, nullptr, 0, 0.0f,
                         nullptr, ws, ws_bytes, stream);
}

extern "C" int nvfp4_quantize_amax(const void* x, int dtype, int64_t rows, int64_t cols,
                                   int64_t ld_x, const nvfp4_quant_params* p,
                                   const nvfp4_qtensor* row_out, const nvfp4_qtensor* col_out,
                                   const float* amax_parts, int64_t n_parts, void* stream) {
    if (!amax_parts) return NVFP4_ERR_NULL;
    return quantize_impl(x, dtype, rows, cols, ld_x, p, row_out, col_out, nullptr, 0, 0.0f,
                         nullptr, nullptr, 0, stream, false, amax_parts, n_parts);
}

extern "C" int nvfp4_quantize_noalloc(const void* x, int dtype, int64_t rows, int64_t cols,
                                      int64_t ld_x, const nvfp4_quant_params* p,
                                      const nvfp4_qtensor* row_out, const nvfp4_qtensor* col_out,
                                      void* stream) {
    return quantize_impl(x, dtype, rows, cols, ld_x, p, row_out, col_out, nullptr, 0, 0.0f,
                         nullptr, nullptr, 0, stream, true);
}

__global__ void k_fill_u16(uint16_t* p, int64_t n, uint16_t v) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = v;
}

extern "C" int nvfp4_quantize_lora(const void* x, int dtype, int64_t rows, int64_t cols,
                                   int64_t ld_x, const nvfp4_quant_params* p,
                                   const nvfp4_qtensor* row_out, const nvfp4_qtensor* col_out,
                                   const uint16_t* lora_a, int64_t rank, float beta,
                                   uint16_t* lora_t, void* ws, size_t ws_bytes, void* stream) {
    if (!p) return NVFP4_ERR_NULL;
    if (dtype != NVFP4_BF16) return NVFP4_ERR_DTYPE;
    if (rank <= 0 || rank % 16 || rank > kLoraMaxRank) return NVFP4_ERR_SHAPE;
    if (rows < 0 || cols < 0 || cols % kLoraStep) return NVFP4_ERR_SHAPE;
    // the first pass's direct loads address 64 input rows and the whole factor with 32-bit
    // byte offsets
    if (ld_x >= ((int64_t)1 << 24) || cols >= ((int64_t)1 << 24)) return NVFP4_ERR_SHAPE;
    if (!lora_a || !lora_t) return NVFP4_ERR_NULL;
    if (((uintptr_t)lora_a & 15) || ((uintptr_t)lora_t & 1)) return NVFP4_ERR_ALIGN;
    if (rows > 0 && cols == 0) {   // an empty contraction: T = 0
        int rc = quantize_impl(x, dtype, rows, cols, ld_x, p, row_out, col_out, nullptr, 0, 0.0f,
                               nullptr, ws, ws_bytes, stream);
        if (rc != NVFP4_OK) return rc;
        const int64_t n = rows * rank;
        k_fill_u16<<<(unsigned)((n + 255) / 256), 256, 0, (hipStream_t)stream>>>(lora_t, n, 0);
        return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
    }
    return quantize_impl(x, dtype, rows, cols, ld_x, p, row_out, col_out, lora_a, rank, beta,
                         rows > 0 ? lora_t : nullptr, ws, ws_bytes, stream);
}

namespace nvfp4 {
void launch_requant_cols(int f, const QArgs& a, hipStream_t st) {
    switch (f) {
    case 0: launch_quant<2, 0>(a, st); break;
    case 2: launch_quant<2, 2>(a, st); break;
    case 8: launch_quant<2, 8>(a, st); break;
    default: launch_quant<2, 10>(a, st); break;
    }
}
}  // namespace nvfp4

extern "C" size_t nvfp4_requantize_cols_workspace_bytes(int64_t rows, int64_t cols) {
    if (rows <= 0 || cols <= 0) return 0;
    return (size_t)amax_parts(rows, cols) * 2 * sizeof(float);
}

extern "C" int nvfp4_requantize_cols(const nvfp4_qtensor* row_in, int64_t rows, int64_t cols,
                                     const nvfp4_quant_params* p, const nvfp4_qtensor* col_out,
                                     void* ws, size_t ws_bytes, void* stream) {
    if (!p || !row_in || !col_out) return NVFP4_ERR_NULL;
    if (rows < 0 || cols < 0 || rows % 16 || cols % 16) return NVFP4_ERR_SHAPE;
    if (p->rowwise || !p->colwise || p->block != NVFP4_BLOCK_1D || p->rht_row ||
        (p->round_col != NVFP4_RNE && p->round_col != NVFP4_SR) ||
        (p->scale46 != 0 && p->scale46 != 1))
        return NVFP4_ERR_MODE;
    hipStream_t st = (hipStream_t)stream;
    if (rows == 0 || cols == 0) {
        if (!col_out->gscale) return NVFP4_ERR_NULL;
        k_fill_scale_one<<<1, 64, 0, st>>>(nullptr, col_out->gscale);
        return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
    }
    int rc;
    if ((rc = check_qtensor(row_in)) != NVFP4_OK) return rc;
    if ((rc = check_qtensor(col_out)) != NVFP4_OK) return rc;
    const size_t need = nvfp4_requantize_cols_workspace_bytes(rows, cols);
    if (!ws || ws_bytes < need) return NVFP4_ERR_WORKSPACE;
    if (!aligned(ws, 16)) return NVFP4_ERR_ALIGN;
    QArgs a;
    a.in_codes = row_in->codes;
    a.in_scales = row_in->scales;
    a.in_sg = row_in->gscale;
    a.x = nullptr;
    a.rows = rows;
    a.cols = cols;
    a.ld = cols;
    a.is_bf16 = 0;
    a.rowwise = 0;
    a.colwise = 1;
    a.block2d = 0;
    a.sr_row = 0;
    a.sr_col = p->round_col == NVFP4_SR;
    a.rht_row = 0;
    a.rht_col = p->rht_col != 0;
    a.scale46 = p->scale46 != 0;
    a.k0 = (uint32_t)p->seed;
    a.k1 = (uint32_t)(p->seed >> 32);
    a.rcodes = nullptr;
    a.rscales = nullptr;
    a.rsg = nullptr;
    a.ccodes = col_out->codes;
    a.cscales = col_out->scales;
    a.csg = col_out->gscale;
    a.partial = (float*)ws;
    a.ntiles = (int)quant_tiles(rows, cols, &a.tiles_c);
    a.lora_a = nullptr;
    a.lora_t = nullptr;
    a.lora_part = nullptr;
    a.lora_r = 0;
    a.lora_parts = 0;
    a.lora_kp = 0;
    a.lora_beta = 0.0f;
    a.npart = (int)amax_parts(rows, cols);
    a.cpart = a.npart;
    a.amax_given = 0;
    launch_requant_cols((a.sr_col << 1) | (a.rht_col << 3), a, st);
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
    if (k % 1024 == 0) {
        const int64_t nwaves = n * (k / 1024);
        k_dequant_w<<<(unsigned)((nwaves + 3) / 4), 256, 0, (hipStream_t)stream>>>(
            q->codes, q->scales, q->gscale, nwaves, k, out_dtype == NVFP4_BF16, out, ld_out);
    } else {
        const int64_t blocks = n * (k / 16);
        const int64_t grid = (blocks + 255) / 256;
        k_dequant<<<(unsigned)grid, 256, 0, (hipStream_t)stream>>>(q->codes, q->scales, q->gscale, n,
                                                                 k, out_dtype == NVFP4_BF16, out, ld_out);
    }
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}
