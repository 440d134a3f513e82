// qadamw.hip -- quantized-state AdamW second moment (encode / decode) for gfx950.
//
// Method: Full-Stack FP4 sec. 3.3 -- (1) y = sqrt(v), (2) subtract the tile-wise mean,
// (3) fast Hadamard transform of the residual, (4) NVFP4 quantization; reconstruction
// v ~ ((s_g s v_hat) H16 + mu)^2.  The gist.science summary (sec. 2.2) stores the tile
// mean in BF16.  Tiles are 16x16, NVFP4 blocks 1x16 along rows, the residual is taken
// against the stored BF16 mean, and the Hadamard is the random one (signs from the seed)
// or the plain normalised H16.
//
// Work decomposition: one lane owns one row of one 16x16 tile, i.e. exactly one 1x16
// NVFP4 block (64 bytes of v: four 16-byte loads).  The 16 lanes of a tile are lanes
// 16k .. 16k+15 of a wave, so the tile sum is an in-register pairwise tree over the
// row followed by xor-shuffles 1, 2, 4, 8 over the 16 row sums -- the same adjacent-
// pair tree in the same order.  A workgroup (4 waves) covers 16 rows x 256 columns.
// Encoding needs the amax of the whole transformed residual first, so it is two passes
// like the quantizer: per-workgroup partial maxima, reduced once by k_max_partials, then
// the encode.
#include "nvfp4.h"
#include "device_common.h"
#include "quantize_kernels.h"   // encode8_rne, encode8_sr, sse8_rne (the quantizer's block encoders)

namespace nvfp4 {

constexpr int QVThreads = 256;
constexpr int QVCols = 256;  // columns per workgroup (16 tiles)

struct QVArgs {
    const float* v;
    int64_t rows, cols;
    uint32_t k0, k1;
    int use_signs;
    uint16_t* mu;
    uint8_t* codes;
    uint8_t* scales;
    float* sg;
    float* partial;      // [nblocks] per-workgroup maxima of the first pass
    const float* amax;   // [1] their maximum (k_max_partials)
    int tiles_c;   // workgroups along columns
    int nblocks;   // workgroups
};

__device__ __forceinline__ float tree16_row(const float y[16]) {
    float t[8], u[4], w[2];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = y[2 * i] + y[2 * i + 1];
#pragma unroll
    for (int i = 0; i < 4; ++i) u[i] = t[2 * i] + t[2 * i + 1];
#pragma unroll
    for (int i = 0; i < 2; ++i) w[i] = u[2 * i] + u[2 * i + 1];
    return w[0] + w[1];
}

// Square roots of one 1x16 row segment y (in place), the tile mean (bf16 bits) and the
// transformed residual e.  The 16 lanes 16k .. 16k+15 hold the rows of one 16x16 tile.
// All 64 lanes must call it (cross-lane shuffles).
__device__ __forceinline__ uint32_t residual_from(float y[16], uint32_t signs, float e[16]) {
    sqrt16_rn(y);
    float s = tree16_row(y);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) s = s + __shfl_xor(s, o, 64);
    const uint32_t mu = f32_to_bf16_rne(s * 0.00390625f);
    const float muf = bf16_to_f32(mu);
#pragma unroll
    for (int i = 0; i < 16; ++i) e[i] = y[i] - muf;
#pragma unroll
    for (int i = 0; i < 16; ++i) e[i] = apply_sign(e[i], signs, i);
    wht16(e);
#pragma unroll
    for (int i = 0; i < 16; ++i) e[i] = e[i] * 0.25f;
    return mu;
}

__device__ __forceinline__ uint32_t residual_block(const QVArgs& a, int64_t r, int64_t c,
                                                   bool valid, uint32_t signs, float e[16]) {
    float y[16];
    if (valid) {
        const float4* p = (const float4*)(a.v + r * a.cols + c);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            float4 f = p[q];
            y[4 * q] = f.x; y[4 * q + 1] = f.y; y[4 * q + 2] = f.z; y[4 * q + 3] = f.w;
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) y[i] = 0.0f;
    }
    return residual_from(y, signs, e);
}

__device__ __forceinline__ void qv_coords(const QVArgs& a, int64_t& r, int64_t& c, bool& valid) {
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int br = blockIdx.x / a.tiles_c, bc = blockIdx.x % a.tiles_c;
    r = (int64_t)br * 16 + (lane & 15);
    c = (int64_t)bc * QVCols + (wid * 4 + (lane >> 4)) * 16;
    valid = r < a.rows && c < a.cols;
}

__device__ __forceinline__ float block_max1(float a, float* red) {
    a = wave_max(a);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
    __syncthreads();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// The tensor maxima from the first pass's per-workgroup partials: one workgroup reads the
// `arrays` (1 or 2) arrays of n partials once and writes their maxima to out[0 .. arrays-1].
// The second pass then reads those instead of every workgroup re-reading all n partials.
// Each thread issues its loads of a round (8 per array) before using any of them, so a round
// costs one memory latency.  The maximum is exact: the reduction order does not change it.
constexpr int kMaxThreads = 1024;
__global__ __launch_bounds__(kMaxThreads) void k_max_partials(const float* partial, int n,
                                                             int arrays, float* out) {
    __shared__ float red[2][kMaxThreads / 64];
    float x = 0.0f, y = 0.0f;
    for (int i0 = threadIdx.x; i0 < n; i0 += 8 * kMaxThreads) {
        float px[8], py[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int i = i0 + u * kMaxThreads;
            px[u] = i < n ? partial[i] : 0.0f;
            py[u] = (arrays > 1 && i < n) ? partial[n + i] : 0.0f;
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) { x = fmaxf(x, px[u]); y = fmaxf(y, py[u]); }
    }
    x = wave_max(x);
    y = wave_max(y);
    if ((threadIdx.x & 63) == 0) { red[0][threadIdx.x >> 6] = x; red[1][threadIdx.x >> 6] = y; }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kMaxThreads / 64; ++w) { x = fmaxf(x, red[0][w]); y = fmaxf(y, red[1][w]); }
        out[0] = x;
        if (arrays > 1) out[1] = y;
    }
}

__global__ __launch_bounds__(QVThreads) void k_qv_pass1(QVArgs a) {
    __shared__ float red[4];
    int64_t r, c;
    bool valid;
    qv_coords(a, r, c, valid);
    const uint32_t signs = a.use_signs ? rht_sign_bits(a.k0, a.k1) : 0u;
    float e[16];
    const uint32_t mu = residual_block(a, r, c, valid, signs, e);
    float am = 0.0f;
    if (valid) {
#pragma unroll
        for (int i = 0; i < 16; ++i) am = fmaxf(am, fabsf(e[i]));
        if ((threadIdx.x & 15) == 0) a.mu[(r / 16) * (a.cols / 16) + c / 16] = (uint16_t)mu;
    }
    am = block_max1(am, red);
    if (threadIdx.x == 0) a.partial[blockIdx.x] = am;
}

__global__ __launch_bounds__(QVThreads) void k_qv_pass2(QVArgs a) {
    __shared__ float rtab[128];   // element reciprocal per scale code
    const float sg = uniform_f(sg_from_amax(a.amax[0]));
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.sg = sg;
    const bool tiny = tiny_scale(sg);
    if (threadIdx.x < 128) rtab[threadIdx.x] = recip_entry(threadIdx.x, sg, tiny);
    __syncthreads();
    const CopyScale csc{sg, __fdiv_rn(1.0f, sg), sg >= 0x1p-92f, rtab, conv_scale(tiny)};

    int64_t r, c;
    bool valid;
    qv_coords(a, r, c, valid);
    const uint32_t signs = a.use_signs ? rht_sign_bits(a.k0, a.k1) : 0u;
    float e[16];
    residual_block(a, r, c, valid, signs, e);
    float bm = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) bm = fmaxf(bm, fabsf(e[i]));
    const uint32_t scode = csc.code(bm, 6.0f, kRcp6);
    float u[16];
    csc.scale8(&e[0], scode, 1.0f, &u[0]);
    csc.scale8(&e[8], scode, 1.0f, &u[8]);
    const uint32_t lo = encode8_rne(&u[0], csc.cs), hi = encode8_rne(&u[8], csc.cs);
    if (valid) {
        *(uint2*)(a.codes + r * (a.cols / 2) + c / 2) = make_uint2(lo, hi);
        a.scales[r * (a.cols / 16) + c / 16] = (uint8_t)scode;
    }
}

__global__ __launch_bounds__(QVThreads) void k_qv_decode(const uint16_t* mu, const uint8_t* codes,
                                                         const uint8_t* scales, const float* gs,
                                                         int64_t rows, int64_t cols, uint32_t k0,
                                                         uint32_t k1, int use_signs, float* out) {
    const int64_t kb = cols / 16;
    const int64_t blk = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (blk >= rows * kb) return;
    const int64_t r = blk / kb, b = blk % kb;
    const uint2 cw = *(const uint2*)(codes + r * (cols / 2) + b * 8);
    const float s = e4m3_value(scales[r * kb + b]);
    const float sg = *gs;
    const float muf = bf16_to_f32(mu[(r / 16) * kb + b]);
    const uint32_t signs = use_signs ? rht_sign_bits(k0, k1) : 0u;
    float w[16];
    uint32_t w2[2] = {cw.x, cw.y};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float2v p0 = fp4x2_to_f32<0>(w2[h]);
        float2v p1 = fp4x2_to_f32<1>(w2[h]);
        float2v p2 = fp4x2_to_f32<2>(w2[h]);
        float2v p3 = fp4x2_to_f32<3>(w2[h]);
        w[8 * h + 0] = p0.x; w[8 * h + 1] = p0.y; w[8 * h + 2] = p1.x; w[8 * h + 3] = p1.y;
        w[8 * h + 4] = p2.x; w[8 * h + 5] = p2.y; w[8 * h + 6] = p3.x; w[8 * h + 7] = p3.y;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = (w[i] * s) * sg;
    wht16(w);
#pragma unroll
    for (int i = 0; i < 16; ++i) w[i] = apply_sign(w[i] * 0.25f, signs, i);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float z = w[i] + muf;
        w[i] = z * z;
    }
    float4* p = (float4*)(out + r * cols + b * 16);
#pragma unroll
    for (int q = 0; q < 4; ++q) p[q] = make_float4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
}

// The same for cols a multiple of 1024, laid out for whole-wave stores (as the dequantizer's
// wide kernel): a wave takes 1024 consecutive elements of one row in four slices of 256, and
// in slice q lane l holds positions 4 (l mod 4) .. + 3 of block 16 q + l / 4, so a block is one
// DPP quad.  The butterfly's stages 1 and 2 stay in-register, stages 4 and 8 pair the lane
// with lane ^ 1 and lane ^ 2: the lower lane forms a + b, the upper b' - b'' as p - w with
// p the partner's value, the same operations on the same operands as wht16.
__global__ __launch_bounds__(QVThreads) void k_qv_decode_w(const uint16_t* mu, const uint8_t* codes,
                                                           const uint8_t* scales, const float* gs,
                                                           int64_t nwaves, int64_t cols, uint32_t k0,
                                                           uint32_t k1, int use_signs, float* out) {
    const int64_t w = (int64_t)blockIdx.x * 4 + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    if (w >= nwaves) return;
    const int lane = threadIdx.x & 63, j = lane & 3;
    const int64_t spans = cols >> 10, kb = cols / 16;
    const int64_t r = w / spans, c0 = (w - r * spans) << 10;
    const float sg = *gs;
    const uint32_t signs = use_signs ? rht_sign_bits(k0, k1) : 0u;
    const float up1 = (j & 1) ? -1.0f : 1.0f, up2 = (j & 2) ? -1.0f : 1.0f;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int64_t c = c0 + q * 256 + 4 * lane, b = c / 16;
        const uint32_t cw = *(const uint16_t*)(codes + r * (cols / 2) + c / 2);
        const float s = e4m3_value(scales[r * kb + b]);
        const float muf = bf16_to_f32(mu[(r / 16) * kb + b]);
        const float2v p0 = fp4x2_to_f32<0>(cw), p1 = fp4x2_to_f32<1>(cw);
        float x[4] = {(p0.x * s) * sg, (p0.y * s) * sg, (p1.x * s) * sg, (p1.y * s) * sg};
        // stages 1 and 2 (positions within the lane)
        float a = x[0] + x[1], bb = x[0] - x[1], cc = x[2] + x[3], d = x[2] - x[3];
        x[0] = a + cc; x[2] = a - cc; x[1] = bb + d; x[3] = bb - d;
        // stage 4: lane ^ 1; stage 8: lane ^ 2
#pragma unroll
        for (int t = 0; t < 4; ++t) x[t] = __builtin_fmaf(x[t], up1, xor1(x[t]));
#pragma unroll
        for (int t = 0; t < 4; ++t) x[t] = __builtin_fmaf(x[t], up2, xor2(x[t]));
        float o[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const float z = apply_sign(x[t] * 0.25f, signs, 4 * j + t) + muf;
            o[t] = z * z;
        }
        *(float4*)(out + r * cols + c) = make_float4(o[0], o[1], o[2], o[3]);
    }
}

// ---------------------------------------------------------------- full AdamW step
// Full-Stack FP4 sec. 2 (moments m = beta1 m + c g, v = beta2 v + (1 - beta2) g^2) and sec.
// 3.3 (m stored through a Hadamard rotation, 4/6 scaling and stochastic rounding; v through
// the pipeline above); decoupled AdamW update w -= lr (bias1 m / (sqrt(bias2 v) + eps) +
// wd w).  Same lane layout as the v kernels (one lane = one 1x16 row block of a 16x16 tile).
// The new s_g of m and of v need the amax of the whole new states, so it is two passes:
// pass 1 forms the moments and their partial maxima (and writes the new tile means);
// pass 2 forms them again, bit for bit, and encodes, and updates w.  The states are read
// from m_in/v_in and written to m_out/v_out, which therefore must not alias.
struct QSArgs {
    float* w;
    const void* g;
    int g_bf16;
    int64_t rows, cols;
    const uint8_t* mc; const uint8_t* ms; const float* msg;     // m in
    uint8_t* mco; uint8_t* mso; float* msgo;                     // m out
    const uint16_t* mu; const uint8_t* vc; const uint8_t* vs; const float* vsg;  // v in
    uint16_t* muo; uint8_t* vco; uint8_t* vso; float* vsgo;      // v out
    float lr, b1, b2, eps, wd, cg, bias1, bias2;
    uint32_t mk0, mk1, sk0, sk1, vk0, vk1;
    int v_use_signs;
    float* partial;      // [2][nblocks]: m and v residual maxima per workgroup
    const float* amax;   // [2]: their maxima (k_max_partials)
    int tiles_c, nblocks;
};

// Decode 16 codes of a row block: (v s) s_g, then the inverse transform D (1/4 H16 x).
__device__ __forceinline__ void decode_rot16(const uint8_t* codes, const uint8_t* scales, float sg,
                                             int64_t r, int64_t c, int64_t cols, uint32_t signs,
                                             float x[16]) {
    const uint2 cw = *(const uint2*)(codes + r * (cols / 2) + c / 2);
    const float s = e4m3_value(scales[r * (cols / 16) + c / 16]);
    const uint32_t w2[2] = {cw.x, cw.y};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const float2v p0 = fp4x2_to_f32<0>(w2[h]), p1 = fp4x2_to_f32<1>(w2[h]);
        const float2v p2 = fp4x2_to_f32<2>(w2[h]), p3 = fp4x2_to_f32<3>(w2[h]);
        x[8 * h + 0] = p0.x; x[8 * h + 1] = p0.y; x[8 * h + 2] = p1.x; x[8 * h + 3] = p1.y;
        x[8 * h + 4] = p2.x; x[8 * h + 5] = p2.y; x[8 * h + 6] = p3.x; x[8 * h + 7] = p3.y;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = (x[i] * s) * sg;
    wht16(x);
#pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = apply_sign(x[i] * 0.25f, signs, i);
}

// New moments of one row block (zeros for lanes outside the tensor).
__device__ __forceinline__ void qs_moments(const QSArgs& a, int64_t r, int64_t c, bool valid,
                                           uint32_t msigns, uint32_t vsigns, float m[16], float v[16]) {
    if (!valid) {
#pragma unroll
        for (int i = 0; i < 16; ++i) { m[i] = 0.0f; v[i] = 0.0f; }
        return;
    }
    float mp[16], vp[16], g[16];
    decode_rot16(a.mc, a.ms, *a.msg, r, c, a.cols, msigns, mp);
    decode_rot16(a.vc, a.vs, *a.vsg, r, c, a.cols, vsigns, vp);
    const float muf = bf16_to_f32(a.mu[(r / 16) * (a.cols / 16) + c / 16]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float z = vp[i] + muf;
        vp[i] = z * z;
    }
    if (a.g_bf16) {
        const uint4* p = (const uint4*)((const uint16_t*)a.g + r * a.cols + c);
#pragma unroll
        for (int q = 0; q < 2; ++q) {
            const uint4 u = p[q];
            const uint32_t ww[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                g[8 * q + 2 * k] = __uint_as_float(ww[k] << 16);
                g[8 * q + 2 * k + 1] = __uint_as_float(ww[k] & 0xFFFF0000u);
            }
        }
    } else {
        const float4* p = (const float4*)((const float*)a.g + r * a.cols + c);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 f = p[q];
            g[4 * q] = f.x; g[4 * q + 1] = f.y; g[4 * q + 2] = f.z; g[4 * q + 3] = f.w;
        }
    }
    const float omb2 = 1.0f - a.b2;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        m[i] = a.b1 * mp[i] + a.cg * g[i];
        v[i] = a.b2 * vp[i] + omb2 * (g[i] * g[i]);
    }
}

// The rotated first moment y = 1/4 H16 (D m).
__device__ __forceinline__ void rot16(const float m[16], uint32_t signs, float y[16]) {
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = apply_sign(m[i], signs, i);
    wht16(y);
#pragma unroll
    for (int i = 0; i < 16; ++i) y[i] = y[i] * 0.25f;
}

__device__ __forceinline__ void qs_coords(const QSArgs& a, int64_t& r, int64_t& c, bool& valid) {
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const int br = blockIdx.x / a.tiles_c, bc = blockIdx.x % a.tiles_c;
    r = (int64_t)br * 16 + (lane & 15);
    c = (int64_t)bc * QVCols + (wid * 4 + (lane >> 4)) * 16;
    valid = r < a.rows && c < a.cols;
}

__global__ __launch_bounds__(QVThreads) void k_qs_pass1(QSArgs a) {
    __shared__ float red[8];
    int64_t r, c;
    bool valid;
    qs_coords(a, r, c, valid);
    const uint32_t msigns = rht_sign_bits(a.mk0, a.mk1);
    const uint32_t vsigns = a.v_use_signs ? rht_sign_bits(a.vk0, a.vk1) : 0u;
    float m[16], v[16], y[16], e[16];
    qs_moments(a, r, c, valid, msigns, vsigns, m, v);
    rot16(m, msigns, y);
    const uint32_t mu = residual_from(v, vsigns, e);
    float am = 0.0f, av = 0.0f;
    if (valid) {
#pragma unroll
        for (int i = 0; i < 16; ++i) { am = fmaxf(am, fabsf(y[i])); av = fmaxf(av, fabsf(e[i])); }
        if ((threadIdx.x & 15) == 0) a.muo[(r / 16) * (a.cols / 16) + c / 16] = (uint16_t)mu;
    }
    block_max2(am, av, red);
    if (threadIdx.x == 0) {
        a.partial[blockIdx.x] = am;
        a.partial[a.nblocks + blockIdx.x] = av;
    }
}

// Five waves per SIMD (96 VGPRs, no spills) instead of four: the pass is long dependent
// arithmetic chains (decodes, square roots, divisions, Philox), and a fifth wave keeps the
// SIMDs issuing more of the time (about 2% at 9216 x 3072, same output).  Six waves (80
// VGPRs) spill and lose 7%.
__global__ __launch_bounds__(QVThreads, 5) void k_qs_pass2(QSArgs a) {
    __shared__ float rtab[2][128];   // element reciprocal per scale code: m, v
    const float sgm = uniform_f(sg_from_amax(a.amax[0])), sgv = uniform_f(sg_from_amax(a.amax[1]));
    if (blockIdx.x == 0 && threadIdx.x == 0) { *a.msgo = sgm; *a.vsgo = sgv; }
    const bool tiny_m = tiny_scale(sgm), tiny_v = tiny_scale(sgv);
    {
        const uint32_t t = threadIdx.x & 127;
        const bool mrow = threadIdx.x < 128;
        rtab[threadIdx.x >> 7][t] = recip_entry(t, mrow ? sgm : sgv, mrow ? tiny_m : tiny_v);
    }
    __syncthreads();
    const CopyScale msc{sgm, __fdiv_rn(1.0f, sgm), sgm >= 0x1p-92f, rtab[0], conv_scale(tiny_m)};
    const CopyScale vsc{sgv, __fdiv_rn(1.0f, sgv), sgv >= 0x1p-92f, rtab[1], conv_scale(tiny_v)};

    int64_t r, c;
    bool valid;
    qs_coords(a, r, c, valid);
    const uint32_t msigns = rht_sign_bits(a.mk0, a.mk1);
    const uint32_t vsigns = a.v_use_signs ? rht_sign_bits(a.vk0, a.vk1) : 0u;
    float m[16], v[16], y[16], e[16];
    qs_moments(a, r, c, valid, msigns, vsigns, m, v);

    // weights
    if (valid) {
        float4* pw = (float4*)(a.w + r * a.cols + c);
        float w[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const float4 f = pw[q];
            w[4 * q] = f.x; w[4 * q + 1] = f.y; w[4 * q + 2] = f.z; w[4 * q + 3] = f.w;
        }
        float rt[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) rt[i] = a.bias2 * v[i];
        sqrt16_rn(rt);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float den = rt[i] + a.eps;
            const float upd = __fdiv_rn(a.bias1 * m[i], den) + a.wd * w[i];
            w[i] = w[i] - a.lr * upd;
        }
#pragma unroll
        for (int q = 0; q < 4; ++q) pw[q] = make_float4(w[4 * q], w[4 * q + 1], w[4 * q + 2], w[4 * q + 3]);
    }

    // m: rotated, 1x16 blocks with 4/6 scaling, stochastic rounding
    rot16(m, msigns, y);
    {
        float bm = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) bm = fmaxf(bm, fabsf(y[i]));
        uint32_t sc = msc.code(bm, 6.0f, kRcp6);
        const uint32_t sc4 = msc.code(bm, 4.0f, 0.25f);
        const float s6 = e4m3_value(sc), s4 = e4m3_value(sc4);
        uint32_t t0, t1, t2, t3;
        float u[16];
        msc.scale8(&y[0], sc, 1.0f, &u[0]);
        msc.scale8(&y[8], sc, 1.0f, &u[8]);
        const float e6 = sse8_rne(&y[0], &u[0], s6, sgm, msc.cs, t0) + sse8_rne(&y[8], &u[8], s6, sgm, msc.cs, t1);
        msc.scale8(&y[0], sc4, 1.0f, &u[0]);
        msc.scale8(&y[8], sc4, 1.0f, &u[8]);
        const float e4 = sse8_rne(&y[0], &u[0], s4, sgm, msc.cs, t2) + sse8_rne(&y[8], &u[8], s4, sgm, msc.cs, t3);
        sc = e4 < e6 ? sc4 : sc;
        msc.scale8(&y[0], sc, 1.0f, &u[0]);
        msc.scale8(&y[8], sc, 1.0f, &u[8]);
        const uint64_t g0 = ((uint64_t)r * (uint64_t)a.cols + (uint64_t)c) >> 3;
        const uint32_t lo = encode8_sr(&u[0], sr_words(g0, 0u, a.sk0, a.sk1), msc.cs);
        const uint32_t hi = encode8_sr(&u[8], sr_words(g0 + 1, 0u, a.sk0, a.sk1), msc.cs);
        if (valid) {
            *(uint2*)(a.mco + r * (a.cols / 2) + c / 2) = make_uint2(lo, hi);
            a.mso[r * (a.cols / 16) + c / 16] = (uint8_t)sc;
        }
    }
    // v: the second-moment pipeline, nearest-even
    residual_from(v, vsigns, e);
    {
        float bm = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) bm = fmaxf(bm, fabsf(e[i]));
        const uint32_t sc = vsc.code(bm, 6.0f, kRcp6);
        float u[16];
        vsc.scale8(&e[0], sc, 1.0f, &u[0]);
        vsc.scale8(&e[8], sc, 1.0f, &u[8]);
        const uint32_t lo = encode8_rne(&u[0], vsc.cs), hi = encode8_rne(&u[8], vsc.cs);
        if (valid) {
            *(uint2*)(a.vco + r * (a.cols / 2) + c / 2) = make_uint2(lo, hi);
            a.vso[r * (a.cols / 16) + c / 16] = (uint8_t)sc;
        }
    }
}

}  // namespace nvfp4

using namespace nvfp4;

static int64_t qv_blocks(int64_t rows, int64_t cols, int* tiles_c) {
    const int64_t tc = (cols + QVCols - 1) / QVCols;
    if (tiles_c) *tiles_c = (int)tc;
    return (rows / 16) * tc;
}

// Workspace: `arrays` arrays of per-workgroup partial maxima, then (16-byte aligned) their
// `arrays` maxima.
static size_t partials_floats(int64_t rows, int64_t cols, int arrays) {
    return ((size_t)qv_blocks(rows, cols, nullptr) * arrays + 3) & ~(size_t)3;
}

extern "C" size_t qadamw_v_workspace_bytes(int64_t rows, int64_t cols) {
    if (rows <= 0 || cols <= 0) return 0;
    return (partials_floats(rows, cols, 1) + 4) * sizeof(float);
}

extern "C" int qadamw_v_encode(const float* v, int64_t rows, int64_t cols, uint64_t seed,
                               int32_t use_signs, uint16_t* mu, const nvfp4_qtensor* q, void* ws,
                               size_t ws_bytes, void* stream) {
    if (!q) return NVFP4_ERR_NULL;
    if (rows < 0 || cols < 0 || rows % 16 || cols % 16) return NVFP4_ERR_SHAPE;
    hipStream_t st = (hipStream_t)stream;
    if (rows == 0 || cols == 0) return NVFP4_OK;
    if (!q->codes || !q->scales || !q->gscale) return NVFP4_ERR_NULL;
    if (!v || !mu) return NVFP4_ERR_NULL;
    if (((uintptr_t)v & 15) || ((uintptr_t)q->codes & 7) || ((uintptr_t)mu & 1) ||
        ((uintptr_t)q->gscale & 3))
        return NVFP4_ERR_ALIGN;
    const size_t need = qadamw_v_workspace_bytes(rows, cols);
    if (!ws || ws_bytes < need) return NVFP4_ERR_WORKSPACE;
    if ((uintptr_t)ws & 15) return NVFP4_ERR_ALIGN;
    QVArgs a;
    a.v = v; a.rows = rows; a.cols = cols;
    a.k0 = (uint32_t)seed; a.k1 = (uint32_t)(seed >> 32);
    a.use_signs = use_signs != 0;
    a.mu = mu; a.codes = q->codes; a.scales = q->scales; a.sg = q->gscale;
    a.partial = (float*)ws;
    a.amax = (float*)ws + partials_floats(rows, cols, 1);
    a.nblocks = (int)qv_blocks(rows, cols, &a.tiles_c);
    k_qv_pass1<<<a.nblocks, QVThreads, 0, st>>>(a);
    k_max_partials<<<1, kMaxThreads, 0, st>>>(a.partial, a.nblocks, 1, (float*)a.amax);
    k_qv_pass2<<<a.nblocks, QVThreads, 0, st>>>(a);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

extern "C" int qadamw_v_decode(const uint16_t* mu, const nvfp4_qtensor* q, int64_t rows,
                               int64_t cols, uint64_t seed, int32_t use_signs, float* v_out,
                               void* stream) {
    if (!q) return NVFP4_ERR_NULL;
    if (rows < 0 || cols < 0 || rows % 16 || cols % 16) return NVFP4_ERR_SHAPE;
    if (rows == 0 || cols == 0) return NVFP4_OK;
    if (!q->codes || !q->scales || !q->gscale || !mu || !v_out) return NVFP4_ERR_NULL;
    if (((uintptr_t)v_out & 15) || ((uintptr_t)q->codes & 7) || ((uintptr_t)mu & 1))
        return NVFP4_ERR_ALIGN;
    if (cols % 1024 == 0) {
        const int64_t nwaves = rows * (cols / 1024);
        k_qv_decode_w<<<(unsigned)((nwaves + 3) / 4), 256, 0, (hipStream_t)stream>>>(
            mu, q->codes, q->scales, q->gscale, nwaves, cols, (uint32_t)seed,
            (uint32_t)(seed >> 32), use_signs != 0, v_out);
    } else {
        const int64_t blocks = rows * (cols / 16);
        k_qv_decode<<<(unsigned)((blocks + 255) / 256), 256, 0, (hipStream_t)stream>>>(
            mu, q->codes, q->scales, q->gscale, rows, cols, (uint32_t)seed, (uint32_t)(seed >> 32),
            use_signs != 0, v_out);
    }
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}

extern "C" size_t qadamw_step_workspace_bytes(int64_t rows, int64_t cols) {
    if (rows <= 0 || cols <= 0) return 0;
    return (partials_floats(rows, cols, 2) + 4) * sizeof(float);
}

extern "C" int qadamw_step(float* w, const void* g, int g_dtype, int64_t rows, int64_t cols,
                           const nvfp4_qtensor* m_in, const nvfp4_qtensor* m_out,
                           const uint16_t* mu_in, const nvfp4_qtensor* v_in, uint16_t* mu_out,
                           const nvfp4_qtensor* v_out, const qadamw_step_params* p, void* ws,
                           size_t ws_bytes, void* stream) {
    if (!p || !m_in || !m_out || !v_in || !v_out) return NVFP4_ERR_NULL;
    if (g_dtype != NVFP4_F32 && g_dtype != NVFP4_BF16) return NVFP4_ERR_DTYPE;
    if (rows < 0 || cols < 0 || rows % 16 || cols % 16) return NVFP4_ERR_SHAPE;
    if (rows == 0 || cols == 0) return NVFP4_OK;
    const nvfp4_qtensor* qs[4] = {m_in, m_out, v_in, v_out};
    for (const nvfp4_qtensor* q : qs) {
        if (!q->codes || !q->scales || !q->gscale) return NVFP4_ERR_NULL;
        if (((uintptr_t)q->codes & 7) || ((uintptr_t)q->gscale & 3)) return NVFP4_ERR_ALIGN;
    }
    if (!w || !g || !mu_in || !mu_out) return NVFP4_ERR_NULL;
    if (((uintptr_t)w & 15) || ((uintptr_t)g & 15) || ((uintptr_t)mu_in & 1) || ((uintptr_t)mu_out & 1))
        return NVFP4_ERR_ALIGN;
    // the states are read by both passes: outputs must not overlap the inputs
    if (m_out->codes == m_in->codes || m_out->scales == m_in->scales || v_out->codes == v_in->codes ||
        v_out->scales == v_in->scales || mu_out == mu_in || m_out->gscale == m_in->gscale ||
        v_out->gscale == v_in->gscale)
        return NVFP4_ERR_MODE;
    const size_t need = qadamw_step_workspace_bytes(rows, cols);
    if (!ws || ws_bytes < need) return NVFP4_ERR_WORKSPACE;
    if ((uintptr_t)ws & 15) return NVFP4_ERR_ALIGN;
    QSArgs a;
    a.w = w; a.g = g; a.g_bf16 = g_dtype == NVFP4_BF16; a.rows = rows; a.cols = cols;
    a.mc = m_in->codes; a.ms = m_in->scales; a.msg = m_in->gscale;
    a.mco = m_out->codes; a.mso = m_out->scales; a.msgo = m_out->gscale;
    a.mu = mu_in; a.vc = v_in->codes; a.vs = v_in->scales; a.vsg = v_in->gscale;
    a.muo = mu_out; a.vco = v_out->codes; a.vso = v_out->scales; a.vsgo = v_out->gscale;
    a.lr = p->lr; a.b1 = p->beta1; a.b2 = p->beta2; a.eps = p->eps; a.wd = p->weight_decay;
    a.cg = p->grad_coef; a.bias1 = p->bias1; a.bias2 = p->bias2;
    a.mk0 = (uint32_t)p->m_rht_seed; a.mk1 = (uint32_t)(p->m_rht_seed >> 32);
    a.sk0 = (uint32_t)p->m_sr_seed; a.sk1 = (uint32_t)(p->m_sr_seed >> 32);
    a.vk0 = (uint32_t)p->v_seed; a.vk1 = (uint32_t)(p->v_seed >> 32);
    a.v_use_signs = p->v_use_signs != 0;
    a.partial = (float*)ws;
    a.amax = (float*)ws + partials_floats(rows, cols, 2);
    a.nblocks = (int)qv_blocks(rows, cols, &a.tiles_c);
    hipStream_t st = (hipStream_t)stream;
    k_qs_pass1<<<a.nblocks, QVThreads, 0, st>>>(a);
    k_max_partials<<<1, kMaxThreads, 0, st>>>(a.partial, a.nblocks, 2, (float*)a.amax);
    k_qs_pass2<<<a.nblocks, QVThreads, 0, st>>>(a);
    return hipGetLastError() == hipSuccess ? NVFP4_OK : NVFP4_ERR_HIP;
}
