// quantize_kernels.h -- NVFP4 quantizer kernels for gfx950 (included by the launch
// units quantize_launch_*.hip, which instantiate the 32 specialisations in parallel
// translation units, and by quantize.hip, which holds the ABI entry points).
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

#pragma once
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
    int scale46;
    uint32_t k0, k1;
    uint8_t* rcodes;
    uint8_t* rscales;
    float* rsg;
    uint8_t* ccodes;
    uint8_t* cscales;
    float* csg;
    // input kind 2 (eq. (2)'s double quantization): the rowwise NVFP4 copy x is decoded from
    const uint8_t* in_codes;
    const uint8_t* in_scales;
    const float* in_sg;
    float* partial;  // [2][npart]: rowwise-copy and columnwise-copy amax per k_amax workgroup
    int tiles_c;
    int ntiles;
    int npart;       // first-pass workgroups, one partial maximum each per copy
    // offset of the columnwise copy's partials in `partial` (npart; 0 when the caller supplies
    // the maxima, which then serve both copies); amax_given: no first pass is launched
    int cpart;
    int amax_given;
    // LoRA-SVD down-projection (lora_t null: none): lora_t[rows][lora_r] = BF16(beta x a^T)
    // with a = lora_a[lora_r][cols]; the first pass leaves one FP32 partial per K-part of
    // lora_kp columns in lora_part[lora_parts][rows][lora_r], the encode pass sums them.
    const uint16_t* lora_a;
    uint16_t* lora_t;
    float* lora_part;
    int lora_r, lora_parts;
    int64_t lora_kp;
    float lora_beta;
};

// One thread's 16-row x 8-column input patch.  bfloat16 stays packed two to a register
// (64 VGPRs rather than 128) and is widened where it is used: a bfloat16 is the upper
// half of the binary32 with the same value.
template <int IN> struct Patch;   // IN: 0 binary32, 1 bfloat16, 2 a rowwise NVFP4 copy

template <> struct Patch<1> {
    uint32_t p[16][4];
    __device__ __forceinline__ void load(const void* x, int64_t ld, int64_t r0, int64_t c0, bool valid) {
        if (!valid) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
#pragma unroll
                for (int h = 0; h < 4; ++h) p[i][h] = 0u;
            return;
        }
        const uint16_t* src = (const uint16_t*)x + r0 * ld + c0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint4 q = *(const uint4*)(src + (int64_t)i * ld);
            p[i][0] = q.x; p[i][1] = q.y; p[i][2] = q.z; p[i][3] = q.w;
        }
    }
    __device__ __forceinline__ float at(int i, int e) const {
        return __uint_as_float((e & 1) ? (p[i][e >> 1] & 0xFFFF0000u) : (p[i][e >> 1] << 16));
    }
    // negate element (i, 2h) where bit 15 of m is set and element (i, 2h + 1) where bit 31 is
    __device__ __forceinline__ void flip(int i, int h, uint32_t m) { p[i][h] ^= m; }
    static __device__ __forceinline__ uint32_t pair_mask(uint32_t b_even, uint32_t b_odd) {
        return (b_even << 15) | (b_odd << 31);
    }
    // max |x| over the patch: on the packed bits with the signs cleared, two at a time
    // (sign-magnitude bit patterns order like the magnitudes)
    __device__ __forceinline__ float amax() const {
        typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
        u16x2 m = {0, 0};
#pragma unroll
        for (int i = 0; i < 16; ++i)
#pragma unroll
            for (int h = 0; h < 4; ++h)
                m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, p[i][h] & 0x7FFF7FFFu));
        return fmaxf(__uint_as_float((uint32_t)m.x << 16), __uint_as_float((uint32_t)m.y << 16));
    }
};

template <> struct Patch<0> {
    float p[16][8];
    __device__ __forceinline__ void load(const void* x, int64_t ld, int64_t r0, int64_t c0, bool valid) {
        if (!valid) {
#pragma unroll
            for (int i = 0; i < 16; ++i)
#pragma unroll
                for (int e = 0; e < 8; ++e) p[i][e] = 0.0f;
            return;
        }
        const float* src = (const float*)x + r0 * ld + c0;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const float4 q0 = *(const float4*)(src + (int64_t)i * ld);
            const float4 q1 = *(const float4*)(src + (int64_t)i * ld + 4);
            p[i][0] = q0.x; p[i][1] = q0.y; p[i][2] = q0.z; p[i][3] = q0.w;
            p[i][4] = q1.x; p[i][5] = q1.y; p[i][6] = q1.z; p[i][7] = q1.w;
        }
    }
    __device__ __forceinline__ float at(int i, int e) const { return p[i][e]; }
    __device__ __forceinline__ void flip(int i, int h, uint32_t m) {   // m as for bfloat16
        p[i][2 * h] = __uint_as_float(__float_as_uint(p[i][2 * h]) ^ (m << 16));
        p[i][2 * h + 1] = __uint_as_float(__float_as_uint(p[i][2 * h + 1]) ^ (m & 0x80000000u));
    }
    static __device__ __forceinline__ uint32_t pair_mask(uint32_t b_even, uint32_t b_odd) {
        return (b_even << 15) | (b_odd << 31);
    }
    __device__ __forceinline__ float amax() const {
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(p[i][e]));
        return m;
    }
};

// A rowwise NVFP4 copy, the input of the columnwise copy in Full-Stack FP4 eq. (2),
// Q_16x1(H^T Q_1x16(X)).  A patch row's 8 columns are one 4-byte group of codes inside one
// 16-element block; the patch keeps those code words and the rows' block scales (32 VGPRs)
// and decodes an element where it is used: fl(fl(v s) s_g), v s being exact.
template <> struct Patch<2> {
    uint32_t p[16];   // 8 E2M1 codes per row, element e in bits 4e..4e+3
    float s[16];      // the row's block scale
    float sg;         // the copy's tensor scale
    __device__ __forceinline__ void load_q(const QArgs& a, int64_t r0, int64_t c0, bool valid) {
        sg = *a.in_sg;
        if (!valid) {
#pragma unroll
            for (int i = 0; i < 16; ++i) { p[i] = 0u; s[i] = 0.0f; }
            return;
        }
        const int64_t cp = a.cols / 2, sp = a.cols / 16;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            p[i] = *(const uint32_t*)(a.in_codes + (r0 + i) * cp + c0 / 2);
            s[i] = e4m3_value(a.in_scales[(r0 + i) * sp + c0 / 16]);
        }
    }
    // the two decoded codes of byte k of row i (k a constant once the callers' loops unroll)
    __device__ __forceinline__ float2v pair(int i, int k) const {
        switch (k) {
            case 0: return fp4x2_to_f32<0>(p[i]);
            case 1: return fp4x2_to_f32<1>(p[i]);
            case 2: return fp4x2_to_f32<2>(p[i]);
            default: return fp4x2_to_f32<3>(p[i]);
        }
    }
    __device__ __forceinline__ float at(int i, int e) const {
        const float2v q = pair(i, e >> 1);
        return ((e & 1) ? q.y : q.x) * s[i] * sg;
    }
    // negating a decoded value is flipping its code's sign bit (bit 3 of the nibble)
    __device__ __forceinline__ void flip(int i, int h, uint32_t m) {   // m as for bfloat16
        p[i] ^= (((m >> 15) & 1u) << (8 * h + 3)) | ((m >> 31) << (8 * h + 7));
    }
    static __device__ __forceinline__ uint32_t pair_mask(uint32_t b_even, uint32_t b_odd) {
        return (b_even << 15) | (b_odd << 31);
    }
    // max |x|: per row from the largest decoded |v| (x -> fl(fl(x s) s_g) is monotone)
    __device__ __forceinline__ float amax() const {
        float m = 0.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float r = 0.0f;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float2v q = pair(i, k);
                r = fmaxf(r, fmaxf(fabsf(q.x), fabsf(q.y)));
            }
            m = fmaxf(m, r * s[i] * sg);
        }
        return m;
    }
};

template <int IN>
__device__ __forceinline__ void load_patch(Patch<IN>& P, const QArgs& a, int64_t r0, int64_t c0,
                                           bool valid) {
    if constexpr (IN == 2) P.load_q(a, r0, c0, valid);
    else P.load(a.x, a.ld, r0, c0, valid);
}

// The random Hadamard transform of a 16-chunk is (1/4) H16 (D v): the sign flips D are
// applied to the packed patch beforehand (flip_row_signs / flip_col_signs: one XOR per
// packed pair), the butterflies here, and the factor 1/4 by the caller (an exact scaling,
// folded into the element reciprocal where that is exact too).
//
// Butterflies of a 16-chunk held as 8 values per lane in a lane pair (the lane with
// half = 0 holds positions 0..7, its neighbour positions 8..15): stages 1, 2, 4
// in-register, stage 8 with lane ^ 1 as one fma with +-1 (w + p, or p - w).
__device__ __forceinline__ void wht_pair8(float w[8], float sgn) {
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
    for (int e = 0; e < 8; ++e) w[e] = __builtin_fmaf(w[e], sgn, xor1(w[e]));
}

// Row signs: element (i, e) of the lane's 8 columns sits at position half * 8 + e of its
// 16-chunk.  Column signs: the patch's 16 rows are one 16-chunk of every column.
template <int IN>
__device__ __forceinline__ uint32_t row_sign_mask(uint32_t signs, int half, int h) {
    const uint32_t s = signs >> (half * 8 + 2 * h);
    return Patch<IN>::pair_mask(s & 1u, (s >> 1) & 1u);
}
__device__ __forceinline__ uint32_t col_sign_mask(uint32_t signs, int i) {
    const uint32_t b = (signs >> i) & 1u;
    return (b << 15) | (b << 31);
}

template <int IN>
__device__ __forceinline__ void flip_signs(Patch<IN>& P, uint32_t signs, int half, bool rows,
                                           bool cols) {
    if constexpr (IN == 2) {   // one XOR per code word: the row signs' nibbles, then column i's
        const uint32_t rs = rows ? (signs >> (half * 8)) & 0xFFu : 0u;
        uint32_t rmask = 0u;
#pragma unroll
        for (int e = 0; e < 8; ++e) rmask |= ((rs >> e) & 1u) << (4 * e + 3);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t cm = cols ? ((signs >> i) & 1u) * 0x88888888u : 0u;
            P.p[i] ^= rmask ^ cm;
        }
        return;
    }
    uint32_t rm[4];
#pragma unroll
    for (int h = 0; h < 4; ++h) rm[h] = rows ? row_sign_mask<IN>(signs, half, h) : 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t cm = cols ? col_sign_mask(signs, i) : 0u;
#pragma unroll
        for (int h = 0; h < 4; ++h) P.flip(i, h, rm[h] ^ cm);
    }
}

// Largest magnitude of 8 (or 16) values, on the bit patterns (the values are |w|).
__device__ __forceinline__ float amax8(const float w[8]) {
    float m = 0.0f;
#pragma unroll
    for (int e = 0; e < 8; ++e) m = fmaxf(m, fabsf(w[e]));
    return m;
}
// max with lane ^ 1 for a non-negative value (integer order of the bit patterns)
__device__ __forceinline__ float pair_max(float v) {
    const uint32_t b = __float_as_uint(v);
    const uint32_t o = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)b, 0xB1, 0xF, 0xF, false);
    return __uint_as_float(max(b, o));
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

// Amax of one 16x8 patch for the rowwise and the columnwise copy (each plain or after its
// Hadamard transform).  The rowwise transform pairs this lane with lane ^ 1 (positions 8..15
// of the 16-chunk when this lane's column is a multiple of 16).  The factor 1/4 is applied
// to the maxima: x -> fl(x / 4) is monotone, so max fl(|w| / 4) = fl(max |w| / 4).
template <int IN, bool RHT_ROW, bool RHT_COL>
__device__ __forceinline__ void patch_amax(const QArgs& a, Patch<IN>& P, uint32_t signs,
                                           int half, float& mr, float& mc) {
    float plain = 0.0f, arow = 0.0f, acol = 0.0f;
    if ((a.rowwise && !RHT_ROW) || (a.colwise && !RHT_COL)) plain = P.amax();
    if (RHT_ROW) {
        flip_signs<IN>(P, signs, half, true, false);
        const float sgn = half ? -1.0f : 1.0f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            float w[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) w[e] = P.at(i, e);
            wht_pair8(w, sgn);
            arow = fmaxf(arow, amax8(w));
        }
        arow = arow * 0.25f;
    }
    if (RHT_COL) {
        flip_signs<IN>(P, signs, half, RHT_ROW, true);   // undo the row signs, apply the column signs
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            float w[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) w[i] = P.at(i, j);
            wht16(w);
            acol = fmaxf(acol, fmaxf(amax8(&w[0]), amax8(&w[8])));
        }
        acol = acol * 0.25f;
    }
    mr = fmaxf(mr, RHT_ROW ? arow : plain);
    mc = fmaxf(mc, RHT_COL ? acol : plain);
}

constexpr int kAmaxWaveCols = 512;   // columns of a k_amax wave tile (64 lanes x 8)

// Specialised on the input dtype and the Hadamard flags (bit 0: rowwise copy, bit 1:
// columnwise copy) so that each variant keeps its 16x8 patch in registers.
template <int IN, int H>
__global__ __launch_bounds__(kThreads) void k_amax(QArgs a) {
    constexpr bool RHT_ROW = H & 1, RHT_COL = (H >> 1) & 1;
    __shared__ float red[8];
    const int t = threadIdx.x, lane = t & 63, wid = t >> 6;
    const uint32_t signs =
        (RHT_ROW || RHT_COL) ? __builtin_amdgcn_readfirstlane(rht_sign_bits(a.k0, a.k1)) : 0u;
    const int64_t wcols = (a.cols + kAmaxWaveCols - 1) / kAmaxWaveCols;
    const int64_t nwt = (a.rows / 16) * wcols;
    float mr = 0.0f, mc = 0.0f;
    for (int64_t w = (int64_t)blockIdx.x * 4 + wid; w < nwt; w += (int64_t)gridDim.x * 4) {
        const int64_t r0 = (w / wcols) * 16;
        const int64_t c0 = (w % wcols) * kAmaxWaveCols + lane * 8;
        Patch<IN> P;
        load_patch(P, a, r0, c0, c0 < a.cols);
        patch_amax<IN, RHT_ROW, RHT_COL>(a, P, signs, lane & 1, mr, mc);
    }
    block_max2(mr, mc, red);
    if (t == 0) {
        a.partial[blockIdx.x] = mr;
        a.partial[a.npart + blockIdx.x] = mc;
    }
}

// Codes for 8 scaled values u (one dword), nearest-even: of u / cs, cs a power of two (1,
// or 2^-64 for the scaled values of a tiny copy; see CopyScale).
__device__ __forceinline__ uint32_t encode8_rne(const float u[8], float cs) {
    uint32_t r = 0;
    r = cvt_fp4x2<0>(r, u[0], u[1], cs);
    r = cvt_fp4x2<1>(r, u[2], u[3], cs);
    r = cvt_fp4x2<2>(r, u[4], u[5], cs);
    r = cvt_fp4x2<3>(r, u[6], u[7], cs);
    return r;
}

// Codes for 8 scaled values (one dword), stochastic (of u / cs, as encode8_rne), with the 4
// Philox words of their group: element 2b takes the low half of word b, element 2b + 1 the
// high half.  Each conversion leaves its code in byte 0 of its result; byte permutes gather
// the even codes into the bytes of one dword and the odd ones into another, which is
// shifted into the high nibbles.
__device__ __forceinline__ uint32_t encode8_sr(const float u[8], const U4& rw, float cs) {
    const uint32_t c0 = cvt_fp4_sr(u[0], rw.x << 16, cs);
    const uint32_t c1 = cvt_fp4_sr(u[1], rw.x & 0xFFFF0000u, cs);
    const uint32_t c2 = cvt_fp4_sr(u[2], rw.y << 16, cs);
    const uint32_t c3 = cvt_fp4_sr(u[3], rw.y & 0xFFFF0000u, cs);
    const uint32_t c4 = cvt_fp4_sr(u[4], rw.z << 16, cs);
    const uint32_t c5 = cvt_fp4_sr(u[5], rw.z & 0xFFFF0000u, cs);
    const uint32_t c6 = cvt_fp4_sr(u[6], rw.w << 16, cs);
    const uint32_t c7 = cvt_fp4_sr(u[7], rw.w & 0xFFFF0000u, cs);
    // selector bytes 0..3 pick bytes of the second operand, 4..7 of the first, 0x0C gives 0
    const uint32_t ev = __builtin_amdgcn_perm(c2, c0, 0x0C0C0400u) |
                        __builtin_amdgcn_perm(c6, c4, 0x04000C0Cu);
    const uint32_t od = __builtin_amdgcn_perm(c3, c1, 0x0C0C0400u) |
                        __builtin_amdgcn_perm(c7, c5, 0x04000C0Cu);
    return ev | (od << 4);
}

// 4/6 adaptive block scaling: squared error of 8 values w quantized nearest-even with block
// scale s (u: the values scaled by it), as the fma chain over the values in order of e_i^2,
// e_i = fma(-(v_i s), s_g, w_i) (v_i the signed decoded code; v_i s is exact).  Also returns
// the 8 codes.
__device__ __forceinline__ float sse8_rne(const float w[8], const float u[8], float s, float sg,
                                          float cs, uint32_t& codes) {
    codes = encode8_rne(u, cs);
    const float2v p[4] = {fp4x2_to_f32<0>(codes), fp4x2_to_f32<1>(codes), fp4x2_to_f32<2>(codes),
                          fp4x2_to_f32<3>(codes)};
    float acc = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float v = (i & 1) ? p[i >> 1].y : p[i >> 1].x;
        const float e = __builtin_fmaf(-(v * s), sg, w[i]);
        acc = __builtin_fmaf(e, e, acc);
    }
    return acc;
}

__device__ __forceinline__ float sg_from_amax(float amax) {
    float sg = __fdiv_rn(amax, 2688.0f);
    return sg == 0.0f ? 1.0f : sg;
}

constexpr float kRcp6 = 1.0f / 6.0f;     // RN(1/6)

// Block-scale arithmetic of one copy for one call.  The code of a block with amax am is
// E4M3(fl(fl(am / k) / s_g)) (k = 6, or 4 for the 4/6 candidate), its element reciprocal
// RN(1 / fl(E4M3 value * s_g)), both exactly as the definitions read:
//  * the two divisions go through div_rn_by when s_g >= 2^-92 (the tensor amax is at
//    least about 2^-80.6).  Then every block whose code can be nonzero has normal
//    operands and quotients, where the corrected division is exact; blocks with quotients
//    below 2^-12 get code 0 either way.  Smaller tensor scales take the plain divisions;
//  * the reciprocal of each of the 128 codes is computed once per workgroup into LDS;
//  * the reciprocal is kept at binary32 precision where its exponent leaves binary32's
//    range: when fl(s s_g) is below about 2^-128 (possible only when s_g < 2^-119), its
//    reciprocal R overflows.  For such a copy (`tiny`, uniform) the table holds
//    R 2^-64 = RN(1 / (fl(s s_g) 2^64)) for every code (the scalings are exact, and every
//    entry and every nonzero scaled element x R 2^-64 is then a normal number), and the
//    E2M1 conversions, which divide by the power of two given as their scale operand, take
//    2^-64: the code is that of fl(x (R 2^-64)) 2^64 = fl(x R).  Where R is finite this is
//    the binary32 product itself.
constexpr float kTinyShift = 0x1p64f;
struct CopyScale {
    float sg, rsg;
    bool fast;
    const float* rtab;
    float cs;   // scale operand of the E2M1 conversions: 1, or 2^-64 for a tiny copy
    __device__ __forceinline__ uint32_t code(float am, float k, float rk) const {
        float z;
        if (fast)
            z = div_rn_by(div_rn_by(am, k, rk), sg, rsg);
        else
            z = __fdiv_rn(__fdiv_rn(am, k), sg);
        return e4m3_encode(z);
    }
    __device__ __forceinline__ float rcp(uint32_t c) const { return rtab[c]; }
    // The scaled values of 8 elements of a block with scale code c (see above); rscale is
    // 1/4 where the rotation's factor is folded into the reciprocal (never in a tiny copy).
    __device__ __forceinline__ void scale8(const float w[8], uint32_t c, float rscale,
                                           float u[8]) const {
        const float r = rtab[c] * rscale;
#pragma unroll
        for (int e = 0; e < 8; ++e) u[e] = w[e] * r;
    }
};

// Whether the reciprocals of a copy with tensor scale sg leave binary32's range: that of
// the smallest nonzero block scale 2^-9, the largest, is infinite.
__device__ __forceinline__ bool tiny_scale(float sg) {
    return __builtin_isinf(__fdiv_rn(1.0f, 0x1p-9f * sg));
}
// The E2M1 conversions' scale operand for a copy (see CopyScale).
__device__ __forceinline__ float conv_scale(bool tiny) { return tiny ? 1.0f / kTinyShift : 1.0f; }
// Table entry for scale code c (0 for the zero scale).
__device__ __forceinline__ float recip_entry(uint32_t c, float sg, bool tiny) {
    const float d = e4m3_value(c) * sg;
    return c ? __fdiv_rn(1.0f, tiny ? d * kTinyShift : d) : 0.0f;
}

__device__ __forceinline__ float uniform_f(float v) {
    return __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(v)));
}

// Tile of workgroup b of n (a bijection of 0..n-1): XCD b mod 8 takes the contiguous run
// of tiles that ends where the next XCD's begins, visited from its end.
__device__ __forceinline__ int xcd_tile(int b, int n) {
    const int x = b & 7, k = b >> 3, q = n >> 3, rem = n & 7;
    const int start = x * q + min(x, rem), len = q + (x < rem ? 1 : 0);
    return start + len - 1 - k;
}

// Specialised on the input dtype and on F: bit 0 rowwise SR, bit 1 columnwise SR,
// bit 2 rowwise Hadamard, bit 3 columnwise Hadamard.  ROW1: the rowwise 1-D copy alone (no
// columnwise copy, 2-D blocks, 4/6 scaling or low-rank term), which leaves out their registers
// and LDS, so that more workgroups are resident.  PLAIN: no 2-D blocks, 4/6 scaling or
// low-rank term (either copy or both), for the same reason (X's row + column-RHT encode:
// 92 VGPRs and five waves per SIMD instead of 106 and four).
//
// The rowwise copy is encoded first, from the patch as loaded (with the row signs flipped in
// place when it is rotated); the patch is then flipped to the column signs and the
// columnwise copy encoded.  A rotated copy's factor 1/4 is folded into the block maximum and
// the element reciprocal (fl(|w'| / 4) = |w'| / 4 and fl(r / 4) = r / 4 exactly) when that is
// exact for every block whose codes can differ: no 4/6 scaling (its squared errors use the
// rotated values themselves) and 2^-92 <= s_g <= 2^110 (no reciprocal is then subnormal,
// and elements small enough to be rounded by the 1/4 quantize to 0 either way).
template <int IN, int F, bool ROW1 = false, bool PLAIN = ROW1>
__global__ __launch_bounds__(kThreads) void k_encode(QArgs a) {
    constexpr bool SR_ROW = F & 1, SR_COL = (F >> 1) & 1;
    constexpr bool RHT_ROW = (F >> 2) & 1, RHT_COL = (F >> 3) & 1;
    __shared__ uint2 ccodes_lds[kTileCols][16];           // [column][16-row slot], slot ^ (column/8)
    __shared__ uint8_t cscales_lds[kTileCols * 17];       // [column][slot], stride 17
    __shared__ float rtab[2][128];                        // element reciprocal per scale code
    __shared__ float red[8];
    const int t = threadIdx.x, pc = t & 15, pr = t >> 4;
    // Workgroups go to the 8 XCDs in turn (workgroup b to XCD b mod 8), each with its own L2.
    // XCD x is given one contiguous run of tiles (ceil or floor of n/8), so that the tiles of
    // one tile row, whose rowwise codes (64 of each 128 bytes) and scales (8 of each 128)
    // share cache lines, are written through one L2.  Within a run the tiles go in reverse
    // order: the first reads are of the rows the amax pass read last, the likeliest still to
    // be cached.
    const int tb = xcd_tile(blockIdx.x, gridDim.x);
    const int tile_r = tb / a.tiles_c, tile_c = tb % a.tiles_c;
    const int64_t r0 = (int64_t)tile_r * kTileRows + pr * 16;
    const int64_t c0 = (int64_t)tile_c * kTileCols + pc * 8;
    const bool valid = r0 < a.rows && c0 < a.cols;
    const int half = pc & 1;

    Patch<IN> P;
    float mr, mc;
    // A rowwise NVFP4 input has a 32-VGPR patch, so its columnwise SR words (64 VGPRs) can be
    // formed up front, overlapping the Philox chains with the load latency; the bf16 and f32
    // patches leave no room for them.
    constexpr bool kEarlyDraws = IN == 2 && SR_COL;
    U4 cdraw[kEarlyDraws ? 8 : 1][2];
    if constexpr (!RHT_ROW) {
        // A first round of the partial maxima (up to 768 per copy, three per thread) is loaded
        // before the patch: vector loads complete in issue order, so the wait for these leaves
        // the patch loads in flight, and the rowwise encode below can start on the first rows
        // of the patch while the later ones are still arriving.
        float pmr[3], pmc[3];
#pragma unroll
        for (int u = 0; u < 3; ++u) {
            const int i = min(t + kThreads * u, a.npart - 1);
            pmr[u] = a.partial[i];
            pmc[u] = a.partial[a.cpart + i];
        }
        // A lane past the tensor's edge (whole 16-row groups and 8-column halves of whole
        // 16-column blocks, so its pair and its column blocks are past it too) encodes the
        // tensor's first patch and stores nothing.  Its loads are not skipped: a branch around
        // them would make the compiler wait for all of them before the first use of the
        // partials.
        load_patch(P, a, valid ? r0 : 0, valid ? c0 : 0, true);
        if constexpr (kEarlyDraws) {
            // the columnwise SR words of all 8 columns, formed while the loads are in flight
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const uint64_t gd = ((uint64_t)(c0 + j) * (uint64_t)a.rows + (uint64_t)r0) >> 3;
                cdraw[j][0] = sr_words(gd, 1u, a.k0, a.k1);
                cdraw[j][1] = sr_words(gd + 1, 1u, a.k0, a.k1);
                asm volatile("" : "+v"(cdraw[j][0].x), "+v"(cdraw[j][0].y), "+v"(cdraw[j][0].z),
                             "+v"(cdraw[j][0].w), "+v"(cdraw[j][1].x), "+v"(cdraw[j][1].y),
                             "+v"(cdraw[j][1].z), "+v"(cdraw[j][1].w));
            }
        }
        // tensor scales from the per-tile partial maxima: the first round loaded above
        // (indices past the last partial read the last one again, which leaves the maximum
        // unchanged), then any beyond 768 (the LoRA first pass can have more workgroups)
        mr = fmaxf(fmaxf(pmr[0], pmr[1]), pmr[2]);
        mc = fmaxf(fmaxf(pmc[0], pmc[1]), pmc[2]);
        for (int i = t + 3 * kThreads; i < a.npart; i += kThreads) {
            mr = fmaxf(mr, a.partial[i]);
            mc = fmaxf(mc, a.partial[a.cpart + i]);
        }
    } else {
        // With the rowwise rotation the whole patch is sign-flipped before the first row is
        // encoded, so nothing starts before the last patch load: the patch goes first and the
        // partials (four loads per copy issued together) after it, the order that needs the
        // fewest registers here.  A lane past the edge loads nothing and stores nothing.
        load_patch(P, a, r0, c0, valid);
        mr = 0.0f;
        mc = 0.0f;
        for (int i0 = t; i0 < a.npart; i0 += 4 * kThreads) {
            float pr[4], pc[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const int i = i0 + u * kThreads;
                pr[u] = i < a.npart ? a.partial[i] : 0.0f;
                pc[u] = i < a.npart ? a.partial[a.cpart + i] : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) { mr = fmaxf(mr, pr[u]); mc = fmaxf(mc, pc[u]); }
        }
    }
    block_max2(mr, mc, red);
    const float sg_r = uniform_f(sg_from_amax(mr)), sg_c = uniform_f(sg_from_amax(mc));
    if (blockIdx.x == 0 && t == 0) {
        if (a.rowwise) *a.rsg = sg_r;
        if ((!ROW1 && a.colwise)) *a.csg = sg_c;
    }
    const bool tiny_r = tiny_scale(sg_r), tiny_c = tiny_scale(sg_c);
    if (t < 128) {
        rtab[0][t] = recip_entry(t, sg_r, tiny_r);
        rtab[1][t] = recip_entry(t, sg_c, tiny_c);
    }
    __syncthreads();
    const CopyScale rsc{sg_r, __fdiv_rn(1.0f, sg_r), sg_r >= 0x1p-92f, rtab[0], conv_scale(tiny_r)};
    const CopyScale csc{sg_c, __fdiv_rn(1.0f, sg_c), sg_c >= 0x1p-92f, rtab[1], conv_scale(tiny_c)};
    const bool fold_r = RHT_ROW && !(!PLAIN && a.scale46) && sg_r >= 0x1p-92f && sg_r <= 0x1p110f;
    const bool fold_c = RHT_COL && !(!PLAIN && a.scale46) && sg_c >= 0x1p-92f && sg_c <= 0x1p110f;
    const uint32_t signs =
        (RHT_ROW || RHT_COL) ? __builtin_amdgcn_readfirstlane(rht_sign_bits(a.k0, a.k1)) : 0u;

    // LoRA-SVD down-projection: T = BF16(beta * sum of the K-part partials, in part order)
    // (after the tensor scales, so that this uniform branch does not stand between the
    // loads above and their first use)
    if ((!PLAIN && a.lora_t)) {
        const int64_t total = a.rows * a.lora_r;
        for (int64_t e = (int64_t)blockIdx.x * kThreads + t; e < total;
             e += (int64_t)gridDim.x * kThreads) {
            float sum = 0.0f;
            for (int q = 0; q < a.lora_parts; ++q) sum += a.lora_part[q * total + e];
            a.lora_t[e] = (uint16_t)f32_to_bf16_rne(sum * a.lora_beta);
        }
    }

    // A rowwise NVFP4 input (IN == 2) asks for the columnwise 1-D copy alone.
    constexpr bool kRowsOrTiles = IN != 2;
    uint32_t scode2d = 0;
    if (kRowsOrTiles && (!PLAIN && a.block2d)) {  // one scale per 16x16 tile = this patch and its neighbour's
        scode2d = rsc.code(pair_max(P.amax()), 6.0f, kRcp6);
    }

    if (kRowsOrTiles && a.rowwise) {
        if (RHT_ROW) flip_signs<IN>(P, signs, half, true, false);
        const float sgn = half ? -1.0f : 1.0f;
        const int64_t rpitch = a.cols / 2, spitch = a.cols / 16;
        uint8_t* const cbase = a.rcodes + r0 * rpitch + c0 / 2;
        uint8_t* const sbase = a.rscales + r0 * spitch + c0 / 16;
        static_for<0, 16>([&](auto I) {
            constexpr int i = decltype(I)::value;
            float w[8];
#pragma unroll
            for (int e = 0; e < 8; ++e) w[e] = P.at(i, e);
            if (RHT_ROW) {
                wht_pair8(w, sgn);
                if (!fold_r) {
#pragma unroll
                    for (int e = 0; e < 8; ++e) w[e] = w[e] * 0.25f;
                }
            }
            uint32_t scode, rcodes = 0;
            bool have = false;   // nearest-even codes already formed by the 4/6 choice
            float rscale = 1.0f; // 1/4 when the rotation's factor is folded in
            if ((!PLAIN && a.block2d)) {
                scode = scode2d;
            } else {
                float am = pair_max(amax8(w));
                if (RHT_ROW && fold_r) { am = am * 0.25f; rscale = 0.25f; }
                scode = rsc.code(am, 6.0f, kRcp6);
                if ((!PLAIN && a.scale46)) {
                    // the block's halves sit in this lane and lane ^ 1; a + b == b + a, so
                    // both lanes form the same (elements 0..7) + (elements 8..15) sum
                    const uint32_t sc4 = rsc.code(am, 4.0f, 0.25f);
                    uint32_t c6, c4;
                    float u[8];
                    rsc.scale8(w, scode, 1.0f, u);
                    float e6 = sse8_rne(w, u, e4m3_value(scode), sg_r, rsc.cs, c6);
                    rsc.scale8(w, sc4, 1.0f, u);
                    float e4 = sse8_rne(w, u, e4m3_value(sc4), sg_r, rsc.cs, c4);
                    e6 += xor1(e6);
                    e4 += xor1(e4);
                    const bool use4 = e4 < e6;
                    scode = use4 ? sc4 : scode;
                    rcodes = use4 ? c4 : c6;
                    have = true;
                }
            }
            uint32_t codes;
            if (SR_ROW) {
                const uint64_t g = ((uint64_t)(r0 + i) * (uint64_t)a.cols + (uint64_t)c0) >> 3;
                const U4 rw = sr_words(g, 0u, a.k0, a.k1);
                float u[8];
                rsc.scale8(w, scode, rscale, u);
                codes = encode8_sr(u, rw, rsc.cs);
            } else if (!have) {
                float u[8];
                rsc.scale8(w, scode, rscale, u);
                codes = encode8_rne(u, rsc.cs);
            } else {
                codes = rcodes;
            }
            if (valid) {
                *(uint32_t*)(cbase + i * rpitch) = codes;
                if (half == 0) sbase[i * spitch] = (uint8_t)scode;
            }
        });
    }

    if ((!ROW1 && a.colwise)) {
        // from the loaded (or row-flipped) signs to the column signs
        if (RHT_COL || RHT_ROW) flip_signs<IN>(P, signs, half, RHT_ROW, RHT_COL);
        static_for<0, 8>([&](auto J) {
            constexpr int j = decltype(J)::value;
            float w[16];
#pragma unroll
            for (int i = 0; i < 16; ++i) w[i] = P.at(i, j);
            if (RHT_COL) {
                wht16(w);
                if (!fold_c) {
#pragma unroll
                    for (int i = 0; i < 16; ++i) w[i] = w[i] * 0.25f;
                }
            }
            uint32_t scode, rlo = 0, rhi = 0;
            bool have = false;   // nearest-even codes already formed by the 4/6 choice
            float rscale = 1.0f;
            if ((!PLAIN && a.block2d)) {
                scode = scode2d;
            } else {
                float am = fmaxf(amax8(&w[0]), amax8(&w[8]));
                if (RHT_COL && fold_c) { am = am * 0.25f; rscale = 0.25f; }
                scode = csc.code(am, 6.0f, kRcp6);
                if ((!PLAIN && a.scale46)) {
                    const uint32_t sc4 = csc.code(am, 4.0f, 0.25f);
                    const float s6 = e4m3_value(scode), s4 = e4m3_value(sc4);
                    uint32_t l6, h6, l4, h4;
                    float u[8];
                    csc.scale8(&w[0], scode, 1.0f, u);
                    float e6 = sse8_rne(&w[0], u, s6, sg_c, csc.cs, l6);
                    csc.scale8(&w[8], scode, 1.0f, u);
                    e6 = e6 + sse8_rne(&w[8], u, s6, sg_c, csc.cs, h6);
                    csc.scale8(&w[0], sc4, 1.0f, u);
                    float e4 = sse8_rne(&w[0], u, s4, sg_c, csc.cs, l4);
                    csc.scale8(&w[8], sc4, 1.0f, u);
                    e4 = e4 + sse8_rne(&w[8], u, s4, sg_c, csc.cs, h4);
                    const bool use4 = e4 < e6;
                    scode = use4 ? sc4 : scode;
                    rlo = use4 ? l4 : l6;
                    rhi = use4 ? h4 : h6;
                    have = true;
                }
            }
            uint32_t lo, hi;
            if (SR_COL) {
                float u[8];
                U4 rlo_w, rhi_w;
                if constexpr (kEarlyDraws) {
                    rlo_w = cdraw[j][0];
                    rhi_w = cdraw[j][1];
                } else {
                    const uint64_t g = ((uint64_t)(c0 + j) * (uint64_t)a.rows + (uint64_t)r0) >> 3;
                    rlo_w = sr_words(g, 1u, a.k0, a.k1);
                    rhi_w = sr_words(g + 1, 1u, a.k0, a.k1);
                }
                csc.scale8(&w[0], scode, rscale, u);
                lo = encode8_sr(u, rlo_w, csc.cs);
                csc.scale8(&w[8], scode, rscale, u);
                hi = encode8_sr(u, rhi_w, csc.cs);
            } else if (!have) {
                float u[8];
                csc.scale8(&w[0], scode, rscale, u);
                lo = encode8_rne(u, csc.cs);
                csc.scale8(&w[8], scode, rscale, u);
                hi = encode8_rne(u, csc.cs);
            } else {
                lo = rlo;
                hi = rhi;
            }
            const int cl = pc * 8 + j;
            ccodes_lds[cl][pr ^ pc] = make_uint2(lo, hi);
            cscales_lds[cl * 17 + pr] = (uint8_t)scode;
        });
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


// ---------------------------------------------------------------- LoRA-SVD first pass
// The quantizer's first pass with the LoRA-SVD down-projection fused in (Full-Stack FP4
// sec. 3.2 eq. (1) and Appendix 9: the down-projection X L1^T reuses the quantizer's input
// read).  Work decomposition: a workgroup takes 64 rows (16 per wave) and one K-part of
// lora_kp columns, in steps of 128 columns; about two workgroups per CU.
// Staging: each step's 64 x 128 input tile and its slice of a (rank x 128) go into one of
// two LDS stages by direct global -> LDS loads, issued one step ahead and waited for
// explicitly, so neither passes through registers and no step waits for loads issued in
// the same step.  (Three stages at one workgroup per CU measured within noise of this;
// four were slower.)  Both are stored as 16-byte chunks, chunk c of row r at r * 16 +
// (c ^ (r mod 16)), which keeps every read below on distinct banks.  Lane (i, g) of a wave
// (i = lane mod 16, g = lane / 16) reads
//  * the 32 consecutive bfloat16 of its row i at columns 32g .. 32g + 31 (four chunks): the
//    A operands of four BF16 MFMAs 16x16x32 (k-step j takes columns 32g + 8j .. +7 as the
//    MFMA's k-slots 8g .. 8g + 7, and the B operands from the slice of a follow the same
//    correspondence, so every column is summed exactly once), and the input of the plain
//    and row-rotated maxima;
//  * rows 0..15 of columns 2 lane and 2 lane + 1 of the wave's 16 x 128 block, for the
//    column rotation.
// The low-rank partial of each K-part goes to lora_part; k_encode sums the parts in order.
constexpr int kLoraStep = 128;
constexpr int kLoraRowsWG = 64;
constexpr int kLoraMaxRank = 64;
constexpr int kLoraStages = 2;
constexpr int kLoraXBytes = kLoraRowsWG * kLoraStep * 2;   // one stage's input tile
typedef __bf16 bf16x8t __attribute__((ext_vector_type(8)));
typedef float f32x4t __attribute__((ext_vector_type(4)));

// One stage: the input tile, then the slice of a (NQ 16-row blocks).
__host__ __device__ constexpr int lora_stage_bytes(int nq) { return kLoraXBytes + nq * 16 * kLoraStep * 2; }

// Direct loads of the step at column c into the stage at LDS address base: slot p =
// 256 k + t of each part receives the global chunk that the layout above puts there.  Input
// rows past the workgroup's valid rows read zeros (offset past the buffer's end).
template <int NQ>
__device__ __forceinline__ void lora_dma(const QArgs& a, int4v rx, int4v ra, uint32_t base, int64_t c,
                                         int t, int wid, int64_t rows_here) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int p = k * kThreads + t, r = p >> 4, ch = (p & 15) ^ (r & 15);
        const uint32_t off = r < rows_here ? (uint32_t)(((int64_t)r * a.ld + c + ch * 8) * 2) : kOutOfRange;
        dma16(rx, base + (uint32_t)(k * kThreads + wid * 64) * 16, off);
    }
#pragma unroll
    for (int k = 0; k < NQ; ++k) {
        const int p = k * kThreads + t, rr = p >> 4, ch = (p & 15) ^ (rr & 15);
        const uint32_t off = (uint32_t)(((int64_t)rr * a.cols + c + ch * 8) * 2);
        dma16(ra, base + kLoraXBytes + (uint32_t)(k * kThreads + wid * 64) * 16, off);
    }
}

// Wait until at most AHEAD stages of this wave's direct loads are outstanding (they complete
// in issue order), then meet the other waves: after it the awaited stage is in LDS and every
// wave is done with the stage about to be refilled.
template <int NQ, int AHEAD>
__device__ __forceinline__ void lora_wait_meet() {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(AHEAD * (4 + NQ)) : "memory");
}

// The partial maxima of one step from the wave's 16 x 128 block wx in LDS; xv holds this
// lane's four chunks of it (see k_amax_lora).
template <int H>
__device__ __forceinline__ void lora_step_amax(const QArgs& a, const uint4 (&xv)[4], uint32_t signs,
                                               const uint4* wx, int lane, float& mr, float& mc) {
    constexpr bool RHT_ROW = H & 1, RHT_COL = (H >> 1) & 1;
    uint32_t xw[16];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        xw[4 * q] = xv[q].x; xw[4 * q + 1] = xv[q].y; xw[4 * q + 2] = xv[q].z; xw[4 * q + 3] = xv[q].w;
    }
    if ((a.rowwise && !RHT_ROW) || (a.colwise && !RHT_COL)) {
        typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
        u16x2 m = {0, 0};
#pragma unroll
        for (int q = 0; q < 16; ++q)
            m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, xw[q] & 0x7FFF7FFFu));
        const float pm = fmaxf(__uint_as_float((uint32_t)m.x << 16), __uint_as_float((uint32_t)m.y << 16));
        if (!RHT_ROW) mr = fmaxf(mr, pm);
        if (!RHT_COL) mc = fmaxf(mc, pm);
    }
    if (RHT_ROW) {
#pragma unroll
        for (int hf = 0; hf < 2; ++hf) {
            float w[16];
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const uint32_t d = xw[8 * hf + e / 2];
                w[e] = apply_sign(__uint_as_float((e & 1) ? (d & 0xFFFF0000u) : (d << 16)), signs, e);
            }
            wht16(w);
            mr = fmaxf(mr, fmaxf(amax8(&w[0]), amax8(&w[8])));
        }
    }
    if (RHT_COL) {
        // rows 0..15 of columns 2 lane, 2 lane + 1: dword lane of each row, whose chunk
        // lane / 4 sits at position (lane / 4) ^ r
        const uint32_t* w32 = (const uint32_t*)wx;
        float w0[16], w1[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            const uint32_t d = w32[r * 64 + ((((lane >> 2) ^ r) & 15) << 2) + (lane & 3)] ^
                               col_sign_mask(signs, r);
            w0[r] = __uint_as_float(d << 16);
            w1[r] = __uint_as_float(d & 0xFFFF0000u);
        }
        wht16(w0);
        wht16(w1);
        mc = fmaxf(mc, fmaxf(fmaxf(amax8(&w0[0]), amax8(&w0[8])), fmaxf(amax8(&w1[0]), amax8(&w1[8]))));
    }
}

template <int NQ>
__device__ __forceinline__ void lora_step_mma(const uint4 (&xv)[4], const uint4* bl, int i, int g,
                                              f32x4t (&acc)[NQ]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const bf16x8t av = __builtin_bit_cast(bf16x8t, xv[j]);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int rr = 16 * q + i;
            const bf16x8t bv = __builtin_bit_cast(bf16x8t, bl[rr * 16 + ((4 * g + j) ^ (rr & 15))]);
            acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, acc[q], 0, 0, 0);
        }
    }
}

template <int H, int NQ>
__global__ __launch_bounds__(kThreads, 1) void k_amax_lora(QArgs a) {
    constexpr bool RHT_ROW = H & 1, RHT_COL = (H >> 1) & 1;
    constexpr int kStage = lora_stage_bytes(NQ);
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    __shared__ float red[8];
    const int t = threadIdx.x, lane = t & 63;
    const int wid = __builtin_amdgcn_readfirstlane(t >> 6);
    const int i = lane & 15, g = lane >> 4;
    const int rblk = blockIdx.x / a.lora_parts, part = blockIdx.x % a.lora_parts;
    const int64_t row0 = (int64_t)rblk * kLoraRowsWG;
    const int64_t rows_here = a.rows - row0 < kLoraRowsWG ? a.rows - row0 : kLoraRowsWG;
    const int64_t kb = (int64_t)part * a.lora_kp;
    const int64_t ke = kb + a.lora_kp < a.cols ? kb + a.lora_kp : a.cols;
    const int nsteps = (int)((ke - kb) / kLoraStep);
    const uint32_t signs =
        (RHT_ROW || RHT_COL) ? __builtin_amdgcn_readfirstlane(rht_sign_bits(a.k0, a.k1)) : 0u;
    const int4v rx = make_rsrc((const uint16_t*)a.x + row0 * a.ld, (uint32_t)(rows_here * a.ld * 2));
    const int4v ra = make_rsrc(a.lora_a, (uint32_t)(a.lora_r * a.cols * 2));
    const uint32_t lds0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)lds;

    f32x4t acc[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) acc[q] = f32x4t{0.0f, 0.0f, 0.0f, 0.0f};
    float mr = 0.0f, mc = 0.0f;

    constexpr int kAhead = kLoraStages - 1;   // steps whose loads are in flight ahead
    for (int j = 0; j < kAhead && j < nsteps; ++j)
        lora_dma<NQ>(a, rx, ra, lds0 + j * kStage, kb + j * kLoraStep, t, wid, rows_here);
    for (int s = 0; s < nsteps; ++s) {
        const int later = nsteps - 1 - s < kAhead - 1 ? nsteps - 1 - s : kAhead - 1;
        if (later >= 2) lora_wait_meet<NQ, 2>();
        else if (later == 1) lora_wait_meet<NQ, 1>();
        else lora_wait_meet<NQ, 0>();
        // every wave is done with step s - 1, whose stage the loads of step s + kAhead refill
        if (s + kAhead < nsteps)
            lora_dma<NQ>(a, rx, ra, lds0 + ((s + kAhead) % kLoraStages) * kStage,
                         kb + (int64_t)(s + kAhead) * kLoraStep, t, wid, rows_here);
        const uint4* xs = (const uint4*)(lds + (s % kLoraStages) * kStage);
        const uint4* wx = xs + wid * 16 * 16;   // the wave's 16 rows
        uint4 xv[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) xv[q] = wx[i * 16 + ((4 * g + q) ^ i)];
        lora_step_amax<H>(a, xv, signs, wx, lane, mr, mc);
        lora_step_mma<NQ>(xv, xs + kLoraXBytes / 16, i, g, acc);
    }
    if (RHT_ROW) mr = mr * 0.25f;
    if (RHT_COL) mc = mc * 0.25f;

    // the K-part's partial of T: lane holds rows 4g .. 4g + 3 of column 16q + i of block q
    const int64_t total = a.rows * a.lora_r;
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t r = row0 + wid * 16 + 4 * g + v;
            if (r < a.rows) a.lora_part[part * total + r * a.lora_r + 16 * q + i] = acc[q][v];
        }
    }
    block_max2(mr, mc, red);
    if (t == 0) {
        a.partial[blockIdx.x] = mr;
        a.partial[a.npart + blockIdx.x] = mc;
    }
}

template <int H, int NQ>
void launch_amax_lora_nq(const QArgs& a, hipStream_t st) {
    constexpr int bytes = kLoraStages * lora_stage_bytes(NQ);
    static_assert(bytes <= 160 * 1024 - 64, "LDS budget");
    (void)hipFuncSetAttribute((const void*)k_amax_lora<H, NQ>, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    k_amax_lora<H, NQ><<<a.npart, kThreads, bytes, st>>>(a);
}

template <int H>
void launch_amax_lora(const QArgs& a, hipStream_t st) {
    switch (a.lora_r / 16) {
    case 1: launch_amax_lora_nq<H, 1>(a, st); break;
    case 2: launch_amax_lora_nq<H, 2>(a, st); break;
    case 3: launch_amax_lora_nq<H, 3>(a, st); break;
    default: launch_amax_lora_nq<H, 4>(a, st); break;
    }
}

template <int IN, int F>
void launch_quant(const QArgs& a, hipStream_t st) {
    if constexpr (IN == 1) {
        if (a.lora_t) launch_amax_lora<(F >> 2)>(a, st);
        else if (!a.amax_given) k_amax<IN, (F >> 2)><<<a.npart, kThreads, 0, st>>>(a);
    } else {
        if (!a.amax_given) k_amax<IN, (F >> 2)><<<a.npart, kThreads, 0, st>>>(a);
    }
    if constexpr ((F & 10) == 0) {   // no columnwise option bits: a rowwise-only variant
        if (a.rowwise && !a.colwise && !a.block2d && !a.scale46 && !a.lora_t) {
            k_encode<IN, F, true><<<a.ntiles, kThreads, 0, st>>>(a);
            return;
        }
    }
    if constexpr (IN != 2) {
        if (!a.block2d && !a.scale46 && !a.lora_t) {
            k_encode<IN, F, false, true><<<a.ntiles, kThreads, 0, st>>>(a);
            return;
        }
    }
    k_encode<IN, F><<<a.ntiles, kThreads, 0, st>>>(a);
}

// Each launch unit covers one dtype and half of the 16 option combinations.
void launch_quant_bf16_lo(int f, const QArgs& a, hipStream_t st);
void launch_quant_bf16_hi(int f, const QArgs& a, hipStream_t st);
void launch_quant_f32_lo(int f, const QArgs& a, hipStream_t st);
void launch_quant_f32_hi(int f, const QArgs& a, hipStream_t st);
void launch_requant_cols(int f, const QArgs& a, hipStream_t st);

}  // namespace nvfp4
