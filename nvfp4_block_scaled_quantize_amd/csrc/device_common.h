// device_common.h -- gfx950 device helpers shared by the NVFP4 kernels.
//
// Format conventions (the pages' NVFP4: Full-Stack FP4 sec. 2; NVFP4 report sec. 2):
//   E2M1 nibble  = sign<<3 | exponent<<1 | mantissa, exponent bias 1
//   E4M3 scale   = OCP "fn" FP8, bias 7, largest finite 448 (0x7E)
//   tensor scale = binary32
// Random bits come from Philox4x32-10 (Salmon et al., SC'11) keyed by the call's
// seed; the counter layout is
//   stochastic rounding, element j of copy c:  (lo32(j/8), hi32(j/8), c, 0x53523136)
//       16 bits = half (j mod 2) of output word ((j/2) mod 4)
//   Hadamard signs:                            (0, 0, 0, 0x52485431), bit i of word 0
//       set means the i-th diagonal entry is -1.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

namespace nvfp4 {

constexpr uint32_t kTagSR = 0x53523136u;
constexpr uint32_t kTagRHT = 0x52485431u;

typedef float float2v __attribute__((ext_vector_type(2)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef _Float16 half8v __attribute__((ext_vector_type(8)));
typedef float float16v __attribute__((ext_vector_type(16)));

// ---------------------------------------------------------------- Philox4x32-10
struct U4 { uint32_t x, y, z, w; };

__device__ __forceinline__ U4 philox10(U4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
        U4 n;
        n.x = (uint32_t)(p1 >> 32) ^ c.y ^ k0;
        n.y = (uint32_t)p1;
        n.z = (uint32_t)(p0 >> 32) ^ c.w ^ k1;
        n.w = (uint32_t)p0;
        c = n;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    return c;
}

// The four output words of the SR draw covering elements 8g .. 8g+7 of copy `copy`.
__device__ __forceinline__ U4 sr_words(uint64_t g, uint32_t copy, uint32_t k0, uint32_t k1) {
    U4 c = {(uint32_t)g, (uint32_t)(g >> 32), copy, kTagSR};
    return philox10(c, k0, k1);
}

__device__ __forceinline__ uint32_t word_of(const U4& w, int i) {
    return i == 0 ? w.x : (i == 1 ? w.y : (i == 2 ? w.z : w.w));
}

// 16 sign bits of the random Hadamard diagonal (bit i set -> -1).
__device__ __forceinline__ uint32_t rht_sign_bits(uint32_t k0, uint32_t k1) {
    U4 c = {0u, 0u, 0u, kTagRHT};
    return philox10(c, k0, k1).x & 0xFFFFu;
}

__device__ __forceinline__ float apply_sign(float v, uint32_t bits, int i) {
    return __uint_as_float(__float_as_uint(v) ^ (((bits >> i) & 1u) << 31));
}

// ---------------------------------------------------------------- E4M3 block scale
// Nearest-even with saturation at 448 for s >= 0.
__device__ __forceinline__ uint32_t e4m3_encode(float s) {
    if (s >= 448.0f) return 0x7Eu;
    if (!(s == s)) return 0u;
    if (s < 0.015625f) {                       // below 2^-6: subnormal step 2^-9
        return (uint32_t)rintf(s * 512.0f);   // exact scaling, nearest-even; 8 = 2^-6
    }
    uint32_t b = __float_as_uint(s);
    b = b + 0x7FFFFu + ((b >> 20) & 1u);      // round the mantissa to 3 bits, ties to even
    return (b >> 20) - 960u;                   // rebias exponent 127 -> 7
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
    uint32_t e = (c >> 3) & 15u, m = c & 7u;
    if (e == 0) return (float)m * 0.001953125f;
    return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// ---------------------------------------------------------------- E2M1 element
// Two binary32 values -> two E2M1 codes (nearest-even, saturating at 6, sign copied),
// written into byte `sel` of `old`.  The hardware conversion at scale 1.0 equals that
// rounding for every finite binary32 input (checked exhaustively on gfx950).
template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4x2(uint32_t old, float a, float b) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, SEL);
}

// Stochastic rounding of a magnitude u >= 0 with 16 random bits: up iff
// frac + r/2^16 >= 1, where frac = (u - c_k) / Delta_k.  Every step is exact.
__device__ __forceinline__ uint32_t sr_mag(float u, uint32_t r16) {
    if (!(u < 6.0f)) return 7u;
    uint32_t k = (uint32_t)(u >= 0.5f) + (uint32_t)(u >= 1.0f) + (uint32_t)(u >= 1.5f) +
                 (uint32_t)(u >= 2.0f) + (uint32_t)(u >= 3.0f) + (uint32_t)(u >= 4.0f);
    float lo = k < 4 ? 0.5f * (float)k : (k == 4 ? 2.0f : (k == 5 ? 3.0f : 4.0f));
    float inv_delta = k < 4 ? 2.0f : (k < 6 ? 1.0f : 0.5f);
    float frac = (u - lo) * inv_delta;
    float need = 1.0f - (float)r16 * (1.0f / 65536.0f);
    return k + (frac >= need ? 1u : 0u);
}

__device__ __forceinline__ uint32_t sr_code(float x, float rcp, uint32_t r16) {
    float u = fabsf(x) * rcp;
    return ((__float_as_uint(x) >> 28) & 8u) | sr_mag(u, r16);
}

// Decode the two E2M1 codes in byte SEL of w to binary32 (exact).
template <int SEL>
__device__ __forceinline__ float2v fp4x2_to_f32(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}
template <int SEL>
__device__ __forceinline__ half2v fp4x2_to_f16(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, SEL);
}

// ---------------------------------------------------------------- misc
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float(bits16 << 16);
}

// bfloat16 nearest-even of a finite binary32 value.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t b = __float_as_uint(f);
    return (b + 0x7FFFu + ((b >> 16) & 1u)) >> 16;
}

// In-register 16-point butterfly, stages h = 1, 2, 4, 8; pair (i, i+h) with bit h of i
// clear becomes (a + b, a - b).  Equals H16 * v in Sylvester order.
__device__ __forceinline__ void wht16(float v[16]) {
#pragma unroll
    for (int h = 1; h < 16; h <<= 1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if ((i & h) == 0) {
                float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
        }
    }
}

// Compile-time loop: f(std::integral_constant<int, I>) for I = B .. E-1, so array
// indices inside f are constants whatever the unroller decides.
template <int B, int E, typename Fn>
__device__ __forceinline__ void static_for(Fn&& f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

}  // namespace nvfp4
