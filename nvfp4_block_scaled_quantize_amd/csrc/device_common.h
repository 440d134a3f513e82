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

// VEC: per-lane counters, the three-way exclusive ors as one v_bitop3_b32 each (truth table
// 0x96).  Otherwise plain exclusive ors, which the compiler keeps on the scalar unit when the
// counter and key are uniform (v_bitop3_b32 is a vector instruction).
template <bool VEC = true>
__device__ __forceinline__ U4 philox10(U4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        uint64_t p0 = (uint64_t)0xD2511F53u * c.x;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c.z;
        U4 n;
        if constexpr (VEC) {
            n.x = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c.y, k0, 0x96);
            n.z = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c.w, k1, 0x96);
        } else {
            n.x = (uint32_t)(p1 >> 32) ^ c.y ^ k0;
            n.z = (uint32_t)(p0 >> 32) ^ c.w ^ k1;
        }
        n.y = (uint32_t)p1;
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

// 16 sign bits of the random Hadamard diagonal (bit i set -> -1).
__device__ __forceinline__ uint32_t rht_sign_bits(uint32_t k0, uint32_t k1) {
    U4 c = {0u, 0u, 0u, kTagRHT};
    return philox10<false>(c, k0, k1).x & 0xFFFFu;
}

__device__ __forceinline__ float apply_sign(float v, uint32_t bits, int i) {
    return __uint_as_float(__float_as_uint(v) ^ (((bits >> i) & 1u) << 31));
}

// ---------------------------------------------------------------- E4M3 block scale
// Nearest-even E4M3 code with saturation at 448 for finite s >= 0: gfx950's OCP FP8
// conversion of min(s, 448).  It equals nearest-even rounding to the E4M3 "fn" grid for
// every non-negative finite binary32 (an exhaustive GPU test compares it with a plain
// search over the grid).
__device__ __forceinline__ uint32_t e4m3_encode(float s) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(s, 448.0f), 0.0f, 0, false) & 0xFFu;
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
    uint32_t e = (c >> 3) & 15u, m = c & 7u;
    if (e == 0) return (float)m * 0.001953125f;
    return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// ---------------------------------------------------------------- E2M1 element
// Two binary32 values -> two E2M1 codes (nearest-even, saturating at 6, sign copied) of
// a / cs and b / cs, written into byte `sel` of `old`.  The scale operand cs is a power of
// two (the conversion uses only its exponent); the division by it is exact.  At cs = 1 the
// hardware conversion equals that rounding for every finite binary32 input, and at
// cs = 2^-64 it equals the conversion of a 2^64 at cs = 1 wherever that is finite (both
// checked exhaustively on gfx950).
template <int SEL>
__device__ __forceinline__ uint32_t cvt_fp4x2(uint32_t old, float a, float b, float cs = 1.0f) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, cs, SEL);
}

// Stochastic rounding of one value v = x * rcp to an E2M1 code with 16 random bits r16: the
// magnitude |v| goes to its upper grid neighbour iff floor(frac * 2^16) + r16 >= 2^16, frac
// being its position between its two grid neighbours (saturating at 6, sign copied).
// gfx950's v_cvt_scalef32_sr_pk_fp4_f32 rounds the first value of its pair by adding bits
// 10..31 of its seed to the 22 leading bits of that fraction and keeping the carry, in the
// subnormal range (|v| < 1, spacing 1/2) as in the normal one.  With seed = r16 << 16 the
// six low added bits are zero, so the carry is the rule's exactly.  The second value of the
// pair is 0.0, whose code is 0 for every seed.  Only byte 0 of the result is defined (code in
// bits 0..3, bits 4..7 zero): the compiler does not carry the builtin's first operand into
// the bytes the instruction leaves alone.  (A GPU test compares the conversion with the
// plain rule for every finite binary32 value.)
// cs: the power-of-two scale operand, as for cvt_fp4x2 (v / cs is rounded; checked against
// v 2^64 at cs = 1 for cs = 2^-64).
__device__ __forceinline__ uint32_t cvt_fp4_sr(float v, uint32_t seed, float cs = 1.0f) {
    const float2v p = {v, 0.0f};
    return __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, p, seed, cs, 0);
}

// Decode the two E2M1 codes in byte SEL of w to binary32 (exact).
template <int SEL>
__device__ __forceinline__ float2v fp4x2_to_f32(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, SEL);
}
// ---------------------------------------------------------------- direct global -> LDS loads
constexpr uint32_t kOutOfRange = 0x80000000u;   // past the end of every direct-load buffer

typedef int int4v __attribute__((ext_vector_type(4)));

// Buffer descriptor of a raw byte buffer: base, no stride, num_records bytes, the data
// format word of untyped 32-bit buffer access.
__device__ __forceinline__ int4v make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t b = (uint64_t)base;
    return int4v{(int)(uint32_t)b, (int)((uint32_t)(b >> 32) & 0xFFFFu), (int)bytes, 0x00020000};
}

// Direct loads (lane l writes its 16 or 4 bytes at LDS address M0 + 16 l or M0 + 4 l; an
// offset past num_records writes zeros).  They are written as assembly so that the compiler
// does not track them: its own bookkeeping would otherwise wait for every pending direct
// load before each LDS read, which would serialise a multi-stage pipeline.  Kernels wait
// for them explicitly (s_waitcnt vmcnt, then a barrier).  The compiler's waits for other
// vector-memory operations do not count them, so they can only wait longer than needed,
// never shorter.
__device__ __forceinline__ void dma16(int4v rsrc, uint32_t lds_addr, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :: "s"(lds_addr), "v"(voff), "s"(rsrc) : "memory", "m0");
}
__device__ __forceinline__ void dma4(int4v rsrc, uint32_t lds_addr, uint32_t voff) {
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
                 :: "s"(lds_addr), "v"(voff), "s"(rsrc) : "memory", "m0");
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

// The value held by lane ^ 1 (a DPP quad permutation [1,0,3,2]: no LDS traffic).
__device__ __forceinline__ float xor1(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}
// The value held by lane ^ 2 (DPP quad permutation [2,3,0,1]).
__device__ __forceinline__ float xor2(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}

// Correctly rounded a / b from r_b = RN(1 / b) (Markstein's correction: q = RN(a r_b) is
// within one ulp, the residual a - q b is exact in one fma, and RN(q + residual * r_b) is
// the correctly rounded quotient while no operand, quotient or residual is subnormal).
// Checked on the host: over every positive binary32 a for b = 6 and b = 4 (all normal
// quotients agree), and over 10^9 random pairs with b >= 2^-92 and a / b in [2^-12, 2^10].
__device__ __forceinline__ float div_rn_by(float a, float b, float rb) {
    const float q = a * rb;
    const float r = __builtin_fmaf(-q, b, a);
    return __builtin_fmaf(r, rb, q);
}

// Correctly rounded square roots of 16 non-negative finite values, in place.  The hardware
// estimate v_sqrt_f32 is within one ulp for inputs of at least 2^-96; the root is then s,
// or s - ulp when (s - ulp) s >= x, or s + ulp when (s + ulp) s < x (residuals by fma,
// exact), which is also right for x = 0.  This is the library square root's own sequence
// for that range, without its rescaling of tiny inputs and its special-value checks.  When
// any lane of the wave holds a value in (0, 2^-96), the whole wave takes sqrtf instead.
__device__ __forceinline__ void sqrt16_rn(float y[16]) {
    // bits - 1 of a value in (0, 2^-96) is below that of 2^-96; 0 wraps to the top
    uint32_t mn = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < 16; ++i) mn = min(mn, __float_as_uint(y[i]) - 1u);
    if (__builtin_amdgcn_ballot_w64(mn < 0x0F7FFFFFu) != 0) {
#pragma unroll
        for (int i = 0; i < 16; ++i) y[i] = sqrtf(y[i]);
        return;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float x = y[i], s = __builtin_amdgcn_sqrtf(x);
        const float sm = __uint_as_float(__float_as_uint(s) - 1u);
        const float sp = __uint_as_float(__float_as_uint(s) + 1u);
        float r = __builtin_fmaf(-sm, s, x) <= 0.0f ? sm : s;
        r = __builtin_fmaf(-sp, s, x) > 0.0f ? sp : r;
        y[i] = r;
    }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

}  // namespace nvfp4
