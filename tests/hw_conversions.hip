// hw_conversions.hip -- test helper (built into tests/libhwcheck.so, loaded only by
// tests/test_gpu_hw_conversions.py): exhaustive comparison, on the GPU, of the gfx950
// conversion instructions the NVFP4 kernels rely on with plain definitions written here.
//
//  * E4M3 block scale: v_cvt_pk_fp8_f32 of min(s, 448) against nearest-even rounding to
//    the OCP E4M3 "fn" grid (bias 7, subnormal step 2^-9, largest finite 448), for every
//    non-negative finite binary32 s.
//  * E2M1 element: v_cvt_scalef32_pk_fp4_f32 at scale 1.0 against the threshold form of
//    nearest-even rounding to {0, 0.5, 1, 1.5, 2, 3, 4, 6} (ties to the even code,
//    saturation at 6, sign copied), for every finite binary32.
//  * E2M1 stochastic rounding: v_cvt_scalef32_sr_pk_fp4_f32 at scale 1.0, first value of
//    the pair with seed r16 << 16 (second value 0.0), against the rule "up iff
//    floor(frac * 2^16) + r16 >= 2^16" (frac: the position between the two grid
//    neighbours, in binary64; saturation at 6, sign copied).  Every finite binary32 with a
//    hashed r16, and every r16 for the multiples of 1/256 in [0, 8) of both signs.
//  * The same two E2M1 conversions with the scale operand 2^-64 (which the kernels pass for
//    tensors whose block-scale reciprocals leave binary32's range) against the conversion
//    of x 2^64 at scale 1.0, for every finite binary32 x with |x| < 2^64 (x 2^64 exact).
// Nothing here is shared with the library's kernels.
#include <hip/hip_runtime.h>
#include <stdint.h>

// Nearest-even E4M3 code of s >= 0 by search over the 127 finite non-negative codes.
__device__ uint32_t e4m3_nearest_even(float s) {
    if (s >= 448.0f) return 0x7Eu;
    uint32_t best = 0;
    float bestd = s;   // distance to code 0
    for (uint32_t c = 1; c < 0x7F; ++c) {
        const uint32_t e = c >> 3, m = c & 7u;
        const float v = e == 0 ? (float)m * 0.001953125f : ldexpf(1.0f + (float)m / 8.0f, (int)e - 7);
        const float d = fabsf(v - s);   // exact: v and s are close or d is not decisive
        if (d < bestd || (d == bestd && (c & 1u) == 0)) { best = c; bestd = d; }
        if (v > s) break;
    }
    return best;
}

__global__ void k_check_e4m3(uint32_t lo, uint32_t n, unsigned long long* bad, uint32_t* first) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const uint32_t bits = lo + i;
    const float s = __uint_as_float(bits);
    const uint32_t ref = e4m3_nearest_even(s);
    const uint32_t hw = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(fminf(s, 448.0f), 0.0f, 0, false) & 0xFFu;
    if (ref != hw && atomicAdd(bad, 1ull) == 0ull) *first = bits;
}

// Threshold form of nearest-even E2M1: each grid midpoint is a tie that goes to the even
// code (0.25 -> 0, 0.75 -> 1.0, 1.25 -> 1.0, 1.75 -> 2.0, 2.5 -> 2.0, 3.5 -> 4.0, 5 -> 4.0).
__device__ uint32_t e2m1_nearest_even(float x) {
    const float u = fabsf(x);
    const uint32_t mag = (u > 0.25f) + (u >= 0.75f) + (u > 1.25f) + (u >= 1.75f) + (u > 2.5f) +
                         (u >= 3.5f) + (u > 5.0f);
    return mag | ((__float_as_uint(x) >> 28) & 8u);
}

__global__ void k_check_e2m1(uint64_t lo, uint32_t n, unsigned long long* bad, uint32_t* first) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const uint32_t bits = (uint32_t)(lo + i);
    if ((bits & 0x7F800000u) == 0x7F800000u) return;   // inf and NaN are outside the contract
    const float x = __uint_as_float(bits);
    const uint32_t ref = e2m1_nearest_even(x);
    const uint32_t hw = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x, 0.0f, 1.0f, 0) & 0xFu;
    if (ref != hw && atomicAdd(bad, 1ull) == 0ull) *first = bits;
}

// Stochastic rounding by its definition, in binary64 (u - grid[k] and the division by the
// spacing are exact there).
__device__ uint32_t e2m1_sr_rule(float x, uint32_t r16) {
    const double grid[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};
    const uint32_t sign = (__float_as_uint(x) >> 28) & 8u;
    const double u = fabs((double)x);
    if (u >= 6.0) return 7u | sign;
    uint32_t k = 0;
    while (k < 7 && grid[k + 1] <= u) ++k;
    const double frac = (u - grid[k]) / (grid[k + 1] - grid[k]);
    const double t = floor(frac * 65536.0);
    return (t + (double)r16 >= 65536.0 ? k + 1 : k) | sign;
}

__device__ uint32_t e2m1_sr_hw(float x, uint32_t r16) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    const f2 p = {x, 0.0f};
    return __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, p, r16 << 16, 1.0f, 0) & 0xFFu;
}

// every finite binary32, r16 from a multiplicative hash of its bits
__global__ void k_check_sr_all(uint64_t lo, uint32_t n, unsigned long long* bad, uint32_t* first) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const uint32_t bits = (uint32_t)(lo + i);
    if ((bits & 0x7F800000u) == 0x7F800000u) return;
    const float x = __uint_as_float(bits);
    const uint32_t r16 = (bits * 0x9E3779B1u) >> 16;
    if (e2m1_sr_rule(x, r16) != e2m1_sr_hw(x, r16) && atomicAdd(bad, 1ull) == 0ull) *first = bits;
}

// index i: r16 = i mod 2^16, x = +-(j / 256) with j = (i >> 17) in [0, 2048), sign bit 16
__global__ void k_check_sr_thresholds(unsigned long long* bad, uint32_t* first) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;   // grid covers exactly 2^28
    const uint32_t r16 = i & 0xFFFFu;
    const float m = (float)(i >> 17) * 0.00390625f;
    const float x = ((i >> 16) & 1u) ? -m : m;
    if (e2m1_sr_rule(x, r16) != e2m1_sr_hw(x, r16) && atomicAdd(bad, 1ull) == 0ull)
        *first = __float_as_uint(x);
}

// every finite x with |x| < 2^64: the conversions at scale 2^-64 equal those of x 2^64 at 1.0
__global__ void k_check_scaled(uint64_t lo, uint32_t n, unsigned long long* bad, uint32_t* first) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const uint32_t bits = (uint32_t)(lo + i);
    if (((bits >> 23) & 0xFFu) >= 127u + 64u) return;    // |x| >= 2^64, inf and NaN
    const float x = __uint_as_float(bits);
    const float xs = x * 0x1p64f;                         // exact
    const uint32_t rne = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, x, 0.0f, 0x1p-64f, 0) & 0xFu;
    const uint32_t rne1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, xs, 0.0f, 1.0f, 0) & 0xFu;
    const uint32_t r16 = (bits * 0x9E3779B1u) >> 16;
    typedef float f2 __attribute__((ext_vector_type(2)));
    const f2 p = {x, 0.0f}, ps = {xs, 0.0f};
    const uint32_t sr = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, p, r16 << 16, 0x1p-64f, 0) & 0xFFu;
    const uint32_t sr1 = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, ps, r16 << 16, 1.0f, 0) & 0xFFu;
    if ((rne != rne1 || sr != sr1) && atomicAdd(bad, 1ull) == 0ull) *first = bits;
}

// Runs the checks; returns 0 and fills counts[0..3] (mismatches: E4M3, E2M1 nearest-even,
// E2M1 stochastic, the two E2M1 conversions at scale 2^-64) and first[0..3] (first
// mismatching input bits), or a HIP error code.
extern "C" int hwcheck_run(unsigned long long* counts, uint32_t* first) {
    unsigned long long* d_bad = nullptr;
    uint32_t* d_first = nullptr;
    if (hipMalloc(&d_bad, 4 * sizeof(unsigned long long)) != hipSuccess) return 1;
    if (hipMalloc(&d_first, 4 * sizeof(uint32_t)) != hipSuccess) return 1;
    (void)hipMemset(d_bad, 0, 4 * sizeof(unsigned long long));
    (void)hipMemset(d_first, 0, 4 * sizeof(uint32_t));
    const uint32_t chunk = 1u << 28;
    const uint32_t nonneg = 0x7F800000u;   // every non-negative finite pattern
    for (uint32_t lo = 0; lo < nonneg; lo += chunk) {
        const uint32_t n = nonneg - lo < chunk ? nonneg - lo : chunk;
        k_check_e4m3<<<(n + 255) / 256, 256>>>(lo, n, d_bad, d_first);
    }
    for (uint64_t lo = 0; lo < (1ull << 32); lo += chunk)
        k_check_e2m1<<<chunk / 256, 256>>>(lo, chunk, d_bad + 1, d_first + 1);
    for (uint64_t lo = 0; lo < (1ull << 32); lo += chunk)
        k_check_sr_all<<<chunk / 256, 256>>>(lo, chunk, d_bad + 2, d_first + 2);
    k_check_sr_thresholds<<<(1u << 28) / 256, 256>>>(d_bad + 2, d_first + 2);
    for (uint64_t lo = 0; lo < (1ull << 32); lo += chunk)
        k_check_scaled<<<chunk / 256, 256>>>(lo, chunk, d_bad + 3, d_first + 3);
    int rc = hipDeviceSynchronize() == hipSuccess ? 0 : 2;
    (void)hipMemcpy(counts, d_bad, 4 * sizeof(unsigned long long), hipMemcpyDeviceToHost);
    (void)hipMemcpy(first, d_first, 4 * sizeof(uint32_t), hipMemcpyDeviceToHost);
    (void)hipFree(d_bad);
    (void)hipFree(d_first);
    return rc;
}
