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

// Runs both checks; returns 0 and fills counts[0..1] (mismatches) and first[0..1] (first
// mismatching input bits), or a HIP error code.
extern "C" int hwcheck_run(unsigned long long* counts, uint32_t* first) {
    unsigned long long* d_bad = nullptr;
    uint32_t* d_first = nullptr;
    if (hipMalloc(&d_bad, 2 * sizeof(unsigned long long)) != hipSuccess) return 1;
    if (hipMalloc(&d_first, 2 * sizeof(uint32_t)) != hipSuccess) return 1;
    hipMemset(d_bad, 0, 2 * sizeof(unsigned long long));
    hipMemset(d_first, 0, 2 * sizeof(uint32_t));
    const uint32_t chunk = 1u << 28;
    const uint32_t nonneg = 0x7F800000u;   // every non-negative finite pattern
    for (uint32_t lo = 0; lo < nonneg; lo += chunk) {
        const uint32_t n = nonneg - lo < chunk ? nonneg - lo : chunk;
        k_check_e4m3<<<(n + 255) / 256, 256>>>(lo, n, d_bad, d_first);
    }
    for (uint64_t lo = 0; lo < (1ull << 32); lo += chunk)
        k_check_e2m1<<<chunk / 256, 256>>>(lo, chunk, d_bad + 1, d_first + 1);
    int rc = hipDeviceSynchronize() == hipSuccess ? 0 : 2;
    hipMemcpy(counts, d_bad, 2 * sizeof(unsigned long long), hipMemcpyDeviceToHost);
    hipMemcpy(first, d_first, 2 * sizeof(uint32_t), hipMemcpyDeviceToHost);
    hipFree(d_bad);
    hipFree(d_first);
    return rc;
}
