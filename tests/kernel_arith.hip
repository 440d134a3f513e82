// kernel_arith.hip -- test helper (built into tests/libkarith.so, loaded only by
// tests/test_gpu_kernel_arith.py): the library's own arithmetic shortcuts, as compiled for
// gfx950 from its device header, checked exhaustively (or on ~10^9 random pairs) on the GPU
// against the definition of correct rounding, evaluated exactly in binary64.
//
//  * sqrt16_rn: the correctly rounded square root of every non-negative finite binary32
//    (the hardware-estimate path for inputs of at least 2^-96, sqrtf below).  r is right iff
//    m_lo^2 < x < m_hi^2 for the midpoints m_lo, m_hi between r and its binary32
//    neighbours (25-bit numbers: their squares are exact in binary64, and no binary32 is
//    such a square), or r = 0 for x = 0.
//  * div_rn_by(a, b, RN(1/b)): the correctly rounded quotient, i.e. m_lo b < a < m_hi b for
//    the midpoints around q (49-bit products, exact in binary64), for every positive finite
//    a with b = 6 and b = 4 (the block-scale divisions), and for 2^30 random pairs with
//    b >= 2^-92 and a / b in [2^-12, 2^10] (the division by the tensor scale).  Quotients
//    below 2^-126 are counted separately: the kernels take no decision on them (they give
//    block-scale code 0 either way).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../nvfp4_block_scaled_quantize_amd/csrc/device_common.h"

using nvfp4::div_rn_by;
using nvfp4::sqrt16_rn;

__device__ double prev_mid(float q) {   // midpoint between q > 0 and its lower neighbour
    return ((double)q + (double)__uint_as_float(__float_as_uint(q) - 1u)) * 0.5;
}
__device__ double next_mid(float q) {
    return ((double)q + (double)__uint_as_float(__float_as_uint(q) + 1u)) * 0.5;
}

__device__ bool sqrt_ok(float x, float r) {
    if (x == 0.0f) return r == 0.0f && !signbit(r);
    if (!(r > 0.0f)) return false;
    const double lo = prev_mid(r), hi = next_mid(r), xd = (double)x;
    return lo * lo < xd && xd < hi * hi;
}

// q is the correctly rounded a / b (a >= 0, b > 0).  Exact ties (possible only among
// subnormal quotients) go to the even neighbour.
__device__ bool quot_ok(float a, float b, float q) {
    const double ad = (double)a, bd = (double)b;
    if (q == 0.0f) return ad < 0x1p-150 * bd || (ad == 0x1p-150 * bd);
    if (!(q > 0.0f)) return false;
    const double lo = prev_mid(q) * bd, hi = next_mid(q) * bd;
    const bool even = (__float_as_uint(q) & 1u) == 0u;
    return (lo < ad || (lo == ad && even)) && (ad < hi || (ad == hi && even));
}

// wrong roots; one lane takes 16 consecutive bit patterns from lo (with_zero: the very first
// is replaced by +0, which the estimate path must also handle)
__global__ void k_check_sqrt(uint32_t lo, uint32_t groups, uint32_t end, int with_zero,
                             unsigned long long* bad, uint32_t* first) {
    const uint32_t g = blockIdx.x * blockDim.x + threadIdx.x;
    if (g >= groups) return;
    float y[16], x[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t bits = lo + 16u * g + (uint32_t)i;
        x[i] = __uint_as_float(bits < end ? bits : lo);
        if (with_zero && g == 0 && i == 0) x[i] = 0.0f;
        y[i] = x[i];
    }
    sqrt16_rn(y);
#pragma unroll
    for (int i = 0; i < 16; ++i)
        if (!sqrt_ok(x[i], y[i]) && atomicAdd(bad, 1ull) == 0ull) *first = __float_as_uint(x[i]);
}

// every positive finite a, fixed b with rb = RN(1 / b); bad[0]: normal quotients wrong,
// bad[1]: subnormal quotients differing from the correctly rounded one
__global__ void k_check_div_fixed(uint32_t lo, uint32_t n, float b, float rb,
                                  unsigned long long* bad, uint32_t* first) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const uint32_t bits = lo + i;
    const float a = __uint_as_float(bits);
    const float q = div_rn_by(a, b, rb);
    if (quot_ok(a, b, q)) return;
    if ((double)a >= 0x1p-126 * (double)b) {
        if (atomicAdd(&bad[0], 1ull) == 0ull) *first = bits;
    } else {
        atomicAdd(&bad[1], 1ull);
    }
}

__device__ uint64_t mix64(uint64_t z) {   // splitmix64 finaliser
    z += 0x9E3779B97F4A7C15ull;
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

// random pairs: b with an exponent in [-92, 127), a quotient q0 with exponent in [-12, 10),
// a = RN(q0 b) (skipped when it is not a normal number)
__global__ void k_check_div_random(uint64_t base, uint32_t n, unsigned long long* bad,
                                   uint32_t* first) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= n) return;
    const uint64_t r = mix64(base + i);
    const uint32_t eb = (uint32_t)((r >> 32) % 219u) + 35u;          // 127 - 92 = 35 .. 253
    const uint32_t eq = (uint32_t)((r >> 24) % 22u) + 115u;          // 127 - 12 = 115 .. 136
    const float b = __uint_as_float((eb << 23) | (uint32_t)(r & 0x7FFFFFu));
    const float q0 = __uint_as_float((eq << 23) | (uint32_t)((r >> 40) & 0x7FFFFFu));
    const float a = q0 * b;
    if (!(a >= 0x1p-126f) || !(a <= 3.4e38f)) return;
    const float q = div_rn_by(a, b, __fdiv_rn(1.0f, b));
    if (!quot_ok(a, b, q) && atomicAdd(bad, 1ull) == 0ull) *first = __float_as_uint(a);
}

// counts: [0] sqrt >= 2^-96, [1] sqrt below, [2] div by 6 (normal quotients), [3] by 6
// (subnormal quotients), [4] div by 4, [5] by 4 subnormal, [6] random pairs.  Returns 0 or
// a HIP error code.
extern "C" int karith_run(unsigned long long* counts, uint32_t* first) {
    unsigned long long* d_bad = nullptr;
    uint32_t* d_first = nullptr;
    if (hipMalloc(&d_bad, 7 * sizeof(unsigned long long)) != hipSuccess) return 1;
    if (hipMalloc(&d_first, 7 * sizeof(uint32_t)) != hipSuccess) return 1;
    (void)hipMemset(d_bad, 0, 7 * sizeof(unsigned long long));
    (void)hipMemset(d_first, 0, 7 * sizeof(uint32_t));
    const uint32_t lo96 = 0x0F800000u, inf = 0x7F800000u;   // bits of 2^-96 and +inf
    {
        const uint32_t groups = (inf - lo96) / 16u;            // exact: both multiples of 16
        k_check_sqrt<<<(groups + 255) / 256, 256>>>(lo96, groups, inf, 1, d_bad, d_first);
        const uint32_t g2 = lo96 / 16u;                        // 0 .. 2^-96 (exclusive)
        k_check_sqrt<<<(g2 + 255) / 256, 256>>>(0u, g2, lo96, 0, d_bad + 1, d_first + 1);
    }
    const uint32_t chunk = 1u << 28;
    for (uint32_t lo = 1; lo < inf; lo += chunk) {
        const uint32_t n = inf - lo < chunk ? inf - lo : chunk;
        k_check_div_fixed<<<(n + 255) / 256, 256>>>(lo, n, 6.0f, 1.0f / 6.0f, d_bad + 2, d_first + 2);
        k_check_div_fixed<<<(n + 255) / 256, 256>>>(lo, n, 4.0f, 0.25f, d_bad + 4, d_first + 4);
    }
    for (uint64_t base = 0; base < (1ull << 30); base += chunk)
        k_check_div_random<<<chunk / 256, 256>>>(base, chunk, d_bad + 6, d_first + 6);
    int rc = hipDeviceSynchronize() == hipSuccess ? 0 : 2;
    (void)hipMemcpy(counts, d_bad, 7 * sizeof(unsigned long long), hipMemcpyDeviceToHost);
    (void)hipMemcpy(first, d_first, 7 * sizeof(uint32_t), hipMemcpyDeviceToHost);
    (void)hipFree(d_bad);
    (void)hipFree(d_first);
    return rc;
}
