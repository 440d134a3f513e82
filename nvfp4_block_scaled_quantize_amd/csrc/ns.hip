// ns.hip -- one quantized Newton-Schulz iteration (NVFP4 Root), composed of the library's
// quantize and GEMM kernels.
//
// Method: Full-Stack FP4 sec. 3.4 (and sec. 2's iteration X_{k+1} = a X + b X (X^T X) +
// c X (X^T X)^2, written for the wide orientation as A = X X^T):
//   qX = Q_1x16(X H), qX' = Q_16x1(H^T X)          one quantize of X, both copies
//   A  = qX qX^T                                     GEMM (the rotations cancel)
//   qA = Q_1x16(A H), qA' = Q_16x1(H^T A)            one quantize of A, both copies
//   B  = b A + c qA qA'                              GEMM with the alpha/beta epilogue
//   qB = Q_1x16(B H)                                 rowwise quantize of B
//   X  = a X + qB qX'                                GEMM with the alpha/beta epilogue, in place
// Every quantization is nearest-even with 4/6 scaling (the pages'), 1x16 / 16x1 blocks, and
// one random Hadamard H per iteration (the seed).  The coefficients are the caller's: the
// pages take shape-specialised ones from Root and do not print them.
#include <hip/hip_runtime.h>
#include "nvfp4.h"

namespace nvfp4 {
// gemm.hip: A A^T on the triangle tiles with K split into parts, then a reduction that
// mirrors (NVFP4_ERR_MODE when the shape does not allow it)
size_t syrk_part_bytes(int64_t m, int64_t k);
int syrk_splitk(const nvfp4_qtensor* a, int64_t m, int64_t k, float* c, int64_t ldc, float* part,
                size_t part_bytes, hipStream_t st);
}  // namespace nvfp4

namespace {

size_t al256(size_t n) { return (n + 255) & ~(size_t)255; }

// One NVFP4 copy of an r x c matrix carved from the workspace.
struct Carve {
    uint8_t* base;
    size_t off;
    uint8_t* take(size_t n) {
        uint8_t* p = base ? base + off : nullptr;
        off += al256(n);
        return p;
    }
    nvfp4_qtensor copy(int64_t r, int64_t c) {
        nvfp4_qtensor q;
        q.codes = take((size_t)(r * c / 2));
        q.scales = take((size_t)(r * c / 16));
        q.gscale = (float*)take(sizeof(float));
        return q;
    }
};

struct NsBuffers {
    nvfp4_qtensor qx, qxc, qa, qac, qb;
    float* a;
    float* b;
    void* qws;
    size_t qws_bytes;
    float* part;          // partial products of A = qX qX^T (none when it is not split)
    size_t part_bytes;
    size_t total;
};

NsBuffers ns_layout(uint8_t* ws, int64_t m, int64_t n, const nvfp4_quant_params* p) {
    NsBuffers L;
    Carve c{ws, 0};
    L.qx = c.copy(m, n);
    L.qxc = c.copy(n, m);
    L.a = (float*)c.take((size_t)(m * m) * sizeof(float));
    L.qa = c.copy(m, m);
    L.qac = c.copy(m, m);
    L.b = (float*)c.take((size_t)(m * m) * sizeof(float));
    L.qb = c.copy(m, m);
    const size_t w1 = nvfp4_quantize_workspace_bytes(m, n, p);
    const size_t w2 = nvfp4_quantize_workspace_bytes(m, m, p);
    L.qws_bytes = w1 > w2 ? w1 : w2;
    L.qws = c.take(L.qws_bytes);
    L.part_bytes = nvfp4::syrk_part_bytes(m, n);
    L.part = L.part_bytes ? (float*)c.take(L.part_bytes) : nullptr;
    L.total = c.off;
    return L;
}

nvfp4_quant_params ns_params(int rowwise_only, uint64_t seed, int scale46) {
    nvfp4_quant_params p;
    p.rowwise = 1;
    p.colwise = rowwise_only ? 0 : 1;
    p.block = NVFP4_BLOCK_1D;
    p.round_row = NVFP4_RNE;
    p.round_col = NVFP4_RNE;
    p.rht_row = 1;
    p.rht_col = rowwise_only ? 0 : 1;
    p.scale46 = scale46 ? 1 : 0;
    p.seed = seed;
    return p;
}

}  // namespace

extern "C" size_t nvfp4_ns_step_workspace_bytes(int64_t m, int64_t n) {
    if (m <= 0 || n <= 0) return 0;
    const nvfp4_quant_params p = ns_params(0, 0, 1);
    return ns_layout(nullptr, m, n, &p).total;
}

extern "C" int nvfp4_ns_step(float* x, int64_t m, int64_t n, float a, float b, float c,
                             uint64_t seed, int32_t scale46, void* ws, size_t ws_bytes,
                             void* stream) {
    if (m < 0 || n < 0 || m % 32 || n % 32) return NVFP4_ERR_SHAPE;
    if (scale46 != 0 && scale46 != 1) return NVFP4_ERR_MODE;
    if (m == 0 || n == 0) return NVFP4_OK;
    if (!x) return NVFP4_ERR_NULL;
    if ((uintptr_t)x & 15) return NVFP4_ERR_ALIGN;
    if (!ws) return NVFP4_ERR_WORKSPACE;
    if ((uintptr_t)ws & 255) return NVFP4_ERR_ALIGN;
    const nvfp4_quant_params pxa = ns_params(0, seed, scale46);
    const nvfp4_quant_params pb = ns_params(1, seed, scale46);
    const NsBuffers L = ns_layout((uint8_t*)ws, m, n, &pxa);
    if (ws_bytes < L.total) return NVFP4_ERR_WORKSPACE;
    int rc;
    // qX, qX'
    if ((rc = nvfp4_quantize(x, NVFP4_F32, m, n, n, &pxa, &L.qx, &L.qxc, L.qws, L.qws_bytes,
                             stream)) != NVFP4_OK)
        return rc;
    // A = qX qX^T: the triangle tiles split along K when that fills the device, else the GEMM
    rc = nvfp4::syrk_splitk(&L.qx, m, n, L.a, m, L.part, L.part_bytes, (hipStream_t)stream);
    if (rc == NVFP4_ERR_MODE) rc = nvfp4_gemm(&L.qx, &L.qx, m, m, n, L.a, m, stream);
    if (rc != NVFP4_OK) return rc;
    // qA, qA'
    if ((rc = nvfp4_quantize(L.a, NVFP4_F32, m, m, m, &pxa, &L.qa, &L.qac, L.qws, L.qws_bytes,
                             stream)) != NVFP4_OK)
        return rc;
    // B = c qA qA' + b A
    if ((rc = nvfp4_gemm_axpby(&L.qa, &L.qac, m, m, m, c, L.a, m, b, L.b, m, stream)) != NVFP4_OK)
        return rc;
    // qB
    if ((rc = nvfp4_quantize(L.b, NVFP4_F32, m, m, m, &pb, &L.qb, nullptr, L.qws, L.qws_bytes,
                             stream)) != NVFP4_OK)
        return rc;
    // X = qB qX' + a X, in place
    return nvfp4_gemm_axpby(&L.qb, &L.qxc, m, n, m, 1.0f, x, n, a, x, n, stream);
}
