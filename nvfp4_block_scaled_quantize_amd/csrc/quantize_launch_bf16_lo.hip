// quantize_launch_bf16_lo.hip -- instantiates the quantizer kernels for bfloat16 input and
// option combinations 0..7 (bit 0 rowwise SR, bit 1 columnwise SR, bit 2 rowwise RHT,
// bit 3 columnwise RHT).
#include "quantize_kernels.h"

namespace nvfp4 {

void launch_quant_bf16_lo(int f, const QArgs& a, hipStream_t st) {
    switch (f) {
#define NVFP4_CASE(F) case F: launch_quant<1, F>(a, st); break;
    NVFP4_CASE(0) NVFP4_CASE(1) NVFP4_CASE(2) NVFP4_CASE(3) NVFP4_CASE(4) NVFP4_CASE(5) NVFP4_CASE(6) NVFP4_CASE(7)
#undef NVFP4_CASE
    }
}

}  // namespace nvfp4
