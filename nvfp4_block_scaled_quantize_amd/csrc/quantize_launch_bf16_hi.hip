// quantize_launch_bf16_hi.hip -- instantiates the quantizer kernels for bfloat16 input and
// option combinations 8..15 (bit 0 rowwise SR, bit 1 columnwise SR, bit 2 rowwise RHT,
// bit 3 columnwise RHT).
#include "quantize_kernels.h"

namespace nvfp4 {

void launch_quant_bf16_hi(int f, const QArgs& a, hipStream_t st) {
    switch (f) {
#define NVFP4_CASE(F) case F: launch_quant<1, F>(a, st); break;
    NVFP4_CASE(8) NVFP4_CASE(9) NVFP4_CASE(10) NVFP4_CASE(11) NVFP4_CASE(12) NVFP4_CASE(13) NVFP4_CASE(14) NVFP4_CASE(15)
#undef NVFP4_CASE
    }
}

}  // namespace nvfp4
