"""The library's arithmetic shortcuts as compiled from its device header
(tests/kernel_arith.hip): sqrt16_rn gives the correctly rounded square root of every
non-negative finite binary32 (the estimate path from 2^-96 up, sqrtf below), and the
corrected division div_rn_by gives the correctly rounded quotient for every positive finite
dividend with divisors 6 and 4 and for 2^30 random pairs with divisors of at least 2^-92 and
quotients in [2^-12, 2^10].  Quotients below 2^-126 (which the kernels never decide on: the
block-scale code is 0 either way) are reported, not required to agree."""
import ctypes
import os

import pytest

pytestmark = pytest.mark.gpu


def test_kernel_arithmetic_exhaustive():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = ctypes.CDLL(os.path.join(os.path.dirname(__file__), "libkarith.so"))
    counts = (ctypes.c_ulonglong * 7)()
    first = (ctypes.c_uint32 * 7)()
    print("kernel arithmetic: sqrt over 2^31 - 2^23 inputs, division by 6 and 4 over 2^31 - 2^23 "
          "dividends each, 2^30 random divisions", flush=True)
    assert lib.karith_run(counts, first) == 0
    print(f"  subnormal quotients off by the corrected division: /6 {counts[3]}, /4 {counts[5]}")
    assert counts[0] == 0, f"sqrt16_rn (estimate path): {counts[0]} wrong, first {first[0]:#010x}"
    assert counts[1] == 0, f"sqrt16_rn (below 2^-96): {counts[1]} wrong, first {first[1]:#010x}"
    assert counts[2] == 0, f"div_rn_by(a, 6): {counts[2]} wrong, first a bits {first[2]:#010x}"
    assert counts[4] == 0, f"div_rn_by(a, 4): {counts[4]} wrong, first a bits {first[4]:#010x}"
    assert counts[6] == 0, f"div_rn_by random pairs: {counts[6]} wrong, first a bits {first[6]:#010x}"
