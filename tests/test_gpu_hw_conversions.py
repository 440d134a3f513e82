"""The conversion instructions the kernels rely on, against plain definitions, over every
input (tests/hw_conversions.hip): the E4M3 block-scale conversion for each non-negative
finite binary32, the E2M1 element conversion at scale 1 for each finite binary32, and the
E2M1 stochastic-rounding conversion (seed r16 << 16) against the rounding rule for each finite
binary32 and for every r16 at the multiples of 1/256 in [0, 8); and both E2M1 conversions at the
scale operand 2^-64 against those of x 2^64 at scale 1, for every finite |x| < 2^64."""
import ctypes
import os

import pytest

pytestmark = pytest.mark.gpu


def test_conversions_exhaustive():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lib = ctypes.CDLL(os.path.join(os.path.dirname(__file__), "libhwcheck.so"))
    counts = (ctypes.c_ulonglong * 4)()
    first = (ctypes.c_uint32 * 4)()
    print("hw conversion check: E4M3 over 2^31 - 2^23 inputs, E2M1 over 2^32, E2M1 SR over 2^32 + 2^28, scaled E2M1 over 2^32", flush=True)
    assert lib.hwcheck_run(counts, first) == 0
    assert counts[0] == 0, f"E4M3: {counts[0]} mismatches, first input bits {first[0]:#010x}"
    assert counts[1] == 0, f"E2M1: {counts[1]} mismatches, first input bits {first[1]:#010x}"
    assert counts[2] == 0, f"E2M1 SR: {counts[2]} mismatches, first input bits {first[2]:#010x}"
    assert counts[3] == 0, f"E2M1 at scale 2^-64: {counts[3]} mismatches, first input bits {first[3]:#010x}"
