"""Host check of the kernels' corrected division (tests/div_rn_check.c): exhaustive over every
positive finite dividend for the block-scale divisors 6 and 4, and 10^8 seeded random pairs
with divisors of at least 2^-92 (the tensor scales that take this path) and quotients in
[2^-12, 2^10].  Every normal quotient must equal the host's correctly rounded division."""
import os
import subprocess
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))


def test_corrected_division_is_correctly_rounded():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "div_rn_check")
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                               "-fopenmp", os.path.join(HERE, "div_rn_check.c"), "-o", exe, "-lm"])
        out = subprocess.check_output([exe, "100000000"], text=True).split()
    print(" ".join(out))
    assert out[0] == "div6" and int(out[1]) == 0, out        # normal quotients of a / 6
    assert out[3] == "div4" and int(out[4]) == 0, out        # normal quotients of a / 4
    assert out[6] == "random" and int(out[7]) == 0, out      # random pairs
    assert int(out[8]) == 100000000
