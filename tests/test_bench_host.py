"""Host logic of bench.py (no GPU): the assignment of traced kernel dispatches to the calls
of the benchmarked step, which the profile summaries rely on, and the refusal of more than
one GPU."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402

# the kernels one step launches, in order, as rocprofv3 names them
STEP = [
    "void nvfp4::k_amax<1, 2>(nvfp4::QArgs)", "void nvfp4::k_encode<1, 8, false>(nvfp4::QArgs)",
    "void nvfp4::k_amax<1, 0>(nvfp4::QArgs)", "void nvfp4::k_encode<1, 0, false>(nvfp4::QArgs)",
    "void nvfp4::k_gemm_dma<4>(nvfp4::GArgs)", "void nvfp4::k_gemm_half<4>(nvfp4::GArgs)",
    "void nvfp4::k_encode<1, 0, true>(nvfp4::QArgs)",          # H: maxima from the GEMM
    "void nvfp4::k_amax<1, 0>(nvfp4::QArgs)", "void nvfp4::k_encode<1, 0, false>(nvfp4::QArgs)",
    "void nvfp4::k_gemm_sk<0>(nvfp4::GArgs)",
    "void nvfp4::k_amax<1, 2>(nvfp4::QArgs)", "void nvfp4::k_encode<1, 11, false>(nvfp4::QArgs)",
    "void nvfp4::k_gemm_sk<0>(nvfp4::GArgs)", "void nvfp4::k_gemm_dma<0>(nvfp4::GArgs)",
    "nvfp4::k_qv_pass1(nvfp4::QVArgs)", "nvfp4::k_max_partials(float const*, int, int, float*)",
    "nvfp4::k_qv_pass2(nvfp4::QVArgs)",
    "nvfp4::k_qv_decode_w(unsigned short const*, unsigned char const*)",
    "nvfp4::k_qs_pass1(nvfp4::QSArgs)", "nvfp4::k_max_partials(float const*, int, int, float*)",
    "nvfp4::k_qs_pass2(nvfp4::QSArgs)",
    "nvfp4::k_dequant_w(unsigned char const*, unsigned char const*)",
]


def test_split_step_assigns_every_dispatch():
    setup = ["nvfp4::k_qs_pass1(nvfp4::QSArgs)", "nvfp4::k_max_partials(float const*, int, int, float*)",
             "nvfp4::k_qs_pass2(nvfp4::QSArgs)"]            # the state set-up before timing
    extras = ["void nvfp4::k_gemm_dma<1>(nvfp4::GArgs)"]
    names = setup + STEP + STEP + extras
    got = bench.split_step(names)
    assert [k for k, _ in got] == [k for k, _ in bench.STEP_ORDER] * 2
    first = len(setup)
    flat = [i for _, idx in got for i in idx]
    assert flat == list(range(first, first + 2 * len(STEP)))       # each dispatch once, in order
    calls = dict(got[:len(bench.STEP_ORDER)])
    assert [names[i].split("(")[0] for i in calls["qadamw_step_Wup"]] == [
        "nvfp4::k_qs_pass1", "nvfp4::k_max_partials", "nvfp4::k_qs_pass2"]
    # FFN-up: whole rounds, then the half-width last round; H's quantize: the encode alone
    assert [names[i].split("(")[0] for i in calls["gemm_ffn_up"]] == [
        "void nvfp4::k_gemm_dma<4>", "void nvfp4::k_gemm_half<4>"]
    assert len(calls["quant_H_row"]) == 1 and len(calls["gemm_wgrad"]) == 1


def test_split_step_rejects_a_partial_step():
    import pytest
    with pytest.raises(SystemExit):
        bench.split_step(STEP[:5])


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
