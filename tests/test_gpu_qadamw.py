"""GPU parity of qadamw_v_encode / qadamw_v_decode against the oracle (bit-exact mean,
codes, scales, tensor scale and reconstructed state), including the full 9216x3072
log-normal second-moment workload."""
import numpy as np
import pytest
import torch

from gpu_util import dev, to_gpu_qtensor

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import nvfp4_block_scaled_quantize_amd as nv
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nv.load_library()
    return nv


def check(nv, oracle, v, seed, use_signs):
    print(f"qadamw case {tuple(v.shape)} seed={seed:#x} signs={use_signs}", flush=True)
    mu, q = nv.qadamw_v_encode(v.to(dev()), seed=seed, use_signs=use_signs)
    torch.cuda.synchronize()
    omu, oq = oracle.qadamw_v_encode(v.numpy(), seed=seed, use_signs=use_signs)
    gmu = mu.cpu().numpy().view(np.uint16)
    assert np.array_equal(gmu, omu), f"{np.count_nonzero(gmu != omu)} tile means differ"
    assert q.gscale.item() == np.float32(oq.sg)
    assert np.array_equal(q.scales.cpu().numpy(), oq.scales)
    assert np.array_equal(q.codes.cpu().numpy(), oq.codes)
    # decode of the oracle's encoding on the GPU vs the oracle's decode
    omu_t = torch.from_numpy(omu.view(np.int16)).to(dev())
    out = nv.qadamw_v_decode(omu_t, to_gpu_qtensor(nv, oq), seed=seed, use_signs=use_signs)
    torch.cuda.synchronize()
    ref = oracle.qadamw_v_decode(omu, oq, seed=seed, use_signs=use_signs)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


# widths that are multiples of 1024 decode in the whole-wave layout
@pytest.mark.parametrize("shape", [(16, 16), (48, 80), (64, 512), (272, 400), (32, 1024), (48, 2048)])
@pytest.mark.parametrize("use_signs", [0, 1])
def test_qadamw_matches_oracle(nv, oracle, shape, use_signs):
    from nvfp4_block_scaled_quantize_amd import synthetic
    v = synthetic.lognormal(shape, 50 + shape[0] + shape[1])
    v[0, :8] = 0.0
    check(nv, oracle, v, 0x5EED5, use_signs)


def test_qadamw_full_size(nv, oracle):
    from nvfp4_block_scaled_quantize_amd import synthetic
    v = synthetic.qadamw()["v"]       # 9216 x 3072 log-normal(-18, 3)
    check(nv, oracle, v, synthetic.RHT_SEED_QADAMW, 1)


def test_qadamw_tiny_values(nv, oracle):
    """Second moments below 2^-96 (normal and subnormal) take the rescaled square root; 2^-96
    itself and everything above take the short one.  Both must round as IEEE sqrt."""
    from nvfp4_block_scaled_quantize_amd import synthetic
    v = synthetic.lognormal((64, 512), 77)
    v[3, :16] = 1e-35
    v[5, 20] = 1e-40                                  # subnormal
    v[7, 3] = 2.0 ** -96                              # the boundary itself (exact in f32)
    v[9, 9] = float(np.nextafter(np.float32(2.0 ** -96), np.float32(0)))
    v[40:56, 256:272] = 3e-33                         # a whole tile of them
    check(nv, oracle, v, 0x5EED5, 1)



def test_qadamw_many_partials(nv, oracle):
    """144000 x 16: 9000 first-pass workgroups, so the tensor maximum is reduced from more
    partials than one round of the reduction's loads covers (8192); the largest value sits in
    the last tile."""
    from nvfp4_block_scaled_quantize_amd import synthetic
    v = synthetic.lognormal((144000, 16), 77)
    v[-1, 3] = float(v.max()) * 4.0
    check(nv, oracle, v, 0x5EED5, 1)
