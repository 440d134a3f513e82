"""GPU parity of the GEMM's balanced (stream-K) schedule.

When the last round of 256 x 256 output tiles would keep at most half of the compute units
busy, nvfp4_gemm runs the whole rounds with one tile per workgroup and either splits each
remaining tile into two K halves on two workgroups (such a tile is summed as fl(head + tail)
of two partial FP32 accumulations) or runs the remaining tiles as twice as many half-width
tiles.  It picks the split for long whole rounds only; NVFP4_GEMM_SK=2 forces the split and
NVFP4_GEMM_SK=3 the half-width tiles, so both are checked here on two ragged shapes with two
K stages per tile (one stage per half): 2000 x 4000 x 192 (8 x 16 = 128 tiles, every one
split) and 4112 x 4112 x 192 (289 tiles: one whole round, then 33 split tiles).  Split:
  * the whole output against the oracle's binary64 GEMM, to the GEMM tolerance;
  * the schedule against one workgroup per tile (NVFP4_GEMM_SK=0), to the same tolerance;
  * the head's fallback (the tail part computed by the head after it claims the tile) is bit
    for bit the normal hand-off: forced from the host with NVFP4_GEMM_SK_TEST=1 (every tail
    skips its hand-off) and NVFP4_GEMM_SK_SPIN=0 (no wait), and with a zero wait alone
    (heads and tails race for each tile);
  * nvfp4_gemm_lora at the same shapes (one workgroup per tile: its epilogue does not take
    the balanced schedule) against the oracle.
Half-width tiles: bit for bit one workgroup per tile (NVFP4_GEMM_SK=0), and what the default
choice runs on these short-K shapes.
"""
import numpy as np
import pytest
import torch

from gpu_util import GEMM_TOL, dev, gemm_errors, to_gpu_qtensor

pytestmark = pytest.mark.gpu

SHAPES = [(2000, 4000, 192), (4112, 4112, 192)]
K = 192
RANK = 32


@pytest.fixture(scope="module")
def nv():
    import nvfp4_block_scaled_quantize_amd as nv
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nv.load_library()
    return nv


@pytest.fixture(scope="module", params=SHAPES, ids=lambda s: "x".join(map(str, s)))
def operands(oracle, request):
    from nvfp4_block_scaled_quantize_amd import synthetic
    M, N, K = request.param
    a = synthetic.outlier_channels((M, K), 4401 + M).to(torch.bfloat16).float().numpy()
    b = synthetic.normal((N, K), 4402 + N, 0.02).to(torch.bfloat16).float().numpy()
    qa, _ = oracle.quantize(a)
    qb, _ = oracle.quantize(b)
    return qa, qb


def cus():
    return torch.cuda.get_device_properties(0).multi_processor_count


def run(nv, qa, qb, monkeypatch, lora=None, **env):
    """nvfp4_gemm (or its LoRA form) with the balanced split forced unless env says otherwise."""
    for k in ("NVFP4_GEMM_SK", "NVFP4_GEMM_SK_SPIN", "NVFP4_GEMM_SK_TEST"):
        monkeypatch.delenv(k, raising=False)
    env.setdefault("NVFP4_GEMM_SK", 2)
    for k, v in env.items():
        monkeypatch.setenv(k, str(v))
    ga, gb = to_gpu_qtensor(nv, qa), to_gpu_qtensor(nv, qb)
    if lora is None:
        c = nv.nvfp4_gemm(ga, gb)
    else:
        c = nv.nvfp4_gemm_lora(ga, gb, lora[0], lora[1])
    torch.cuda.synchronize()
    return c


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_shapes_take_the_balanced_schedule(M, N, K):
    tiles = ((M + 255) // 256) * ((N + 255) // 256)
    g = cus() & ~7
    print(f"tiles {tiles}, workgroups {g}", flush=True)
    assert 0 < tiles % g <= g // 2 and (K + 127) // 128 >= 2


def test_balanced_full_matrix_vs_oracle(nv, oracle, operands, monkeypatch):
    qa, qb = operands
    M, N = qa.shape[0], qb.shape[0]
    print(f"balanced gemm {M}x{N}x{K}", flush=True)
    c = run(nv, qa, qb, monkeypatch)
    ref, absdot = oracle.gemm_f64(qa, qb)
    fro, nw = gemm_errors(c.cpu().numpy(), ref, absdot)
    print(f"  frobenius {fro:.3e} normwise {nw:.3e}")
    assert fro <= GEMM_TOL and nw <= GEMM_TOL
    # against one workgroup per tile: both within the tolerance of the exact product
    d = run(nv, qa, qb, monkeypatch, NVFP4_GEMM_SK=0)
    fro2, nw2 = gemm_errors(d.cpu().numpy(), ref, absdot)
    assert fro2 <= GEMM_TOL and nw2 <= GEMM_TOL


@pytest.mark.parametrize("env", [dict(NVFP4_GEMM_SK_TEST=1, NVFP4_GEMM_SK_SPIN=0),
                                 dict(NVFP4_GEMM_SK_SPIN=0)])
def test_fallback_is_bitwise_the_handoff(nv, operands, monkeypatch, env):
    qa, qb = operands
    print(f"balanced gemm fallback {env}", flush=True)
    c = run(nv, qa, qb, monkeypatch)
    f = run(nv, qa, qb, monkeypatch, **env)
    assert torch.equal(c.view(torch.int32), f.view(torch.int32))
    # twice in a row: the per-launch flags do not leak between calls
    f2 = run(nv, qa, qb, monkeypatch, **env)
    assert torch.equal(c.view(torch.int32), f2.view(torch.int32))


def test_balanced_lora(nv, oracle, operands, monkeypatch):
    from nvfp4_block_scaled_quantize_amd import synthetic
    qa, qb = operands
    M, N = qa.shape[0], qb.shape[0]
    t = synthetic.normal((M, RANK), 4403, 0.5).to(torch.bfloat16)
    lb = synthetic.normal((N, RANK), 4404, 0.02).to(torch.bfloat16)
    tg, lg = t.to(dev()), lb.to(dev())
    print(f"balanced gemm lora rank {RANK}", flush=True)
    c = run(nv, qa, qb, monkeypatch, lora=(tg, lg))
    bits = lambda x: x.view(torch.int16).numpy().view(np.uint16)
    ref, absdot = oracle.gemm_lora_f64(qa, qb, bits(t), bits(lb))
    fro, nw = gemm_errors(c.cpu().numpy(), ref, absdot)
    print(f"  frobenius {fro:.3e} normwise {nw:.3e}")
    assert fro <= GEMM_TOL and nw <= GEMM_TOL


def test_balanced_graph_replays(nv, operands, monkeypatch):
    """Replays of one captured launch share its epoch: each must still see only its own
    hand-offs (the flags are cleared by their last user), with eager GEMMs in between."""
    qa, qb = operands
    M, N = qa.shape[0], qb.shape[0]
    print(f"balanced gemm under graph capture {M}x{N}x{K}", flush=True)
    ref = run(nv, qa, qb, monkeypatch)
    d = dev()
    ga, gb = to_gpu_qtensor(nv, qa), to_gpu_qtensor(nv, qb)
    out = torch.empty((M, N), dtype=torch.float32, device=d)
    s = torch.cuda.Stream(device=d)
    s.wait_stream(torch.cuda.current_stream(d))
    with torch.cuda.stream(s):
        nv.nvfp4_gemm(ga, gb, out=out)             # warm-up on the capture stream
    torch.cuda.current_stream(d).wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        nv.nvfp4_gemm(ga, gb, out=out)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        other = nv.nvfp4_gemm(ga, gb)              # an eager launch with its own epoch
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int32), ref.view(torch.int32)), f"replay {rep}"
        assert torch.equal(other.view(torch.int32), ref.view(torch.int32)), f"eager {rep}"


def test_half_width_tiles_are_the_per_tile_sums(nv, operands, monkeypatch):
    qa, qb = operands
    print(f"half-width last round {qa.shape[0]}x{qb.shape[0]}x{K}", flush=True)
    per_tile = run(nv, qa, qb, monkeypatch, NVFP4_GEMM_SK=0)
    half = run(nv, qa, qb, monkeypatch, NVFP4_GEMM_SK=3)
    auto = run(nv, qa, qb, monkeypatch, NVFP4_GEMM_SK=1)
    assert torch.equal(half.view(torch.int32), per_tile.view(torch.int32))
    assert torch.equal(auto.view(torch.int32), half.view(torch.int32))


@pytest.mark.parametrize("M,N,Kf", [(8192, 3072, 9216), (8192, 9216, 3072)])
def test_half_width_full_size(nv, monkeypatch, M, N, Kf):
    """The step's FFN-down / dgrad shape (one whole round, 128 tiles left, 72 K stages) and the
    FP32 FFN-up shape (four whole rounds, 128 left), with the half-width last round forced:
    bit for bit one workgroup per tile.  GPU-quantized operands (the quantizer is checked bit
    for bit against the oracle elsewhere)."""
    from nvfp4_block_scaled_quantize_amd import synthetic
    print(f"half-width last round at full size {M}x{N}x{Kf}", flush=True)
    a = synthetic.outlier_channels((M, Kf), 7001).to(torch.bfloat16).to(dev())
    b = synthetic.normal((N, Kf), 7002, 0.02).to(torch.bfloat16).to(dev())
    qa, _ = nv.nvfp4_quantize(a, nv.quant_params(rowwise=True))
    qb, _ = nv.nvfp4_quantize(b, nv.quant_params(rowwise=True))
    del a, b
    for k in ("NVFP4_GEMM_SK", "NVFP4_GEMM_SK_SPIN", "NVFP4_GEMM_SK_TEST"):
        monkeypatch.delenv(k, raising=False)
    monkeypatch.setenv("NVFP4_GEMM_SK", "0")
    per_tile = nv.nvfp4_gemm(qa, qb)
    monkeypatch.setenv("NVFP4_GEMM_SK", "3")
    half = nv.nvfp4_gemm(qa, qb)
    torch.cuda.synchronize()
    assert torch.equal(half.view(torch.int32), per_tile.view(torch.int32))
