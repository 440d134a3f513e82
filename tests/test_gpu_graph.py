"""The entry points under HIP graph capture: a chain of calls (both quantizes, the GEMM, the
dequantizer, the second-moment encode and decode, one Newton-Schulz step) is captured once
with pre-allocated buffers and replayed three times, with eager work that overwrites every
output in between; each replay must reproduce the eager results bit for bit.  The library
issues no allocation, memset or synchronisation, so all of its work is capturable."""
import pytest
import torch

from gpu_util import dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    import nvfp4_block_scaled_quantize_amd as nv
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    nv.load_library()
    return nv


def test_graph_replays_match_eager(nv):
    from nvfp4_block_scaled_quantize_amd import synthetic
    d = dev()
    print("graph capture: quantize, gemm, dequantize, qadamw v, ns step", flush=True)
    X = synthetic.outlier_channels((512, 768), 41).to(torch.bfloat16).to(d)
    W = synthetic.normal((384, 768), 42, 0.02).to(torch.bfloat16).to(d)
    v = synthetic.lognormal((256, 512), 43).to(d)
    Xns0 = synthetic.normal((64, 192), 44, 0.1).to(d)
    px = nv.quant_params(rowwise=True, colwise=True, rht_col=True, seed=9)
    pw = nv.quant_params(rowwise=True, colwise=True, block2d=True)
    qx = (nv.QTensor.empty(512, 768, d), nv.QTensor.empty(768, 512, d))
    qw = (nv.QTensor.empty(384, 768, d), nv.QTensor.empty(768, 384, d))
    wsx = torch.empty(max(nv.nvfp4_quantize_workspace_bytes(512, 768, px), 16), dtype=torch.uint8, device=d)
    wsw = torch.empty(max(nv.nvfp4_quantize_workspace_bytes(384, 768, pw), 16), dtype=torch.uint8, device=d)
    C = torch.empty((512, 384), dtype=torch.float32, device=d)
    deq = torch.empty((384, 768), dtype=torch.float32, device=d)
    mu = torch.empty((16, 32), dtype=torch.int16, device=d)
    qv = nv.QTensor.empty(256, 512, d)
    wsv = torch.empty(max(nv.qadamw_v_workspace_bytes(256, 512), 16), dtype=torch.uint8, device=d)
    vout = torch.empty_like(v)
    Xns = torch.empty_like(Xns0)
    wsns = torch.empty(nv.load_library().nvfp4_ns_step_workspace_bytes(64, 192), dtype=torch.uint8, device=d)

    def chain():
        nv.nvfp4_quantize(X, px, qx[0], qx[1], wsx)
        nv.nvfp4_quantize(W, pw, qw[0], qw[1], wsw)
        nv.nvfp4_gemm(qx[0], qw[0], out=C)
        nv.nvfp4_dequantize(qw[0], out=deq)
        nv.qadamw_v_encode(v, 7, True, mu, qv, wsv)
        nv.qadamw_v_decode(mu, qv, 7, True, out=vout)
        nv.nvfp4_ns_step(Xns, 2.0, -1.5, 0.5, 11, True, wsns)

    outs = lambda: [qx[0].codes, qx[0].scales, qx[0].gscale, qx[1].codes, qx[1].scales, qx[1].gscale,
                    qw[0].codes, qw[1].codes, C, deq, mu, qv.codes, qv.scales, vout, Xns]

    Xns.copy_(Xns0)
    chain()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs()]

    s = torch.cuda.Stream(device=d)
    s.wait_stream(torch.cuda.current_stream(d))
    with torch.cuda.stream(s):
        Xns.copy_(Xns0)
        chain()                                    # warm-up on the capture stream
    torch.cuda.current_stream(d).wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs():
            o.zero_()                              # eager work between replays
        Xns.copy_(Xns0)                            # the Newton-Schulz step updates X in place
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (o, r) in enumerate(zip(outs(), ref)):
            assert torch.equal(o, r), f"replay {rep}: output {k} differs from the eager run"
