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


def test_graph_replays_the_step_calls(nv):
    """The calls of the benchmarked step that the chain above leaves out, captured and
    replayed the same way: the bf16 GEMM whose last round runs as half-width tiles (272
    tiles: one round of 256, then 16 tiles as 32 half-width ones, with the tile maxima zeroed
    by the first launch and combined by atomics in the second), the quantize that takes those
    maxima, the balanced FP32 GEMM (384 tiles: its 128 last ones split over K with the
    hand-off flags), the stochastically rounded quantize with a column rotation, and the
    quantized-state AdamW step (which updates the weights in place)."""
    from nvfp4_block_scaled_quantize_amd import synthetic
    d = dev()
    print("graph capture: bf16 gemm (half-width round), quantize with maxima, balanced gemm, "
          "SR quantize, qadamw step", flush=True)
    P = nv.quant_params
    A = synthetic.outlier_channels((4352, 192), 61).to(torch.bfloat16).to(d)
    B = synthetic.normal((4096, 192), 62, 0.02).to(torch.bfloat16).to(d)
    E = synthetic.outlier_channels((4096, 256), 63).to(torch.bfloat16).to(d)
    F = synthetic.normal((6144, 256), 64, 0.02).to(torch.bfloat16).to(d)
    G = synthetic.normal((512, 768), 65, 1.0).to(torch.bfloat16).to(d)
    w0 = synthetic.normal((256, 512), 66, 0.02).to(d)
    grad = synthetic.normal((256, 512), 67, 1e-3).to(torch.bfloat16).to(d)
    qa, _ = nv.nvfp4_quantize(A, P(rowwise=True))
    qb, _ = nv.nvfp4_quantize(B, P(rowwise=True, block2d=True))
    qe, _ = nv.nvfp4_quantize(E, P(rowwise=True))
    qf, _ = nv.nvfp4_quantize(F, P(rowwise=True))
    H = torch.empty((4352, 4096), dtype=torch.bfloat16, device=d)
    T = torch.empty((nv.load_library().nvfp4_gemm_tiles(4352, 4096),), dtype=torch.float32, device=d)
    qh = nv.QTensor.empty(4352, 4096, d)
    C = torch.empty((4096, 6144), dtype=torch.float32, device=d)
    psr = P(rowwise=True, colwise=True, round_row=nv.NVFP4_SR, round_col=nv.NVFP4_SR, rht_col=True,
            seed=13)
    qg = (nv.QTensor.empty(512, 768, d), nv.QTensor.empty(768, 512, d))
    wsg = torch.empty(max(nv.nvfp4_quantize_workspace_bytes(512, 768, psr), 16), dtype=torch.uint8, device=d)
    pst = nv.qadamw_step_params(1e-3, 0.9, 0.95, 1e-8, 0.01, m_rht_seed=3, m_sr_seed=4, v_seed=5)
    # one step from the zero state gives the states every replayed step reads
    z = nv.QTensor(torch.zeros((256, 256), dtype=torch.uint8, device=d),
                   torch.zeros((256, 32), dtype=torch.uint8, device=d), torch.ones((1,), device=d))
    zmu = torch.zeros((16, 32), dtype=torch.int16, device=d)
    w = w0.clone()
    m, mu, v = nv.qadamw_step(w, grad, z, zmu, z, pst)
    torch.cuda.synchronize()
    m2, v2 = nv.QTensor.empty(256, 512, d), nv.QTensor.empty(256, 512, d)
    mu2 = torch.empty_like(mu)
    wss = torch.empty(max(nv.qadamw_step_workspace_bytes(256, 512), 16), dtype=torch.uint8, device=d)

    def chain():
        nv.nvfp4_gemm_bf16(qa, qb, out=H, tile_amax=T)
        nv.nvfp4_quantize(H, P(rowwise=True), qh, None, amax_parts=T)
        nv.nvfp4_gemm(qe, qf, out=C)
        nv.nvfp4_quantize(G, psr, qg[0], qg[1], wsg)
        nv.qadamw_step(w, grad, m, mu, v, pst, m2, mu2, v2, wss)

    outs = lambda: [H, T, qh.codes, qh.scales, qh.gscale, C, qg[0].codes, qg[0].scales, qg[1].codes,
                    qg[1].scales, w, m2.codes, m2.scales, mu2, v2.codes, v2.scales]

    w.copy_(w0)
    chain()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs()]
    s = torch.cuda.Stream(device=d)
    s.wait_stream(torch.cuda.current_stream(d))
    with torch.cuda.stream(s):
        w.copy_(w0)
        chain()
    torch.cuda.current_stream(d).wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain()
    torch.cuda.synchronize()
    for rep in range(3):
        for o in outs():
            o.zero_()
        T.fill_(-1.0)
        w.copy_(w0)
        nv.nvfp4_gemm(qe, qf)                     # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, (o, r) in enumerate(zip(outs(), ref)):
            assert torch.equal(o, r), f"replay {rep}: output {k} differs from the eager run"
