"""Every entry point captured in a HIP graph and replayed: each replay, with
eager work and synchronisations between replays, must reproduce the eager
result bit for bit (the kernels are deterministic and take no host state)."""
import numpy as np
import pytest

import synth
from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a HIP device")]


def test_graph_replays_match_eager():
    import torch
    import weight_quantized_decode_q8_amd as qg

    dev = "cuda"
    # Q2 with split-K (partials + reduce), g128
    M2, K2 = 5120, 17408
    blob, x = synth.q2_inputs(M2, K2, 128, seed=31)
    W2 = qg.Q2Weight.from_blocks(blob, M2, K2, 128)
    x_d = torch.from_numpy(x).to(dev)
    xq = torch.empty(K2, dtype=torch.int8, device=dev)
    sc = torch.empty(1, dtype=torch.float32, device=dev)
    suma = torch.empty(K2 // 64, dtype=torch.int32, device=dev)
    y2 = torch.empty(M2, dtype=torch.float32, device=dev)
    ws2 = torch.empty(max(1, qg.qgemv_q2_ws_bytes(M2, K2, 128, 4)), dtype=torch.uint8, device=dev)
    # q8_row GEMV
    q, rs, xs = synth.q8row_inputs(1000, 1028, seed=32)
    W8 = qg.Q8RowWeight.from_host(q, rs)
    xs_d = torch.from_numpy(xs).to(dev)
    y8 = torch.empty(1000, dtype=torch.float32, device=dev)
    # batched GEMM, auto limbs, with one outlier row (both limb paths)
    qb, rsb, xsb = synth.q8gemm_inputs(256, 600, 2048, seed=33)
    xsb[200, 5] = 4000.0
    Wb = qg.Q8RowWeight.from_host(qb, rsb)
    xsb_d = torch.from_numpy(xsb).to(dev)
    yb = torch.empty((256, 600), dtype=torch.float32, device=dev)
    wsb = torch.empty(qg.qgemm_q8row_batched_ws_bytes(256, 2048), dtype=torch.uint8, device=dev)

    # column prescale and the batched product that forms it (second workspace)
    gg, uu, cc = (torch.from_numpy(a).to(dev) for a in synth.gate_inputs(256, 2048, seed=34))
    act = torch.empty((256, 2048), dtype=torch.float32, device=dev)
    ys = torch.empty((256, 600), dtype=torch.float32, device=dev)
    wss = torch.empty(qg.qgemm_q8row_batched_ws_bytes(256, 2048), dtype=torch.uint8, device=dev)

    def path():
        qg.qquant_act_i8(x_d, xq, sc, suma)
        qg.qgemv_q2(W2, xq, suma, sc, y2, ws2, split_k=4)
        W8.gemv(xs_d, y8)
        qg.qgemm_q8row_batched(Wb.packed, Wb.rs, xsb_d, yb, 256, 600, 2048, wsb, xs_limbs=0)
        qg.qact_silu_mul_pre(gg, uu, cc, act)
        qg.qgemm_q8row_batched_silu(Wb.packed, Wb.rs, gg, uu, cc, ys, 256, 600, 2048, wss, xs_limbs=0)

    path()
    torch.cuda.synchronize()
    outs = (xq, sc, suma, y2, y8, yb, act, ys)
    ref = [t.clone() for t in outs]

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        path()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        path()
    for rep in range(4):
        for t in outs:   # eager work between replays
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("xq", "act_scale", "suma", "y_q2", "y_q8", "y_gemm", "act", "y_gemm_silu"),
                              outs, ref):
            assert torch.equal(t, r), f"replay {rep}: {name} differs from the eager result"
    assert np.isfinite(yb.cpu().numpy()).all()


def test_graph_replays_fused_forms():
    """The fused FFN forms and a batched launch, captured and replayed."""
    import torch
    import weight_quantized_decode_q8_amd as qg

    dev = "cuda"
    D, F = 1024, 2048
    rng = np.random.Generator(np.random.PCG64(41))
    h = torch.from_numpy(rng.standard_normal(D).astype(np.float32)).to(dev)
    nw = torch.from_numpy((1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32)).to(dev)
    Wg = qg.Q2Weight.from_blocks(synth.q2_inputs(F, D, 128, seed=42)[0], F, D, 128)
    Wu = qg.Q2Weight.from_blocks(synth.q2_inputs(F, D, 128, seed=43)[0], F, D, 128)
    Wd = qg.Q2Weight.from_blocks(synth.q2_inputs(D, F, 128, seed=44)[0], D, F, 128)
    Wx = [qg.Q2Weight.from_blocks(synth.q2_inputs(300 + 64 * n, D, 128, seed=45 + n)[0], 300 + 64 * n, D, 128)
          for n in range(3)]
    xq1 = torch.empty(D, dtype=torch.int8, device=dev)
    sc1 = torch.empty(1, device=dev)
    su1 = torch.empty(D // 64, dtype=torch.int32, device=dev)
    g = torch.empty(F, device=dev)
    u = torch.empty(F, device=dev)
    t = torch.empty(F, device=dev)
    xq2 = torch.empty(F, dtype=torch.int8, device=dev)
    sc2 = torch.empty(1, device=dev)
    su2 = torch.empty(F // 64, dtype=torch.int32, device=dev)
    hout = torch.empty(D, device=dev)
    ys = [torch.empty(W.M, device=dev) for W in Wx]
    ws_gu = torch.empty(max(1, qg.qgemv_q2_dual_ws_bytes(F, D, 128, 2)), dtype=torch.uint8, device=dev)
    ws_d = torch.empty(max(1, qg.qgemv_q2_ws_bytes(D, F, 128, 2)), dtype=torch.uint8, device=dev)

    t2 = torch.empty(F, device=dev)
    xq3 = torch.empty(F, dtype=torch.int8, device=dev)
    sc3 = torch.empty(1, device=dev)
    su3 = torch.empty(F // 64, dtype=torch.int32, device=dev)
    # the two-launch block: producers and split reduce inside the GEMV launches
    # (workspaces zero-filled once; every replay must leave them zero again)
    t4 = torch.empty(F, device=dev)
    h4 = torch.empty(D, device=dev)
    g5 = torch.empty(F, device=dev)
    u5 = torch.empty(F, device=dev)
    ws_glu = qg.qgemv_q2_gate_up_glu_x_workspace(F, dev)
    ws_x = qg.qgemv_q2_x_workspace(D, F, 128, 3, dev)

    def path():
        qg.qgemv_q2_gate_up_glu_x(Wg, Wu, h, qg.QG_GLU_SILU, t4, ws_glu, norm_w=nw, eps=1e-6)
        qg.qgemv_q2_x(Wd, t4, h4, accum=h, ws=ws_x, split_k=3)
        qg.qgemv_q2_dual_x(Wg, Wu, h, g5, u5, norm_w=nw, eps=1e-6)
        qg.qquant_rmsnorm_i8(h, nw, 1e-6, xq1, sc1, su1)
        qg.qgemv_q2_gate_up_glu(Wg, Wu, xq1, su1, sc1, qg.QG_GLU_SILU, t2, xq3, sc3, su3)
        qg.qgemv_q2_dual(Wg, Wu, xq1, su1, sc1, g, u, ws_gu, split_k=2)
        qg.qquant_glu_i8(g, u, qg.QG_GLU_SILU, t, xq2, sc2, su2)
        qg.qgemv_q2_accum(Wd, xq2, su2, sc2, h, hout, ws_d, split_k=2)
        qg.qgemv_q2_batch([(W, xq1, su1, sc1, y) + ((h[:W.M],) if W.M <= D and n == 0 else ())
                           for n, (W, y) in enumerate(zip(Wx, ys))])

    outs = (xq1, sc1, su1, g, u, t, xq2, sc2, su2, hout, t2, xq3, sc3, su3, *ys, t4, h4, g5, u5)
    path()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        path()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        path()
    for rep in range(4):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o, r), f"replay {rep}: output {n} differs from the eager result"
        assert int(torch.count_nonzero(ws_glu).item()) == 0 and int(torch.count_nonzero(ws_x).item()) == 0, \
            f"replay {rep}: a workspace was not left all zero"
        # eager work on the same workspaces between replays
        qg.qgemv_q2_x(Wd, t4, h4, accum=h, ws=ws_x, split_k=2)
    torch.cuda.synchronize()
    assert torch.equal(t4, t2), "the two-launch block's t differs from the fused kernel's"


def test_graph_replays_prefill_forms():
    """Row-batched producers and the batched Q2 product (with a K split), captured and replayed."""
    import torch
    import weight_quantized_decode_q8_amd as qg

    dev = "cuda"
    nb, D, F = 40, 1024, 2048
    rng = np.random.Generator(np.random.PCG64(51))
    H = torch.from_numpy(rng.standard_normal((nb, D)).astype(np.float32)).to(dev)
    nw = torch.from_numpy((1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32)).to(dev)
    Wg = qg.Q2Weight.from_blocks(synth.q2_inputs(F, D, 64, seed=52)[0], F, D, 64)
    Wd = qg.Q2Weight.from_blocks(synth.q2_inputs(D, F, 64, seed=53)[0], D, F, 64)
    xq1 = torch.empty((nb, D), dtype=torch.int8, device=dev)
    sc1 = torch.empty(nb, device=dev)
    su1 = torch.empty((nb, D // 64), dtype=torch.int32, device=dev)
    G = torch.empty((nb, F), device=dev)
    xq2 = torch.empty((nb, F), dtype=torch.int8, device=dev)
    sc2 = torch.empty(nb, device=dev)
    su2 = torch.empty((nb, F // 64), dtype=torch.int32, device=dev)
    Hout = torch.empty((nb, D), device=dev)
    ws1 = torch.empty(max(1, qg.qgemm_q2_batched_ws_bytes(F, D, 64, nb)), dtype=torch.uint8, device=dev)
    ws2 = torch.empty(max(1, qg.qgemm_q2_batched_ws_bytes(D, F, 64, nb)), dtype=torch.uint8, device=dev)
    assert qg.qgemm_q2_batched_ws_bytes(D, F, 64, nb) > 0

    Wu = qg.Q2Weight.from_blocks(synth.q2_inputs(F, D, 64, seed=54)[0], F, D, 64)
    U = torch.empty((nb, F), device=dev)
    G2 = torch.empty((nb, F), device=dev)
    ws3 = torch.empty(max(1, qg.qgemm_q2_batched_dual_ws_bytes(F, D, 64, nb)), dtype=torch.uint8, device=dev)

    def path():
        qg.qquant_rmsnorm_i8_rows(H, nw, 1e-6, xq1, sc1, su1)
        qg.qgemm_q2_batched(Wg, xq1, su1, sc1, G, ws=ws1)
        qg.qgemm_q2_batched_dual(Wg, Wu, xq1, su1, sc1, G2, U, ws=ws3)
        qg.qquant_glu_i8_rows(G, G, qg.QG_GLU_SIGMOID, G, xq2, sc2, su2)
        qg.qgemm_q2_batched(Wd, xq2, su2, sc2, Hout, accum=H, ws=ws2)

    outs = (xq1, sc1, su1, G, xq2, sc2, su2, Hout, G2, U)
    path()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        path()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        path()
    for rep in range(4):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for n, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o, r), f"replay {rep}: output {n} differs from the eager result"
