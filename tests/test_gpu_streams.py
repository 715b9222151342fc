"""Re-entrancy across streams: the entry points keep no global state, so
independent calls enqueued on three streams at once (each with its own
buffers and workspace) give exactly the results they give one at a time."""
import numpy as np
import pytest

import synth
from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a HIP device")]


def test_concurrent_streams_match_sequential():
    import torch
    import weight_quantized_decode_q8_amd as qg

    dev = "cuda"
    # stream A: Q2 split-K GEMV with its quantiser
    M2, K2 = 5120, 17408
    blob, x = synth.q2_inputs(M2, K2, 128, seed=91)
    W2 = qg.Q2Weight.from_blocks(blob, M2, K2, 128)
    x_d = torch.from_numpy(x).to(dev)
    xq = torch.empty(K2, dtype=torch.int8, device=dev)
    sc = torch.empty(1, device=dev)
    su = torch.empty(K2 // 64, dtype=torch.int32, device=dev)
    y2 = torch.empty(M2, device=dev)
    ws2 = torch.empty(max(1, qg.qgemv_q2_ws_bytes(M2, K2, 128, 4)), dtype=torch.uint8, device=dev)
    # stream B: batched q8_row GEMM (its own workspace)
    q, rs, xs = synth.q8gemm_inputs(256, 600, 2048, seed=92)
    Wb = qg.Q8RowWeight.from_host(q, rs)
    xs_d = torch.from_numpy(xs).to(dev)
    yb = torch.empty((256, 600), device=dev)
    wsb = torch.empty(qg.qgemm_q8row_batched_ws_bytes(256, 2048), dtype=torch.uint8, device=dev)
    # stream C: the same Q2 matrix on other token rows, batched, and a prescale
    X = synth.rng_for(93).standard_normal((64, K2)).astype(np.float32)
    Xd = torch.from_numpy(X).to(dev)
    xqr = torch.empty((64, K2), dtype=torch.int8, device=dev)
    scr = torch.empty(64, device=dev)
    sur = torch.empty((64, K2 // 64), dtype=torch.int32, device=dev)
    yr = torch.empty((64, M2), device=dev)
    wsr = torch.empty(max(1, qg.qgemm_q2_batched_ws_bytes(M2, K2, 128, 64)), dtype=torch.uint8, device=dev)
    g, u, c = (torch.from_numpy(a).to(dev) for a in synth.gate_inputs(64, K2, seed=94))
    act = torch.empty((64, K2), device=dev)

    def work_a(s):
        qg.qquant_act_i8(x_d, xq, sc, su, stream=s)
        qg.qgemv_q2(W2, xq, su, sc, y2, ws2, split_k=4, stream=s)

    def work_b(s):
        qg.qgemm_q8row_batched(Wb.packed, Wb.rs, xs_d, yb, 256, 600, 2048, wsb, stream=s)

    def work_c(s):
        qg.qquant_act_i8_rows(Xd, xqr, scr, sur, stream=s)
        qg.qgemm_q2_batched(W2, xqr, sur, scr, yr, ws=wsr, stream=s)
        qg.qact_silu_mul_pre(g, u, c, act, stream=s)

    outs = (xq, sc, su, y2, yb, xqr, scr, sur, yr, act)
    cur = torch.cuda.current_stream()
    for w in (work_a, work_b, work_c):
        w(cur)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    streams = [torch.cuda.Stream() for _ in range(3)]
    for rep in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        for _ in range(4):  # several rounds in flight at once on the three streams
            for w, s in zip((work_a, work_b, work_c), streams):
                w(s)
        torch.cuda.synchronize()
        for n, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o, r), f"round {rep}: output {n} differs under concurrent streams"


def test_concurrent_streams_one_launch_forms():
    """The one-launch split forms on three streams at once, each stream with
    its own workspaces: qgemv_q2_x with split 3 and a residual, the gate|up
    pair with the SiLU gate and the RMSNorm inside, and the balanced q8_row
    launch; every output as the one-at-a-time result, bit for bit."""
    import torch
    import weight_quantized_decode_q8_amd as qg

    dev = "cuda"
    D, F = 1024, 4096
    Wd = [qg.Q2Weight.from_blocks(synth.q2_inputs(D, F, 128, seed=95 + n)[0], D, F, 128) for n in range(3)]
    Wg = qg.Q2Weight.from_blocks(synth.q2_inputs(F, D, 128, seed=99)[0], F, D, 128)
    Wu = qg.Q2Weight.from_blocks(synth.q2_inputs(F, D, 128, seed=100)[0], F, D, 128)
    r = synth.rng_for(101)
    xs = [torch.from_numpy(r.standard_normal(F).astype(np.float32)).to(dev) for _ in range(3)]
    hs = [torch.from_numpy(r.standard_normal(D).astype(np.float32)).to(dev) for _ in range(3)]
    nw = torch.from_numpy((1.0 + 0.1 * r.standard_normal(D)).astype(np.float32)).to(dev)
    q8, rs8, xs8 = synth.q8row_inputs(64 * 300 + 9, 1028, seed=102)
    W8 = qg.Q8RowWeight.from_host(q8, rs8)
    xs8_d = torch.from_numpy(xs8).to(dev)
    ys = [torch.empty(D, device=dev) for _ in range(3)]
    ts = [torch.empty(F, device=dev) for _ in range(3)]
    y8 = [torch.empty(W8.M, device=dev) for _ in range(3)]
    wsx = [qg.qgemv_q2_x_workspace(D, F, 128, 3, dev) for _ in range(3)]
    wsg = [qg.qgemv_q2_gate_up_glu_x_workspace(F, dev) for _ in range(3)]
    ws8 = [W8.workspace(dev) for _ in range(3)]

    def work(n, s):
        qg.qgemv_q2_x(Wd[n], xs[n], ys[n], accum=hs[n], ws=wsx[n], split_k=3, stream=s)
        qg.qgemv_q2_gate_up_glu_x(Wg, Wu, hs[n], qg.QG_GLU_SILU, ts[n], wsg[n], norm_w=nw, eps=1e-6, stream=s)
        W8.gemv_balanced(xs8_d, y8[n], ws8[n], stream=s)

    outs = ys + ts + y8
    cur = torch.cuda.current_stream()
    for n in range(3):
        work(n, cur)
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    streams = [torch.cuda.Stream() for _ in range(3)]
    for rep in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        for _ in range(4):
            for n, s in enumerate(streams):
                work(n, s)
        torch.cuda.synchronize()
        for k, (o, rr) in enumerate(zip(outs, ref)):
            assert torch.equal(o, rr), f"round {rep}: output {k} differs under concurrent streams"
    for w in wsx + wsg + ws8:
        assert int(torch.count_nonzero(w).item()) == 0
