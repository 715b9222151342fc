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
