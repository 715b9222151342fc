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

    def path():
        qg.qquant_act_i8(x_d, xq, sc, suma)
        qg.qgemv_q2(W2, xq, suma, sc, y2, ws2, split_k=4)
        W8.gemv(xs_d, y8)
        qg.qgemm_q8row_batched(Wb.packed, Wb.rs, xsb_d, yb, 256, 600, 2048, wsb, xs_limbs=0)

    path()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (xq, sc, suma, y2, y8, yb)]

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
        for t in (xq, sc, suma, y2, y8, yb):   # eager work between replays
            t.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("xq", "act_scale", "suma", "y_q2", "y_q8", "y_gemm"),
                              (xq, sc, suma, y2, y8, yb), ref):
            assert torch.equal(t, r), f"replay {rep}: {name} differs from the eager result"
    assert np.isfinite(yb.cpu().numpy()).all()
