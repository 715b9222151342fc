"""The in-launch handshakes (split-K partials, the gate|up halves and the
lm_head's split tail meeting through device-scope atomics and per-tile
arrival counters) over many calls from one graph.  Every call's outputs are
kept in a slot of their own and must equal the first eager run bit for bit,
and every workspace must be zero after each replay (a missed or doubled
arrival would leave a count or a partial behind).  The decode FFN launches
run at the benched decode shapes: gate|up 2 x 17408 x 5120 with the
quantiser inside, the 5120 x 17408 down projection with its split 3 inside,
and the fused form with the RMSNorm, the SiLU gate, the tile maxima and the
residual."""
import numpy as np
import pytest

import synth
from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a HIP device")]

STEPS_PER_GRAPH = 100
REPLAYS = 200


def test_decode_ffn_launches_identical_over_20000_graph_steps():
    import torch
    import weight_quantized_decode_q8_amd as qg
    W = {}
    for n in ("q2_g128_gate_17408x5120", "q2_g128_up_17408x5120", "q2_g128_down_5120x17408"):
        c = synth.CONFIGS[n]
        blob, x = synth.config_inputs(n)
        W[n] = (qg.Q2Weight.from_blocks(blob, c["M"], c["K"], c["group"]), torch.from_numpy(x).cuda())
    Wg, xg = W["q2_g128_gate_17408x5120"]
    Wu, _ = W["q2_g128_up_17408x5120"]
    Wd, xd = W["q2_g128_down_5120x17408"]
    F, D = Wg.M, Wg.K
    yg, yu, yd = torch.empty(F, device="cuda"), torch.empty(F, device="cuda"), torch.empty(D, device="cuda")
    rng = np.random.Generator(np.random.PCG64(77))
    h = torch.from_numpy(rng.standard_normal(D).astype(np.float32)).cuda()
    nw = torch.from_numpy((1 + 0.1 * rng.standard_normal(D)).astype(np.float32)).cuda()
    t, tmax, hout = torch.empty(F, device="cuda"), torch.empty(F // 64, device="cuda"), torch.empty(D, device="cuda")
    wsd = qg.qgemv_q2_x_workspace(D, F, 128, 0)
    wsg = qg.qgemv_q2_gate_up_glu_x_workspace(F)
    wsd2 = qg.qgemv_q2_x_workspace(D, F, 128, 0)
    assert qg.qgemv_q2_x_auto_split(D, F, 128) == 3

    def step():
        qg.qgemv_q2_dual_x(Wg, Wu, xg, yg, yu, stream=torch.cuda.current_stream())
        qg.qgemv_q2_x(Wd, xd, yd, ws=wsd, split_k=0, stream=torch.cuda.current_stream())
        qg.qgemv_q2_gate_up_glu_x(Wg, Wu, h, qg.QG_GLU_SILU, t, wsg, norm_w=nw, eps=1e-6, tmax=tmax,
                                  stream=torch.cuda.current_stream())
        qg.qgemv_q2_x(Wd, t, hout, accum=h, ws=wsd2, split_k=0, xmax=tmax, stream=torch.cuda.current_stream())

    outs = (yg, yu, yd, t, hout)
    step()
    torch.cuda.synchronize()
    ref = torch.cat([v.clone() for v in outs])
    slots = torch.empty(STEPS_PER_GRAPH, ref.numel(), device="cuda")

    def keep(k):
        o = 0
        for v in outs:
            slots[k, o:o + v.numel()].copy_(v)
            o += v.numel()

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for k in range(STEPS_PER_GRAPH):
                step()
                keep(k)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        slots.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        diff = (slots != ref.unsqueeze(0)).any(dim=1)
        assert not bool(diff.any()), f"replay {r}: steps {torch.nonzero(diff).flatten().tolist()[:8]} differ"
        for w in (wsd, wsg, wsd2):
            assert int(torch.count_nonzero(w).item()) == 0, f"replay {r}: a workspace is not left zero"


def test_balanced_q8row_split_tail_identical_over_20000_graph_calls():
    """qgemv_q8row_balanced with 296 row tiles (40 past the full round, each
    split 7 ways along K like the 248320-row lm_head's tail, the pieces
    meeting through arrival counters): 20,000 calls from one graph, every
    call's output kept and equal to the first eager call bit for bit, the
    workspace zero after each replay."""
    import torch
    import weight_quantized_decode_q8_amd as qg
    M, K = 64 * 296, 5120
    q, rs, xs = synth.q8row_inputs(M, K, seed=91)
    W = qg.Q8RowWeight.from_host(q, rs)
    x = torch.from_numpy(xs).cuda()
    y = torch.empty(M, device="cuda")
    ws = W.workspace("cuda")
    assert ws is not None and ws.numel() > 0
    W.gemv_balanced(x, y, ws)
    torch.cuda.synchronize()
    ref = y.clone()
    slots = torch.empty(STEPS_PER_GRAPH, M, device="cuda")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for k in range(STEPS_PER_GRAPH):
                W.gemv_balanced(x, y, ws, stream=torch.cuda.current_stream())
                slots[k].copy_(y)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        slots.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        diff = (slots != ref.unsqueeze(0)).any(dim=1)
        assert not bool(diff.any()), f"replay {r}: calls {torch.nonzero(diff).flatten().tolist()[:8]} differ"
        assert int(torch.count_nonzero(ws).item()) == 0, f"replay {r}: the workspace is not left zero"
