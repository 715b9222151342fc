"""The balanced q8_row GEMV (qgemv_q8row_balanced) through the C-ABI: the row
tiles past the last full round over the 256 CUs are split along K and their
pieces' row sums meet in a workspace.  Outputs of the full rounds' tiles
must equal qgemv_q8row bit for bit, every output must be within
|y - y_ref| <= 2e-5 * sum_i |w_i x_i| of the fp64 oracle, and the workspace
must be left all zero."""
import numpy as np
import pytest

import oracle
import synth
from conftest import gpu_available
from test_gpu_canary import Guarded, check, ws_guarded
from test_gpu_parity import dev, host, qg, within

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a HIP device")]


def bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def run_both(W, xs, ws):
    import torch
    y0 = torch.full((W.M,), float("nan"), device="cuda")
    y1 = torch.full((W.M,), float("nan"), device="cuda")
    W.gemv(dev(xs), y0)
    W.gemv_balanced(dev(xs), y1, ws)
    return host(y0), host(y1)


def full_rows(M, K):
    """Rows of the tiles that run as whole tiles in the balanced launch."""
    tiles = -(-M // 64)
    n = qg().lib().qgemv_q8row_balanced_ws_bytes(M, K)
    rest = tiles % 256 if n else 0
    return min(M, (tiles - rest) * 64)


@pytest.mark.parametrize("M,K", [(100, 512), (64 * 256, 512), (64 * 257, 1024), (64 * 300 + 17, 2052),
                                 (64 * 511, 96), (64 * 600 + 5, 5120)])
def test_balanced_matches_plain_and_oracle(M, K):
    import torch
    q, rs, xs = synth.q8row_inputs(M, K, seed=M + K + 11)
    W = qg().Q8RowWeight.from_host(q, rs)
    ws = W.workspace()
    y0, y1 = run_both(W, xs, ws)
    f = full_rows(M, K)
    assert np.array_equal(bits(y1[:f]), bits(y0[:f])), "full-round tiles differ from qgemv_q8row"
    yref, mass = oracle.q8row_gemv(q, rs, xs)
    within(y1, yref, mass, what=f"balanced q8_row {M}x{K}")
    if ws is not None:
        assert int(torch.count_nonzero(ws).item()) == 0, "workspace not left all zero"


def test_balanced_lm_head_as_benched():
    """The 248320 x 5120 lm_head (3880 tiles: 3840 in full rounds, 40 split
    7 ways): sampled rows of every part against the oracle, the full-round
    rows against qgemv_q8row bit for bit; two calls on one workspace."""
    import torch
    q, rs, xs = synth.config_inputs("q8row_lm_head_248320x5120")
    W = qg().Q8RowWeight.from_host(q, rs)
    M, K = q.shape
    assert qg().lib().qgemv_q8row_balanced_ws_bytes(M, K) == 256 + 40 * 7 * 64 * 4
    ws = W.workspace()
    y0, y1 = run_both(W, xs, ws)
    y1b = torch.empty(M, device="cuda")
    W.gemv_balanced(dev(xs), y1b, ws)
    y1b = host(y1b)
    assert np.array_equal(bits(y1), bits(y1b)), "second call on the same workspace differs"
    assert np.array_equal(bits(y1[:3840 * 64]), bits(y0[:3840 * 64]))
    rows = np.unique(np.concatenate([np.arange(0, M, 4099), np.arange(3840 * 64, M, 7), [M - 1]]))
    yref, mass = oracle.q8row_gemv(q, rs, xs, rows=rows)
    within(y1[rows], yref, mass, what="balanced lm_head sampled")
    assert int(torch.count_nonzero(ws).item()) == 0


@pytest.mark.parametrize("M,K", [(64 * 257, 1024), (64 * 300 + 17, 2052)])
def test_balanced_canary(M, K):
    """Nothing written outside y and the workspace (guard regions)."""
    import torch
    q, rs, xs = synth.q8row_inputs(M, K, seed=M + 5)
    W = qg().Q8RowWeight.from_host(q, rs)
    y = Guarded(M, torch.float32)
    ws = ws_guarded(qg().lib().qgemv_q8row_balanced_ws_bytes(M, K))
    ws.t.zero_()
    W.gemv_balanced(dev(xs), y.t, ws.t)
    check(y, ws)
    assert int(torch.count_nonzero(ws.t).item()) == 0


def test_balanced_graph_replays():
    """Captured in a HIP graph and replayed with eager calls on the same
    workspace in between: every replay gives the eager result bit for bit and
    leaves the workspace all zero."""
    import torch
    M, K = 64 * 300 + 17, 2052
    q, rs, xs = synth.q8row_inputs(M, K, seed=77)
    W = qg().Q8RowWeight.from_host(q, rs)
    ws = W.workspace()
    xd = dev(xs)
    y = torch.empty(M, device="cuda")
    W.gemv_balanced(xd, y, ws)
    torch.cuda.synchronize()
    ref = y.clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        W.gemv_balanced(xd, y, ws)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        W.gemv_balanced(xd, y, ws)
    for rep in range(4):
        y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"replay {rep} differs from the eager result"
        assert int(torch.count_nonzero(ws).item()) == 0, f"replay {rep} left the workspace non-zero"
        W.gemv_balanced(xd, y, ws)  # eager call on the same workspace between replays
