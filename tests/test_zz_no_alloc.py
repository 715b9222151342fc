"""qgemv_q2_noalloc: the Q2 GEMV whose split-K partials live in the library's
static device scratch instead of a caller workspace.

Its output must equal qgemv_q2 with the same split and its own workspace,
bit for bit, and stay within the oracle's bound.  Two calls in a row (the
second on a smaller matrix, whose partials overwrite only part of what the
first left in the scratch), then the first shape again.
"""
import numpy as np
import pytest

import oracle
import synth
from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a HIP device")]


def _run(m, blob, M, K, group, x, split_k):
    import torch
    W = m.Q2Weight.from_blocks(blob, M, K, group)
    xs = torch.from_numpy(x).to("cuda")
    xq = torch.empty(K, dtype=torch.int8, device="cuda")
    sc = torch.empty(1, dtype=torch.float32, device="cuda")
    suma = torch.empty(K // 64, dtype=torch.int32, device="cuda")
    m.qquant_act_i8(xs, xq, sc, suma)
    y_ws = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    nws = m.qgemv_q2_ws_bytes(M, K, group, split_k)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda") if nws else None
    m.qgemv_q2(W, xq, suma, sc, y_ws, ws, split_k)
    y_na = torch.full((M,), float("nan"), dtype=torch.float32, device="cuda")
    m.qgemv_q2_noalloc(W, xq, suma, sc, y_na, split_k)
    torch.cuda.synchronize()
    return y_ws.cpu().numpy(), y_na.cpu().numpy(), xq.cpu().numpy(), sc.cpu().numpy()[0]


def _check(m, blob, M, K, group, x, split_k, rows, what):
    y_ws, y_na, xq, sc = _run(m, blob, M, K, group, x, split_k)
    assert np.array_equal(y_na.view(np.uint32), y_ws.view(np.uint32)), f"{what}: differs from qgemv_q2"
    yref, mass = oracle.q2_gemv(blob, M, K, group, xq, sc, rows=rows)
    got = y_na if rows is None else y_na[rows]
    err = np.abs(got.astype(np.float64) - yref)
    assert np.all(err <= 2e-5 * mass), f"{what}: max err/bound {np.max(err / (2e-5 * mass))}"


def test_noalloc_matches_workspace_entry_two_calls():
    import weight_quantized_decode_q8_amd as m
    print("qgemv_q2_noalloc: down 5120x17408 g128 split 3, then 300x2048 g64 split 4", flush=True)
    blob, x = synth.config_inputs("q2_g128_down_5120x17408")
    rng = synth.rng_for(515)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(5120 - 64, 5120), rng.integers(0, 5120, 400)]))
    _check(m, blob, 5120, 17408, 128, x, 3, rows, "down, split 3")
    blob2, x2 = synth.q2_inputs(300, 2048, 64, seed=516)
    _check(m, blob2, 300, 2048, 64, x2, 4, None, "300x2048, split 4")
    # auto split on the first shape again (the scratch now holds the second call's partials)
    _check(m, blob, 5120, 17408, 128, x, 0, rows, "down, auto split")


@pytest.mark.parametrize("M,K,group,split_k", [(1, 64, 64, 1), (65, 192, 64, 3), (129, 1024, 128, 16),
                                               (4096, 4096, 64, 0)])
def test_noalloc_shapes(M, K, group, split_k):
    import weight_quantized_decode_q8_amd as m
    print(f"qgemv_q2_noalloc {M}x{K} g{group} split {split_k}", flush=True)
    blob, x = synth.q2_inputs(M, K, group, seed=M + K + split_k)
    _check(m, blob, M, K, group, x, split_k, None, f"{M}x{K} g{group} split {split_k}")


def test_noalloc_rejects_partials_beyond_the_scratch():
    import torch
    import weight_quantized_decode_q8_amd as m
    M, K = 16400, 4096
    W = m.Q2Weight(torch.empty(m.lib().qg_q2_codes_bytes(M, K), dtype=torch.uint8, device="cuda"),
                   torch.empty(M * K // 64, dtype=torch.int16, device="cuda"), M, K, 64)
    xq = torch.zeros(K, dtype=torch.int8, device="cuda")
    sc = torch.zeros(1, dtype=torch.float32, device="cuda")
    suma = torch.zeros(K // 64, dtype=torch.int32, device="cuda")
    y = torch.empty(M, dtype=torch.float32, device="cuda")
    with pytest.raises(m.QGError, match="static scratch"):
        m.qgemv_q2_noalloc(W, xq, suma, sc, y, 16)
