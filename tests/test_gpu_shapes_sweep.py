"""A seeded sweep over random valid shapes for every product: rows not a
multiple of 64, K tails, both group sizes, every split factor, token counts
around the 128-row tiles, each limb mode; every output against the oracle
(integer outputs bit for bit, f32 within |y - y_ref| <= 2e-5 sum_i |w_i x_i|).

QG_SWEEP_CASES sets the number of seeds per product (default 24); case n
always draws the same shape, so a longer run extends the default one."""
import os

import numpy as np
import pytest

import oracle
import synth
from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a HIP device")]

REL = 2e-5
N_CASES = int(os.environ.get("QG_SWEEP_CASES", "24"))


def _within(y, yref, mass, what):
    err = np.abs(np.asarray(y, np.float64) - yref)
    bad = ~(err <= REL * mass)
    assert not bad.any(), f"{what}: {int(bad.sum())} outputs outside the bound"


@pytest.mark.parametrize("case", range(N_CASES))
def test_sweep_q8row_gemv(case):
    import torch
    import weight_quantized_decode_q8_amd as qg
    r = synth.rng_for(30000 + case)
    M = int(r.integers(1, 700))
    K = 4 * int(r.integers(1, 1500))
    q, rs, xs = synth.q8row_inputs(M, K, rng=r)
    W = qg.Q8RowWeight.from_host(q, rs)
    y = torch.empty(M, device="cuda")
    W.gemv(torch.from_numpy(xs).cuda(), y)
    yref, mass = oracle.q8row_gemv(q, rs, xs)
    _within(y.cpu().numpy(), yref, mass, f"q8row M={M} K={K}")


@pytest.mark.parametrize("case", range(N_CASES))
def test_sweep_q2_gemv(case):
    import torch
    import weight_quantized_decode_q8_amd as qg
    r = synth.rng_for(31000 + case)
    group = int(r.choice([64, 128]))
    M = int(r.integers(1, 900))
    K = group * int(r.integers(1, 40))
    split = int(r.integers(0, 17))
    blob, x = synth.q2_inputs(M, K, group, seed=31500 + case)
    W = qg.Q2Weight.from_blocks(blob, M, K, group)
    xq = torch.empty(K, dtype=torch.int8, device="cuda")
    sc = torch.empty(1, device="cuda")
    su = torch.empty(K // 64, dtype=torch.int32, device="cuda")
    qg.qquant_act_i8(torch.from_numpy(x).cuda(), xq, sc, su)
    ws = torch.empty(max(1, qg.qgemv_q2_ws_bytes(M, K, group, split)), dtype=torch.uint8, device="cuda")
    y = torch.empty(M, device="cuda")
    dots = torch.empty((M, K // 64), dtype=torch.int32, device="cuda")
    qg.qgemv_q2_dots(W, xq, su, sc, y, dots, ws, split_k=split)
    rq, rsc, rsu = oracle.act_quant_i8(x)
    assert np.array_equal(xq.cpu().numpy(), rq) and np.array_equal(su.cpu().numpy(), rsu)
    assert np.array_equal(dots.cpu().numpy(), oracle.q2_dots(blob, M, K, group, rq))
    yref, mass = oracle.q2_gemv(blob, M, K, group, rq, rsc)
    _within(y.cpu().numpy(), yref, mass, f"q2 M={M} K={K} g{group} split {split}")


@pytest.mark.parametrize("case", range(N_CASES))
def test_sweep_q2_product(case):
    import torch
    import weight_quantized_decode_q8_amd as qg
    r = synth.rng_for(32000 + case)
    group = int(r.choice([64, 128]))
    nb = int(r.integers(1, 300))
    M = int(r.integers(1, 700))
    K = group * int(r.integers(1, 24))
    blob, _ = synth.q2_inputs(M, K, group, seed=32500 + case)
    W = qg.Q2Weight.from_blocks(blob, M, K, group)
    X = (r.standard_normal((nb, K)) * r.uniform(0.1, 10.0, (nb, 1))).astype(np.float32)
    xq = torch.empty((nb, K), dtype=torch.int8, device="cuda")
    sc = torch.empty(nb, device="cuda")
    su = torch.empty((nb, K // 64), dtype=torch.int32, device="cuda")
    qg.qquant_act_i8_rows(torch.from_numpy(X).cuda(), xq, sc, su)
    n = qg.qgemm_q2_batched_ws_bytes(M, K, group, nb)
    y = torch.empty((nb, M), device="cuda")
    qg.qgemm_q2_batched(W, xq, su, sc, y, ws=torch.empty(n, dtype=torch.uint8, device="cuda") if n else None)
    xq_h, sc_h = xq.cpu().numpy(), sc.cpu().numpy()
    yref, mass = oracle.q2_gemm(blob, M, K, group, xq_h, sc_h)
    _within(y.cpu().numpy(), yref, mass, f"q2 product nb={nb} M={M} K={K} g{group}")


@pytest.mark.parametrize("case", range(N_CASES))
def test_sweep_q8row_gemm(case):
    import torch
    import weight_quantized_decode_q8_amd as qg
    r = synth.rng_for(33000 + case)
    nb = int(r.integers(1, 300))
    M = int(r.integers(1, 600))
    K = 4 * int(r.integers(1, 600))
    limbs = int(r.choice([0, 3]))
    q, rs, _ = synth.q8row_inputs(M, K, rng=r)
    xs = (r.standard_normal((nb, K)) * r.uniform(0.01, 100.0, (nb, 1))).astype(np.float32)
    W = qg.Q8RowWeight.from_host(q, rs)
    y = torch.empty((nb, M), device="cuda")
    ws = torch.empty(qg.qgemm_q8row_batched_ws_bytes(nb, K), dtype=torch.uint8, device="cuda")
    qg.qgemm_q8row_batched(W.packed, W.rs, torch.from_numpy(xs).cuda(), y, nb, M, K, ws, xs_limbs=limbs)
    yref, mass = oracle.q8row_gemm(q, rs, xs)
    _within(y.cpu().numpy(), yref, mass, f"gemm nb={nb} M={M} K={K} limbs={limbs}")


@pytest.mark.parametrize("case", range(N_CASES))
def test_sweep_producers(case):
    """RMSNorm + quantiser and the gated products + quantiser over random row
    counts, lengths and scales: every code, scale and group sum bit for bit."""
    import torch
    import weight_quantized_decode_q8_amd as qg
    r = synth.rng_for(34000 + case)
    nb = int(r.integers(1, 40))
    K = 64 * int(r.integers(1, 300))
    kind = int(r.integers(0, 2))
    eps = float(r.choice([0.0, 1e-6, 1e-5]))
    X = (r.standard_normal((nb, K)) * r.uniform(0.01, 30.0, (nb, 1))).astype(np.float32)
    G = (2.5 * r.standard_normal((nb, K))).astype(np.float32)
    w = (1.0 + 0.1 * r.standard_normal(K)).astype(np.float32)
    xq = torch.empty((nb, K), dtype=torch.int8, device="cuda")
    sc = torch.empty(nb, device="cuda")
    su = torch.empty((nb, K // 64), dtype=torch.int32, device="cuda")
    qg.qquant_rmsnorm_i8_rows(torch.from_numpy(X).cuda(), torch.from_numpy(w).cuda(), eps, xq, sc, su)
    xq_h, sc_h, su_h = xq.cpu().numpy(), sc.cpu().numpy(), su.cpu().numpy()
    for b in range(nb):
        _, rq, rsc, rsu = oracle.rmsnorm_quant_i8(X[b], w, eps)
        assert np.array_equal(xq_h[b], rq) and sc_h[b] == rsc and np.array_equal(su_h[b], rsu), f"rmsnorm row {b}"
    t = torch.empty((nb, K), device="cuda")
    qg.qquant_glu_i8_rows(torch.from_numpy(G).cuda(), torch.from_numpy(X).cuda(), kind, t, xq, sc, su)
    t_h, xq_h, sc_h, su_h = t.cpu().numpy(), xq.cpu().numpy(), sc.cpu().numpy(), su.cpu().numpy()
    for b in range(nb):
        rt, rq, rsc, rsu = oracle.glu_quant_i8(G[b], X[b], kind)
        assert np.array_equal(t_h[b].view(np.uint32), rt.view(np.uint32)), f"gated product row {b}"
        assert np.array_equal(xq_h[b], rq) and sc_h[b] == rsc and np.array_equal(su_h[b], rsu), f"glu row {b}"


@pytest.mark.parametrize("case", range(N_CASES // 2))
def test_sweep_q2_batch_jobs(case):
    """Random job tables for the batched GEMV launch: own shapes, activations
    and residuals, one group size per launch."""
    import torch
    import weight_quantized_decode_q8_amd as qg
    r = synth.rng_for(35000 + case)
    group = int(r.choice([64, 128]))
    njobs = int(r.integers(1, 17))
    jobs, refs = [], []
    for j in range(njobs):
        M = int(r.integers(1, 500))
        K = group * int(r.integers(1, 20))
        blob, x = synth.q2_inputs(M, K, group, seed=35500 + 100 * case + j)
        W = qg.Q2Weight.from_blocks(blob, M, K, group)
        xq = torch.empty(K, dtype=torch.int8, device="cuda")
        sc = torch.empty(1, device="cuda")
        su = torch.empty(K // 64, dtype=torch.int32, device="cuda")
        qg.qquant_act_i8(torch.from_numpy(x).cuda(), xq, sc, su)
        y = torch.empty(M, device="cuda")
        acc = r.standard_normal(M).astype(np.float32) if r.random() < 0.5 else None
        jobs.append((W, xq, su, sc, y) + ((torch.from_numpy(acc).cuda(),) if acc is not None else ()))
        refs.append((blob, M, K, x, acc, y))
    qg.qgemv_q2_batch(jobs)
    for blob, M, K, x, acc, y in refs:
        rq, rsc, _ = oracle.act_quant_i8(x)
        if acc is None:
            yref, mass = oracle.q2_gemv(blob, M, K, group, rq, rsc)
            _within(y.cpu().numpy(), yref, mass, f"batch job {M}x{K}")
        else:
            yref, mass = oracle.q2_gemv_accum(blob, M, K, group, rq, rsc, acc)
            err = np.abs(y.cpu().numpy().astype(np.float64) - yref)
            assert np.all(err <= REL * mass + 2.0 ** -24 * np.abs(yref)), f"batch job with residual {M}x{K}"


@pytest.mark.parametrize("case", range(N_CASES))
def test_sweep_q2_in_launch_forms(case):
    """qgemv_q2_x (random split, residual or not), qgemv_q2_dual_x and
    qgemv_q2_gate_up_glu_x (with or without the RMSNorm) on random shapes, one
    shared workspace per form across the sweep's calls: each output against
    the oracle on the oracle's own quantised vector, the workspaces left zero."""
    import torch
    import weight_quantized_decode_q8_amd as qg
    r = synth.rng_for(36000 + case)
    group = int(r.choice([64, 128]))
    M = int(r.integers(1, 1400))
    K = group * int(r.integers(1, 60))
    split = int(r.integers(0, 17))
    blob, x = synth.q2_inputs(M, K, group, seed=36500 + case)
    b1, _ = synth.q2_inputs(M, K, group, seed=36700 + case)
    W = qg.Q2Weight.from_blocks(blob, M, K, group)
    W1 = qg.Q2Weight.from_blocks(b1, M, K, group)
    xd = torch.from_numpy(x).cuda()
    rq, rsc, _ = oracle.act_quant_i8(x)
    ws = qg.qgemv_q2_x_workspace(M, K, group, split)
    acc = synth.rng_for(36900 + case).standard_normal(M).astype(np.float32) if case % 2 else None
    y = torch.empty(M, device="cuda")
    qg.qgemv_q2_x(W, xd, y, accum=None if acc is None else torch.from_numpy(acc).cuda(), ws=ws, split_k=split)
    if acc is None:
        yref, mass = oracle.q2_gemv(blob, M, K, group, rq, rsc)
    else:
        yref, mass = oracle.q2_gemv_accum(blob, M, K, group, rq, rsc, acc)
        mass = mass + (2.0 ** -24 / REL) * np.abs(yref)
    _within(y.cpu().numpy(), yref, mass, f"qgemv_q2_x M={M} K={K} g{group} split={split}")
    if ws is not None:
        assert int(torch.count_nonzero(ws).item()) == 0
    norm = (case % 3 == 0) and K <= 16384
    nw = (1.0 + 0.1 * synth.rng_for(37000 + case).standard_normal(K)).astype(np.float32)
    if norm:
        _, rq, rsc, _ = oracle.rmsnorm_quant_i8(x, nw, 1e-6)
    y0, y1 = torch.empty(M, device="cuda"), torch.empty(M, device="cuda")
    qg.qgemv_q2_dual_x(W, W1, xd, y0, y1, norm_w=torch.from_numpy(nw).cuda() if norm else None, eps=1e-6)
    for b, yy, nm in ((blob, y0, "gate"), (b1, y1, "up")):
        yref, mass = oracle.q2_gemv(b, M, K, group, rq, rsc)
        _within(yy.cpu().numpy(), yref, mass, f"qgemv_q2_dual_x {nm} M={M} K={K} g{group} norm={norm}")
    # the gated product of those two outputs, formed in the launch: the same
    # bits as the product of the dual outputs by the producers' rule
    wsg = qg.qgemv_q2_gate_up_glu_x_workspace(M)
    t = torch.empty(M, device="cuda")
    kind = int(case % 2)
    qg.qgemv_q2_gate_up_glu_x(W, W1, xd, kind, t, wsg, norm_w=torch.from_numpy(nw).cuda() if norm else None, eps=1e-6)
    Mp = -(-M // 64) * 64  # the oracle's producer quantises whole groups: pad g, u with zeros
    gp, up = np.zeros(Mp, np.float32), np.zeros(Mp, np.float32)
    gp[:M], up[:M] = y0.cpu().numpy(), y1.cpu().numpy()
    tref = oracle.glu_quant_i8(gp, up, kind)[0][:M]
    assert np.array_equal(t.cpu().numpy().view(np.uint32), tref.view(np.uint32)), "gated product differs"
    assert int(torch.count_nonzero(wsg).item()) == 0


@pytest.mark.parametrize("case", range(N_CASES // 3))
def test_sweep_q8row_balanced(case):
    """qgemv_q8row_balanced on random row counts past one full round of 256
    tiles and random K (tails included): every output against the oracle."""
    import torch
    import weight_quantized_decode_q8_amd as qg
    r = synth.rng_for(38000 + case)
    M = 64 * 256 + int(r.integers(1, 64 * 300))
    K = 4 * int(r.integers(1, 400))
    q, rs, xs = synth.q8row_inputs(M, K, rng=r)
    W = qg.Q8RowWeight.from_host(q, rs)
    ws = W.workspace()
    y = torch.empty(M, device="cuda")
    W.gemv_balanced(torch.from_numpy(xs).cuda(), y, ws)
    yref, mass = oracle.q8row_gemv(q, rs, xs)
    _within(y.cpu().numpy(), yref, mass, f"q8row balanced M={M} K={K}")
    if ws is not None:
        assert int(torch.count_nonzero(ws).item()) == 0
