"""Out-of-bounds writes: every output and workspace sits in the middle of a
larger buffer whose guard regions hold a bit pattern; each entry point runs
on ragged shapes (rows not a multiple of 64, K tails, token counts not a
multiple of 128) and the guards must come back untouched.  (Reads past an
input are not provoked on purpose; the kernels' read guards are checked by
reading the code and by the parity tests on these shapes.)"""
import numpy as np
import pytest

import synth
from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a HIP device")]

GUARD_BYTES = 1 << 16
PATTERN = 0xA5


class Guarded:
    """A device buffer of n elements of dtype with GUARD_BYTES of pattern on each side."""

    def __init__(self, shape, dtype):
        import torch
        self.shape = tuple(shape) if isinstance(shape, (tuple, list)) else (shape,)
        n = int(np.prod(self.shape))
        esz = torch.empty(0, dtype=dtype).element_size()
        self.g = GUARD_BYTES // esz
        self.raw = torch.full((2 * GUARD_BYTES + n * esz,), PATTERN, dtype=torch.uint8, device="cuda")
        self.t = self.raw[GUARD_BYTES:GUARD_BYTES + n * esz].view(dtype).view(self.shape)
        self.nbytes = n * esz

    def intact(self):
        import torch
        lo = self.raw[:GUARD_BYTES]
        hi = self.raw[GUARD_BYTES + self.nbytes:]
        return bool(torch.all(lo == PATTERN)) and bool(torch.all(hi == PATTERN))


def ws_guarded(nbytes):
    import torch
    return Guarded(max(1, nbytes), torch.uint8)


def check(*bufs):
    import torch
    torch.cuda.synchronize()
    for n, b in enumerate(bufs):
        assert b.intact(), f"buffer {n} (shape {b.shape}): a guard byte was written"


def test_canary_quantisers_and_producers():
    import torch
    import weight_quantized_decode_q8_amd as qg
    for nb, K in ((1, 64), (3, 1088), (130, 192)):
        X = torch.from_numpy(synth.rng_for(nb + K).standard_normal((nb, K)).astype(np.float32)).cuda()
        w = torch.from_numpy((1.0 + 0.1 * synth.rng_for(5).standard_normal(K)).astype(np.float32)).cuda()
        xq, sc, su = Guarded((nb, K), torch.int8), Guarded(nb, torch.float32), Guarded((nb, K // 64), torch.int32)
        qg.qquant_act_i8_rows(X, xq.t, sc.t, su.t)
        check(xq, sc, su)
        qg.qquant_rmsnorm_i8_rows(X, w, 1e-6, xq.t, sc.t, su.t)
        check(xq, sc, su)
        t = Guarded((nb, K), torch.float32)
        qg.qquant_glu_i8_rows(X, X, qg.QG_GLU_SILU, t.t, xq.t, sc.t, su.t)
        check(xq, sc, su, t)
        act = Guarded((nb, K), torch.float32)
        qg.qact_silu_mul_pre(X, X, w, act.t)
        check(act)
    # odd row length for the prescale (scalar path)
    g = torch.from_numpy(synth.rng_for(6).standard_normal((5, 37)).astype(np.float32)).cuda()
    act = Guarded((5, 37), torch.float32)
    qg.qact_silu_mul_pre(g, g, None, act.t)
    check(act)


@pytest.mark.parametrize("M,K", [(1, 4), (100, 1028), (65, 4100)])
def test_canary_q8row_gemv(M, K):
    import torch
    import weight_quantized_decode_q8_amd as qg
    q, rs, xs = synth.q8row_inputs(M, K, seed=M + K)
    W = qg.Q8RowWeight.from_host(q, rs)
    y = Guarded(M, torch.float32)
    W.gemv(torch.from_numpy(xs).cuda(), y.t)
    check(y)


@pytest.mark.parametrize("M,K,group,split", [(100, 1024, 128, 3), (65, 640, 64, 0), (300, 4096, 64, 16), (17408, 640, 64, 0), (128, 1024, 128, 1)])
def test_canary_q2_gemvs(M, K, group, split):
    import torch
    import weight_quantized_decode_q8_amd as qg
    blob, x = synth.q2_inputs(M, K, group, seed=M * 3 + K)
    blob1, _ = synth.q2_inputs(M, K, group, seed=M * 3 + K + 1)
    W, W1 = qg.Q2Weight.from_blocks(blob, M, K, group), qg.Q2Weight.from_blocks(blob1, M, K, group)
    xq = torch.empty(K, dtype=torch.int8, device="cuda")
    sc = torch.empty(1, device="cuda")
    su = torch.empty(K // 64, dtype=torch.int32, device="cuda")
    qg.qquant_act_i8(torch.from_numpy(x).cuda(), xq, sc, su)
    n1 = qg.qgemv_q2_ws_bytes(M, K, group, split)
    ws = ws_guarded(n1)                                    # exactly the one-matrix workspace
    ws2 = ws_guarded(qg.qgemv_q2_dual_ws_bytes(M, K, group, split))
    wsv = ws.t if n1 else None
    y, y1 = Guarded(M, torch.float32), Guarded(M, torch.float32)
    dots = Guarded((M, K // 64), torch.int32)
    qg.qgemv_q2(W, xq, su, sc, y.t, wsv, split_k=split)
    check(y, ws)
    qg.qgemv_q2_dots(W, xq, su, sc, y.t, dots.t, wsv, split_k=split)
    check(y, dots, ws)
    res = torch.ones(M, device="cuda")
    qg.qgemv_q2_accum(W, xq, su, sc, res, y.t, wsv, split_k=split)
    check(y, ws)
    qg.qgemv_q2_dual(W, W1, xq, su, sc, y.t, y1.t, ws2.t if n1 else None, split_k=split)
    check(y, y1, ws2)
    if M % 64 == 0:
        t, xq2 = Guarded(M, torch.float32), Guarded(M, torch.int8)
        sc2, su2 = Guarded(1, torch.float32), Guarded(M // 64, torch.int32)
        qg.qgemv_q2_gate_up_glu(W, W1, xq, su, sc, qg.QG_GLU_SILU, t.t, xq2.t, sc2.t, su2.t)
        check(t, xq2, sc2, su2)
    ys = [Guarded(M, torch.float32) for _ in range(3)]
    qg.qgemv_q2_batch([(W, xq, su, sc, ys[0].t), (W1, xq, su, sc, ys[1].t), (W, xq, su, sc, ys[2].t, res)])
    check(*ys)


@pytest.mark.parametrize("nb,M,K,group", [(3, 100, 1024, 128), (130, 300, 640, 64), (40, 5120 + 64, 2048, 128)])
def test_canary_q2_products(nb, M, K, group):
    import torch
    import weight_quantized_decode_q8_amd as qg
    blob, _ = synth.q2_inputs(M, K, group, seed=nb + M)
    blob1, _ = synth.q2_inputs(M, K, group, seed=nb + M + 1)
    W, W1 = qg.Q2Weight.from_blocks(blob, M, K, group), qg.Q2Weight.from_blocks(blob1, M, K, group)
    X = torch.from_numpy(synth.rng_for(nb).standard_normal((nb, K)).astype(np.float32)).cuda()
    xq = torch.empty((nb, K), dtype=torch.int8, device="cuda")
    sc = torch.empty(nb, device="cuda")
    su = torch.empty((nb, K // 64), dtype=torch.int32, device="cuda")
    qg.qquant_act_i8_rows(X, xq, sc, su)
    n1 = qg.qgemm_q2_batched_ws_bytes(M, K, group, nb)
    ws = ws_guarded(n1)
    ws2 = ws_guarded(qg.qgemm_q2_batched_dual_ws_bytes(M, K, group, nb))
    y, y1 = Guarded((nb, M), torch.float32), Guarded((nb, M), torch.float32)
    qg.qgemm_q2_batched(W, xq, su, sc, y.t, ws=ws.t if n1 else None)
    check(y, ws)
    qg.qgemm_q2_batched(W, xq, su, sc, y.t, accum=torch.ones((nb, M), device="cuda"), ws=ws.t if n1 else None)
    check(y, ws)
    qg.qgemm_q2_batched_dual(W, W1, xq, su, sc, y.t, y1.t, ws=ws2.t if n1 else None)
    check(y, y1, ws2)


@pytest.mark.parametrize("nb,M,K", [(1, 1, 4), (3, 100, 68), (130, 257, 1028), (200, 300, 516)])
def test_canary_q8row_gemm(nb, M, K):
    import torch
    import weight_quantized_decode_q8_amd as qg
    q, rs, xs = synth.q8gemm_inputs(nb, M, K, seed=nb * 7 + K)
    W = qg.Q8RowWeight.from_host(q, rs)
    xs_d = torch.from_numpy(xs).cuda()
    ws = ws_guarded(qg.qgemm_q8row_batched_ws_bytes(nb, K))
    y = Guarded((nb, M), torch.float32)
    for limbs in (0, 2, 3):
        qg.qgemm_q8row_batched(W.packed, W.rs, xs_d, y.t, nb, M, K, ws.t, xs_limbs=limbs)
        check(y, ws)
    g, u, c = (torch.from_numpy(a).cuda() for a in synth.gate_inputs(nb, K, seed=K))
    qg.qgemm_q8row_batched_silu(W.packed, W.rs, g, u, c, y.t, nb, M, K, ws.t)
    check(y, ws)


@pytest.mark.parametrize("M,K,group,split", [(1, 64, 64, 1), (100, 1088, 64, 3), (130, 640, 128, 0),
                                             (5000, 2048, 128, 5), (16400, 256, 64, 1)])
def test_canary_q2_in_launch_forms(M, K, group, split):
    """qgemv_q2_x (its split partials and counters), qgemv_q2_dual_x and
    qgemv_q2_gate_up_glu_x (g and u meeting in the workspace) on ragged
    shapes: nothing written outside the outputs and workspaces, and the
    workspaces left all zero."""
    import torch
    import weight_quantized_decode_q8_amd as qg
    b0, x = synth.q2_inputs(M, K, group, seed=M + K + 7)
    b1, _ = synth.q2_inputs(M, K, group, seed=M + K + 8)
    W0 = qg.Q2Weight.from_blocks(b0, M, K, group)
    W1 = qg.Q2Weight.from_blocks(b1, M, K, group)
    xd = torch.from_numpy(x).cuda()
    nw = torch.ones(K, device="cuda")
    y, y1 = Guarded(M, torch.float32), Guarded(M, torch.float32)
    ws = ws_guarded(qg.qgemv_q2_x_ws_bytes(M, K, group, split))
    ws.t.zero_()
    acc = torch.from_numpy(synth.rng_for(M).standard_normal(M).astype(np.float32)).cuda()
    qg.qgemv_q2_x(W0, xd, y.t, accum=acc, ws=ws.t if ws.nbytes > 1 else None, split_k=split)
    check(y, ws)
    assert int(torch.count_nonzero(ws.t).item()) == 0
    qg.qgemv_q2_dual_x(W0, W1, xd, y.t, y1.t, norm_w=nw if K <= 16384 else None, eps=1e-6)
    check(y, y1)
    wsg = ws_guarded(qg.lib().qgemv_q2_gate_up_glu_x_ws_bytes(M))
    wsg.t.zero_()
    qg.qgemv_q2_gate_up_glu_x(W0, W1, xd, qg.QG_GLU_SIGMOID, y.t, wsg.t)
    check(y, wsg)
    assert int(torch.count_nonzero(wsg.t).item()) == 0


def test_canary_detects_a_stray_write():
    """The guard check itself: one byte changed just past (or just before) the
    buffer is reported."""
    import torch
    b = Guarded((3, 5), torch.float32)
    assert b.intact()
    b.raw[GUARD_BYTES + b.nbytes] = 0
    assert not b.intact()
    b = Guarded(7, torch.int8)
    b.raw[GUARD_BYTES - 1] = 0
    assert not b.intact()
