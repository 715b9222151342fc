"""The extensions of the Q2 GEMV, through the C-ABI: gate and up in one
launch against a shared quantized activation (qgemv_q2_dual), the residual
added in the epilogue (qgemv_q2_accum), and up to 16 independent GEMVs in
one launch (qgemv_q2_batch).

The first two must equal the unfused calls bit for bit (the qxmx page claims
exactly that for gemv_dpas8_dual and tmatvec_accum), the batch must where it
uses the same waves per tile; all are checked against the fp64 oracle:
|y - y_ref| <= 2e-5 * sum_i |w_i x_i| per output, plus, for the residual, one
binary32 rounding of the final add (2^-24 |y_ref|).
"""
import numpy as np
import pytest

import oracle
import synth
from conftest import gpu_available
from test_gpu_parity import REL, dev, gpu_act_quant, host, qg, sub_blob, within

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a HIP device")]

U32 = 2.0 ** -24


def _torch():
    import torch
    return torch


def _ws(nbytes):
    torch = _torch()
    return torch.empty(nbytes, dtype=torch.uint8, device="cuda") if nbytes else None


def gpu_single(W, xq, sc, suma, split_k):
    torch = _torch()
    m = qg()
    y = torch.empty(W.M, dtype=torch.float32, device="cuda")
    m.qgemv_q2(W, xq, suma, sc, y, _ws(m.qgemv_q2_ws_bytes(W.M, W.K, W.group, split_k)), split_k)
    return host(y)


def gpu_dual(W0, W1, xq, sc, suma, split_k):
    torch = _torch()
    m = qg()
    y0 = torch.empty(W0.M, dtype=torch.float32, device="cuda")
    y1 = torch.empty(W0.M, dtype=torch.float32, device="cuda")
    ws = _ws(m.qgemv_q2_dual_ws_bytes(W0.M, W0.K, W0.group, split_k))
    m.qgemv_q2_dual(W0, W1, xq, suma, sc, y0, y1, ws, split_k)
    return host(y0), host(y1)


def gpu_accum(W, xq, sc, suma, accum, split_k, in_place=False):
    torch = _torch()
    m = qg()
    a = dev(accum)
    y = a if in_place else torch.empty(W.M, dtype=torch.float32, device="cuda")
    m.qgemv_q2_accum(W, xq, suma, sc, a, y, _ws(m.qgemv_q2_ws_bytes(W.M, W.K, W.group, split_k)), split_k)
    return host(y)


def bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


# ------------------------------------------------------------- dual GEMV --
@pytest.mark.parametrize("M,K,group,split", [(1, 64, 64, 1), (64, 256, 64, 1), (130, 640, 128, 0),
                                             (300, 2048, 64, 4), (200, 4096, 128, 3),
                                             (4100, 1024, 128, 0), (70, 1536, 64, 16)])
def test_dual_equals_two_calls(M, K, group, split):
    m = qg()
    b0, x = synth.q2_inputs(M, K, group, seed=1000 + M + K)
    b1, _ = synth.q2_inputs(M, K, group, seed=2000 + M + K)
    W0 = m.Q2Weight.from_blocks(b0, M, K, group)
    W1 = m.Q2Weight.from_blocks(b1, M, K, group)
    xq_h, sc_h, _, (xq, sc, suma) = gpu_act_quant(x)
    y0, y1 = gpu_dual(W0, W1, xq, sc, suma, split)
    assert np.array_equal(bits(y0), bits(gpu_single(W0, xq, sc, suma, split)))
    assert np.array_equal(bits(y1), bits(gpu_single(W1, xq, sc, suma, split)))
    for blob, y, name in ((b0, y0, "gate"), (b1, y1, "up")):
        yref, mass = oracle.q2_gemv(blob, M, K, group, xq_h, sc_h)
        within(y, yref, mass, what=f"dual {name} {M}x{K} g{group} S={split}")


def test_dual_c3_gate_up():
    """The FFN gate and up matrices of the 17408 x 5120 g128 workload, one activation."""
    m = qg()
    c = synth.CONFIGS["q2_g128_gate_17408x5120"]
    M, K, group = c["M"], c["K"], c["group"]
    bg, x = synth.config_inputs("q2_g128_gate_17408x5120")
    bu, _ = synth.config_inputs("q2_g128_up_17408x5120")
    Wg = m.Q2Weight.from_blocks(bg, M, K, group)
    Wu = m.Q2Weight.from_blocks(bu, M, K, group)
    xq_h, sc_h, _, (xq, sc, suma) = gpu_act_quant(x)
    yg, yu = gpu_dual(Wg, Wu, xq, sc, suma, 0)
    assert np.array_equal(bits(yg), bits(gpu_single(Wg, xq, sc, suma, 0)))
    assert np.array_equal(bits(yu), bits(gpu_single(Wu, xq, sc, suma, 0)))
    rng = synth.rng_for(551)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(M - 64, M), rng.integers(0, M, 1200)]))
    for blob, y, name in ((bg, yg, "gate"), (bu, yu, "up")):
        yref, mass = oracle.q2_gemv(blob, M, K, group, xq_h, sc_h, rows=rows)
        within(y[rows], yref, mass, what=f"gate|up dual 17408x5120 {name}")


def test_dual_same_weight_twice():
    """Both slots may name one matrix: two identical outputs."""
    m = qg()
    b, x = synth.q2_inputs(256, 1024, 64, seed=31)
    W = m.Q2Weight.from_blocks(b, 256, 1024, 64)
    _, _, _, (xq, sc, suma) = gpu_act_quant(x)
    y0, y1 = gpu_dual(W, W, xq, sc, suma, 2)
    assert np.array_equal(bits(y0), bits(y1))
    assert np.array_equal(bits(y0), bits(gpu_single(W, xq, sc, suma, 2)))


# ----------------------------------------------------- residual epilogue --
def _accum_check(blob, M, K, group, x, accum, split, rows=None, what=""):
    m = qg()
    W = m.Q2Weight.from_blocks(blob, M, K, group)
    xq_h, sc_h, _, (xq, sc, suma) = gpu_act_quant(x)
    y = gpu_accum(W, xq, sc, suma, accum, split)
    # the unfused order: the GEMV, then a separate binary32 add
    y_plain = gpu_single(W, xq, sc, suma, split)
    assert np.array_equal(bits(y), bits(y_plain + accum)), f"{what}: not the unfused result"
    y_in = gpu_accum(W, xq, sc, suma, accum, split, in_place=True)
    assert np.array_equal(bits(y_in), bits(y)), f"{what}: in-place differs"
    if rows is None:
        yref, mass = oracle.q2_gemv_accum(blob, M, K, group, xq_h, sc_h, accum)
        within(y, yref, mass + U32 / REL * np.abs(yref), what=what)
    else:
        yref, mass = oracle.q2_gemv_accum(blob, M, K, group, xq_h, sc_h, accum, rows=rows)
        within(y[rows], yref, mass + U32 / REL * np.abs(yref), what=what)


@pytest.mark.parametrize("M,K,group,split", [(1, 64, 64, 1), (65, 192, 64, 1), (129, 640, 128, 0),
                                             (300, 2048, 128, 4), (5000, 256, 64, 0), (96, 3072, 64, 16)])
def test_accum_equals_gemv_then_add(M, K, group, split):
    blob, x = synth.q2_inputs(M, K, group, seed=3000 + M + K)
    accum = (synth.rng_for(3100 + M).standard_normal(M) * 3.0).astype(np.float32)
    _accum_check(blob, M, K, group, x, accum, split, what=f"accum {M}x{K} g{group} S={split}")


def test_accum_c3_down_residual():
    """The 5120 x 17408 down projection added to a residual stream (auto split)."""
    c = synth.CONFIGS["q2_g128_down_5120x17408"]
    M, K, group = c["M"], c["K"], c["group"]
    blob, x = synth.config_inputs("q2_g128_down_5120x17408")
    accum = synth.rng_for(552).standard_normal(M).astype(np.float32)
    rng = synth.rng_for(553)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(M - 64, M), rng.integers(0, M, 600)]))
    _accum_check(blob, M, K, group, x, accum, 0, rows=rows, what="down 5120x17408 + residual")


def test_accum_zero_projection_returns_residual():
    """All codes 1 (every weight 0): y is the residual, bit for bit."""
    from oracle_pins import encode_q2
    rng = synth.rng_for(554)
    M, K = 130, 512
    codes = np.ones((M, K), np.uint8)
    d_bits = np.abs(rng.normal(0, 0.02, size=(M, K // 128))).astype(np.float16).view(np.uint16)
    blob = encode_q2(codes, d_bits, 128)
    accum = rng.standard_normal(M).astype(np.float32)
    m = qg()
    W = m.Q2Weight.from_blocks(blob, M, K, 128)
    _, _, _, (xq, sc, suma) = gpu_act_quant(rng.standard_normal(K, dtype=np.float32))
    for split in (1, 4):
        y = gpu_accum(W, xq, sc, suma, accum, split)
        assert np.array_equal(bits(y), bits(accum + np.float32(0.0)))


# ------------------------------------------------------- batched launch --
def _batch_case(specs, group, seed):
    """specs: list of (M, K, with_accum).  Returns per-job host data and device jobs."""
    m = qg()
    torch = _torch()
    host_jobs, dev_jobs = [], []
    acts = {}
    for n, (M, K, with_acc) in enumerate(specs):
        blob, _ = synth.q2_inputs(M, K, group, seed=seed + 17 * n)
        if K not in acts:
            x = synth.activation(K, seed + 1000 + K)
            acts[K] = (x, gpu_act_quant(x))
        x, (xq_h, sc_h, _, (xq, sc, suma)) = acts[K]
        W = m.Q2Weight.from_blocks(blob, M, K, group)
        y = torch.empty(M, dtype=torch.float32, device="cuda")
        accum = (synth.rng_for(seed + 31 * n).standard_normal(M) * 2).astype(np.float32) if with_acc else None
        job = (W, xq, suma, sc, y) + ((dev(accum),) if with_acc else ())
        dev_jobs.append(job)
        host_jobs.append(dict(blob=blob, M=M, K=K, W=W, xq=xq, sc=sc, suma=suma, xq_h=xq_h, sc_h=sc_h,
                              accum=accum, y=y))
    return host_jobs, dev_jobs


def _check_batch(specs, group, seed, exact):
    hj, dj = _batch_case(specs, group, seed)
    qg().qgemv_q2_batch(dj)
    for n, j in enumerate(hj):
        y = host(j["y"])
        if j["accum"] is None:
            single = gpu_single(j["W"], j["xq"], j["sc"], j["suma"], 1)
            yref, mass = oracle.q2_gemv(j["blob"], j["M"], j["K"], group, j["xq_h"], j["sc_h"])
        else:
            single = gpu_accum(j["W"], j["xq"], j["sc"], j["suma"], j["accum"], 1)
            yref, mass = oracle.q2_gemv_accum(j["blob"], j["M"], j["K"], group, j["xq_h"], j["sc_h"], j["accum"])
            mass = mass + U32 / REL * np.abs(yref)
        if exact:
            assert np.array_equal(bits(y), bits(single)), f"job {n}: differs from the single call"
        within(y, yref, mass, what=f"batch job {n} {j['M']}x{j['K']} g{group}")


@pytest.mark.parametrize("group", [64, 128])
def test_batch_small_jobs_equal_single_calls(group):
    # every job and the launch below 256 row tiles: 16 waves per tile everywhere
    specs = [(64, 256, False), (130, 1024, True), (1, 128, False), (1000, 512, True), (257, 2048, False)]
    _check_batch(specs, group, 5000 + group, exact=True)


def test_batch_sixteen_jobs_shared_activation():
    specs = [(100 + 37 * n, 1024, n % 3 == 0) for n in range(16)]
    _check_batch(specs, 128, 5200, exact=sum((M + 63) // 64 for M, _, _ in specs) < 256)


def test_batch_large_jobs_equal_single_calls():
    # every job and the launch at 256 row tiles or more: 8 waves per tile everywhere
    specs = [(16384, 1024, False), (17408, 640, True)]
    _check_batch(specs, 128, 5300, exact=True)


def test_batch_mixed_sizes_within_bound():
    # small jobs in a launch of >= 256 tiles: only the summation order changes
    specs = [(16384, 512, False), (200, 1024, True), (64, 2048, False)]
    _check_batch(specs, 64, 5400, exact=False)


@pytest.mark.parametrize("M,K,group,kind", [(17408, 5120, 128, 0), (17408, 5120, 128, 1), (2048, 1024, 64, 0),
                                            (64, 640, 64, 1), (4096, 4096, 128, 0)])
def test_gate_up_glu_equals_dual_then_glu(M, K, group, kind):
    """The gate|up GEMV with the gated product in its epilogue and the
    quantiser after it (cortiq moe_gate_up) gives t, xq, act_scale and suma
    bit for bit as qgemv_q2_dual (split 1) followed by qquant_glu_i8."""
    import torch
    m = qg()
    bg, x = synth.q2_inputs(M, K, group, seed=9100 + M)
    bu, _ = synth.q2_inputs(M, K, group, seed=9101 + M)
    Wg, Wu = m.Q2Weight.from_blocks(bg, M, K, group), m.Q2Weight.from_blocks(bu, M, K, group)
    xq = torch.empty(K, dtype=torch.int8, device="cuda")
    sc = torch.empty(1, device="cuda")
    su = torch.empty(K // 64, dtype=torch.int32, device="cuda")
    m.qquant_act_i8(dev(x), xq, sc, su)
    t = torch.full((M,), float("nan"), device="cuda")
    xq2 = torch.empty(M, dtype=torch.int8, device="cuda")
    sc2 = torch.empty(1, device="cuda")
    su2 = torch.empty(M // 64, dtype=torch.int32, device="cuda")
    m.qgemv_q2_gate_up_glu(Wg, Wu, xq, su, sc, kind, t, xq2, sc2, su2)
    g = torch.empty(M, device="cuda")
    u = torch.empty(M, device="cuda")
    m.qgemv_q2_dual(Wg, Wu, xq, su, sc, g, u, None, split_k=1)
    t_r = torch.empty(M, device="cuda")
    xq_r = torch.empty(M, dtype=torch.int8, device="cuda")
    sc_r = torch.empty(1, device="cuda")
    su_r = torch.empty(M // 64, dtype=torch.int32, device="cuda")
    m.qquant_glu_i8(g, u, kind, t_r, xq_r, sc_r, su_r)
    torch.cuda.synchronize()
    assert torch.equal(t.view(torch.int32), t_r.view(torch.int32)), "t differs"
    assert torch.equal(xq2, xq_r) and torch.equal(sc2.view(torch.int32), sc_r.view(torch.int32)) and torch.equal(su2, su_r)
