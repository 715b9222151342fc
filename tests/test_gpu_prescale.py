"""The column prescale act = silu(g) * u * col (cortiq pages, silu_mul_pre)
and the batched q8_row product that forms it in its activation prep (the
Metal page's q8_mul_mm_silu), through the C-ABI.

act is binary32 arithmetic with every step fixed, so it must equal the
oracle bit for bit; the products are held to |y - y_ref| <= 2e-5 *
sum_i |w_i act_i| against the fp64 oracle, and the fused product must equal
the two-step path (prescale, then the product) bit for bit."""
import numpy as np
import pytest

import oracle
import synth
from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a HIP device")]

REL = 2e-5


def qg():
    import weight_quantized_decode_q8_amd as m
    return m


def dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def within(y, yref, mass, what):
    err = np.abs(y.astype(np.float64) - yref)
    lim = REL * mass
    bad = ~(err <= lim)
    if bad.any():
        j = np.unravel_index(int(np.argmax(np.where(np.isnan(err), np.inf, err - lim))), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())}/{y.size} outside bound; worst {j}: "
                             f"y={y[j]!r} ref={yref[j]!r} err={err[j]:.3e} lim={lim[j]:.3e}")


@pytest.mark.parametrize("rows,n,col", [(1, 17408, True), (1, 5120, False), (1, 100, True), (1, 3, False),
                                        (3, 37, True), (5, 64, False), (512, 5120, True)])
def test_prescale_bit_exact(rows, n, col):
    import torch
    g, u, c = synth.gate_inputs(rows, n, seed=rows * 1000 + n, col=col)
    g[0, : min(n, 4)] = np.array([0.0, 100.0, -100.0, 30.0], np.float32)[: min(n, 4)]
    ref = oracle.silu_mul_pre(g, u, c)
    act = torch.full((rows, n), float("nan"), device="cuda")
    qg().qact_silu_mul_pre(dev(g), dev(u), None if c is None else dev(c), act)
    torch.cuda.synchronize()
    assert np.array_equal(act.cpu().numpy(), ref), f"rows={rows} n={n} col={col}"


def test_prescale_in_place_and_unaligned():
    """act may be g or u itself; an odd element offset takes the scalar path."""
    import torch
    rows, n = 4, 1000
    g, u, c = synth.gate_inputs(rows, n, seed=71)
    ref = oracle.silu_mul_pre(g, u, c)
    gd, ud = dev(g), dev(u)
    qg().qact_silu_mul_pre(gd, ud, dev(c), gd)       # over g
    torch.cuda.synchronize()
    assert np.array_equal(gd.cpu().numpy(), ref)
    gd = dev(g)
    qg().qact_silu_mul_pre(gd, ud, dev(c), ud)       # over u
    torch.cuda.synchronize()
    assert np.array_equal(ud.cpu().numpy(), ref)
    # views one element into larger buffers: 4-byte but not 16-byte aligned
    gb, ub, cb = dev(np.concatenate([[0.0], g.ravel()]).astype(np.float32)), \
        dev(np.concatenate([[0.0], u.ravel()]).astype(np.float32)), dev(np.concatenate([[0.0], c]).astype(np.float32))
    out = torch.full((rows * n + 1,), float("nan"), device="cuda")
    qg().qact_silu_mul_pre(gb[1:].view(rows, n), ub[1:].view(rows, n), cb[1:], out[1:].view(rows, n))
    torch.cuda.synchronize()
    assert np.array_equal(out[1:].cpu().numpy().reshape(rows, n), ref)


def test_decode_chain_q8():
    """The q8_row decode FFN of the cortiq pages' MoE block: gate and up
    matvecs, the column prescale, the down matvec.  Each stage is checked on
    the GPU's own input to it: the prescale bit for bit, the matvecs within
    the bound."""
    import torch
    m = qg()
    D, F = 1024, 2816
    r = synth.rng_for(72)
    qgt, rsg, x = synth.q8row_inputs(F, D, rng=r)
    qup, rsu, _ = synth.q8row_inputs(F, D, rng=r)
    qdn, rsd, _ = synth.q8row_inputs(D, F, rng=r)
    col = r.uniform(0.5, 2.0, F).astype(np.float32)
    Wg, Wu, Wd = m.Q8RowWeight.from_host(qgt, rsg), m.Q8RowWeight.from_host(qup, rsu), m.Q8RowWeight.from_host(qdn, rsd)
    xd = dev(x)
    g = torch.empty(F, device="cuda")
    u = torch.empty(F, device="cuda")
    act = torch.empty(F, device="cuda")
    y = torch.empty(D, device="cuda")
    Wg.gemv(xd, g)
    Wu.gemv(xd, u)
    m.qact_silu_mul_pre(g, u, dev(col), act)
    Wd.gemv(act, y)
    torch.cuda.synchronize()
    gh, uh, ah, yh = (t.cpu().numpy() for t in (g, u, act, y))
    for name, q, rs, out in (("gate", qgt, rsg, gh), ("up", qup, rsu, uh)):
        ref, mass = oracle.q8row_gemv(q, rs, x)
        within(out, ref, mass, name)
    assert np.array_equal(ah, oracle.silu_mul_pre(gh, uh, col))
    ref, mass = oracle.q8row_gemv(qdn, rsd, ah)
    within(yh, ref, mass, "down")


def fused_and_two_step(q, rs, g, u, c, limbs):
    import torch
    m = qg()
    nb, K = g.shape
    M = q.shape[0]
    W = m.Q8RowWeight.from_host(q, rs)
    gd, ud, cd = dev(g), dev(u), (None if c is None else dev(c))
    ws = torch.empty(m.qgemm_q8row_batched_ws_bytes(nb, K), dtype=torch.uint8, device="cuda")
    yf = torch.full((nb, M), float("nan"), device="cuda")
    m.qgemm_q8row_batched_silu(W.packed, W.rs, gd, ud, cd, yf, nb, M, K, ws, xs_limbs=limbs)
    act = torch.empty((nb, K), device="cuda")
    m.qact_silu_mul_pre(gd, ud, cd, act)
    y2 = torch.full((nb, M), float("nan"), device="cuda")
    m.qgemm_q8row_batched(W.packed, W.rs, act, y2, nb, M, K, ws, xs_limbs=limbs)
    torch.cuda.synchronize()
    return yf.cpu().numpy(), y2.cpu().numpy(), act.cpu().numpy()


@pytest.mark.parametrize("limbs", [0, 2, 3])
@pytest.mark.parametrize("nb,M,K,col", [(1, 64, 64, True), (130, 257, 1028, True), (200, 300, 516, False),
                                        (64, 1000, 2048, True)])
def test_gemm_silu_fused(nb, M, K, col, limbs):
    q, rs, _ = synth.q8row_inputs(M, K, seed=73 + nb + M)
    g, u, c = synth.gate_inputs(nb, K, seed=74 + K, col=col)
    yf, y2, act = fused_and_two_step(q, rs, g, u, c, limbs)
    assert np.array_equal(yf, y2), f"fused != two-step ({nb}x{M}x{K}, limbs {limbs})"
    act_ref = oracle.silu_mul_pre(g, u, c)
    assert np.array_equal(act, act_ref)
    if limbs != 2:  # the 16-bit form is a caller's choice outside the bound's guarantee
        yref, mass = oracle.q8row_gemm(q, rs, act_ref)
        within(yf, yref, mass, f"fused silu gemm {nb}x{M}x{K} limbs={limbs}")


def test_gemm_silu_fused_full_size():
    """The prefill down-projection shape of the q8_row pages' FFN width, 512
    rows: fused equals two-step everywhere; sampled outputs against the oracle."""
    nb, M, K = 512, 5120, 17408
    r = synth.rng_for(75)
    q, rs, _ = synth.q8row_inputs(M, K, rng=r)
    g, u, c = synth.gate_inputs(nb, K, seed=76)
    yf, y2, act = fused_and_two_step(q, rs, g, u, c, 0)
    assert np.array_equal(yf, y2)
    bs = r.integers(0, nb, 24)
    act_ref = oracle.silu_mul_pre(g[bs], u[bs], c)
    assert np.array_equal(act[bs], act_ref)
    rows = r.integers(0, M, 64)
    for j, b in enumerate(bs):
        yref, mass = oracle.q8row_gemv(q, rs, act_ref[j], rows=rows)
        within(yf[b, rows], yref, mass, f"full-size fused row {b}")
