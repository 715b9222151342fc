"""The decode Q2 GEMVs with the activation quantiser in the same launch, through
the C-ABI: qgemv_q2_x (one matrix, split-K added by the last workgroup of
each row tile, optional residual), qgemv_q2_dual_x (the gate|up pair,
optionally RMSNorm-ed) and qgemv_q2_gate_up_glu_x (the pair with the gated
product in its epilogue).

Each must equal the multi-launch chain it replaces bit for bit (the
quantiser, RMSNorm and gated product of the qxmx page's producers, then
gemv_dpas8 / gemv_dpas8_dual / gemv_reduce), and the one-matrix form is also
checked against the fp64 oracle: |y - y_ref| <= 2e-5 * sum_i |w_i x_i|.
"""
import numpy as np
import pytest

import oracle
import synth
from conftest import gpu_available
from test_gpu_parity import dev, gpu_act_quant, host, qg, within

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a HIP device")]


def _torch():
    import torch
    return torch


def bits(a):
    return np.asarray(a, np.float32).view(np.uint32)


def _empty(n):
    torch = _torch()
    return torch.full((n,), float("nan"), dtype=torch.float32, device="cuda")


def chain_single(W, x, split, accum=None):
    """qquant_act_i8 then qgemv_q2 / qgemv_q2_accum (the launches replaced),
    with the split qgemv_q2_x uses (its automatic choice for split 0)."""
    torch = _torch()
    m = qg()
    split = split or m.qgemv_q2_x_auto_split(W.M, W.K, W.group)
    _, _, _, (xq, sc, suma) = gpu_act_quant(x)
    y = _empty(W.M)
    n = m.qgemv_q2_ws_bytes(W.M, W.K, W.group, split)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda") if n else None
    if accum is None:
        m.qgemv_q2(W, xq, suma, sc, y, ws, split)
    else:
        m.qgemv_q2_accum(W, xq, suma, sc, dev(accum), y, ws, split)
    return host(y)


def fused_single(W, x, split, accum=None, ws=None, in_place=False):
    m = qg()
    if ws is None:
        ws = m.qgemv_q2_x_workspace(W.M, W.K, W.group, split)
    a = dev(accum) if accum is not None else None
    y = a if in_place else _empty(W.M)
    m.qgemv_q2_x(W, dev(x), y, accum=a, ws=ws, split_k=split)
    return host(y)


SHAPES = [(1, 64, 64, 1), (64, 256, 64, 1), (130, 640, 128, 0), (300, 2048, 64, 4), (200, 4096, 128, 3),
          (70, 1536, 64, 16), (4100, 1024, 128, 0), (16448, 512, 64, 1), (777, 32768, 128, 1),
          (777, 32768, 128, 5), (16448, 16384, 128, 1), (16448, 16384, 64, 2), (100, 8256, 64, 1), (64, 32768, 64, 0)]


@pytest.mark.parametrize("M,K,group,split", SHAPES)
def test_q2_x_equals_quant_then_gemv(M, K, group, split):
    m = qg()
    blob, x = synth.q2_inputs(M, K, group, seed=7000 + M + K)
    W = m.Q2Weight.from_blocks(blob, M, K, group)
    y = fused_single(W, x, split)
    assert np.array_equal(bits(y), bits(chain_single(W, x, split))), "differs from qquant_act_i8 + qgemv_q2"
    if M * K <= 4096 * 4096:
        rq, rsc, _ = oracle.act_quant_i8(x)
        yref, mass = oracle.q2_gemv(blob, M, K, group, rq, rsc)
        within(y, yref, mass, what=f"qgemv_q2_x {M}x{K} g{group} S{split}")


@pytest.mark.parametrize("M,K,group,split,in_place", [(300, 2048, 64, 4, False), (130, 640, 128, 1, True),
                                                      (5120, 17408, 128, 0, False), (5120, 17408, 128, 0, True),
                                                      (1000, 8192, 128, 7, True)])
def test_q2_x_residual(M, K, group, split, in_place):
    m = qg()
    blob, x = synth.q2_inputs(M, K, group, seed=7100 + M)
    W = m.Q2Weight.from_blocks(blob, M, K, group)
    acc = np.random.Generator(np.random.PCG64(7101 + M)).standard_normal(M).astype(np.float32)
    y = fused_single(W, x, split, accum=acc, in_place=in_place)
    assert np.array_equal(bits(y), bits(chain_single(W, x, split, accum=acc)))


def test_q2_x_counters_reset_between_calls():
    """One workspace through calls of different shapes and splits: every call
    leaves the whole workspace (arrival counters and partials) at zero, so
    each result equals the chain."""
    torch = _torch()
    m = qg()
    ws = torch.zeros(m.qgemv_q2_x_ws_bytes(5120, 17408, 128, 16), dtype=torch.uint8, device="cuda")
    for (M, K, group, split) in [(5120, 17408, 128, 2), (5120, 17408, 128, 2), (300, 2048, 64, 4),
                                 (5120, 17408, 128, 16), (70, 1536, 64, 3)]:
        blob, x = synth.q2_inputs(M, K, group, seed=7200 + M + split)
        W = m.Q2Weight.from_blocks(blob, M, K, group)
        y = fused_single(W, x, split, ws=ws)
        assert np.array_equal(bits(y), bits(chain_single(W, x, split))), (M, K, split)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(ws).item()) == 0, "workspace not left all zero"


def test_q2_x_zero_vector():
    m = qg()
    M, K, group = 200, 1024, 128
    blob, _ = synth.q2_inputs(M, K, group, seed=7300)
    W = m.Q2Weight.from_blocks(blob, M, K, group)
    y = fused_single(W, np.zeros(K, np.float32), 2)
    assert np.all(y == 0.0)


def _pair(M, K, group, seed):
    m = qg()
    bg, x = synth.q2_inputs(M, K, group, seed=seed)
    bu, _ = synth.q2_inputs(M, K, group, seed=seed + 1)
    return m.Q2Weight.from_blocks(bg, M, K, group), m.Q2Weight.from_blocks(bu, M, K, group), x


def _quant_chain(x, norm_w, eps):
    """The producer the in-launch quantiser replaces: (xq, act_scale, suma) on the device."""
    torch = _torch()
    m = qg()
    K = x.size
    xq = torch.empty(K, dtype=torch.int8, device="cuda")
    sc = torch.empty(1, dtype=torch.float32, device="cuda")
    su = torch.empty(K // 64, dtype=torch.int32, device="cuda")
    if norm_w is None:
        m.qquant_act_i8(dev(x), xq, sc, su)
    else:
        m.qquant_rmsnorm_i8(dev(x), dev(norm_w), eps, xq, sc, su)
    return xq, sc, su


PAIR_SHAPES = [(1, 64, 64), (130, 640, 128), (512, 1024, 64), (300, 2048, 128), (16448, 512, 64),
               (17408, 5120, 128)]


@pytest.mark.parametrize("M,K,group", PAIR_SHAPES)
@pytest.mark.parametrize("norm", [False, True])
def test_dual_x_equals_quant_then_dual(M, K, group, norm):
    m = qg()
    Wg, Wu, x = _pair(M, K, group, 7400 + M + K)
    rng = np.random.Generator(np.random.PCG64(7402 + M))
    nw = (1.0 + 0.1 * rng.standard_normal(K)).astype(np.float32) if norm else None
    eps = 1e-6
    y0, y1 = _empty(M), _empty(M)
    m.qgemv_q2_dual_x(Wg, Wu, dev(x), y0, y1, norm_w=dev(nw) if norm else None, eps=eps)
    xq, sc, su = _quant_chain(x, nw, eps)
    r0, r1 = _empty(M), _empty(M)
    m.qgemv_q2_dual(Wg, Wu, xq, su, sc, r0, r1, None, split_k=1)
    assert np.array_equal(bits(host(y0)), bits(host(r0))), "gate output differs"
    assert np.array_equal(bits(host(y1)), bits(host(r1))), "up output differs"


@pytest.mark.parametrize("M,K,group", PAIR_SHAPES)
@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("norm", [False, True])
def test_gate_up_glu_x_equals_chain(M, K, group, kind, norm):
    """t equals the quantiser (or RMSNorm+quantiser), the dual GEMV with
    split 1 and the gated product of qquant_glu_i8, bit for bit."""
    torch = _torch()
    m = qg()
    Wg, Wu, x = _pair(M, K, group, 7500 + M + K)
    rng = np.random.Generator(np.random.PCG64(7502 + M))
    nw = (1.0 + 0.1 * rng.standard_normal(K)).astype(np.float32) if norm else None
    eps = 1e-5
    t = _empty(M)
    ws = m.qgemv_q2_gate_up_glu_x_workspace(M)
    m.qgemv_q2_gate_up_glu_x(Wg, Wu, dev(x), kind, t, ws, norm_w=dev(nw) if norm else None, eps=eps)
    xq, sc, su = _quant_chain(x, nw, eps)
    g, u = _empty(M), _empty(M)
    m.qgemv_q2_dual(Wg, Wu, xq, su, sc, g, u, None, split_k=1)
    Kt = -(-M // 64) * 64
    if M % 64 == 0:
        tr = _empty(M)
        m.qquant_glu_i8(g, u, kind, tr, torch.empty(M, dtype=torch.int8, device="cuda"),
                        torch.empty(1, device="cuda"), torch.empty(Kt // 64, dtype=torch.int32, device="cuda"))
        tr = host(tr)
    else:
        # the quantising producer needs a multiple of 64: pad g, u with zeros
        gp = torch.zeros(Kt, device="cuda")
        up = torch.zeros(Kt, device="cuda")
        gp[:M] = g
        up[:M] = u
        tp = torch.empty(Kt, device="cuda")
        m.qquant_glu_i8(gp, up, kind, tp, torch.empty(Kt, dtype=torch.int8, device="cuda"),
                        torch.empty(1, device="cuda"), torch.empty(Kt // 64, dtype=torch.int32, device="cuda"))
        tr = host(tp)[:M]
    assert np.array_equal(bits(host(t)), bits(tr)), "t differs"
    assert int(torch.count_nonzero(ws).item()) == 0, "workspace not left all zero"


def test_ffn_block_two_launches_equals_fused_chain():
    """The decode FFN block at the pages' model shapes (g128, gate/up
    17408 x 5120, down 5120 x 17408): RMSNorm+quantiser, gate|up with the
    SiLU gate, quantiser, down with the residual -- as two launches
    (qgemv_q2_gate_up_glu_x, qgemv_q2_x) and as the five-launch chain
    (qquant_rmsnorm_i8, qgemv_q2_gate_up_glu [two launches], qgemv_q2_accum
    with the same split and its reduce), bit for bit."""
    torch = _torch()
    m = qg()
    D, F, group = 5120, 17408, 128
    Wg, Wu, _ = _pair(F, D, group, 7600)
    bd, _ = synth.q2_inputs(D, F, group, seed=7602)
    Wd = m.Q2Weight.from_blocks(bd, D, F, group)
    rng = np.random.Generator(np.random.PCG64(7603))
    h = rng.standard_normal(D).astype(np.float32)
    nw = (1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    resid = rng.standard_normal(D).astype(np.float32)
    eps = 1e-6
    # two launches
    t = _empty(F)
    m.qgemv_q2_gate_up_glu_x(Wg, Wu, dev(h), 0, t, m.qgemv_q2_gate_up_glu_x_workspace(F), norm_w=dev(nw), eps=eps)
    y = _empty(D)
    m.qgemv_q2_x(Wd, t, y, accum=dev(resid), ws=m.qgemv_q2_x_workspace(D, F, group, 0), split_k=0)
    # the chain
    xq, sc, su = _quant_chain(h, nw, eps)
    t_r = _empty(F)
    xq2 = torch.empty(F, dtype=torch.int8, device="cuda")
    sc2 = torch.empty(1, device="cuda")
    su2 = torch.empty(F // 64, dtype=torch.int32, device="cuda")
    m.qgemv_q2_gate_up_glu(Wg, Wu, xq, su, sc, 0, t_r, xq2, sc2, su2)
    y_r = _empty(D)
    S = m.qgemv_q2_x_auto_split(D, F, group)
    n = m.qgemv_q2_ws_bytes(D, F, group, S)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda") if n else None
    m.qgemv_q2_accum(Wd, xq2, su2, sc2, dev(resid), y_r, ws, S)
    assert np.array_equal(bits(host(t)), bits(host(t_r))), "t differs"
    assert np.array_equal(bits(host(y)), bits(host(y_r))), "y differs"
    # and the down projection against the oracle, from the chain's own t
    tq, tsc, _ = oracle.act_quant_i8(host(t_r))
    rows = np.arange(0, D, 37)
    yref, mass = oracle.q2_gemv_accum(bd, D, F, group, tq, tsc, resid, rows=rows)
    within(host(y)[rows], yref, mass + np.abs(yref) * 2.0 ** -24 / 2e-5, what="FFN block down")


def test_decode_ffn_workloads_as_benched():
    """The decode step's Q2 workloads (g128 gate and up 17408 x 5120, down
    5120 x 17408, the seeded inputs and the launch configuration the bench
    times: the pair with the quantiser inside, the down projection with the
    quantiser and its automatic split inside): sampled rows against the fp64
    oracle on the oracle's own quantised activations, every row against the
    six-launch chain bit for bit."""
    m = qg()
    blobs, xs, Ws = {}, {}, {}
    for n in ("q2_g128_gate_17408x5120", "q2_g128_up_17408x5120", "q2_g128_down_5120x17408"):
        c = synth.CONFIGS[n]
        blobs[n], xs[n] = synth.config_inputs(n)
        Ws[n] = m.Q2Weight.from_blocks(blobs[n], c["M"], c["K"], c["group"])
    Wg, Wu = Ws["q2_g128_gate_17408x5120"], Ws["q2_g128_up_17408x5120"]
    Wd = Ws["q2_g128_down_5120x17408"]
    x_gu, x_dn = xs["q2_g128_gate_17408x5120"], xs["q2_g128_down_5120x17408"]
    yg, yu = _empty(Wg.M), _empty(Wg.M)
    m.qgemv_q2_dual_x(Wg, Wu, dev(x_gu), yg, yu)
    S = m.qgemv_q2_x_auto_split(Wd.M, Wd.K, Wd.group)
    assert S == 3
    yd = _empty(Wd.M)
    m.qgemv_q2_x(Wd, dev(x_dn), yd, ws=m.qgemv_q2_x_workspace(Wd.M, Wd.K, Wd.group, 0), split_k=0)
    yg, yu, yd = host(yg), host(yu), host(yd)
    assert np.array_equal(bits(yg), bits(chain_single(Wg, x_gu, 1)))
    assert np.array_equal(bits(yu), bits(chain_single(Wu, x_gu, 1)))
    assert np.array_equal(bits(yd), bits(chain_single(Wd, x_dn, S)))
    for name, W, x, y in (("q2_g128_gate_17408x5120", Wg, x_gu, yg), ("q2_g128_up_17408x5120", Wu, x_gu, yu),
                          ("q2_g128_down_5120x17408", Wd, x_dn, yd)):
        rq, rsc, _ = oracle.act_quant_i8(x)
        rows = np.unique(np.concatenate([np.arange(0, W.M, 97), [W.M - 1]]))
        yref, mass = oracle.q2_gemv(blobs[name], W.M, W.K, W.group, rq, rsc, rows=rows)
        within(y[rows], yref, mass, what=name)


@pytest.mark.parametrize("kind", [0, 1])
def test_gate_up_glu_x_t_within_oracle_bound(kind):
    """t of the fused gate|up launch (RMSNorm + quantiser inside, the gated
    product in the epilogue) held directly to the fp64 oracle at the decode
    shape (g128, 17408 x 5120), every row.  The oracle gives g, u (fp64, on
    its own quantised activation) and their yardsticks m_g, m_u; with
    |g - g_ref| <= 2e-5 m_g and |u - u_ref| <= 2e-5 m_u, the mean value
    theorem bounds t = u * f(g) (f = silu, |f'| < 1.1; or f = sigmoid,
    |f'| <= 1/4) by
        |dt| <= c (|u_ref| + du) dg + (|f(g_ref)| + c dg) du + 6 ulp(t_ref),
    the last term the binary32 evaluation of exp, 1 + e, the quotient and
    the product (four roundings)."""
    m = qg()
    M, K, group = 17408, 5120, 128
    bg, x = synth.q2_inputs(M, K, group, seed=7700)
    bu, _ = synth.q2_inputs(M, K, group, seed=7701)
    Wg, Wu = m.Q2Weight.from_blocks(bg, M, K, group), m.Q2Weight.from_blocks(bu, M, K, group)
    rng = np.random.Generator(np.random.PCG64(7702))
    nw = (1.0 + 0.1 * rng.standard_normal(K)).astype(np.float32)
    eps = 1e-6
    t = _empty(M)
    m.qgemv_q2_gate_up_glu_x(Wg, Wu, dev(x), kind, t, m.qgemv_q2_gate_up_glu_x_workspace(M),
                             norm_w=dev(nw), eps=eps)
    t = host(t).astype(np.float64)
    _, xq, sc, _ = oracle.rmsnorm_quant_i8(x, nw, eps)
    g, mg = oracle.q2_gemv(bg, M, K, group, xq, sc)
    u, mu = oracle.q2_gemv(bu, M, K, group, xq, sc)
    sig = 1.0 / (1.0 + np.exp(-g))
    f, c = (g * sig, 1.1) if kind == 0 else (sig, 0.25)
    t_ref = u * f
    dg, du = 2e-5 * mg, 2e-5 * mu
    bound = c * (np.abs(u) + du) * dg + (np.abs(f) + c * dg) * du + 6.0 * 2.0 ** -24 * np.abs(t_ref)
    err = np.abs(t - t_ref)
    assert np.all(np.isfinite(t))
    bad = err > bound
    assert not bad.any(), (f"{int(bad.sum())} of {M} t outside the bound; worst ratio "
                           f"{np.max(err / bound):.3f}")


@pytest.mark.parametrize("M,K,group,kind", [(130, 640, 128, 0), (300, 2048, 128, 1), (16448, 512, 64, 0),
                                            (17408, 5120, 128, 0)])
def test_gate_up_glu_x_tmax_is_each_tiles_max(M, K, group, kind):
    """tmax[tile] = max |t| over the tile's rows, bit for bit, and t itself is
    the same as without tmax."""
    torch = _torch()
    m = qg()
    Wg, Wu, x = _pair(M, K, group, 7800 + M)
    tiles = -(-M // 64)
    ws = m.qgemv_q2_gate_up_glu_x_workspace(M)
    t0 = _empty(M)
    m.qgemv_q2_gate_up_glu_x(Wg, Wu, dev(x), kind, t0, ws)
    t1 = _empty(M)
    tmax = torch.full((tiles,), float("nan"), dtype=torch.float32, device="cuda")
    m.qgemv_q2_gate_up_glu_x(Wg, Wu, dev(x), kind, t1, ws, tmax=tmax)
    t0, t1, tmax = host(t0), host(t1), host(tmax)
    assert np.array_equal(bits(t0), bits(t1))
    pad = np.zeros(tiles * 64, np.float32)
    pad[:M] = np.abs(t1)
    assert np.array_equal(bits(tmax), bits(pad.reshape(tiles, 64).max(axis=1)))
    assert int(torch.count_nonzero(ws).item()) == 0


@pytest.mark.parametrize("M,K,group,split", [(1, 64, 64, 1), (65, 192, 64, 3), (300, 2048, 128, 0),
                                             (129, 4096, 64, 16), (4096, 4096, 64, 0), (5120, 17408, 128, 0),
                                             (5120, 17408, 128, 1), (64, 32768, 64, 5)])
@pytest.mark.parametrize("nparts", [1, 7, 512])
def test_q2_x_with_partial_maxima_equals_whole_vector(M, K, group, split, nparts):
    """Given partial maxima of |x| (here over nparts ragged chunks), each
    workgroup reads only its split of x: y is bit-identical to the launch
    that finds the max over the whole vector, residual included."""
    torch = _torch()
    m = qg()
    blob, x = synth.q2_inputs(M, K, group, seed=7900 + M + K + split)
    W = m.Q2Weight.from_blocks(blob, M, K, group)
    rng = np.random.Generator(np.random.PCG64(7901 + M))
    resid = rng.standard_normal(M).astype(np.float32)
    cuts = np.linspace(0, K, min(nparts, K) + 1).astype(int)
    parts = np.array([np.max(np.abs(x[a:b])) for a, b in zip(cuts[:-1], cuts[1:])], np.float32)
    ws = m.qgemv_q2_x_workspace(M, K, group, split)
    y0, y1 = _empty(M), _empty(M)
    m.qgemv_q2_x(W, dev(x), y0, accum=dev(resid), ws=ws, split_k=split)
    m.qgemv_q2_x(W, dev(x), y1, accum=dev(resid), ws=ws, split_k=split, xmax=dev(parts))
    assert np.array_equal(bits(host(y0)), bits(host(y1)))
    assert ws is None or int(torch.count_nonzero(ws).item()) == 0


def test_ffn_block_with_tile_maxima_equals_two_launches():
    """The decode FFN block with the gate|up launch's tile maxima handed to
    the down projection (which then reads only its split of t): y bit-
    identical to the block without them, at the pages' model shapes."""
    torch = _torch()
    m = qg()
    D, F, group = 5120, 17408, 128
    Wg, Wu, _ = _pair(F, D, group, 7600)
    bd, _ = synth.q2_inputs(D, F, group, seed=7602)
    Wd = m.Q2Weight.from_blocks(bd, D, F, group)
    rng = np.random.Generator(np.random.PCG64(7603))
    h = rng.standard_normal(D).astype(np.float32)
    nw = (1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32)
    eps = 1e-6
    ws_g = m.qgemv_q2_gate_up_glu_x_workspace(F)
    ws_d = m.qgemv_q2_x_workspace(D, F, group, 0)
    ys = []
    for use_parts in (False, True):
        t = _empty(F)
        tmax = torch.empty(F // 64, dtype=torch.float32, device="cuda") if use_parts else None
        m.qgemv_q2_gate_up_glu_x(Wg, Wu, dev(h), 0, t, ws_g, norm_w=dev(nw), eps=eps, tmax=tmax)
        y = dev(h)
        m.qgemv_q2_x(Wd, t, y, accum=y, ws=ws_d, split_k=0, xmax=tmax)
        ys.append(host(y))
    assert np.array_equal(bits(ys[0]), bits(ys[1]))


def test_stamped_launches_equal_product_launches():
    """The timeline probe's stamped entry points run the product kernels: the
    same bits as qgemv_q2_gate_up_glu_x / qgemv_q2_x, and every workgroup's
    four stamps in order (start <= prologue <= tile sum <= exit)."""
    torch = _torch()
    m = qg()
    F, D, group = 1152, 512, 128
    Wg, Wu, x = _pair(F, D, group, 7960)
    bd, _ = synth.q2_inputs(D, F, group, seed=7961)
    Wd = m.Q2Weight.from_blocks(bd, D, F, group)
    ws = m.qgemv_q2_gate_up_glu_x_workspace(F)
    tiles = -(-F // 64)
    t0, t1 = _empty(F), _empty(F)
    tm0 = torch.empty(tiles, device="cuda")
    tm1 = torch.empty(tiles, device="cuda")
    m.qgemv_q2_gate_up_glu_x(Wg, Wu, dev(x), 0, t0, ws, tmax=tm0)
    st_g = torch.zeros(4 * 2 * tiles, dtype=torch.int64, device="cuda")
    m.qg_probe_q2_gate_up_glu_x_stamped(Wg, Wu, dev(x), 0, t1, ws, st_g, tmax=tm1)
    S = m.qgemv_q2_x_auto_split(D, F, group)
    wsd = m.qgemv_q2_x_workspace(D, F, group, S)
    y0, y1 = _empty(D), _empty(D)
    m.qgemv_q2_x(Wd, t0, y0, ws=wsd, split_k=S, xmax=tm0)
    st_d = torch.zeros(4 * (-(-D // 64)) * S, dtype=torch.int64, device="cuda")
    m.qg_probe_q2_x_stamped(Wd, t1, y1, st_d, ws=wsd, split_k=S, xmax=tm1)
    assert np.array_equal(bits(host(t0)), bits(host(t1))) and np.array_equal(bits(host(y0)), bits(host(y1)))
    for st in (st_g, st_d):
        a = host(st).reshape(-1, 4)
        assert np.all(a > 0) and np.all(np.diff(a, axis=1) >= 0)


def test_peak_probes_run():
    """The measurement probes run and report plausible figures: the streaming
    read writes nothing (the sentinel is never met), the MFMA loops fill their
    sink and report a shader clock between 0.5 and 3 GHz."""
    import torch
    m = qg()
    buf = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(2048, dtype=torch.int32, device="cuda")
    m.qg_probe_stream_read(buf, 0x5EED1E55, sink, 2048, 8)
    torch.cuda.synchronize()
    assert int(torch.count_nonzero(sink).item()) == 0
    khz = m.qg_probe_wall_clock_khz()
    assert khz > 0
    for kind in (0, 1):
        s = torch.zeros(64 * 256, dtype=torch.float32, device="cuda")
        clocks = torch.zeros(2, dtype=torch.int64, device="cuda")
        m.qg_probe_mfma(kind, 50, 64, s, clocks)
        torch.cuda.synchronize()
        cyc, ticks = (int(v) for v in clocks.cpu())
        assert ticks > 0 and 0.5e6 < cyc / (ticks / khz) < 3e6
    # matrix-core + vector-ALU loops and the LDS read loop fill their sinks
    for mf, nf in ((1, 0), (1, 4), (0, 4)):
        s = torch.full((64 * 512,), float("nan"), dtype=torch.float32, device="cuda")
        m.qg_probe_mfma_valu(mf, nf, 20, 64, 2, s)
        torch.cuda.synchronize()
        assert bool(torch.isfinite(s).all().item())
    for w in (4, 8, 16):
        si = torch.full((64 * 64 * 8,), -1, dtype=torch.int32, device="cuda")
        m.qg_probe_lds_read(w, 20, 64, 8, si)
        torch.cuda.synchronize()
        assert int((si == -1).sum().item()) < si.numel()
