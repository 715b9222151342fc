"""The fused activation producers through the C-ABI (qquant_rmsnorm_i8,
qquant_glu_i8) against the oracle.

Everything they write is decided in binary32 on both sides, so the check is
bit-exact: the gated product t, the int8 codes, act_scale and the group sums.
"""
import numpy as np
import pytest

import oracle
import synth
from conftest import gpu_available
from test_gpu_parity import dev, host, qg

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a HIP device")]


def _torch():
    import torch
    return torch


def _outs(K):
    torch = _torch()
    return (torch.empty(K, dtype=torch.int8, device="cuda"),
            torch.empty(1, dtype=torch.float32, device="cuda"),
            torch.empty(K // 64, dtype=torch.int32, device="cuda"))


def gpu_rmsnorm(x, w, eps):
    xq, sc, suma = _outs(x.size)
    qg().qquant_rmsnorm_i8(dev(x), dev(w), eps, xq, sc, suma)
    return host(xq), host(sc)[0], host(suma)


def gpu_glu(g, u, kind, t_mode="separate"):
    """t_mode: 'separate' (own buffer), 'in_u' or 'in_g' (in place)."""
    torch = _torch()
    K = g.size
    xq, sc, suma = _outs(K)
    gd, ud = dev(g), dev(u)
    t = {"separate": torch.empty(K, dtype=torch.float32, device="cuda"), "in_u": ud, "in_g": gd}[t_mode]
    qg().qquant_glu_i8(gd, ud, kind, t, xq, sc, suma)
    return host(t), host(xq), host(sc)[0], host(suma)


def same_bits(a, b):
    return np.array_equal(np.asarray(a, np.float32).view(np.uint32), np.asarray(b, np.float32).view(np.uint32))


def assert_quant_equal(got, ref, what):
    xq, sc, suma = got
    rxq, rsc, rsuma = ref
    assert np.array_equal(xq, rxq), f"{what}: {int((xq != rxq).sum())} codes differ"
    assert same_bits(sc, rsc), f"{what}: act_scale {sc!r} vs {rsc!r}"
    assert np.array_equal(suma, rsuma), f"{what}: suma differs"


# ----------------------------------------------------------------- RMSNorm --
@pytest.mark.parametrize("K,scale,eps,seed", [(64, 1.0, 1e-6, 1), (192, 1e-3, 1e-5, 2), (4096, 1.0, 1e-6, 3),
                                              (5120, 1.0, 1e-6, 4), (5120, 40.0, 0.0, 5), (17408, 1.0, 1e-5, 6),
                                              (65536, 0.25, 1e-6, 7)])
def test_rmsnorm_quant_bit_exact(K, scale, eps, seed):
    rng = synth.rng_for(4000 + seed)
    x = (rng.standard_normal(K) * scale).astype(np.float32)
    w = (1.0 + 0.1 * rng.standard_normal(K)).astype(np.float32)
    _, rxq, rsc, rsuma = oracle.rmsnorm_quant_i8(x, w, eps)
    assert_quant_equal(gpu_rmsnorm(x, w, eps), (rxq, rsc, rsuma), f"rmsnorm K={K}")


def test_rmsnorm_closed_forms():
    rng = synth.rng_for(4010)
    K = 1024
    w = rng.standard_normal(K).astype(np.float32)
    ref = oracle.act_quant_i8(w)
    # unit x, eps 0: the quantiser of w itself
    assert_quant_equal(gpu_rmsnorm(np.ones(K, np.float32), w, 0.0), ref, "unit x")
    # unit x, eps 3: inv = 1/2 exactly, same codes, half the scale
    xq, sc, suma = gpu_rmsnorm(np.ones(K, np.float32), w, 3.0)
    assert np.array_equal(xq, ref[0]) and sc == ref[1] * np.float32(0.5) and np.array_equal(suma, ref[2])
    # two-level x (1, 7): codes 18 and 127
    x = np.tile(np.array([1.0, 7.0], np.float32), K // 2)
    xq, _, _ = gpu_rmsnorm(x, np.ones(K, np.float32), 0.0)
    assert np.array_equal(xq, np.tile(np.array([18, 127], np.int8), K // 2))


def test_rmsnorm_zero_vector_with_eps():
    xq, sc, suma = gpu_rmsnorm(np.zeros(256, np.float32), np.ones(256, np.float32), 1e-6)
    assert sc == 0.0 and np.all(xq == 0) and np.all(suma == 0)


# ----------------------------------------------------------- gated product --
@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("K,seed", [(64, 1), (320, 2), (5120, 3), (17408, 4), (65536, 5)])
def test_glu_quant_bit_exact(kind, K, seed):
    rng = synth.rng_for(4100 + seed)
    g = (rng.standard_normal(K) * 2.5).astype(np.float32)
    u = rng.standard_normal(K).astype(np.float32)
    rt, rxq, rsc, rsuma = oracle.glu_quant_i8(g, u, kind)
    t, xq, sc, suma = gpu_glu(g, u, kind)
    assert same_bits(t, rt), f"t: {int((t.view(np.uint32) != rt.view(np.uint32)).sum())} differ"
    assert_quant_equal((xq, sc, suma), (rxq, rsc, rsuma), f"glu kind={kind} K={K}")


@pytest.mark.parametrize("kind", [0, 1])
def test_glu_extreme_gates(kind):
    """Gates where exp(-g) underflows to a subnormal or 0, overflows to inf, is 1."""
    K = 256
    rng = synth.rng_for(4120 + kind)
    g = rng.choice(np.array([0.0, -0.0, 100.0, -100.0, 87.5, -87.5, 88.8, -88.8, 103.9, -104.0, 150.0,
                             -150.0, 1e-7, -1e-7, 20.0, -20.0], np.float32), size=K).astype(np.float32)
    u = rng.standard_normal(K).astype(np.float32)
    rt, rxq, rsc, rsuma = oracle.glu_quant_i8(g, u, kind)
    t, xq, sc, suma = gpu_glu(g, u, kind)
    assert same_bits(t, rt)
    assert_quant_equal((xq, sc, suma), (rxq, rsc, rsuma), f"glu extremes kind={kind}")


@pytest.mark.parametrize("kind", [0, 1])
def test_glu_gate_sweep_vs_oracle(kind):
    """Gates spread evenly over the binary32 bit patterns of [-110, 110]
    (both signs, from 1e-30 up: exp(-g) from 1 through overflow and
    underflow): t, the codes, the scale and the group sums bit-exact against
    the oracle."""
    K = 65536
    pos_lo = int(np.array([1e-30], np.float32).view(np.uint32)[0])
    pos_hi = int(np.array([110.0], np.float32).view(np.uint32)[0])
    bits = np.linspace(pos_lo, pos_hi, K // 2).astype(np.uint32)
    g = np.concatenate([bits.view(np.float32), -bits.view(np.float32)])
    g = g[synth.rng_for(4140 + kind).permutation(K)].astype(np.float32)
    u = synth.rng_for(4142 + kind).standard_normal(K).astype(np.float32)
    rt, rxq, rsc, rsuma = oracle.glu_quant_i8(g, u, kind)
    t, xq, sc, suma = gpu_glu(g, u, kind)
    assert same_bits(t, rt), f"t: {int((t.view(np.uint32) != rt.view(np.uint32)).sum())} differ"
    assert_quant_equal((xq, sc, suma), (rxq, rsc, rsuma), f"glu sweep kind={kind}")


@pytest.mark.parametrize("mode", ["in_u", "in_g"])
def test_glu_output_modes(mode):
    rng = synth.rng_for(4130)
    K = 4096
    g = (rng.standard_normal(K) * 2.0).astype(np.float32)
    u = rng.standard_normal(K).astype(np.float32)
    rt, rxq, rsc, rsuma = oracle.glu_quant_i8(g, u, 0)
    t, xq, sc, suma = gpu_glu(g, u, 0, mode)
    assert same_bits(t, rt)
    assert_quant_equal((xq, sc, suma), (rxq, rsc, rsuma), f"glu t={mode}")


# ---------------------------------------------------- batches of token rows --
@pytest.mark.parametrize("nb,K", [(1, 64), (5, 320), (64, 5120), (33, 17408)])
def test_rmsnorm_quant_rows_bit_exact(nb, K):
    torch = _torch()
    rng = synth.rng_for(4200 + nb)
    X = (rng.standard_normal((nb, K)) * rng.uniform(0.01, 30.0, size=(nb, 1))).astype(np.float32)
    w = (1.0 + 0.1 * rng.standard_normal(K)).astype(np.float32)
    xq = torch.empty((nb, K), dtype=torch.int8, device="cuda")
    sc = torch.empty(nb, dtype=torch.float32, device="cuda")
    suma = torch.empty((nb, K // 64), dtype=torch.int32, device="cuda")
    qg().qquant_rmsnorm_i8_rows(dev(X), dev(w), 1e-6, xq, sc, suma)
    xq, sc, suma = host(xq), host(sc), host(suma)
    for b in range(nb):
        _, rxq, rsc, rsu = oracle.rmsnorm_quant_i8(X[b], w, 1e-6)
        assert_quant_equal((xq[b], sc[b], suma[b]), (rxq, rsc, rsu), f"rmsnorm row {b}")


@pytest.mark.parametrize("kind", [0, 1])
@pytest.mark.parametrize("nb,K", [(1, 64), (7, 1088), (48, 17408), (64, 1088), (72, 17408), (64, 18496)])
def test_glu_quant_rows_bit_exact(kind, nb, K):
    """Below 64 rows the two-launch form, from 64 rows one workgroup per row
    holding its t in LDS (K <= 18432; 18496 takes the two-launch form)."""
    torch = _torch()
    rng = synth.rng_for(4300 + nb + kind)
    G = (rng.standard_normal((nb, K)) * 2.5).astype(np.float32)
    U = rng.standard_normal((nb, K)).astype(np.float32)
    t = torch.empty((nb, K), dtype=torch.float32, device="cuda")
    xq = torch.empty((nb, K), dtype=torch.int8, device="cuda")
    sc = torch.empty(nb, dtype=torch.float32, device="cuda")
    suma = torch.empty((nb, K // 64), dtype=torch.int32, device="cuda")
    qg().qquant_glu_i8_rows(dev(G), dev(U), kind, t, xq, sc, suma)
    t, xq, sc, suma = host(t), host(xq), host(sc), host(suma)
    for b in range(nb):
        rt, rxq, rsc, rsu = oracle.glu_quant_i8(G[b], U[b], kind)
        assert same_bits(t[b], rt), f"row {b}: t differs"
        assert_quant_equal((xq[b], sc[b], suma[b]), (rxq, rsc, rsu), f"glu row {b}")


@pytest.mark.parametrize("kind", [0, 1])
def test_glu_quant_rows_in_place(kind):
    """The one-launch batch form with t written over g, then over u."""
    torch = _torch()
    nb, K = 96, 5120
    rng = synth.rng_for(4400 + kind)
    G = (rng.standard_normal((nb, K)) * 2.5).astype(np.float32)
    U = rng.standard_normal((nb, K)).astype(np.float32)
    for over in ("g", "u"):
        g_d, u_d = dev(G), dev(U)
        t = g_d if over == "g" else u_d
        xq = torch.empty((nb, K), dtype=torch.int8, device="cuda")
        sc = torch.empty(nb, dtype=torch.float32, device="cuda")
        suma = torch.empty((nb, K // 64), dtype=torch.int32, device="cuda")
        qg().qquant_glu_i8_rows(g_d, u_d, kind, t, xq, sc, suma)
        th, xq, sc, suma = host(t), host(xq), host(sc), host(suma)
        for b in (0, 1, nb // 2, nb - 1):
            rt, rxq, rsc, rsu = oracle.glu_quant_i8(G[b], U[b], kind)
            assert same_bits(th[b], rt), f"row {b}: t over {over} differs"
            assert_quant_equal((xq[b], sc[b], suma[b]), (rxq, rsc, rsu), f"glu row {b}, t over {over}")
