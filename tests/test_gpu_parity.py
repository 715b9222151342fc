"""Parity of the HIP path (through the C-ABI) with the CPU oracle.

Integer results (the quantised activations, their group sums, the Q2 unit
dots) must be bit-exact.  Every f32 output must satisfy
    |y - y_ref| <= 2e-5 * sum_i |w_i x_i|
per output, with y_ref and the sum from the fp64 oracle.  Full-size
workloads are checked on sampled rows the oracle computes one by one, in the
launch configuration the bench times.
"""
import numpy as np
import pytest

import oracle
import synth
from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a HIP device")]

REL = 2e-5


def _torch():
    import torch
    return torch


def dev(a):
    return _torch().from_numpy(np.ascontiguousarray(a)).to("cuda")


def host(t):
    _torch().cuda.synchronize()
    return t.cpu().numpy()


def within(y, yref, mass, rel=REL, what=""):
    y = np.asarray(y, np.float64)
    err = np.abs(y - yref)
    lim = rel * mass
    bad = err > lim
    if bad.any():
        j = int(np.argmax(err - lim))
        raise AssertionError(f"{what}: {int(bad.sum())}/{y.size} outputs outside the bound; "
                             f"worst at {j}: y={y[j]!r} ref={yref[j]!r} err={err[j]:.3e} lim={lim[j]:.3e}")


def qg():
    import weight_quantized_decode_q8_amd as m
    return m


# ------------------------------------------------------- activation quant --
def gpu_act_quant(x):
    torch = _torch()
    K = x.size
    xq = torch.empty(K, dtype=torch.int8, device="cuda")
    sc = torch.empty(1, dtype=torch.float32, device="cuda")
    suma = torch.empty(K // 64, dtype=torch.int32, device="cuda")
    qg().qquant_act_i8(dev(x), xq, sc, suma)
    return host(xq), host(sc)[0], host(suma), (xq, sc, suma)


def assert_quant_exact(x):
    xq, sc, suma, _ = gpu_act_quant(x)
    rq, rsc, rsuma = oracle.act_quant_i8(x)
    assert np.array_equal(xq, rq), f"{int((xq != rq).sum())} xq differ"
    assert np.float32(sc).view(np.uint32) == np.float32(rsc).view(np.uint32), (sc, rsc)
    assert np.array_equal(suma, rsuma)


@pytest.mark.parametrize("K,scale,seed", [(64, 1.0, 1), (192, 1e-3, 2), (1088, 300.0, 3),
                                          (4096, 1.0, 4), (5120, 1.0, 5), (17408, 1.0, 6),
                                          (65536, 1.0, 7)])
def test_act_quant_bit_exact(K, scale, seed):
    assert_quant_exact((synth.activation(K, seed) * np.float32(scale)).astype(np.float32))


def test_act_quant_ties_and_signs():
    # the hand example plus exact half-way points in both signs
    x = np.zeros(128, np.float32)
    x[:5] = [127, 0.5, 1.5, -0.5, -2.5]
    x[5:16] = np.arange(11) - 5.5
    x[64] = -127.0
    assert_quant_exact(x)
    xq, sc, suma, _ = gpu_act_quant(x)
    assert list(xq[:5]) == [127, 1, 2, -1, -3] and sc == 1.0


def test_act_quant_zero_vector():
    xq, sc, suma, _ = gpu_act_quant(np.zeros(256, np.float32))
    assert sc == 0.0 and np.all(xq == 0) and np.all(suma == 0)


# ------------------------------------------------------------- q8_row GEMV --
def gpu_q8row(q, rs, xs):
    torch = _torch()
    W = qg().Q8RowWeight.from_host(q, rs)
    y = torch.empty(q.shape[0], dtype=torch.float32, device="cuda")
    W.gemv(dev(xs), y)
    return host(y)


@pytest.mark.parametrize("M,K", [(1, 4), (1, 16), (3, 12), (63, 20), (64, 64), (65, 100),
                                 (130, 1028), (200, 4100), (64, 17408)])
def test_q8row_small_shapes(M, K):
    q, rs, xs = synth.q8row_inputs(M, K, seed=M * 7 + K)
    y = gpu_q8row(q, rs, xs)
    yref, mass = oracle.q8row_gemv(q, rs, xs)
    within(y, yref, mass, what=f"q8row {M}x{K}")


def test_q8row_config_c1_all_outputs():
    q, rs, xs = synth.config_inputs("q8row_256x512")
    y = gpu_q8row(q, rs, xs)
    yref, mass = oracle.q8row_gemv(q, rs, xs)
    within(y, yref, mass, what="q8row 256x512")


def test_q8row_int8_min_and_zero_rows():
    rng = synth.rng_for(99)
    M, K = 128, 512
    q = rng.integers(-128, 128, size=(M, K), dtype=np.int8)
    q[5, :] = -128
    rs = rng.uniform(0.001, 0.01, M).astype(np.float32)
    rs[7] = 0.0
    q[9, :] = 0
    xs = rng.standard_normal(K, dtype=np.float32)
    y = gpu_q8row(q, rs, xs)
    yref, mass = oracle.q8row_gemv(q, rs, xs)
    within(y, yref, mass, what="int8 min")
    assert y[7] == 0.0 and y[9] == 0.0


def test_q8row_config_c4_sampled_rows():
    q, rs, xs = synth.config_inputs("q8row_lm_head_248320x5120")
    M = q.shape[0]
    y = gpu_q8row(q, rs, xs)
    assert np.all(np.isfinite(y))
    rng = synth.rng_for(404)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(M - 64, M),
                                     rng.integers(0, M, 6000)]))
    yref, mass = oracle.q8row_gemv(q, rs, xs, rows=rows)
    within(y[rows], yref, mass, what="lm_head 248320x5120 sampled")


# ------------------------------------------------------------------ Q2 GEMV --
def sub_blob(blob, M, K, group, rows):
    """Blocks of the given rows only (blocks are row-major)."""
    rb = (K // group) * (2 + group // 4)
    return blob.reshape(M, rb)[rows].reshape(-1)


def gpu_q2(blob, M, K, group, x, split_k=0, want_dots=True):
    torch = _torch()
    m = qg()
    W = m.Q2Weight.from_blocks(blob, M, K, group)
    xq_h, sc_h, suma_h, (xq, sc, suma) = gpu_act_quant(x)
    y = torch.empty(M, dtype=torch.float32, device="cuda")
    nws = m.qgemv_q2_ws_bytes(M, K, group, split_k)
    ws = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda") if nws else None
    if want_dots:
        dots = torch.empty((M, K // 64), dtype=torch.int32, device="cuda")
        m.qgemv_q2_dots(W, xq, suma, sc, y, dots, ws, split_k)
        return host(y), host(dots), xq_h, sc_h
    m.qgemv_q2(W, xq, suma, sc, y, ws, split_k)
    return host(y), None, xq_h, sc_h


def check_q2(blob, M, K, group, x, split_k=0, rows=None, what=""):
    y, dots, xq, sc = gpu_q2(blob, M, K, group, x, split_k)
    rq, rsc, _ = oracle.act_quant_i8(x)
    assert np.array_equal(xq, rq) and sc == rsc
    if rows is None:
        rdots = oracle.q2_dots(blob, M, K, group, rq)
        assert np.array_equal(dots, rdots), f"{what}: {int((dots != rdots).sum())} dots differ"
        yref, mass = oracle.q2_gemv(blob, M, K, group, rq, rsc)
        within(y, yref, mass, what=what)
    else:
        sb = sub_blob(blob, M, K, group, rows)
        rdots = oracle.q2_dots(sb, len(rows), K, group, rq)
        assert np.array_equal(dots[rows], rdots), f"{what}: {int((dots[rows] != rdots).sum())} dots differ"
        yref, mass = oracle.q2_gemv(blob, M, K, group, rq, rsc, rows=rows)
        within(y[rows], yref, mass, what=what)
    return y, dots


@pytest.mark.parametrize("M,K,group", [(1, 64, 64), (3, 128, 128), (65, 192, 64), (100, 256, 128),
                                       (64, 1024, 128), (129, 640, 128), (200, 4096, 64)])
def test_q2_small_shapes(M, K, group):
    blob, x = synth.q2_inputs(M, K, group, seed=M + 3 * K + group)
    check_q2(blob, M, K, group, x, what=f"q2 {M}x{K} g{group}")


def test_q2_config_c2_all_outputs():
    blob, x = synth.config_inputs("q2_g64_4096x4096")
    check_q2(blob, 4096, 4096, 64, x, what="Q2 g64 4096x4096")


@pytest.mark.parametrize("name", ["q2_g128_gate_17408x5120", "q2_g128_up_17408x5120", "q2_g128_down_5120x17408"])
def test_q2_config_c3_sampled_rows(name):
    c = synth.CONFIGS[name]
    blob, x = synth.config_inputs(name)
    M, K = c["M"], c["K"]
    rng = synth.rng_for(333)
    rows = np.unique(np.concatenate([np.arange(64), np.arange(M - 64, M), rng.integers(0, M, 1500)]))
    check_q2(blob, M, K, 128, x, rows=rows, what=name)


@pytest.mark.parametrize("group", [64, 128])
def test_q2_split_invariance(group):
    M, K = 300, 2048
    blob, x = synth.q2_inputs(M, K, group, seed=77 + group)
    y1, d1 = check_q2(blob, M, K, group, x, split_k=1, what="S=1")
    for S in (2, 3, 4, 8, 16):
        yS, dS = check_q2(blob, M, K, group, x, split_k=S, what=f"S={S}")
        assert np.array_equal(dS, d1), f"dots depend on split {S}"


def test_q2_codes_one_gives_zero_and_subnormal_scales():
    from oracle_pins import encode_q2
    rng = synth.rng_for(5)
    M, K = 70, 256
    codes = rng.integers(0, 4, size=(M, K), dtype=np.uint8)
    codes[:10] = 1
    d_bits = np.abs(rng.normal(0, 0.02, size=(M, K // 64))).astype(np.float16).view(np.uint16)
    d_bits[10:20] = rng.integers(1, 0x400, size=(10, K // 64), dtype=np.uint16)  # subnormal
    blob = encode_q2(codes, d_bits, 64)
    x = rng.standard_normal(K, dtype=np.float32)
    y, _ = check_q2(blob, M, K, 64, x, what="special")
    assert np.all(y[:10] == 0.0)


def test_q2_g128_equals_g64_split_blocks():
    from oracle_pins import encode_q2
    rng = synth.rng_for(6)
    M, K = 130, 512
    codes = rng.integers(0, 4, size=(M, K), dtype=np.uint8)
    d128 = np.abs(rng.normal(0, 0.02, size=(M, K // 128))).astype(np.float16).view(np.uint16)
    b128 = encode_q2(codes, d128, 128)
    b64 = encode_q2(codes, np.repeat(d128, 2, axis=1), 64)
    x = rng.standard_normal(K, dtype=np.float32)
    y128, d_128, _, _ = gpu_q2(b128, M, K, 128, x, split_k=1)
    y64, d_64, _, _ = gpu_q2(b64, M, K, 64, x, split_k=1)
    assert np.array_equal(d_128, d_64)
    yref, mass = oracle.q2_gemv(b128, M, K, 128, *oracle.act_quant_i8(x)[:2])
    within(y128, yref, mass, what="g128")
    within(y64, yref, mass, what="g64")


def test_q2_plain_entry_matches_dots_entry():
    blob, x = synth.q2_inputs(256, 1024, 128, seed=8)
    y_plain, _, _, _ = gpu_q2(blob, 256, 1024, 128, x, want_dots=False)
    y_dots, _, _, _ = gpu_q2(blob, 256, 1024, 128, x, want_dots=True)
    assert np.array_equal(y_plain, y_dots)


def test_q2_workspace_too_small_is_rejected():
    torch = _torch()
    m = qg()
    blob, x = synth.q2_inputs(128, 1024, 64, seed=9)
    W = m.Q2Weight.from_blocks(blob, 128, 1024, 64)
    _, _, _, (xq, sc, suma) = gpu_act_quant(x)
    y = torch.empty(128, dtype=torch.float32, device="cuda")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(m.QGError):
        m.qgemv_q2(W, xq, suma, sc, y, ws, split_k=4)
