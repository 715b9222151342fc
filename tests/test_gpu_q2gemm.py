"""The batched (prefill) Q2 product and the row-batched quantiser, through
the C-ABI, against the oracle: per-row quantisation bit for bit, the product
within |y - y_ref| <= 2e-5 * sum_i |w_i x_i| per output (plus one binary32
rounding, 2^-24 |y_ref|, when a residual is added)."""
import numpy as np
import pytest

import oracle
import synth
from conftest import gpu_available
from test_gpu_parity import REL, dev, host, qg, within

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a HIP device")]

U32 = 2.0 ** -24


def _torch():
    import torch
    return torch


def gpu_quant_rows(X):
    torch = _torch()
    nb, K = X.shape
    xq = torch.empty((nb, K), dtype=torch.int8, device="cuda")
    sc = torch.empty(nb, dtype=torch.float32, device="cuda")
    suma = torch.empty((nb, K // 64), dtype=torch.int32, device="cuda")
    qg().qquant_act_i8_rows(dev(X), xq, sc, suma)
    return xq, sc, suma


def token_rows(nb, K, seed):
    rng = synth.rng_for(seed)
    # rows of different magnitudes, as tokens of a prefill batch
    return (rng.standard_normal((nb, K)) * rng.uniform(0.05, 20.0, size=(nb, 1))).astype(np.float32)


@pytest.mark.parametrize("nb,K", [(1, 64), (3, 192), (130, 1024), (512, 5120)])
def test_quant_rows_bit_exact(nb, K):
    X = token_rows(nb, K, 6000 + nb)
    xq, sc, suma = (host(t) for t in gpu_quant_rows(X))
    for b in range(nb):
        rq, rsc, rsu = oracle.act_quant_i8(X[b])
        assert np.array_equal(xq[b], rq), f"row {b}: codes differ"
        assert np.float32(sc[b]).view(np.uint32) == np.float32(rsc).view(np.uint32), f"row {b}: scale"
        assert np.array_equal(suma[b], rsu), f"row {b}: suma"


def run_gemm(blob, M, K, group, X, accum=None, in_place=False):
    torch = _torch()
    m = qg()
    W = m.Q2Weight.from_blocks(blob, M, K, group)
    xq, sc, suma = gpu_quant_rows(X)
    nb = X.shape[0]
    nws = m.qgemm_q2_batched_ws_bytes(M, K, group, nb)
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda") if nws else None
    if in_place:
        y = dev(accum)
        m.qgemm_q2_batched(W, xq, suma, sc, y, accum=y, ws=ws)
    else:
        y = torch.empty((nb, M), dtype=torch.float32, device="cuda")
        m.qgemm_q2_batched(W, xq, suma, sc, y, accum=None if accum is None else dev(accum), ws=ws)
    return host(y), host(xq), host(sc)


@pytest.mark.parametrize("nb,M,K,group", [(1, 64, 64, 64), (5, 100, 256, 128), (128, 272, 1024, 64),
                                          (129, 545, 640, 128), (200, 300, 2048, 64), (256, 1088, 512, 128)])
def test_q2_gemm_small_all_outputs(nb, M, K, group):
    blob, _ = synth.q2_inputs(M, K, group, seed=6100 + M + K)
    X = token_rows(nb, K, 6200 + nb)
    y, xq, sc = run_gemm(blob, M, K, group, X)
    yref, mass = oracle.q2_gemm(blob, M, K, group, xq, sc)
    within(y.reshape(-1), yref.reshape(-1), mass.reshape(-1), what=f"q2 gemm nb={nb} {M}x{K} g{group}")


@pytest.mark.parametrize("in_place", [False, True])
def test_q2_gemm_residual(in_place):
    nb, M, K, group = 96, 700, 1536, 128
    blob, _ = synth.q2_inputs(M, K, group, seed=6300)
    X = token_rows(nb, K, 6301)
    acc = (synth.rng_for(6302).standard_normal((nb, M)) * 3).astype(np.float32)
    y, xq, sc = run_gemm(blob, M, K, group, X, accum=acc, in_place=in_place)
    yref, mass = oracle.q2_gemm(blob, M, K, group, xq, sc, accum=acc)
    within(y.reshape(-1), yref.reshape(-1), (mass + U32 / REL * np.abs(yref)).reshape(-1), what="q2 gemm + residual")


def test_q2_gemm_c3_gate_prefill_sampled():
    """The 17408 x 5120 g128 gate matrix over 512 prefill tokens, sampled entries."""
    c = synth.CONFIGS["q2_g128_gate_17408x5120"]
    M, K, group = c["M"], c["K"], c["group"]
    blob, _ = synth.config_inputs("q2_g128_gate_17408x5120")
    nb = 512
    X = token_rows(nb, K, 6400)
    y, xq, sc = run_gemm(blob, M, K, group, X)
    assert np.all(np.isfinite(y))
    rng = synth.rng_for(6401)
    bs = np.concatenate([rng.integers(0, nb, 3000), np.full(64, nb - 1), np.zeros(64, np.int64)])
    os_ = np.concatenate([rng.integers(0, M, 3000), np.arange(M - 64, M), np.arange(64)])
    yref, mass = oracle.q2_gemm(blob, M, K, group, xq, sc, entries=(bs, os_))
    within(y[bs, os_], yref, mass, what="gate 17408x5120 prefill")


def test_q2_gemm_c3_down_prefill_split_sampled():
    """The 5120 x 17408 g128 down matrix over 512 tokens: its tiles take a K split."""
    c = synth.CONFIGS["q2_g128_down_5120x17408"]
    M, K, group = c["M"], c["K"], c["group"]
    assert qg().qgemm_q2_batched_ws_bytes(M, K, group, 512) > 0
    blob, _ = synth.config_inputs("q2_g128_down_5120x17408")
    X = token_rows(512, K, 6450)
    acc = synth.rng_for(6451).standard_normal((512, M)).astype(np.float32)
    y, xq, sc = run_gemm(blob, M, K, group, X, accum=acc)
    rng = synth.rng_for(6452)
    bs = np.concatenate([rng.integers(0, 512, 1500), np.full(32, 511)])
    os_ = np.concatenate([rng.integers(0, M, 1500), np.arange(M - 32, M)])
    yref, mass = oracle.q2_gemm(blob, M, K, group, xq, sc, accum=acc, entries=(bs, os_))
    within(y[bs, os_], yref, mass + U32 / REL * np.abs(yref), what="down 5120x17408 prefill + residual")


@pytest.mark.parametrize("M,in_place", [(17000, True), (16999, False), (16998, True)])
def test_q2_gemm_residual_one_split_ragged(M, in_place):
    """A residual on a product that takes no K split (63 row tiles x 3 token
    tiles), ragged in rows and tokens, in place and not, with M % 4 == 0 (16-byte
    output stores) and not: the residual of every output is read before the
    workgroup's first store, so y may be the residual itself."""
    nb, K, group = 300, 1024, 128
    assert qg().qgemm_q2_batched_ws_bytes(M, K, group, nb) == 0
    blob, _ = synth.q2_inputs(M, K, group, seed=6460 + M)
    X = token_rows(nb, K, 6461)
    acc = (synth.rng_for(6462).standard_normal((nb, M)) * 3).astype(np.float32)
    y, xq, sc = run_gemm(blob, M, K, group, X, accum=acc, in_place=in_place)
    rng = synth.rng_for(6463)
    bs = np.concatenate([rng.integers(0, nb, 2000), np.full(64, nb - 1), np.zeros(64, np.int64), np.full(64, 255)])
    os_ = np.concatenate([rng.integers(0, M, 2000), np.arange(M - 64, M), np.arange(64), np.arange(M - 64, M)])
    yref, mass = oracle.q2_gemm(blob, M, K, group, xq, sc, accum=acc, entries=(bs, os_))
    within(y[bs, os_], yref, mass + U32 / REL * np.abs(yref), what=f"q2 gemm {M} rows + residual, no split")


@pytest.mark.parametrize("K,group", [(32768, 128), (16384, 64)])
def test_q2_gemm_long_rows_split(K, group):
    """Long rows over a K split of the occupancy rule (16 row tiles x 4 token
    tiles: S = 4, 64 scale groups per split), sampled entries and the edges
    held to the oracle's bound."""
    nb, M = 512, 4352
    groups = K // group
    S = qg().qgemm_q2_batched_ws_bytes(M, K, group, nb) // (nb * M * 4)
    assert S == 4 and groups // S == 64, (S, groups)
    blob, _ = synth.q2_inputs(M, K, group, seed=6480 + group)
    X = token_rows(nb, K, 6481 + group)
    y, xq, sc = run_gemm(blob, M, K, group, X)
    rng = synth.rng_for(6482 + group)
    bs = np.concatenate([rng.integers(0, nb, 1200), np.full(32, nb - 1), np.zeros(32, np.int64)])
    os_ = np.concatenate([rng.integers(0, M, 1200), np.arange(M - 32, M), np.arange(32)])
    yref, mass = oracle.q2_gemm(blob, M, K, group, xq, sc, entries=(bs, os_))
    within(y[bs, os_], yref, mass, what=f"long rows {M}x{K} g{group}")


@pytest.mark.parametrize("nb,M,K,group", [(40, 300, 1024, 64), (7, 64, 256, 128), (5, 100, 5120, 128)])
def test_q2_gemm_split_small_shapes(nb, M, K, group):
    """Few tiles: K is split (several splits, short last split; at 100 x 5120
    g128, 40 groups over 16 splits of 3 leave the last two splits empty, and
    their zero partials must not disturb the sum)."""
    assert qg().qgemm_q2_batched_ws_bytes(M, K, group, nb) > 0
    blob, _ = synth.q2_inputs(M, K, group, seed=6460 + M)
    X = token_rows(nb, K, 6470 + nb)
    y, xq, sc = run_gemm(blob, M, K, group, X)
    yref, mass = oracle.q2_gemm(blob, M, K, group, xq, sc)
    within(y.reshape(-1), yref.reshape(-1), mass.reshape(-1), what=f"split nb={nb} {M}x{K}")


def test_q2_gemm_token_rows_match_gemv_bound():
    """Each token row of the product also matches the GEMV oracle of that token."""
    nb, M, K, group = 7, 130, 512, 64
    blob, _ = synth.q2_inputs(M, K, group, seed=6500)
    X = token_rows(nb, K, 6501)
    y, xq, sc = run_gemm(blob, M, K, group, X)
    for b in range(nb):
        yr, mr = oracle.q2_gemv(blob, M, K, group, xq[b], sc[b])
        within(y[b], yr, mr, what=f"token {b}")


@pytest.mark.parametrize("nb,M,K,group", [(40, 300, 1024, 128), (130, 600, 2048, 64), (512, 17408, 5120, 128)])
def test_q2_gemm_dual_equals_two_calls(nb, M, K, group):
    """The gate|up pair launch (the page's gemm_gpu_v4_dual) gives both outputs
    bit for bit as two one-matrix launches, with and without a K split; the
    small shapes are also held to the oracle's bound."""
    torch = _torch()
    m = qg()
    b0, _ = synth.q2_inputs(M, K, group, seed=7000 + M)
    b1, _ = synth.q2_inputs(M, K, group, seed=7001 + M)
    W0 = m.Q2Weight.from_blocks(b0, M, K, group)
    W1 = m.Q2Weight.from_blocks(b1, M, K, group)
    X = token_rows(nb, K, 7002 + nb)
    xq, sc, suma = gpu_quant_rows(X)
    n1 = m.qgemm_q2_batched_ws_bytes(M, K, group, nb)
    n2 = m.qgemm_q2_batched_dual_ws_bytes(M, K, group, nb)
    assert n2 == 2 * n1
    ws1 = torch.empty(n1, dtype=torch.uint8, device="cuda") if n1 else None
    ws2 = torch.empty(n2, dtype=torch.uint8, device="cuda") if n2 else None
    y0 = torch.full((nb, M), float("nan"), device="cuda")
    y1 = torch.full((nb, M), float("nan"), device="cuda")
    m.qgemm_q2_batched_dual(W0, W1, xq, suma, sc, y0, y1, ws=ws2)
    r0 = torch.full((nb, M), float("nan"), device="cuda")
    r1 = torch.full((nb, M), float("nan"), device="cuda")
    m.qgemm_q2_batched(W0, xq, suma, sc, r0, ws=ws1)
    m.qgemm_q2_batched(W1, xq, suma, sc, r1, ws=ws1)
    torch.cuda.synchronize()
    assert torch.equal(y0, r0) and torch.equal(y1, r1), f"pair launch differs ({nb}x{M}x{K} g{group})"
    if nb * M <= 200000:
        xq_h, sc_h = host(xq), host(sc)
        for blob, out in ((b0, y0), (b1, y1)):
            yref, mass = oracle.q2_gemm(blob, M, K, group, xq_h, sc_h)
            within(host(out).reshape(-1), yref.reshape(-1), mass.reshape(-1), what=f"pair {nb}x{M}x{K} g{group}")
