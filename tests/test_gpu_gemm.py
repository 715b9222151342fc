"""Parity of the batched q8_row GEMM (int8 MFMA, exact int8 activation limbs)
with the fp64 oracle, through the C-ABI.  Bound per output:
|y - y_ref| <= 2e-5 * sum_i |w_i x_i|."""
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


def gpu_gemm(q, rs, xs, limbs):
    import torch
    m = qg()
    nb, K = xs.shape
    M = q.shape[0]
    W = m.Q8RowWeight.from_host(q, rs)
    x = torch.from_numpy(np.ascontiguousarray(xs)).cuda()
    y = torch.full((nb, M), float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(m.qgemm_q8row_batched_ws_bytes(nb, K), dtype=torch.uint8, device="cuda")
    m.qgemm_q8row_batched(W.packed, W.rs, x, y, nb, M, K, ws, xs_limbs=limbs)
    torch.cuda.synchronize()
    return y.cpu().numpy()


def within(y, yref, mass, what):
    err = np.abs(y.astype(np.float64) - yref)
    lim = REL * mass
    bad = ~(err <= lim)
    if bad.any():
        j = np.unravel_index(int(np.argmax(np.where(np.isnan(err), np.inf, err - lim))), err.shape)
        raise AssertionError(f"{what}: {int(bad.sum())}/{y.size} outside bound; worst {j}: "
                             f"y={y[j]!r} ref={yref[j]!r} err={err[j]:.3e} lim={lim[j]:.3e}")


SHAPES = [(1, 1, 4), (1, 64, 64), (3, 100, 68), (130, 257, 1028), (128, 256, 5120),
          (200, 300, 516), (64, 1000, 2048)]


@pytest.mark.parametrize("limbs", [0, 3])
@pytest.mark.parametrize("nb,M,K", SHAPES)
def test_gemm_small_shapes(nb, M, K, limbs):
    q, rs, xs = synth.q8gemm_inputs(nb, M, K, seed=nb + 7 * M + 13 * K)
    y = gpu_gemm(q, rs, xs, limbs)
    yref, mass = oracle.q8row_gemm(q, rs, xs)
    within(y, yref, mass, f"gemm {nb}x{M}x{K} limbs={limbs}")


@pytest.mark.parametrize("nb,M,K", [s for s in SHAPES if s[2] >= 512])
def test_gemm_two_limbs_where_its_error_model_holds(nb, M, K):
    # 16-bit activations: within the bound for N(0,1) rows of K >= 512.
    # Auto mode picks, per 128 rows of xs, one of the two forms: each group
    # of its output equals the 2-limb or the 3-limb result bit for bit.
    q, rs, xs = synth.q8gemm_inputs(nb, M, K, seed=nb + 7 * M + 13 * K)
    y2 = gpu_gemm(q, rs, xs, 2)
    y3 = gpu_gemm(q, rs, xs, 3)
    y0 = gpu_gemm(q, rs, xs, 0)
    yref, mass = oracle.q8row_gemm(q, rs, xs)
    within(y2, yref, mass, f"gemm {nb}x{M}x{K} limbs=2")
    for g in range(0, nb, 128):
        assert np.array_equal(y0[g:g + 128], y2[g:g + 128]) or np.array_equal(y0[g:g + 128], y3[g:g + 128])


def test_gemm_auto_picks_three_limbs_for_short_rows():
    # K = 4 or 64: too few terms for the 16-bit rounding to average out
    for nb, M, K in [(1, 1, 4), (3, 100, 68)]:
        q, rs, xs = synth.q8gemm_inputs(nb, M, K, seed=K)
        assert np.array_equal(gpu_gemm(q, rs, xs, 0), gpu_gemm(q, rs, xs, 3))


def test_gemm_auto_picks_three_limbs_for_outlier_rows():
    nb, M, K = 256, 512, 2048
    q, rs, xs = synth.q8gemm_inputs(nb, M, K, seed=5)
    xs[130, 17] = 3000.0      # activation outliers in the third 64-row tile
    xs[200, 1000] = -800.0    # and in the fourth
    y0 = gpu_gemm(q, rs, xs, 0)
    y2 = gpu_gemm(q, rs, xs, 2)
    y3 = gpu_gemm(q, rs, xs, 3)
    yref, mass = oracle.q8row_gemm(q, rs, xs)
    within(y0, yref, mass, "auto")
    within(y3, yref, mass, "3 limbs")
    # rows 128..255 hold outliers: auto runs the 3-limb kernel there, the
    # 2-limb kernel on rows 0..127; the kernels are deterministic.
    assert np.array_equal(y0[128:], y3[128:])
    assert np.array_equal(y0[:128], y2[:128])
    # the 16-bit form cannot hold these rows: it leaves the bound
    err2 = np.abs(y2[128:].astype(np.float64) - yref[128:])
    assert np.any(err2 > REL * mass[128:])


def test_gemm_zero_and_int8_min_rows():
    nb, M, K = 70, 130, 256
    q, rs, xs = synth.q8gemm_inputs(nb, M, K, seed=6)
    q[3, :] = -128
    xs[5, :] = 0.0
    rs[9] = 0.0
    for limbs in (0, 3):
        y = gpu_gemm(q, rs, xs, limbs)
        yref, mass = oracle.q8row_gemm(q, rs, xs)
        within(y, yref, mass, f"special limbs={limbs}")
        assert np.all(y[5] == 0.0) and np.all(y[:, 9] == 0.0)


def test_gemm_config_c5_sampled_entries():
    c = synth.CONFIGS["q8row_gemm_512x17408x5120"]
    q, rs, xs = synth.config_inputs("q8row_gemm_512x17408x5120")
    nb, M, K = c["nb"], c["M"], c["K"]
    y = gpu_gemm(q, rs, xs, 0)
    assert np.all(np.isfinite(y))
    rng = synth.rng_for(555)
    bs = np.concatenate([np.repeat(np.arange(nb), 4), rng.integers(0, nb, 20000)])
    os_ = np.concatenate([np.tile([0, 1, M - 2, M - 1], nb), rng.integers(0, M, 20000)])
    yref, mass = oracle.q8row_gemm(q, rs, xs, entries=(bs, os_))
    within(y[bs, os_], yref, mass, "GEMM 512x17408x5120 sampled")


def test_gemm_workspace_too_small_is_rejected():
    import torch
    m = qg()
    q, rs, xs = synth.q8gemm_inputs(4, 64, 64, seed=1)
    W = m.Q8RowWeight.from_host(q, rs)
    x = torch.from_numpy(xs).cuda()
    y = torch.empty((4, 64), dtype=torch.float32, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    with pytest.raises(m.QGError):
        m.qgemm_q8row_batched(W.packed, W.rs, x, y, 4, 64, 64, ws)


def test_gemm_largest_k_extreme_values():
    """K = 131068, the largest the entry point takes: every weight -128 (or
    127) against activation rows whose limbs reach the limb range's ends, so
    each limb's int32 sum comes close to 2^31 without wrapping."""
    nb, M, K = 4, 64, 131068
    r = synth.rng_for(97)
    q = r.integers(-127, 128, (M, K), dtype=np.int8)
    q[0, :] = -128
    q[1, :] = 127
    rs = r.uniform(0.001, 0.01, M).astype(np.float32)
    xs = r.standard_normal((nb, K)).astype(np.float32)
    xs[0, :] = -3.0                                   # a constant row: top limb -126 everywhere
    xs[1, :] = np.where(np.arange(K) % 2 == 0, 3.0, -3.0 + 2.0 ** -14).astype(np.float32)
    for limbs in (0, 3):
        y = gpu_gemm(q, rs, xs, limbs)
        yref, mass = oracle.q8row_gemm(q, rs, xs)
        within(y, yref, mass, f"largest K, limbs={limbs}")


# ---- the accuracy contract: sparse weight rows ------------------------------
def _sparse_case(nb, M, K, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    q = rng.integers(-127, 128, (M, K), dtype=np.int8)
    n1 = min(1024, M // 3)
    q[: 2 * n1] = 0
    for o in range(n1):                                    # one-hot rows
        q[o, rng.integers(0, K)] = rng.choice([-1, 1]) * rng.integers(1, 128)
    for o in range(n1, 2 * n1):                            # one non-zero per 64
        cols = np.arange(0, K, 64) + rng.integers(0, 64, K // 64)
        q[o, cols] = rng.integers(-127, 128, K // 64)
    rs = rng.uniform(0.001, 0.01, M).astype(np.float32)
    return q, rs, rng, n1


def _contract_u(xs_row, limbs):
    from test_gemm_error_model import exponent
    e = exponent(xs_row)
    return 2.0 ** (e - 1) * (257 if limbs == 2 else 1)


def test_gemm_sparse_rows_inside_contract_c5_shape():
    """One-hot rows and rows with one non-zero per 64 at the batched
    workload's shape (512 x 17408 x 5120), 3 limbs, activation rows whose
    entries are at least a fifth of the row maximum: condition (C) of the
    contract holds for every sampled output (checked here), and so must the
    2e-5 bound."""
    nb, M, K = 512, 17408, 5120
    q, rs, rng, n1 = _sparse_case(nb, M, K, 9200)
    xs = (rng.choice([-1.0, 1.0], (nb, K)) * rng.uniform(0.2, 1.0, (nb, K))
          * rng.uniform(0.1, 10.0, (nb, 1))).astype(np.float32)
    y = gpu_gemm(q, rs, xs, 3)
    bs = np.concatenate([rng.integers(0, nb, 6000), rng.integers(0, nb, 2000)])
    os_ = np.concatenate([rng.integers(0, 2 * n1, 6000), rng.integers(2 * n1, M, 2000)])
    yref, mass = oracle.q8row_gemm(q, rs, xs, entries=(bs, os_))
    A = np.abs(q.astype(np.int64)).sum(axis=1)
    u = np.array([_contract_u(xs[b], 3) for b in range(nb)])
    assert np.all(rs[os_].astype(np.float64) * u[bs] * A[os_] <= 1.9e-5 * mass), "case outside (C)"
    within(y[bs, os_], yref, mass, "sparse rows, 3 limbs")


@pytest.mark.skip(reason="outside the accuracy contract of qgemm_q8row_batched: one-hot weight rows whose "
                         "non-zero meets an activation far below its row's maximum break condition (C) for every "
                         "fixed-point limb count, and the fixed point then leaves the 2e-5 bound (the CPU error "
                         "model in test_gemm_error_model.py shows it); kept as the recorded out-of-class case")
def test_gemm_auto_one_hot_rows_on_small_activations_outside_contract():
    nb, M, K = 512, 17408, 5120
    rng = np.random.Generator(np.random.PCG64(9201))
    xs = rng.standard_normal((nb, K)).astype(np.float32)
    q = np.zeros((M, K), np.int8)
    for o in range(M):
        q[o, int(np.argmin(np.abs(xs[o % nb])))] = 127
    rs = rng.uniform(0.001, 0.01, M).astype(np.float32)
    y = gpu_gemm(q, rs, xs, 0)
    os_ = np.arange(0, M, 7)
    bs = os_ % nb
    yref, mass = oracle.q8row_gemm(q, rs, xs, entries=(bs, os_))
    within(y[bs, os_], yref, mass, "one-hot rows on the smallest activations, auto")


@pytest.mark.parametrize("limbs", [0, 2, 3])
def test_gemm_non_finite_rows_give_nan(limbs):
    """A row of xs holding an infinity or a NaN gives NaN for all its
    outputs; the other rows are unaffected and within the bound."""
    nb, M, K = 130, 300, 640
    q, rs, xs = synth.q8gemm_inputs(nb, M, K, seed=9202)
    xs = xs.copy()
    xs[3, 17] = np.inf
    xs[70, 5] = -np.inf
    xs[129, 600] = np.nan
    y = gpu_gemm(q, rs, xs, limbs)
    bad = [3, 70, 129]
    assert np.all(np.isnan(y[bad]))
    good = np.setdiff1d(np.arange(nb), bad)
    yref, mass = oracle.q8row_gemm(q, rs, xs[good])
    within(y[good], yref, mass, f"finite rows beside non-finite ones, limbs={limbs}")
