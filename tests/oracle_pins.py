"""Pins of the CPU oracle to facts outside itself.

Each pin takes an ``oracle.Oracle`` and raises AssertionError when the oracle
disagrees with what the pages or the mathematics fix: hand-worked examples
(``tests/golden``), library routines (numpy's binary16 decoder, numpy fp64
matmul), an independent encoder, brute force on tiny inputs, closed-form
special cases and exact invariants.  ``test_oracle.py`` runs them on the
oracle; ``test_oracle_mutants.py`` runs them on deliberately broken copies of
the oracle and requires that every copy fails at least one pin.
"""
from __future__ import annotations

import json
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _close(a, b, rel=1e-12, abs_=0.0):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    err = np.abs(a - b)
    lim = rel * np.abs(b) + abs_
    assert np.all(err <= lim), f"max err {err.max()} (limit {lim.flat[np.argmax(err - lim)]})"


# ---- independent encoder of GGUF-style Q2 blocks (test side) -------------
def encode_q2(codes: np.ndarray, d_bits: np.ndarray, group: int) -> np.ndarray:
    """codes uint8 [M][K] in 0..3, d_bits uint16 [M][K/group] -> block blob.

    Byte j of a block holds codes 4j..4j+3 at bit offsets 0, 2, 4, 6.
    """
    M, K = codes.shape
    ng = K // group
    c = codes.reshape(M, ng, group // 4, 4).astype(np.uint8)
    qs = c[..., 0] | (c[..., 1] << 2) | (c[..., 2] << 4) | (c[..., 3] << 6)
    blob = np.empty((M, ng, 2 + group // 4), np.uint8)
    blob[:, :, 0] = (d_bits & 0xFF).astype(np.uint8)
    blob[:, :, 1] = (d_bits >> 8).astype(np.uint8)
    blob[:, :, 2:] = qs
    return blob.reshape(-1)


def f16_values(d_bits):
    return np.asarray(d_bits, np.uint16).view(np.float16).astype(np.float64)


# ---- binary16 -------------------------------------------------------------
def pin_f16_all_vs_numpy(orc):
    bits = np.arange(1 << 16, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = np.array([orc.f16_to_f64(int(b)) for b in bits])
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def pin_f16_golden(orc):
    for bits, val in _golden("f16_points.json")["points"]:
        got = orc.f16_to_f64(bits)
        assert got == val and np.signbit(got) == np.signbit(val), (bits, got, val)


# ---- q8_row ---------------------------------------------------------------
def pin_q8row_hand(orc):
    g = _golden("q8row_hand.json")
    y, m = orc.q8row_gemv(np.array(g["q"], np.int8), np.array(g["rs"], np.float32),
                          np.array(g["xs"], np.float32))
    assert np.array_equal(y, np.array(g["y"])), y
    assert np.array_equal(m, np.array(g["mass"])), m


def pin_q8row_vs_numpy_matmul(orc):
    rng = np.random.Generator(np.random.PCG64(11))
    for M, K in [(1, 4), (7, 36), (33, 260)]:
        q = rng.integers(-128, 128, size=(M, K), dtype=np.int8)
        rs = rng.uniform(0.001, 0.01, M).astype(np.float32)
        xs = rng.standard_normal(K, dtype=np.float32)
        W = rs.astype(np.float64)[:, None] * q.astype(np.float64)
        ref = W @ xs.astype(np.float64)
        y, m = orc.q8row_gemv(q, rs, xs)
        _close(y, ref, rel=1e-12, abs_=1e-12)
        _close(m, np.abs(W) @ np.abs(xs.astype(np.float64)), rel=1e-12)


def pin_q8row_rows_subset(orc):
    rng = np.random.Generator(np.random.PCG64(12))
    q = rng.integers(-127, 128, size=(20, 16), dtype=np.int8)
    rs = rng.uniform(0.001, 0.01, 20).astype(np.float32)
    xs = rng.standard_normal(16, dtype=np.float32)
    y, _ = orc.q8row_gemv(q, rs, xs)
    rows = np.array([19, 0, 7, 7])
    ys, _ = orc.q8row_gemv(q, rs, xs, rows=rows)
    assert np.array_equal(ys, y[rows])


def pin_q8gemm_hand(orc):
    g = _golden("q8gemm_hand.json")
    y, _ = orc.q8row_gemm(np.array(g["q"], np.int8), np.array(g["rs"], np.float32),
                          np.array(g["xs"], np.float32))
    assert np.array_equal(y, np.array(g["y"])), y


def pin_q8gemm_vs_numpy(orc):
    rng = np.random.Generator(np.random.PCG64(13))
    nb, M, K = 5, 9, 68
    q = rng.integers(-127, 128, size=(M, K), dtype=np.int8)
    rs = rng.uniform(0.001, 0.01, M).astype(np.float32)
    xs = rng.standard_normal((nb, K), dtype=np.float32)
    W = rs.astype(np.float64)[:, None] * q.astype(np.float64)
    ref = xs.astype(np.float64) @ W.T
    y, m = orc.q8row_gemm(q, rs, xs)
    _close(y, ref, rel=1e-12, abs_=1e-12)
    _close(m, np.abs(xs.astype(np.float64)) @ np.abs(W).T, rel=1e-12)
    bs = np.array([4, 0, 2])
    os_ = np.array([8, 3, 0])
    ye, _ = orc.q8row_gemm(q, rs, xs, entries=(bs, os_))
    assert np.array_equal(ye, y[bs, os_])
    for b in range(nb):
        yb, _ = orc.q8row_gemv(q, rs, xs[b])
        _close(y[b], yb, rel=1e-14, abs_=1e-14)


# ---- activation quantisation ---------------------------------------------
def pin_act_quant_tie(orc):
    g = _golden("act_quant_tie.json")
    x = np.zeros(g["K"], np.float32)
    x[: len(g["x_head"])] = g["x_head"]
    xq, sc, suma = orc.act_quant_i8(x)
    assert list(xq[: len(g["xq_head"])]) == g["xq_head"], xq[:8]
    assert np.all(xq[len(g["xq_head"]):] == 0)
    assert sc == np.float32(g["act_scale"])
    assert list(suma) == g["suma"]


def _bits(v):
    return int(np.asarray(v, np.float32).reshape(()).view(np.uint32))


def _from_bits(b):
    return np.array([int(b, 16)], np.uint32).view(np.float32)[0]


def pin_act_quant_reciprocal(orc):
    """Reciprocal then multiply, as the page writes it: a division by the
    scale would turn the 84 of this vector into 85."""
    g = _golden("act_quant_reciprocal.json")
    x = np.zeros(g["K"], np.float32)
    x[: len(g["x_head_bits"])] = [_from_bits(b) for b in g["x_head_bits"]]
    xq, sc, suma = orc.act_quant_i8(x)
    assert list(xq[: len(g["xq_head"])]) == g["xq_head"], xq[:4]
    assert np.all(xq[len(g["xq_head"]):] == 0)
    assert _bits(sc) == int(g["act_scale_bits"], 16), hex(_bits(sc))
    assert list(suma) == g["suma"]


def pin_act_quant_invariants(orc):
    rng = np.random.Generator(np.random.PCG64(14))
    for K, scale in [(64, 1.0), (128, 3e-3), (4096, 1.0), (5120, 250.0), (17408, 1.0)]:
        x = (rng.standard_normal(K) * scale).astype(np.float32)
        xq, sc, suma = orc.act_quant_i8(x)
        amax = np.max(np.abs(x))
        assert sc == np.float32(amax) / np.float32(127.0)
        j = int(np.argmax(np.abs(x)))
        assert abs(int(xq[j])) == 127 and np.sign(xq[j]) == np.sign(x[j])
        assert np.max(np.abs(xq.astype(np.int32))) == 127
        r = np.abs(xq.astype(np.float64) - x.astype(np.float64) / np.float64(sc))
        assert np.all(r <= 0.5 + 1e-5), r.max()
        assert np.array_equal(suma, xq.astype(np.int32).reshape(-1, 64).sum(axis=1))


def pin_act_quant_pow2(orc):
    rng = np.random.Generator(np.random.PCG64(15))
    x = rng.standard_normal(1024).astype(np.float32)
    xq0, sc0, s0 = orc.act_quant_i8(x)
    for k in (-20, -3, -1, 1, 5, 30):
        xq, sc, s = orc.act_quant_i8((x * np.float32(2.0 ** k)).astype(np.float32))
        assert np.array_equal(xq, xq0) and np.array_equal(s, s0)
        assert sc == np.float32(sc0 * np.float32(2.0 ** k))


def pin_act_quant_zero(orc):
    xq, sc, suma = orc.act_quant_i8(np.zeros(128, np.float32))
    assert sc == 0.0 and not np.isnan(sc)
    assert np.all(xq == 0) and np.all(suma == 0)


# ---- Q2 -----------------------------------------------------------------
def _hand_block(case):
    group = case["group"]
    qs = np.full(group // 4, case["qs_fill"], np.uint8)
    for k, v in case["qs_set"].items():
        qs[int(k)] = v
    blob = np.empty(2 + group // 4, np.uint8)
    blob[0] = case["d_bits"] & 0xFF
    blob[1] = case["d_bits"] >> 8
    blob[2:] = qs
    return blob


def pin_q2_blocks_hand(orc):
    tie = _golden("act_quant_tie.json")
    for case in _golden("q2_blocks_hand.json")["cases"]:
        group = case["group"]
        blob = _hand_block(case)
        w = orc.q2_dequant(blob, 1, group, group)[0]
        if "w_head" in case:
            assert list(w[: len(case["w_head"])]) == case["w_head"], (case["name"], w[:8])
        for k, v in case.get("w_at", {}).items():
            assert w[int(k)] == v, (case["name"], k, w[int(k)])
        if "dot" in case:
            x = np.zeros(group, np.float32)
            x[: len(tie["x_head"])] = tie["x_head"]
            xq, sc, _ = orc.act_quant_i8(x)
            dots = orc.q2_dots(blob, 1, group, group, xq)
            assert dots[0, 0] == case["dot"], dots
            y, _ = orc.q2_gemv(blob, 1, group, group, xq, sc)
            assert y[0] == case["y"], y


def pin_q2_roundtrip_encoder(orc):
    rng = np.random.Generator(np.random.PCG64(16))
    for group, M, K in [(64, 3, 192), (128, 2, 384)]:
        codes = rng.integers(0, 4, size=(M, K), dtype=np.uint8)
        d_bits = np.abs(rng.normal(0, 0.02, size=(M, K // group))).astype(np.float16).view(np.uint16)
        d_bits[0, 0] = 0x0001  # a subnormal scale
        blob = encode_q2(codes, d_bits, group)
        w = orc.q2_dequant(blob, M, K, group)
        ref = np.repeat(f16_values(d_bits), group, axis=1) * (codes.astype(np.float64) - 1.0)
        assert np.array_equal(w, ref)


def _q2_case(rng, M, K, group):
    codes = rng.integers(0, 4, size=(M, K), dtype=np.uint8)
    d_bits = np.abs(rng.normal(0, 0.02, size=(M, K // group))).astype(np.float16).view(np.uint16)
    return codes, d_bits, encode_q2(codes, d_bits, group)


def pin_q2_dots_brute(orc):
    rng = np.random.Generator(np.random.PCG64(17))
    for group, M, K in [(64, 4, 256), (128, 3, 384)]:
        codes, _, _ = _q2_case(rng, M, K, group)
        ones = np.full((M, K // group), 0x3C00, np.uint16)  # d = 1.0
        blob = encode_q2(codes, ones, group)
        x = rng.standard_normal(K).astype(np.float32)
        xq, _, _ = orc.act_quant_i8(x)
        dots = orc.q2_dots(blob, M, K, group, xq)
        ref = ((codes.astype(np.int64) - 1) * xq.astype(np.int64)).reshape(M, K // 64, 64).sum(-1)
        assert np.array_equal(dots, ref)


def pin_q2_gemv_vs_dense(orc):
    rng = np.random.Generator(np.random.PCG64(18))
    for group, M, K in [(64, 5, 320), (128, 6, 640)]:
        codes, d_bits, blob = _q2_case(rng, M, K, group)
        x = rng.standard_normal(K).astype(np.float32)
        xq, sc, _ = orc.act_quant_i8(x)
        W = np.repeat(f16_values(d_bits), group, axis=1) * (codes.astype(np.float64) - 1.0)
        xd = np.float64(sc) * xq.astype(np.float64)
        y, m = orc.q2_gemv(blob, M, K, group, xq, sc)
        _close(y, W @ xd, rel=1e-12, abs_=1e-15)
        _close(m, np.abs(W) @ np.abs(xd), rel=1e-12)
        rows = np.array([M - 1, 0])
        yr, _ = orc.q2_gemv(blob, M, K, group, xq, sc, rows=rows)
        assert np.array_equal(yr, y[rows])


def pin_q2_g128_is_two_g64(orc):
    rng = np.random.Generator(np.random.PCG64(19))
    M, K = 3, 512
    codes, d128, blob128 = _q2_case(rng, M, K, 128)
    blob64 = encode_q2(codes, np.repeat(d128, 2, axis=1), 64)
    x = rng.standard_normal(K).astype(np.float32)
    xq, sc, _ = orc.act_quant_i8(x)
    assert np.array_equal(orc.q2_dequant(blob128, M, K, 128), orc.q2_dequant(blob64, M, K, 64))
    assert np.array_equal(orc.q2_dots(blob128, M, K, 128, xq), orc.q2_dots(blob64, M, K, 64, xq))
    assert np.array_equal(orc.q2_gemv(blob128, M, K, 128, xq, sc)[0],
                          orc.q2_gemv(blob64, M, K, 64, xq, sc)[0])


def pin_q2_codes_one_zero(orc):
    rng = np.random.Generator(np.random.PCG64(20))
    M, K = 4, 256
    codes = np.ones((M, K), np.uint8)
    d_bits = np.abs(rng.normal(0, 0.02, size=(M, K // 64))).astype(np.float16).view(np.uint16)
    blob = encode_q2(codes, d_bits, 64)
    xq, sc, _ = orc.act_quant_i8(rng.standard_normal(K).astype(np.float32))
    y, _ = orc.q2_gemv(blob, M, K, 64, xq, sc)
    assert np.all(y == 0.0)
    assert np.all(orc.q2_dots(blob, M, K, 64, xq) == 0)


def pin_q2_pow2(orc):
    rng = np.random.Generator(np.random.PCG64(21))
    M, K = 6, 384
    _, _, blob = _q2_case(rng, M, K, 128)
    x = rng.standard_normal(K).astype(np.float32)
    xq0, sc0, _ = orc.act_quant_i8(x)
    y0, _ = orc.q2_gemv(blob, M, K, 128, xq0, sc0)
    for k in (-7, 3, 12):
        xq, sc, _ = orc.act_quant_i8((x * np.float32(2.0 ** k)).astype(np.float32))
        y, _ = orc.q2_gemv(blob, M, K, 128, xq, sc)
        assert np.array_equal(y, y0 * 2.0 ** k)


# ---- Q2 GEMV plus residual ------------------------------------------------
def pin_q2_accum_hand(orc):
    """The hand block with y = 126 (codes 2, d = 1, tie activation) plus a residual."""
    tie = _golden("act_quant_tie.json")
    case = [c for c in _golden("q2_blocks_hand.json")["cases"] if "dot" in c][0]
    blob = _hand_block(case)
    x = np.zeros(64, np.float32)
    x[: len(tie["x_head"])] = tie["x_head"]
    xq, sc, _ = orc.act_quant_i8(x)
    for a, want in [(0.5, 126.5), (-126.0, 0.0), (0.0, 126.0), (-1000.25, -874.25)]:
        y, _ = orc.q2_gemv_accum(blob, 1, 64, 64, xq, sc, np.array([a], np.float32))
        assert y[0] == want, (a, y)


def pin_q2_accum_zero_projection(orc):
    """All codes 1: the projection is exactly 0, so the result is the residual itself."""
    rng = np.random.Generator(np.random.PCG64(22))
    M, K = 7, 256
    codes = np.ones((M, K), np.uint8)
    d_bits = np.abs(rng.normal(0, 0.02, size=(M, K // 128))).astype(np.float16).view(np.uint16)
    blob = encode_q2(codes, d_bits, 128)
    xq, sc, _ = orc.act_quant_i8(rng.standard_normal(K).astype(np.float32))
    acc = rng.standard_normal(M).astype(np.float32)
    y, _ = orc.q2_gemv_accum(blob, M, K, 128, xq, sc, acc)
    assert np.array_equal(y, acc.astype(np.float64))


def pin_q2_accum_rows_subset(orc):
    """A row subset returns exactly those rows of the full result, residual included."""
    rng = np.random.Generator(np.random.PCG64(23))
    M, K = 9, 192
    _, _, blob = _q2_case(rng, M, K, 64)
    xq, sc, _ = orc.act_quant_i8(rng.standard_normal(K).astype(np.float32))
    acc = (rng.standard_normal(M) * 100).astype(np.float32)
    y, m = orc.q2_gemv_accum(blob, M, K, 64, xq, sc, acc)
    rows = [8, 2, 5]
    ys, ms = orc.q2_gemv_accum(blob, M, K, 64, xq, sc, acc, rows=rows)
    assert np.array_equal(ys, y[rows]) and np.array_equal(ms, m[rows])
    y0, m0 = orc.q2_gemv(blob, M, K, 64, xq, sc)
    assert np.array_equal(m, m0)


# ---- batched Q2 ---------------------------------------------------------------
def _q2_rows_case(orc, rng, nb, M, K, group):
    _, _, blob = _q2_case(rng, M, K, group)
    X = (rng.standard_normal((nb, K)) * rng.uniform(0.1, 10.0, size=(nb, 1))).astype(np.float32)
    q = [orc.act_quant_i8(X[b]) for b in range(nb)]
    xq = np.stack([t[0] for t in q])
    sc = np.array([t[1] for t in q], np.float32)
    return blob, xq, sc


def pin_q2_gemm_rows_are_gemvs(orc):
    """One token of the batched product is the GEMV of that token's activation."""
    rng = np.random.Generator(np.random.PCG64(29))
    nb, M, K = 5, 7, 384
    blob, xq, sc = _q2_rows_case(orc, rng, nb, M, K, 128)
    y, m = orc.q2_gemm(blob, M, K, 128, xq, sc)
    for b in range(nb):
        yb, mb = orc.q2_gemv(blob, M, K, 128, xq[b], sc[b])
        assert np.array_equal(y[b], yb) and np.array_equal(m[b], mb)


def pin_q2_gemm_vs_dense(orc):
    """Dense dequantised weights times sc[b] * xq[b] by numpy's fp64 matmul."""
    rng = np.random.Generator(np.random.PCG64(30))
    for group, nb, M, K in [(64, 4, 6, 256), (128, 3, 5, 512)]:
        blob, xq, sc = _q2_rows_case(orc, rng, nb, M, K, group)
        w = orc.q2_dequant(blob, M, K, group)
        ref = (xq.astype(np.float64) * sc.astype(np.float64)[:, None]) @ w.T
        y, _ = orc.q2_gemm(blob, M, K, group, xq, sc)
        _close(y, ref, rel=1e-12, abs_=1e-12)


def pin_q2_gemm_entries_and_residual(orc):
    """Listed entries equal the full output; a residual adds per (b, o)."""
    rng = np.random.Generator(np.random.PCG64(31))
    nb, M, K = 4, 9, 192
    blob, xq, sc = _q2_rows_case(orc, rng, nb, M, K, 64)
    y, m = orc.q2_gemm(blob, M, K, 64, xq, sc)
    bs = np.array([3, 0, 2, 1, 3])
    os_ = np.array([8, 4, 0, 7, 1])
    ye, me = orc.q2_gemm(blob, M, K, 64, xq, sc, entries=(bs, os_))
    assert np.array_equal(ye, y[bs, os_]) and np.array_equal(me, m[bs, os_])
    acc = np.round(rng.standard_normal((nb, M)) * 8).astype(np.float32)  # integers: the sums are exact
    ya, _ = orc.q2_gemm(blob, M, K, 64, xq, sc, accum=acc)
    codes_one = encode_q2(np.ones((M, K), np.uint8), np.full((M, K // 64), 0x3C00, np.uint16), 64)
    y0, _ = orc.q2_gemm(codes_one, M, K, 64, xq, sc, accum=acc)
    assert np.array_equal(y0, acc.astype(np.float64))
    _close(ya, y + acc.astype(np.float64), rel=1e-15, abs_=1e-12)


# ---- RMSNorm + quantiser ----------------------------------------------------
def pin_rmsnorm_unit_vector(orc):
    """x = 1 everywhere and eps = 0: mean(x^2) = 1 exactly, inv = 1, so the
    normalised vector is w itself and the outputs are the quantiser's on w."""
    rng = np.random.Generator(np.random.PCG64(24))
    for K in (64, 128, 5120):
        w = rng.standard_normal(K).astype(np.float32)
        v, xq, sc, suma = orc.rmsnorm_quant_i8(np.ones(K, np.float32), w, 0.0)
        xq0, sc0, s0 = orc.act_quant_i8(w)
        assert np.array_equal(v, w) and np.array_equal(xq, xq0) and sc == sc0 and np.array_equal(suma, s0)


def pin_rmsnorm_eps(orc):
    """x = 1, eps = 3: mean + eps = 4, sqrt = 2, inv = 1/2 exactly, so v = w/2:
    the same codes as the quantiser on w and half its scale."""
    rng = np.random.Generator(np.random.PCG64(25))
    K = 256
    w = rng.standard_normal(K).astype(np.float32)
    v, xq, sc, suma = orc.rmsnorm_quant_i8(np.ones(K, np.float32), w, 3.0)
    xq0, sc0, s0 = orc.act_quant_i8(w)
    assert np.array_equal(v, w * np.float32(0.5))
    assert np.array_equal(xq, xq0) and sc == sc0 * np.float32(0.5) and np.array_equal(suma, s0)


def pin_rmsnorm_two_level(orc):
    """x alternating 1, 7 with w = 1 and eps = 0: mean(x^2) = 25, inv = f32(1/5);
    the 7s carry the maximum (code 127) and the 1s get round(127/7) = 18."""
    K = 128
    x = np.tile(np.array([1.0, 7.0], np.float32), K // 2)
    v, xq, sc, suma = orc.rmsnorm_quant_i8(x, np.ones(K, np.float32), 0.0)
    inv = np.float32(1.0) / np.float32(5.0)
    assert v[0] == inv and v[1] == np.float32(np.float32(7.0) * inv)
    assert np.array_equal(xq, np.tile(np.array([18, 127], np.int8), K // 2))
    assert list(suma) == [32 * (18 + 127)] * (K // 64)


def _rmsnorm_golden(orc, name, x, w):
    g = _golden(name)
    v, xq, sc, suma = orc.rmsnorm_quant_i8(x, w, g["eps"])
    n = len(g["v_bits_head"])
    assert [_bits(a) for a in v[:n]] == [int(b, 16) for b in g["v_bits_head"]], [hex(_bits(a)) for a in v[:n]]
    assert _bits(sc) == int(g["act_scale_bits"], 16), hex(_bits(sc))
    assert list(xq[: len(g["xq_head"])]) == g["xq_head"], xq[:4]
    assert list(suma) == g["suma"], suma
    return v, xq


def pin_rmsnorm_sum_of_squares_binary64(orc):
    """x = [4096, 1 x 1023]: the binary64 sum of squares is 16778239 where a
    binary32 one stays at 2^24, and the scale tells the two apart."""
    K = 1024
    x = np.ones(K, np.float32)
    x[0] = 4096.0
    v, xq = _rmsnorm_golden(orc, "rmsnorm_sum_of_squares.json", x, np.ones(K, np.float32))
    assert np.all(v[1:] == v[1]) and np.all(xq[1:] == 0)


def pin_rmsnorm_product_order(orc):
    """x alternating 1, 7 and w alternating 1, 1.5: (x*inv)*w rounds the 7s
    to 0x40066666, x*(inv*w) to 0x40066667."""
    K = 128
    x = np.tile(np.array([1.0, 7.0], np.float32), K // 2)
    w = np.tile(np.array([1.0, 1.5], np.float32), K // 2)
    v, xq = _rmsnorm_golden(orc, "rmsnorm_product_order.json", x, w)
    assert np.array_equal(v, np.tile(v[:2], K // 2)) and np.array_equal(xq, np.tile(xq[:2], K // 2))


def pin_rmsnorm_pow2(orc):
    """With eps = 0 the norm is invariant under x -> 2^k x (every step exact)."""
    rng = np.random.Generator(np.random.PCG64(26))
    K = 1024
    x = rng.standard_normal(K).astype(np.float32)
    w = (1.0 + 0.1 * rng.standard_normal(K)).astype(np.float32)
    ref = orc.rmsnorm_quant_i8(x, w, 0.0)
    for k in (-9, -1, 2, 13):
        got = orc.rmsnorm_quant_i8((x * np.float32(2.0 ** k)).astype(np.float32), w, 0.0)
        assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
        assert got[2] == ref[2] and np.array_equal(got[3], ref[3])


# ---- gated product + quantiser ----------------------------------------------
def pin_glu_saturated_gate(orc):
    """g = 100: exp(-100) is far below half an ulp of 1, so 1 + e = 1 and
    silu(g) = g, sigmoid(g) = 1 exactly: t = 100 u and t = u."""
    rng = np.random.Generator(np.random.PCG64(27))
    K = 320
    u = rng.standard_normal(K).astype(np.float32)
    g = np.full(K, 100.0, np.float32)
    t, xq, sc, suma = orc.glu_quant_i8(g, u, 0)
    ref = (np.float32(100.0) * u).astype(np.float32)
    xq0, sc0, s0 = orc.act_quant_i8(ref)
    assert np.array_equal(t, ref) and np.array_equal(xq, xq0) and sc == sc0 and np.array_equal(suma, s0)
    t, xq, sc, suma = orc.glu_quant_i8(g, u, 1)
    xq0, sc0, s0 = orc.act_quant_i8(u)
    assert np.array_equal(t, u) and np.array_equal(xq, xq0) and sc == sc0 and np.array_equal(suma, s0)


def pin_glu_zero_gate(orc):
    """g = 0: exp(0) = 1, so silu(0) = 0 and sigmoid(0) = 1/2 exactly."""
    rng = np.random.Generator(np.random.PCG64(28))
    K = 192
    u = rng.standard_normal(K).astype(np.float32)
    g = np.zeros(K, np.float32)
    t, xq, sc, suma = orc.glu_quant_i8(g, u, 0)
    assert np.all(t == 0.0) and np.all(xq == 0) and sc == 0.0 and np.all(suma == 0)
    t, xq, sc, suma = orc.glu_quant_i8(g, u, 1)
    xq0, sc0, s0 = orc.act_quant_i8(u)
    assert np.array_equal(t, u * np.float32(0.5))
    assert np.array_equal(xq, xq0) and sc == sc0 * np.float32(0.5) and np.array_equal(suma, s0)


def pin_glu_identities(orc):
    """sigmoid(g) + sigmoid(-g) = 1 and silu(g) - silu(-g) = g, to a few binary32 ulps."""
    g = np.linspace(-12.0, 12.0, 256).astype(np.float32)
    one = np.ones_like(g)
    sp = orc.glu_quant_i8(g, one, 1)[0].astype(np.float64)
    sn = orc.glu_quant_i8(-g, one, 1)[0].astype(np.float64)
    assert np.all(np.abs(sp + sn - 1.0) <= 2.0 ** -22)
    lp = orc.glu_quant_i8(g, one, 0)[0].astype(np.float64)
    ln = orc.glu_quant_i8(-g, one, 0)[0].astype(np.float64)
    assert np.all(np.abs((lp - ln) - g.astype(np.float64)) <= 2.0 ** -20 * (1.0 + np.abs(g)))



# ---- silu * mul * column prescale -------------------------------------------
def pin_silu_pre_values(orc):
    """Closed forms: silu(0) = 0; sigmoid(ln 3) = 3/4, so silu(ln 3) = 0.75 ln 3
    (to a few ulps: exp(-ln 3) = 1/3 is rounded); for g = 30, exp(-30) is below
    half an ulp of 1, so silu(30) = 30 exactly; for g = -100, exp(100)
    overflows binary32 and silu(-100) = -0."""
    g = np.array([0.0, np.log(3.0), 30.0, -100.0], np.float32)
    act = orc.silu_mul_pre(g, np.ones(4, np.float32))
    assert act[0] == 0.0 and act[2] == 30.0 and act[3] == 0.0
    assert abs(float(act[1]) - 0.75 * float(g[1])) <= 2.0 ** -21 * float(g[1])


def pin_silu_pre_vs_fp64(orc):
    """Against the definition x u c / (1 + exp(-x)) in fp64: five binary32
    roundings, so within 2^-21 relative."""
    rng = np.random.Generator(np.random.PCG64(61))
    n = 1000
    g = (3.0 * rng.standard_normal(n)).astype(np.float32)
    u = rng.standard_normal(n).astype(np.float32)
    c = rng.uniform(0.5, 2.0, n).astype(np.float32)
    act = orc.silu_mul_pre(g, u, c).astype(np.float64)
    gd, ud, cd = g.astype(np.float64), u.astype(np.float64), c.astype(np.float64)
    ref = gd * ud * cd / (1.0 + np.exp(-gd))
    assert np.all(np.abs(act - ref) <= 2.0 ** -21 * np.abs(ref))


def pin_silu_pre_odd_identity(orc):
    """silu(g) - silu(-g) = g (since sigmoid(g) + sigmoid(-g) = 1), to a few ulps."""
    g = np.linspace(-12.0, 12.0, 256).astype(np.float32)
    one = np.ones_like(g)
    lp = orc.silu_mul_pre(g, one).astype(np.float64)
    ln = orc.silu_mul_pre(-g, one).astype(np.float64)
    assert np.all(np.abs((lp - ln) - g.astype(np.float64)) <= 2.0 ** -20 * (1.0 + np.abs(g)))


def pin_silu_pre_scaling(orc):
    """Powers of two in u and col pass through every rounding exactly; no column
    field is the same as a column of ones."""
    rng = np.random.Generator(np.random.PCG64(62))
    n = 300
    g = (2.0 * rng.standard_normal(n)).astype(np.float32)
    u = rng.standard_normal(n).astype(np.float32)
    c = rng.uniform(0.25, 4.0, n).astype(np.float32)
    ref = orc.silu_mul_pre(g, u, c)
    assert np.array_equal(orc.silu_mul_pre(g, u), orc.silu_mul_pre(g, u, np.ones(n, np.float32)))
    assert np.array_equal(orc.silu_mul_pre(g, u * np.float32(8.0), c), ref * np.float32(8.0))
    assert np.array_equal(orc.silu_mul_pre(g, u, c * np.float32(0.25)), ref * np.float32(0.25))
    assert np.array_equal(orc.silu_mul_pre(g, u, np.full(n, 2.0, np.float32)),
                          orc.silu_mul_pre(g, u) * np.float32(2.0))


def pin_silu_pre_rows(orc):
    """Rows share the column field: every element of a [rows][n] call equals the
    one-element call on (g[r, i], u[r, i], col[i]), and a row without a column
    equals the gated product of the quantising producer."""
    rng = np.random.Generator(np.random.PCG64(63))
    rows, n = 3, 37
    g = (2.0 * rng.standard_normal((rows, n))).astype(np.float32)
    u = rng.standard_normal((rows, n)).astype(np.float32)
    c = rng.uniform(0.5, 2.0, n).astype(np.float32)
    act = orc.silu_mul_pre(g, u, c)
    for r in range(rows):
        for i in range(n):
            one = orc.silu_mul_pre(g[r, i:i + 1], u[r, i:i + 1], c[i:i + 1])
            assert act[r, i] == one[0], (r, i)
        t = orc.glu_quant_i8(np.pad(g[r], (0, 64 - n)), np.pad(u[r], (0, 64 - n)), 0)[0][:n]
        assert np.array_equal(orc.silu_mul_pre(g[r], u[r]), t)

ALL_PINS = {name: fn for name, fn in sorted(globals().items()) if name.startswith("pin_")}
