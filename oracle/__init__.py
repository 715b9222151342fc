"""CPU oracle for the weight-only-quantized decode products (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product (the HIP library and its
binding) never imports it, and it never imports the product.

The arithmetic lives in ``qoracle.c`` (plain C, fp64 accumulation, the
activation quantiser in IEEE binary32); this module only builds that file
with gcc and marshals numpy arrays into it.  Each wrapper names the page and
function whose definition it follows (see ``qoracle.c`` for the full list).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qoracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared", "-std=c99"]

def build(src: str = _SRC, out: str = _LIB) -> str:
    """Compile a copy of the oracle's C source with gcc (always recompiles)."""
    tmp = out + ".tmp"
    subprocess.run(["gcc", *_CFLAGS, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _rows(rows):
    if rows is None:
        return None, None, 0
    r, p = _c(rows, np.int64)
    return r, p, len(r)


class Oracle:
    """numpy front end of one built copy of the oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.qo_f16_to_f64.restype = ctypes.c_double
        lib.qo_f16_to_f64.argtypes = [ctypes.c_uint16]
        lib.qo_q8row_gemv.restype = None
        lib.qo_q8row_gemv.argtypes = [P, P, P, I64, I64, P, I64, P, P]
        lib.qo_q8row_gemm.restype = None
        lib.qo_q8row_gemm.argtypes = [P, P, P, I64, I64, I64, P, P, I64, P, P]
        lib.qo_q2_dequant.restype = None
        lib.qo_q2_dequant.argtypes = [P, I64, I64, ctypes.c_int, P]
        lib.qo_act_quant_i8.restype = None
        lib.qo_act_quant_i8.argtypes = [P, I64, P, P, P]
        lib.qo_q2_dots.restype = None
        lib.qo_q2_dots.argtypes = [P, I64, I64, ctypes.c_int, P, P]
        lib.qo_q2_gemv.restype = None
        lib.qo_q2_gemv.argtypes = [P, I64, I64, ctypes.c_int, P, ctypes.c_float, P, I64, P, P]
        lib.qo_q2_gemv_accum.restype = None
        lib.qo_q2_gemv_accum.argtypes = [P, I64, I64, ctypes.c_int, P, ctypes.c_float, P, P, I64, P, P]
        lib.qo_q2_gemm.restype = None
        lib.qo_q2_gemm.argtypes = [P, I64, I64, ctypes.c_int, P, P, I64, P, P, P, I64, P, P]
        lib.qo_rmsnorm_quant_i8.restype = None
        lib.qo_rmsnorm_quant_i8.argtypes = [P, P, I64, ctypes.c_float, P, P, P, P]
        lib.qo_glu_quant_i8.restype = None
        lib.qo_glu_quant_i8.argtypes = [P, P, I64, ctypes.c_int, P, P, P, P]
        lib.qo_silu_mul_pre.restype = None
        lib.qo_silu_mul_pre.argtypes = [P, P, P, I64, I64, P]
        self.lib = lib

    def f16_to_f64(self, bits: int) -> float:
        """IEEE binary16 bit pattern -> float (subnormals as m * 2^-24)."""
        return self.lib.qo_f16_to_f64(int(bits) & 0xFFFF)

    def q8row_gemv(self, q, rs, xs, rows=None):
        """y[o] = rs[o] * sum_i q[o,i] xs[i] in fp64 (cortiq pages, q8_matvec).

        Returns ``(y, mass)`` with ``mass[o] = sum_i |rs[o] q[o,i] xs[i]|``.
        ``rows`` selects a subset of rows (outputs in that order).
        """
        q, qp = _c(q, np.int8)
        M, K = q.shape
        rs, rsp = _c(rs, np.float32)
        xs, xp = _c(xs, np.float32)
        assert rs.shape == (M,) and xs.shape == (K,)
        r, rp, n = _rows(rows)
        n = M if r is None else n
        y = np.empty(n, np.float64)
        m = np.empty(n, np.float64)
        self.lib.qo_q8row_gemv(qp, rsp, xp, M, K, rp, n, y.ctypes.data, m.ctypes.data)
        return y, m

    def q8row_gemm(self, q, rs, xs, entries=None):
        """y[b,o] = rs[o] * sum_i q[o,i] xs[b,i] in fp64 (cortiq pages, q8_matmat).

        ``entries=None`` gives the full ``[nb][M]`` output; else a pair
        ``(bs, os)`` of index arrays gives those entries only.  Returns (y, mass).
        """
        q, qp = _c(q, np.int8)
        M, K = q.shape
        rs, rsp = _c(rs, np.float32)
        xs, xp = _c(xs, np.float32)
        nb = xs.shape[0]
        assert xs.shape == (nb, K) and rs.shape == (M,)
        if entries is None:
            y = np.empty((nb, M), np.float64)
            m = np.empty((nb, M), np.float64)
            self.lib.qo_q8row_gemm(qp, rsp, xp, nb, M, K, None, None, 0,
                                   y.ctypes.data, m.ctypes.data)
            return y, m
        bs, bp = _c(entries[0], np.int64)
        os_, op = _c(entries[1], np.int64)
        n = len(bs)
        y = np.empty(n, np.float64)
        m = np.empty(n, np.float64)
        self.lib.qo_q8row_gemm(qp, rsp, xp, nb, M, K, bp, op, n, y.ctypes.data, m.ctypes.data)
        return y, m

    def q2_dequant(self, blob, M, K, group):
        """Dense w[o][i] = d * (code - 1) (qxmx page, dequant_embd)."""
        b, bp = _c(blob, np.uint8)
        assert b.size == M * (K // group) * (2 + group // 4)
        w = np.empty((M, K), np.float64)
        self.lib.qo_q2_dequant(bp, M, K, group, w.ctypes.data)
        return w

    def act_quant_i8(self, x):
        """Per-vector int8 quantisation in binary32 (qxmx page, gpu_rmsnorm_quant).

        Returns ``(xq int8[K], act_scale float32, suma int32[K/64])``.
        """
        x, xp = _c(x, np.float32)
        K = x.size
        xq = np.empty(K, np.int8)
        sc = np.zeros(1, np.float32)
        suma = np.empty(K // 64, np.int32)
        self.lib.qo_act_quant_i8(xp, K, xq.ctypes.data, sc.ctypes.data,
                                 suma.ctypes.data if K // 64 else None)
        return xq, sc[0], suma

    def q2_dots(self, blob, M, K, group, xq):
        """Exact int32 dots per 64-wide unit: sum (code - 1) * xq (qxmx page, gemv_dpas8)."""
        b, bp = _c(blob, np.uint8)
        xq, xqp = _c(xq, np.int8)
        dots = np.empty((M, K // 64), np.int32)
        self.lib.qo_q2_dots(bp, M, K, group, xqp, dots.ctypes.data)
        return dots

    def q2_gemv(self, blob, M, K, group, xq, sc, rows=None):
        """y[o] = sc * sum_u d(u) * dots[o][u] in fp64 (qxmx page, gemv_dpas8 + gemv_reduce).

        Returns ``(y, mass)`` with ``mass[o] = sum_i |w_oi| |sc xq_i|``.
        """
        b, bp = _c(blob, np.uint8)
        xq, xqp = _c(xq, np.int8)
        r, rp, n = _rows(rows)
        n = M if r is None else n
        y = np.empty(n, np.float64)
        m = np.empty(n, np.float64)
        self.lib.qo_q2_gemv(bp, M, K, group, xqp, ctypes.c_float(float(sc)), rp, n,
                            y.ctypes.data, m.ctypes.data)
        return y, m

    def q2_gemv_accum(self, blob, M, K, group, xq, sc, accum, rows=None):
        """q2_gemv plus a residual: y[o] = proj[o] + accum[o] in fp64 (qxmx page, tmatvec_accum).

        Returns ``(y, mass)``; mass as q2_gemv.
        """
        b, bp = _c(blob, np.uint8)
        xq, xqp = _c(xq, np.int8)
        a, ap = _c(accum, np.float32)
        assert a.size == M
        r, rp, n = _rows(rows)
        n = M if r is None else n
        y = np.empty(n, np.float64)
        m = np.empty(n, np.float64)
        self.lib.qo_q2_gemv_accum(bp, M, K, group, xqp, ctypes.c_float(float(sc)), ap, rp, n,
                                  y.ctypes.data, m.ctypes.data)
        return y, m

    def q2_gemm(self, blob, M, K, group, xq, sc, accum=None, entries=None):
        """Batched Q2: y[b,o] = sc[b] * sum_u d(o,u) * dot(b,o,u) (+ accum[b,o]) in fp64
        (qxmx page, ffn_forward_b with gemm_gpu_v4).

        xq is int8 [nb][K] (row b quantised with scale sc[b]); ``entries=None``
        gives the full ``[nb][M]`` output, else ``(bs, os)`` index arrays.
        Returns (y, mass).
        """
        b, bp = _c(blob, np.uint8)
        xq, xqp = _c(xq, np.int8)
        sc, scp = _c(sc, np.float32)
        nb = sc.size
        assert xq.shape == (nb, K)
        ap = None
        if accum is not None:
            accum, ap = _c(accum, np.float32)
            assert accum.shape == (nb, M)
        if entries is None:
            y = np.empty((nb, M), np.float64)
            m = np.empty((nb, M), np.float64)
            self.lib.qo_q2_gemm(bp, M, K, group, xqp, scp, nb, ap, None, None, 0, y.ctypes.data, m.ctypes.data)
            return y, m
        bs, bsp = _c(entries[0], np.int64)
        os_, osp = _c(entries[1], np.int64)
        n = len(bs)
        y = np.empty(n, np.float64)
        m = np.empty(n, np.float64)
        self.lib.qo_q2_gemm(bp, M, K, group, xqp, scp, nb, ap, bsp, osp, n, y.ctypes.data, m.ctypes.data)
        return y, m

    def rmsnorm_quant_i8(self, x, w, eps):
        """RMSNorm in binary32 then the int8 quantiser (qxmx page, gpu_rmsnorm_quant).

        Returns ``(v float32[K], xq int8[K], act_scale float32, suma int32[K/64])``
        where v = (x * inv) * w, inv = 1 / sqrt(f32(sum x^2 / K) + eps).
        """
        x, xp = _c(x, np.float32)
        w, wp = _c(w, np.float32)
        K = x.size
        assert w.size == K
        v = np.empty(K, np.float32)
        xq = np.empty(K, np.int8)
        sc = np.zeros(1, np.float32)
        suma = np.empty(K // 64, np.int32)
        self.lib.qo_rmsnorm_quant_i8(xp, wp, K, ctypes.c_float(float(eps)), v.ctypes.data, xq.ctypes.data,
                                     sc.ctypes.data, suma.ctypes.data if K // 64 else None)
        return v, xq, sc[0], suma

    def glu_quant_i8(self, g, u, kind):
        """Gated product in binary32 then the int8 quantiser (qxmx page,
        gpu_swiglu_quant / gpu_silu_mul_quant for kind 0, gpu_sigmoid_mul_quant for kind 1).

        Returns ``(t float32[K], xq int8[K], act_scale float32, suma int32[K/64])``.
        """
        g, gp = _c(g, np.float32)
        u, up = _c(u, np.float32)
        K = g.size
        assert u.size == K and kind in (0, 1)
        t = np.empty(K, np.float32)
        xq = np.empty(K, np.int8)
        sc = np.zeros(1, np.float32)
        suma = np.empty(K // 64, np.int32)
        self.lib.qo_glu_quant_i8(gp, up, K, kind, t.ctypes.data, xq.ctypes.data, sc.ctypes.data,
                                 suma.ctypes.data if K // 64 else None)
        return t, xq, sc[0], suma

    def silu_mul_pre(self, g, u, col=None):
        """act = silu(g) * u * col in binary32 (cortiq pages, silu_mul_pre): the
        down projection's prescaled input.  g, u [n] or [rows][n]; col [n] or
        None (no column field).  Returns float32 of g's shape.
        """
        g = np.asarray(g, np.float32)
        shape = g.shape
        n = shape[-1] if g.ndim else 1
        rows = g.size // n if n else 0
        g, gp = _c(g, np.float32)
        u, up = _c(u, np.float32)
        assert u.shape == shape
        cp = None
        if col is not None:
            col, cp = _c(col, np.float32)
            assert col.shape == (n,)
        act = np.empty(shape, np.float32)
        self.lib.qo_silu_mul_pre(gp, up, cp, rows, n, act.ctypes.data)
        return act


_default = None


def default() -> Oracle:
    """The oracle built from qoracle.c in this folder (built on first use)."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB):
            build()
        _default = Oracle(_LIB)
    return _default


def f16_to_f64(bits):
    return default().f16_to_f64(bits)


def q8row_gemv(q, rs, xs, rows=None):
    return default().q8row_gemv(q, rs, xs, rows)


def q8row_gemm(q, rs, xs, entries=None):
    return default().q8row_gemm(q, rs, xs, entries)


def q2_dequant(blob, M, K, group):
    return default().q2_dequant(blob, M, K, group)


def act_quant_i8(x):
    return default().act_quant_i8(x)


def q2_dots(blob, M, K, group, xq):
    return default().q2_dots(blob, M, K, group, xq)


def q2_gemv(blob, M, K, group, xq, sc, rows=None):
    return default().q2_gemv(blob, M, K, group, xq, sc, rows)


def q2_gemv_accum(blob, M, K, group, xq, sc, accum, rows=None):
    return default().q2_gemv_accum(blob, M, K, group, xq, sc, accum, rows)


def rmsnorm_quant_i8(x, w, eps):
    return default().rmsnorm_quant_i8(x, w, eps)


def glu_quant_i8(g, u, kind):
    return default().glu_quant_i8(g, u, kind)


def silu_mul_pre(g, u, col=None):
    return default().silu_mul_pre(g, u, col)


def q2_gemm(blob, M, K, group, xq, sc, accum=None, entries=None):
    return default().q2_gemm(blob, M, K, group, xq, sc, accum, entries)
