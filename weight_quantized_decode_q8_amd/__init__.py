"""Python binding of libqgemv.so, the weight-only-quantized decode library.

Argument marshalling only: every step of the computation runs in the
library's HIP kernels (device entry points) or its C++ host repack.  Device
tensors are torch tensors used as plain device memory; the stream is torch's
current stream unless one is given.  Nothing here falls back to any other
implementation: if the library is missing, or an entry point returns an
error, a ``QGError`` is raised.

Entry points mirror ``include/qgemv.h`` one for one, with the same names.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqgemv.so")

QG_OK, QG_EINVAL, QG_ELAUNCH = 0, 1, 2


class QGError(RuntimeError):
    """A non-OK status from the library (or the library is not built)."""

    def __init__(self, fn, status, message):
        super().__init__(f"{fn}: status {status}: {message}")
        self.status = status


class qg_q2_weight(ctypes.Structure):
    _fields_ = [("codes", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("M", ctypes.c_int64), ("K", ctypes.c_int64),
                ("group", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class qg_q2_job(ctypes.Structure):
    _fields_ = [("w", qg_q2_weight), ("xq", ctypes.c_void_p), ("suma", ctypes.c_void_p),
                ("act_scale", ctypes.c_void_p), ("accum", ctypes.c_void_p), ("y", ctypes.c_void_p)]


QG_Q2_BATCH_MAX = 16

_P, _I64, _SZ, _I = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t, ctypes.c_int
_SIGS = {
    "qg_status_string": (ctypes.c_char_p, [_I]),
    "qg_last_error": (ctypes.c_char_p, []),
    "qg_abi_version": (_I, []),
    "qg_q8row_packed_bytes": (_SZ, [_I64, _I64]),
    "qg_repack_q8row": (_I, [_P, _I64, _I64, _P, _SZ]),
    "qg_unpack_q8row": (_I, [_P, _SZ, _I64, _I64, _P]),
    "qgemv_q8row": (_I, [_P, _P, _P, _P, _I64, _I64, _P]),
    "qg_q2_blocks_bytes": (_SZ, [_I64, _I64, _I]),
    "qg_q2_codes_bytes": (_SZ, [_I64, _I64]),
    "qg_q2_scales_bytes": (_SZ, [_I64, _I64, _I]),
    "qg_repack_q2": (_I, [_P, _SZ, _I64, _I64, _I, _P, _SZ, _P, _SZ]),
    "qg_unpack_q2": (_I, [_P, _SZ, _P, _SZ, _I64, _I64, _I, _P, _SZ]),
    "qquant_act_i8": (_I, [_P, _I64, _P, _P, _P, _P]),
    "qquant_act_i8_rows": (_I, [_P, _I64, _I64, _P, _P, _P, _P]),
    "qquant_rmsnorm_i8": (_I, [_P, _P, _I64, ctypes.c_float, _P, _P, _P, _P]),
    "qquant_glu_i8": (_I, [_P, _P, _I64, _I, _P, _P, _P, _P, _P]),
    "qquant_rmsnorm_i8_rows": (_I, [_P, _P, _I64, _I64, ctypes.c_float, _P, _P, _P, _P]),
    "qquant_glu_i8_rows": (_I, [_P, _P, _I64, _I64, _I, _P, _P, _P, _P, _P]),
    "qgemv_q2_ws_bytes": (_SZ, [_I64, _I64, _I, _I]),
    "qgemv_q2_auto_split": (_I, [_I64, _I64, _I]),
    "qgemv_q2": (_I, [ctypes.POINTER(qg_q2_weight), _P, _P, _P, _P, _P, _SZ, _I, _P]),
    "qgemv_q2_noalloc": (_I, [ctypes.POINTER(qg_q2_weight), _P, _P, _P, _P, _I, _P]),
    "qgemv_q2_dots": (_I, [ctypes.POINTER(qg_q2_weight), _P, _P, _P, _P, _P, _P, _SZ, _I, _P]),
    "qgemv_q2_accum": (_I, [ctypes.POINTER(qg_q2_weight), _P, _P, _P, _P, _P, _P, _SZ, _I, _P]),
    "qgemv_q2_dual_ws_bytes": (_SZ, [_I64, _I64, _I, _I]),
    "qgemv_q2_dual": (_I, [ctypes.POINTER(qg_q2_weight), ctypes.POINTER(qg_q2_weight), _P, _P, _P, _P, _P, _P,
                           _SZ, _I, _P]),
    "qgemv_q2_batch": (_I, [ctypes.POINTER(qg_q2_job), _I, _P]),
    "qgemv_q2_gate_up_glu": (_I, [ctypes.POINTER(qg_q2_weight), ctypes.POINTER(qg_q2_weight), _P, _P, _P, _I, _P, _P,
                                  _P, _P, _P]),
    "qgemv_q8row_balanced_ws_bytes": (_SZ, [_I64, _I64]),
    "qgemv_q8row_balanced": (_I, [_P, _P, _P, _P, _I64, _I64, _P, _SZ, _P]),
    "qgemv_q2_x_ws_bytes": (_SZ, [_I64, _I64, _I, _I]),
    "qgemv_q2_x_auto_split": (_I, [_I64, _I64, _I]),
    "qgemv_q2_x": (_I, [ctypes.POINTER(qg_q2_weight), _P, _P, _I64, _P, _P, _P, _SZ, _I, _P]),
    "qgemv_q2_dual_x": (_I, [ctypes.POINTER(qg_q2_weight), ctypes.POINTER(qg_q2_weight), _P, _P, ctypes.c_float,
                             _P, _P, _P]),
    "qgemv_q2_gate_up_glu_x_ws_bytes": (_SZ, [_I64]),
    "qgemv_q2_gate_up_glu_x": (_I, [ctypes.POINTER(qg_q2_weight), ctypes.POINTER(qg_q2_weight), _P, _P,
                                    ctypes.c_float, _I, _P, _P, _P, _SZ, _P]),
    "qgemm_q2_batched": (_I, [ctypes.POINTER(qg_q2_weight), _P, _P, _P, _P, _P, _I64, _P, _SZ, _P]),
    "qgemm_q2_batched_ws_bytes": (_SZ, [_I64, _I64, _I, _I64]),
    "qgemm_q2_batched_dual": (_I, [ctypes.POINTER(qg_q2_weight), ctypes.POINTER(qg_q2_weight), _P, _P, _P, _P, _P,
                                   _I64, _P, _SZ, _P]),
    "qgemm_q2_batched_dual_ws_bytes": (_SZ, [_I64, _I64, _I, _I64]),
    "qgemm_q8row_batched_ws_bytes": (_SZ, [_I64, _I64]),
    "qgemm_q8row_batched": (_I, [_P, _P, _P, _P, _I64, _I64, _I64, _I, _P, _SZ, _P]),
    "qgemm_q8row_batched_silu": (_I, [_P, _P, _P, _P, _P, _P, _I64, _I64, _I64, _I, _P, _SZ, _P]),
    "qact_silu_mul_pre": (_I, [_P, _P, _P, _P, _I64, _I64, _P]),
    # measurement probes (include/qgemv_probes.h), not the product path
    "qg_probe_stream_read": (_I, [_P, _SZ, ctypes.c_uint, _P, _I, _I, _P]),
    "qg_probe_mfma": (_I, [_I, _I, _I, _P, _P, _P]),
    "qg_probe_wall_clock_khz": (_I, [ctypes.POINTER(ctypes.c_int)]),
    "qg_probe_mfma_valu": (_I, [_I, _I, _I, _I, _I, _P, _SZ, _P]),
    "qg_probe_lds_read": (_I, [_I, _I, _I, _I, _P, _SZ, _P]),
    "qg_probe_q2_x_stamped": (_I, [ctypes.POINTER(qg_q2_weight), _P, _P, _I64, _P, _P, _P, _SZ, _I, _P, _P]),
    "qg_probe_q2_gate_up_glu_x_stamped": (_I, [ctypes.POINTER(qg_q2_weight), ctypes.POINTER(qg_q2_weight), _P, _P,
                                               ctypes.c_float, _I, _P, _P, _P, _SZ, _P, _P]),
}

_lib = None


def lib():
    """The loaded library (raises QGError when it has not been built)."""
    global _lib
    if _lib is None:
        # Load torch first so that the HIP runtime soname the library needs
        # resolves to the runtime torch already uses: one runtime per process,
        # so torch's streams and allocations are valid handles here.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        if not os.path.exists(LIB_PATH):
            raise QGError("load", -1, f"{LIB_PATH} is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(fn, status):
    if status != QG_OK:
        raise QGError(fn, status, lib().qg_last_error().decode())


def _np_ptr(a):
    return a.ctypes.data_as(ctypes.c_void_p)


def _dev(t, dtype, name):
    """Device pointer of a contiguous torch tensor of the given dtype."""
    if t is None:
        return None
    if not t.is_cuda:
        raise QGError(name, QG_EINVAL, "tensor is not on a HIP device")
    if t.dtype != dtype:
        raise QGError(name, QG_EINVAL, f"dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise QGError(name, QG_EINVAL, "tensor is not contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


# ---------------------------------------------------------------- q8_row --
def q8row_packed_bytes(M: int, K: int) -> int:
    return lib().qg_q8row_packed_bytes(M, K)


def repack_q8row(q: np.ndarray) -> np.ndarray:
    """Host: row-major int8 [M][K] -> T64 image (uint8, flat)."""
    q = np.ascontiguousarray(q, dtype=np.int8)
    M, K = q.shape
    n = lib().qg_q8row_packed_bytes(M, K)
    if n == 0:
        raise QGError("qg_repack_q8row", QG_EINVAL, f"bad shape {q.shape}")
    out = np.empty(n, np.uint8)
    _check("qg_repack_q8row", lib().qg_repack_q8row(_np_ptr(q), M, K, _np_ptr(out), n))
    return out


def unpack_q8row(packed: np.ndarray, M: int, K: int) -> np.ndarray:
    packed = np.ascontiguousarray(packed, dtype=np.uint8)
    q = np.empty((M, K), np.int8)
    _check("qg_unpack_q8row", lib().qg_unpack_q8row(_np_ptr(packed), packed.nbytes, M, K, _np_ptr(q)))
    return q


def qgemv_q8row(qpacked, rs, xs, y, M: int, K: int, stream=None):
    """y[o] = rs[o] * sum_i q[o,i] xs[i] on the device (all torch tensors)."""
    import torch
    _check("qgemv_q8row", lib().qgemv_q8row(
        _dev(qpacked, torch.uint8, "qpacked"), _dev(rs, torch.float32, "rs"),
        _dev(xs, torch.float32, "xs"), _dev(y, torch.float32, "y"), M, K, _stream(stream)))


def qgemv_q8row_balanced(qpacked, rs, xs, y, M: int, K: int, ws, stream=None):
    """qgemv_q8row with the last partial round of row tiles split along K; ws all zero (calls leave it so)."""
    import torch
    _check("qgemv_q8row_balanced", lib().qgemv_q8row_balanced(
        _dev(qpacked, torch.uint8, "qpacked"), _dev(rs, torch.float32, "rs"), _dev(xs, torch.float32, "xs"),
        _dev(y, torch.float32, "y"), M, K, _dev(ws, torch.uint8, "ws"), 0 if ws is None else ws.numel(),
        _stream(stream)))


@dataclass
class Q8RowWeight:
    """A q8_row matrix resident on the device: T64 image + row scales."""
    packed: object  # torch.uint8 device tensor
    rs: object      # torch.float32 device tensor [M]
    M: int
    K: int

    @classmethod
    def from_host(cls, q: np.ndarray, rs: np.ndarray, device="cuda"):
        import torch
        packed = torch.from_numpy(repack_q8row(q)).to(device)
        rs_t = torch.from_numpy(np.ascontiguousarray(rs, np.float32)).to(device)
        return cls(packed, rs_t, q.shape[0], q.shape[1])

    def gemv(self, xs, y, stream=None):
        qgemv_q8row(self.packed, self.rs, xs, y, self.M, self.K, stream)

    def workspace(self, device="cuda"):
        """The zero-filled workspace gemv_balanced needs (None when it needs none)."""
        import torch
        n = lib().qgemv_q8row_balanced_ws_bytes(self.M, self.K)
        return torch.zeros(n, dtype=torch.uint8, device=device) if n else None

    def gemv_balanced(self, xs, y, ws, stream=None):
        """The same GEMV with the last partial round of row tiles split along K over the GPU."""
        qgemv_q8row_balanced(self.packed, self.rs, xs, y, self.M, self.K, ws, stream)


# -------------------------------------------------------------------- Q2 --
def q2_blocks_bytes(M, K, group):
    return lib().qg_q2_blocks_bytes(M, K, group)


def repack_q2(blocks: np.ndarray, M: int, K: int, group: int):
    """Host: GGUF-style block blob -> (codes uint8 plane, scales uint16 plane)."""
    blocks = np.ascontiguousarray(blocks, dtype=np.uint8).reshape(-1)
    nc = lib().qg_q2_codes_bytes(M, K)
    ns = lib().qg_q2_scales_bytes(M, K, group)
    if nc == 0 or ns == 0:
        raise QGError("qg_repack_q2", QG_EINVAL, f"bad shape M={M} K={K} group={group}")
    codes = np.empty(nc, np.uint8)
    scales = np.empty(ns // 2, np.uint16)
    _check("qg_repack_q2", lib().qg_repack_q2(_np_ptr(blocks), blocks.nbytes, M, K, group,
                                              _np_ptr(codes), nc, _np_ptr(scales), ns))
    return codes, scales


def unpack_q2(codes: np.ndarray, scales: np.ndarray, M: int, K: int, group: int) -> np.ndarray:
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint16)
    out = np.empty(lib().qg_q2_blocks_bytes(M, K, group), np.uint8)
    _check("qg_unpack_q2", lib().qg_unpack_q2(_np_ptr(codes), codes.nbytes, _np_ptr(scales), scales.nbytes,
                                              M, K, group, _np_ptr(out), out.nbytes))
    return out


def qquant_act_i8(x, xq, act_scale, suma, stream=None):
    """Per-vector int8 quantisation of x (f32[K]) into xq, act_scale[1], suma[K/64]."""
    import torch
    _check("qquant_act_i8", lib().qquant_act_i8(
        _dev(x, torch.float32, "x"), x.numel(), _dev(xq, torch.int8, "xq"),
        _dev(act_scale, torch.float32, "act_scale"), _dev(suma, torch.int32, "suma"), _stream(stream)))


def qquant_act_i8_rows(x, xq, act_scale, suma, stream=None):
    """Row-wise int8 quantisation of x (f32 [nb][K]): xq [nb][K], act_scale [nb], suma [nb][K/64]."""
    import torch
    nb, K = x.shape
    _check("qquant_act_i8_rows", lib().qquant_act_i8_rows(
        _dev(x, torch.float32, "x"), nb, K, _dev(xq, torch.int8, "xq"),
        _dev(act_scale, torch.float32, "act_scale"), _dev(suma, torch.int32, "suma"), _stream(stream)))


QG_GLU_SILU, QG_GLU_SIGMOID = 0, 1


def qquant_rmsnorm_i8(x, w, eps, xq, act_scale, suma, stream=None):
    """RMSNorm of x with weights w, then the int8 quantiser (one launch)."""
    import torch
    _check("qquant_rmsnorm_i8", lib().qquant_rmsnorm_i8(
        _dev(x, torch.float32, "x"), _dev(w, torch.float32, "w"), x.numel(), float(eps),
        _dev(xq, torch.int8, "xq"), _dev(act_scale, torch.float32, "act_scale"),
        _dev(suma, torch.int32, "suma"), _stream(stream)))


def qquant_glu_i8(g, u, kind, t, xq, act_scale, suma, stream=None):
    """t = silu(g) * u (kind 0) or u * sigmoid(g) (kind 1), then the int8 quantiser; t may be g or u."""
    import torch
    _check("qquant_glu_i8", lib().qquant_glu_i8(
        _dev(g, torch.float32, "g"), _dev(u, torch.float32, "u"), g.numel(), int(kind),
        _dev(t, torch.float32, "t"), _dev(xq, torch.int8, "xq"),
        _dev(act_scale, torch.float32, "act_scale"), _dev(suma, torch.int32, "suma"), _stream(stream)))


def qquant_rmsnorm_i8_rows(x, w, eps, xq, act_scale, suma, stream=None):
    """RMSNorm (shared weights w [K]) then the int8 quantiser on each row of x [nb][K]."""
    import torch
    nb, K = x.shape
    _check("qquant_rmsnorm_i8_rows", lib().qquant_rmsnorm_i8_rows(
        _dev(x, torch.float32, "x"), _dev(w, torch.float32, "w"), nb, K, float(eps),
        _dev(xq, torch.int8, "xq"), _dev(act_scale, torch.float32, "act_scale"),
        _dev(suma, torch.int32, "suma"), _stream(stream)))


def qquant_glu_i8_rows(g, u, kind, t, xq, act_scale, suma, stream=None):
    """The gated product and the int8 quantiser on each row of g, u [nb][K]."""
    import torch
    nb, K = g.shape
    _check("qquant_glu_i8_rows", lib().qquant_glu_i8_rows(
        _dev(g, torch.float32, "g"), _dev(u, torch.float32, "u"), nb, K, int(kind),
        _dev(t, torch.float32, "t"), _dev(xq, torch.int8, "xq"),
        _dev(act_scale, torch.float32, "act_scale"), _dev(suma, torch.int32, "suma"), _stream(stream)))


def qact_silu_mul_pre(g, u, col, act, stream=None):
    """act = silu(g) * u * col (col None: no column field); g, u, act [n] or
    [rows][n], col [n]; act may be g or u."""
    import torch
    n = g.shape[-1]
    rows = g.numel() // n
    _check("qact_silu_mul_pre", lib().qact_silu_mul_pre(
        _dev(g, torch.float32, "g"), _dev(u, torch.float32, "u"), _dev(col, torch.float32, "col"),
        _dev(act, torch.float32, "act"), rows, n, _stream(stream)))


def qgemv_q2_ws_bytes(M, K, group, split_k=0) -> int:
    return lib().qgemv_q2_ws_bytes(M, K, group, split_k)


def qgemv_q2_auto_split(M, K, group) -> int:
    return lib().qgemv_q2_auto_split(M, K, group)


@dataclass
class Q2Weight:
    """A Q2 matrix resident on the device: the two T64 planes."""
    codes: object   # torch.uint8 device tensor
    scales: object  # torch.int16 device tensor (binary16 bit patterns)
    M: int
    K: int
    group: int

    @classmethod
    def from_blocks(cls, blocks: np.ndarray, M: int, K: int, group: int, device="cuda"):
        import torch
        c, s = repack_q2(blocks, M, K, group)
        return cls(torch.from_numpy(c).to(device), torch.from_numpy(s.view(np.int16)).to(device), M, K, group)

    def desc(self) -> qg_q2_weight:
        import torch
        return qg_q2_weight(_dev(self.codes, torch.uint8, "codes").value,
                            _dev(self.scales, torch.int16, "scales").value,
                            self.M, self.K, self.group, 0)


def qgemv_q2(w: Q2Weight, xq, suma, act_scale, y, ws=None, split_k=0, stream=None):
    """y = act_scale * sum_u d * dot_u on the device; ws is a uint8 tensor or None."""
    import torch
    d = w.desc()
    wsp = _dev(ws, torch.uint8, "ws")
    _check("qgemv_q2", lib().qgemv_q2(
        ctypes.byref(d), _dev(xq, torch.int8, "xq"), _dev(suma, torch.int32, "suma"),
        _dev(act_scale, torch.float32, "act_scale"), _dev(y, torch.float32, "y"),
        wsp, 0 if ws is None else ws.numel(), split_k, _stream(stream)))


def qgemv_q2_noalloc(w: Q2Weight, xq, suma, act_scale, y, split_k=0, stream=None):
    """qgemv_q2 with its split-K partials in the library's static device
    scratch: no workspace, no allocation.  Calls overlapping on one GPU race."""
    import torch
    d = w.desc()
    _check("qgemv_q2_noalloc", lib().qgemv_q2_noalloc(
        ctypes.byref(d), _dev(xq, torch.int8, "xq"), _dev(suma, torch.int32, "suma"),
        _dev(act_scale, torch.float32, "act_scale"), _dev(y, torch.float32, "y"), split_k, _stream(stream)))


def qgemv_q2_dots(w: Q2Weight, xq, suma, act_scale, y, dots, ws=None, split_k=0, stream=None):
    """qgemv_q2 that also writes the exact int32 unit dots [M][K/64]."""
    import torch
    d = w.desc()
    wsp = _dev(ws, torch.uint8, "ws")
    _check("qgemv_q2_dots", lib().qgemv_q2_dots(
        ctypes.byref(d), _dev(xq, torch.int8, "xq"), _dev(suma, torch.int32, "suma"),
        _dev(act_scale, torch.float32, "act_scale"), _dev(y, torch.float32, "y"),
        _dev(dots, torch.int32, "dots"), wsp, 0 if ws is None else ws.numel(), split_k, _stream(stream)))


def qgemv_q2_accum(w: Q2Weight, xq, suma, act_scale, accum, y, ws=None, split_k=0, stream=None):
    """y = (act_scale * sum_u d * dot_u) + accum, two f32 roundings; accum may be y itself."""
    import torch
    d = w.desc()
    wsp = _dev(ws, torch.uint8, "ws")
    _check("qgemv_q2_accum", lib().qgemv_q2_accum(
        ctypes.byref(d), _dev(xq, torch.int8, "xq"), _dev(suma, torch.int32, "suma"),
        _dev(act_scale, torch.float32, "act_scale"), _dev(accum, torch.float32, "accum"),
        _dev(y, torch.float32, "y"), wsp, 0 if ws is None else ws.numel(), split_k, _stream(stream)))


def qgemv_q2_dual_ws_bytes(M, K, group, split_k=0) -> int:
    return lib().qgemv_q2_dual_ws_bytes(M, K, group, split_k)


def qgemv_q2_dual(w0: Q2Weight, w1: Q2Weight, xq, suma, act_scale, y0, y1, ws=None, split_k=0, stream=None):
    """Two Q2 GEMVs of one shape (gate, up) against one quantized activation, one launch."""
    import torch
    d0, d1 = w0.desc(), w1.desc()
    wsp = _dev(ws, torch.uint8, "ws")
    _check("qgemv_q2_dual", lib().qgemv_q2_dual(
        ctypes.byref(d0), ctypes.byref(d1), _dev(xq, torch.int8, "xq"), _dev(suma, torch.int32, "suma"),
        _dev(act_scale, torch.float32, "act_scale"), _dev(y0, torch.float32, "y0"), _dev(y1, torch.float32, "y1"),
        wsp, 0 if ws is None else ws.numel(), split_k, _stream(stream)))


def qgemv_q2_gate_up_glu(w_gate: Q2Weight, w_up: Q2Weight, xq, suma, act_scale, kind, t, xq_out, act_scale_out,
                         suma_out, stream=None):
    """Gate|up GEMV with t = silu(g)*u (kind 0) or u*sigmoid(g) (kind 1) formed in its epilogue,
    then the int8 quantiser of t: two launches, bit-identical to qgemv_q2_dual + qquant_glu_i8."""
    import torch
    dg, du = w_gate.desc(), w_up.desc()
    _check("qgemv_q2_gate_up_glu", lib().qgemv_q2_gate_up_glu(
        ctypes.byref(dg), ctypes.byref(du), _dev(xq, torch.int8, "xq"), _dev(suma, torch.int32, "suma"),
        _dev(act_scale, torch.float32, "act_scale"), int(kind), _dev(t, torch.float32, "t"),
        _dev(xq_out, torch.int8, "xq_out"), _dev(act_scale_out, torch.float32, "act_scale_out"),
        _dev(suma_out, torch.int32, "suma_out"), _stream(stream)))


def qgemv_q2_batch(jobs, stream=None):
    """Independent Q2 GEMVs in one launch.  jobs: sequence of
    (Q2Weight, xq, suma, act_scale, y) or (Q2Weight, xq, suma, act_scale, y, accum)."""
    import torch
    arr = (qg_q2_job * max(1, len(jobs)))()
    for n, job in enumerate(jobs):
        w, xq, suma, sc, y = job[:5]
        accum = job[5] if len(job) > 5 else None
        arr[n] = qg_q2_job(w.desc(), _dev(xq, torch.int8, "xq"), _dev(suma, torch.int32, "suma"),
                           _dev(sc, torch.float32, "act_scale"), _dev(accum, torch.float32, "accum"),
                           _dev(y, torch.float32, "y"))
    _check("qgemv_q2_batch", lib().qgemv_q2_batch(arr, len(jobs), _stream(stream)))


def qgemv_q2_x_ws_bytes(M, K, group, split_k=0) -> int:
    return lib().qgemv_q2_x_ws_bytes(M, K, group, split_k)


def qgemv_q2_x_auto_split(M, K, group) -> int:
    return lib().qgemv_q2_x_auto_split(M, K, group)


def qgemv_q2_x_workspace(M, K, group, split_k=0, device="cuda"):
    """A zero-filled workspace for qgemv_q2_x (it must start all zero; calls leave it so), or None."""
    import torch
    n = qgemv_q2_x_ws_bytes(M, K, group, split_k)
    return torch.zeros(n, dtype=torch.uint8, device=device) if n else None


def qgemv_q2_x(w: Q2Weight, x, y, accum=None, ws=None, split_k=0, stream=None, xmax=None):
    """y = Q2 GEMV of the f32 vector x, quantised inside the launch (+ accum); one launch.
    ws: from qgemv_q2_x_workspace (all zero) when the split is above 1.
    xmax: None, or a float32 device tensor of partial maxima of |x| (the tmax
    of qgemv_q2_gate_up_glu_x), so each workgroup reads only its split of x."""
    import torch
    d = w.desc()
    _check("qgemv_q2_x", lib().qgemv_q2_x(
        ctypes.byref(d), _dev(x, torch.float32, "x"), _dev(xmax, torch.float32, "xmax"),
        0 if xmax is None else xmax.numel(), _dev(accum, torch.float32, "accum"),
        _dev(y, torch.float32, "y"), _dev(ws, torch.uint8, "ws"), 0 if ws is None else ws.numel(), split_k,
        _stream(stream)))


def qgemv_q2_dual_x(w0: Q2Weight, w1: Q2Weight, x, y0, y1, norm_w=None, eps=0.0, stream=None):
    """The gate|up pair against x quantised (after RMSNorm with norm_w, eps) inside the launch."""
    import torch
    d0, d1 = w0.desc(), w1.desc()
    _check("qgemv_q2_dual_x", lib().qgemv_q2_dual_x(
        ctypes.byref(d0), ctypes.byref(d1), _dev(x, torch.float32, "x"), _dev(norm_w, torch.float32, "norm_w"),
        float(eps), _dev(y0, torch.float32, "y0"), _dev(y1, torch.float32, "y1"), _stream(stream)))


def qgemv_q2_gate_up_glu_x_workspace(M, device="cuda"):
    """The zero-filled workspace qgemv_q2_gate_up_glu_x needs (calls leave it all zero)."""
    import torch
    return torch.zeros(lib().qgemv_q2_gate_up_glu_x_ws_bytes(M), dtype=torch.uint8, device=device)


def qgemv_q2_gate_up_glu_x(w_gate: Q2Weight, w_up: Q2Weight, x, kind, t, ws, norm_w=None, eps=0.0, stream=None,
                           tmax=None):
    """t = silu(g)*u (kind 0) or u*sigmoid(g) (kind 1) of the gate|up pair, x quantised in the launch.
    ws: from qgemv_q2_gate_up_glu_x_workspace.  tmax: None, or a float32 device
    tensor of ceil(M/64) entries that receives max|t| of each row tile."""
    import torch
    dg, du = w_gate.desc(), w_up.desc()
    _check("qgemv_q2_gate_up_glu_x", lib().qgemv_q2_gate_up_glu_x(
        ctypes.byref(dg), ctypes.byref(du), _dev(x, torch.float32, "x"), _dev(norm_w, torch.float32, "norm_w"),
        float(eps), int(kind), _dev(t, torch.float32, "t"), _dev(tmax, torch.float32, "tmax"),
        _dev(ws, torch.uint8, "ws"),
        0 if ws is None else ws.numel(), _stream(stream)))


def qgemm_q2_batched_ws_bytes(M, K, group, nb) -> int:
    return lib().qgemm_q2_batched_ws_bytes(M, K, group, nb)


def qgemm_q2_batched(w: Q2Weight, xq, suma, act_scale, y, accum=None, ws=None, stream=None):
    """Batched Q2: y[b,o] = act_scale[b] * sum_g d * dot(b,o,g) (+ accum), y [nb][M]; ws a uint8 tensor or None."""
    import torch
    d = w.desc()
    nb = act_scale.numel()
    _check("qgemm_q2_batched", lib().qgemm_q2_batched(
        ctypes.byref(d), _dev(xq, torch.int8, "xq"), _dev(suma, torch.int32, "suma"),
        _dev(act_scale, torch.float32, "act_scale"), _dev(accum, torch.float32, "accum"),
        _dev(y, torch.float32, "y"), nb, _dev(ws, torch.uint8, "ws"), 0 if ws is None else ws.numel(),
        _stream(stream)))


def qgemm_q2_batched_dual_ws_bytes(M, K, group, nb) -> int:
    return lib().qgemm_q2_batched_dual_ws_bytes(M, K, group, nb)


def qgemm_q2_batched_dual(w0: Q2Weight, w1: Q2Weight, xq, suma, act_scale, y0, y1, ws=None, stream=None):
    """Gate|up pair of the batched Q2 product in one launch: y0, y1 [nb][M] from w0, w1
    (same shape) against the same token rows; bit-identical to two qgemm_q2_batched calls."""
    import torch
    d0, d1 = w0.desc(), w1.desc()
    nb = act_scale.numel()
    _check("qgemm_q2_batched_dual", lib().qgemm_q2_batched_dual(
        ctypes.byref(d0), ctypes.byref(d1), _dev(xq, torch.int8, "xq"), _dev(suma, torch.int32, "suma"),
        _dev(act_scale, torch.float32, "act_scale"), _dev(y0, torch.float32, "y0"), _dev(y1, torch.float32, "y1"),
        nb, _dev(ws, torch.uint8, "ws"), 0 if ws is None else ws.numel(), _stream(stream)))


# ------------------------------------------------------ batched q8_row GEMM --
def qgemm_q8row_batched_ws_bytes(nb: int, K: int) -> int:
    return lib().qgemm_q8row_batched_ws_bytes(nb, K)


def qgemm_q8row_batched(qpacked, rs, xs, y, nb: int, M: int, K: int, ws, xs_limbs: int = 0, stream=None):
    """y[b,o] = rs[o] * sum_i q[o,i] xs[b,i] (xs [nb][K], y [nb][M]); ws a uint8 tensor."""
    import torch
    _check("qgemm_q8row_batched", lib().qgemm_q8row_batched(
        _dev(qpacked, torch.uint8, "qpacked"), _dev(rs, torch.float32, "rs"),
        _dev(xs, torch.float32, "xs"), _dev(y, torch.float32, "y"), nb, M, K, xs_limbs,
        _dev(ws, torch.uint8, "ws"), 0 if ws is None else ws.numel(), _stream(stream)))


def qgemm_q8row_batched_silu(qpacked, rs, g, u, col, y, nb: int, M: int, K: int, ws, xs_limbs: int = 0,
                             stream=None):
    """y[b,o] = rs[o] * sum_i q[o,i] act[b,i] with act = silu(g) * u * col formed in the
    product's prep (g, u [nb][K]; col [K] or None); ws as for qgemm_q8row_batched."""
    import torch
    _check("qgemm_q8row_batched_silu", lib().qgemm_q8row_batched_silu(
        _dev(qpacked, torch.uint8, "qpacked"), _dev(rs, torch.float32, "rs"),
        _dev(g, torch.float32, "g"), _dev(u, torch.float32, "u"), _dev(col, torch.float32, "col"),
        _dev(y, torch.float32, "y"), nb, M, K, xs_limbs,
        _dev(ws, torch.uint8, "ws"), 0 if ws is None else ws.numel(), _stream(stream)))


# ---- measurement probes (include/qgemv_probes.h): not the product path ----
def qg_probe_stream_read(buf, sentinel, sink, workgroups, loads=8, stream=None):
    """Read the uint8 device tensor buf once (16-byte non-temporal loads, `loads` in flight per lane);
    sink: int32[workgroups]."""
    import torch
    _check("qg_probe_stream_read", lib().qg_probe_stream_read(
        _dev(buf, torch.uint8, "buf"), buf.numel(), sentinel & 0xFFFFFFFF, _dev(sink, torch.int32, "sink"),
        int(workgroups), int(loads), _stream(stream)))


def qg_probe_mfma(kind, iters, workgroups, sink, clocks, stream=None):
    """Matrix-core loop: kind 0 int8 16x16x64, 1 fp16 16x16x32; sink f32[workgroups*256], clocks int64[2]."""
    import torch
    _check("qg_probe_mfma", lib().qg_probe_mfma(
        int(kind), int(iters), int(workgroups), _dev(sink, torch.float32, "sink"),
        _dev(clocks, torch.int64, "clocks"), _stream(stream)))


def qg_probe_mfma_valu(mfma, fmas, iters, workgroups, waves_per_simd, sink, stream=None):
    """Matrix-core and vector-ALU work together or apart (qgemv_probes.h);
    sink: float32[workgroups * 256 * waves_per_simd]."""
    import torch
    _check("qg_probe_mfma_valu", lib().qg_probe_mfma_valu(
        int(mfma), int(fmas), int(iters), int(workgroups), int(waves_per_simd),
        _dev(sink, torch.float32, "sink"), sink.numel(), _stream(stream)))


def qg_probe_lds_read(bytes_per_lane, iters, workgroups, waves, sink, stream=None):
    """LDS read rate probe (qgemv_probes.h); sink: int32[workgroups * 64 * waves]."""
    import torch
    _check("qg_probe_lds_read", lib().qg_probe_lds_read(
        int(bytes_per_lane), int(iters), int(workgroups), int(waves),
        _dev(sink, torch.int32, "sink"), sink.numel(), _stream(stream)))


def qg_probe_wall_clock_khz():
    khz = ctypes.c_int(0)
    _check("qg_probe_wall_clock_khz", lib().qg_probe_wall_clock_khz(ctypes.byref(khz)))
    return khz.value


def qg_probe_q2_x_stamped(w: Q2Weight, x, y, stamps, accum=None, ws=None, split_k=0, xmax=None, stream=None):
    """qgemv_q2_x with four wall-clock stamps per workgroup into the int64 device tensor stamps."""
    import torch
    d = w.desc()
    _check("qg_probe_q2_x_stamped", lib().qg_probe_q2_x_stamped(
        ctypes.byref(d), _dev(x, torch.float32, "x"), _dev(xmax, torch.float32, "xmax"),
        0 if xmax is None else xmax.numel(), _dev(accum, torch.float32, "accum"), _dev(y, torch.float32, "y"),
        _dev(ws, torch.uint8, "ws"), 0 if ws is None else ws.numel(), split_k, _dev(stamps, torch.int64, "stamps"),
        _stream(stream)))


def qg_probe_q2_gate_up_glu_x_stamped(w_gate: Q2Weight, w_up: Q2Weight, x, kind, t, ws, stamps, norm_w=None,
                                      eps=0.0, tmax=None, stream=None):
    """qgemv_q2_gate_up_glu_x with four wall-clock stamps per workgroup."""
    import torch
    dg, du = w_gate.desc(), w_up.desc()
    _check("qg_probe_q2_gate_up_glu_x_stamped", lib().qg_probe_q2_gate_up_glu_x_stamped(
        ctypes.byref(dg), ctypes.byref(du), _dev(x, torch.float32, "x"), _dev(norm_w, torch.float32, "norm_w"),
        float(eps), int(kind), _dev(t, torch.float32, "t"), _dev(tmax, torch.float32, "tmax"),
        _dev(ws, torch.uint8, "ws"), ws.numel(), _dev(stamps, torch.int64, "stamps"), _stream(stream)))
