"""Host-side checks of the C-ABI library: it loads, exports every declared
symbol, its repacks place every byte where the header says, and invalid
arguments are rejected before anything is launched.  No GPU needed: the
device entry points are only called with arguments that fail validation."""
import ctypes
import glob
import os
import re

import numpy as np
import pytest

import weight_quantized_decode_q8_amd as qg
from oracle_pins import encode_q2

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def declared_functions():
    names = []
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        src = open(h).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w\s\*]*?\b([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M):
            if m.group(1) not in ("if", "sizeof"):
                names.append(m.group(1))
    return sorted(set(names))


def test_header_declares_entry_points():
    names = declared_functions()
    for n in ("qgemv_q8row", "qgemv_q2", "qquant_act_i8", "qg_repack_q2", "qg_repack_q8row"):
        assert n in names


@pytest.mark.parametrize("name", declared_functions())
def test_library_exports(name):
    assert hasattr(ctypes.CDLL(qg.LIB_PATH), name), name


def test_abi_and_status_strings():
    L = qg.lib()
    assert L.qg_abi_version() == 7
    assert L.qg_status_string(0) == b"QG_OK"
    assert L.qg_status_string(1) == b"QG_EINVAL"
    assert L.qg_status_string(2) == b"QG_ELAUNCH"


def test_sizes():
    L = qg.lib()
    assert L.qg_q8row_packed_bytes(256, 512) == 256 * 512
    assert L.qg_q8row_packed_bytes(65, 20) == 128 * 32
    assert L.qg_q8row_packed_bytes(10, 6) == 0
    assert L.qg_q2_blocks_bytes(4096, 4096, 64) == 4096 * 64 * 18
    assert L.qg_q2_blocks_bytes(17408, 5120, 128) == 17408 * 40 * 34
    assert L.qg_q2_codes_bytes(100, 256) == 128 * 64
    assert L.qg_q2_scales_bytes(100, 256, 128) == 128 * 2 * 2
    assert L.qg_q2_scales_bytes(100, 200, 128) == 0
    for M, K, g in [(4096, 4096, 64), (17408, 5120, 128), (5120, 17408, 128), (1, 64, 64)]:
        S = L.qgemv_q2_auto_split(M, K, g)
        assert 1 <= S <= 16
        ws = L.qgemv_q2_ws_bytes(M, K, g, 0)
        assert ws == (0 if S == 1 else S * ((M + 63) // 64 * 64) * 4)
    assert L.qgemv_q2_ws_bytes(100, 256, 64, 1) == 0
    assert L.qgemv_q2_ws_bytes(100, 256, 64, 4) == 4 * 128 * 4


@pytest.mark.parametrize("M,K", [(1, 4), (63, 16), (64, 20), (70, 36), (130, 1028)])
def test_q8_repack_layout(M, K):
    rng = np.random.Generator(np.random.PCG64(M * 1000 + K))
    q = rng.integers(-128, 128, size=(M, K), dtype=np.int8)
    p = qg.repack_q8row(q)
    Mp, Kp = -(-M // 64) * 64, -(-K // 16) * 16
    assert p.size == Mp * Kp
    o, i = np.meshgrid(np.arange(M), np.arange(K), indexing="ij")
    where = ((o // 64) * (Kp // 16) + i // 16) * 1024 + (o % 64) * 16 + i % 16
    assert np.array_equal(p[where].view(np.int8), q)
    mask = np.ones(p.size, bool)
    mask[where.reshape(-1)] = False
    assert np.all(p[mask] == 0)  # padding is zero
    assert np.array_equal(qg.unpack_q8row(p, M, K), q)


def decode_t64_codes(codes, M, K):
    """Codes [M][K] read back from the T64 code plane per the header's layout."""
    tiles = -(-M // 64)
    nu = K // 64
    u8 = codes.reshape(tiles, nu, 64, 4, 4)            # [tile][unit][row][word j][byte]
    words = u8.astype(np.uint32)
    w = words[..., 0] | (words[..., 1] << 8) | (words[..., 2] << 16) | (words[..., 3] << 24)
    out = np.empty((tiles, 64, nu, 4, 4, 4), np.uint8)  # [tile][row][unit][j][a][b]
    for a in range(4):
        for b in range(4):
            out[:, :, :, :, a, b] = ((w >> (8 * b + 2 * a)) & 3).transpose(0, 2, 1, 3)
    return out.reshape(tiles * 64, K)[:M]


@pytest.mark.parametrize("M,K,group", [(1, 64, 64), (65, 192, 64), (100, 256, 128), (64, 1024, 128)])
def test_q2_repack_layout(M, K, group):
    rng = np.random.Generator(np.random.PCG64(M + K + group))
    codes = rng.integers(0, 4, size=(M, K), dtype=np.uint8)
    d_bits = rng.integers(0, 1 << 15, size=(M, K // group), dtype=np.uint16)
    blob = encode_q2(codes, d_bits, group)
    cplane, splane = qg.repack_q2(blob, M, K, group)
    tiles = -(-M // 64)
    assert cplane.size == tiles * 64 * K // 4
    assert np.array_equal(decode_t64_codes(cplane, M, K), codes)
    s = splane.reshape(tiles, K // group, 64).transpose(0, 2, 1).reshape(tiles * 64, K // group)
    assert np.array_equal(s[:M], d_bits)
    assert np.all(s[M:] == 0)
    assert np.all(decode_t64_codes(cplane, tiles * 64, K)[M:] == 0)
    assert np.array_equal(qg.unpack_q2(cplane, splane, M, K, group), blob)


def _einval(status):
    assert status == qg.QG_EINVAL
    assert qg.lib().qg_last_error()


def test_einval_paths():
    L = qg.lib()
    P = ctypes.c_void_p
    a16 = P(0x10000)  # never dereferenced: every call below fails validation
    # q8_row GEMV
    _einval(L.qgemv_q8row(None, a16, a16, a16, 64, 64, None))
    _einval(L.qgemv_q8row(a16, a16, a16, a16, 0, 64, None))
    _einval(L.qgemv_q8row(a16, a16, a16, a16, 64, 62, None))
    _einval(L.qgemv_q8row(P(0x10004), a16, a16, a16, 64, 64, None))
    _einval(L.qgemv_q8row(a16, a16, P(0x10004), a16, 64, 64, None))
    # activation quantiser
    _einval(L.qquant_act_i8(a16, 100, a16, a16, a16, None))
    _einval(L.qquant_act_i8(a16, 0, a16, a16, a16, None))
    _einval(L.qquant_act_i8(None, 64, a16, a16, a16, None))
    _einval(L.qquant_act_i8(P(0x10008), 64, a16, a16, a16, None))
    # fused producers
    F = ctypes.c_float
    _einval(L.qquant_rmsnorm_i8(None, a16, 64, F(1e-6), a16, a16, a16, None))
    _einval(L.qquant_rmsnorm_i8(a16, a16, 100, F(1e-6), a16, a16, a16, None))
    _einval(L.qquant_rmsnorm_i8(a16, P(0x10008), 64, F(1e-6), a16, a16, a16, None))
    _einval(L.qquant_rmsnorm_i8(a16, a16, 64, F(-1.0), a16, a16, a16, None))
    _einval(L.qquant_rmsnorm_i8(a16, a16, 64, F(float("nan")), a16, a16, a16, None))
    _einval(L.qquant_rmsnorm_i8(a16, a16, 64, F(float("inf")), a16, a16, a16, None))
    _einval(L.qquant_rmsnorm_i8(a16, a16, 64, F(1e-6), None, a16, a16, None))
    _einval(L.qquant_glu_i8(a16, a16, 64, 2, a16, a16, a16, a16, None))
    _einval(L.qquant_glu_i8(a16, a16, 64, -1, a16, a16, a16, a16, None))
    _einval(L.qquant_glu_i8(a16, None, 64, 0, a16, a16, a16, a16, None))
    _einval(L.qquant_glu_i8(a16, a16, 64, 0, None, a16, a16, a16, None))     # t is required
    _einval(L.qquant_glu_i8(a16, a16, 32, 0, a16, a16, a16, a16, None))
    _einval(L.qquant_glu_i8(P(0x10004), a16, 64, 1, a16, a16, a16, a16, None))
    _einval(L.qquant_glu_i8(a16, a16, 64, 1, P(0x10008), a16, a16, a16, None))  # t misaligned
    _einval(L.qquant_glu_i8(P(0x20000), P(0x30000), 64, 0, P(0x20010), a16, a16, a16, None))  # t inside g
    _einval(L.qquant_glu_i8(P(0x20000), P(0x30000), 64, 0, P(0x2FFF0), a16, a16, a16, None))  # t over u
    _einval(L.qquant_rmsnorm_i8_rows(a16, a16, 0, 64, F(1e-6), a16, a16, a16, None))
    _einval(L.qquant_rmsnorm_i8_rows(a16, a16, 4, 96, F(1e-6), a16, a16, a16, None))
    _einval(L.qquant_rmsnorm_i8_rows(a16, a16, 4, 64, F(-2.0), a16, a16, a16, None))
    _einval(L.qquant_glu_i8_rows(a16, a16, 0, 64, 0, a16, a16, a16, a16, None))
    _einval(L.qquant_glu_i8_rows(a16, a16, 4, 64, 5, a16, a16, a16, a16, None))
    _einval(L.qquant_glu_i8_rows(P(0x20000), P(0x30000), 4, 64, 0, P(0x20100), a16, a16, a16, None))  # t in g
    # Q2 GEMV
    w = qg.qg_q2_weight(0x10000, 0x20000, 128, 256, 64, 0)
    bad = [qg.qg_q2_weight(0x10000, 0x20000, 128, 256, 96, 0),
           qg.qg_q2_weight(0x10000, 0x20000, 128, 200, 64, 0),
           qg.qg_q2_weight(0x10000, 0x20000, 0, 256, 64, 0),
           qg.qg_q2_weight(0, 0x20000, 128, 256, 64, 0),
           qg.qg_q2_weight(0x10008, 0x20000, 128, 256, 64, 0),
           qg.qg_q2_weight(0x10000, 0x20000, 128, 256, 64, 7)]
    for b in bad:
        _einval(L.qgemv_q2(ctypes.byref(b), a16, a16, a16, a16, None, 0, 1, None))
    _einval(L.qgemv_q2(None, a16, a16, a16, a16, None, 0, 1, None))
    _einval(L.qgemv_q2(ctypes.byref(w), a16, a16, a16, a16, None, 0, 17, None))
    _einval(L.qgemv_q2(ctypes.byref(w), a16, a16, a16, a16, None, 0, -1, None))
    _einval(L.qgemv_q2(ctypes.byref(w), a16, a16, a16, a16, None, 0, 4, None))        # no workspace
    _einval(L.qgemv_q2(ctypes.byref(w), a16, a16, a16, a16, a16, 100, 4, None))       # too small
    _einval(L.qgemv_q2(ctypes.byref(w), P(0x10004), a16, a16, a16, None, 0, 1, None))  # xq misaligned
    _einval(L.qgemv_q2_dots(ctypes.byref(w), a16, a16, a16, a16, None, None, 0, 1, None))
    # the entry point without a workspace: the same checks, and splits whose
    # partials exceed the static scratch (16 * 16448 floats > 1 MiB)
    for b in bad:
        _einval(L.qgemv_q2_noalloc(ctypes.byref(b), a16, a16, a16, a16, 1, None))
    _einval(L.qgemv_q2_noalloc(None, a16, a16, a16, a16, 1, None))
    _einval(L.qgemv_q2_noalloc(ctypes.byref(w), a16, a16, a16, a16, 17, None))
    _einval(L.qgemv_q2_noalloc(ctypes.byref(w), a16, a16, a16, a16, -1, None))
    wbig = qg.qg_q2_weight(0x10000, 0x20000, 16400, 4096, 64, 0)
    assert L.qgemv_q2_ws_bytes(16400, 4096, 64, 16) == 16 * 16448 * 4 > (1 << 20)
    _einval(L.qgemv_q2_noalloc(ctypes.byref(wbig), a16, a16, a16, a16, 16, None))
    assert b"static scratch" in L.qg_last_error()
    # residual epilogue: null accum, accum partly overlapping y
    _einval(L.qgemv_q2_accum(ctypes.byref(w), a16, a16, a16, None, a16, None, 0, 1, None))
    _einval(L.qgemv_q2_accum(ctypes.byref(w), a16, a16, a16, P(0x10010), a16, None, 0, 1, None))
    for b in bad:
        _einval(L.qgemv_q2_accum(ctypes.byref(b), a16, a16, a16, P(0x40000), a16, None, 0, 1, None))
    # two matrices in one launch: shape mismatch, overlapping or null outputs,
    # no second weight, short workspace (twice the one-matrix size)
    w1 = qg.qg_q2_weight(0x30000, 0x40000, 128, 256, 64, 0)
    for other in (qg.qg_q2_weight(0x30000, 0x40000, 64, 256, 64, 0),
                  qg.qg_q2_weight(0x30000, 0x40000, 128, 512, 64, 0),
                  qg.qg_q2_weight(0x30000, 0x40000, 128, 256, 128, 0)):
        _einval(L.qgemv_q2_dual(ctypes.byref(w), ctypes.byref(other), a16, a16, a16, a16, P(0x50000),
                                None, 0, 1, None))
    for b in bad:
        _einval(L.qgemv_q2_dual(ctypes.byref(w), ctypes.byref(b), a16, a16, a16, a16, P(0x50000),
                                None, 0, 1, None))
    _einval(L.qgemv_q2_dual(ctypes.byref(w), None, a16, a16, a16, a16, P(0x50000), None, 0, 1, None))
    _einval(L.qgemv_q2_dual(ctypes.byref(w), ctypes.byref(w1), a16, a16, a16, a16, P(0x10100),
                            None, 0, 1, None))
    _einval(L.qgemv_q2_dual(ctypes.byref(w), ctypes.byref(w1), a16, a16, a16, a16, None, None, 0, 1, None))
    one = L.qgemv_q2_ws_bytes(128, 256, 64, 4)
    assert L.qgemv_q2_dual_ws_bytes(128, 256, 64, 4) == 2 * one > 0
    _einval(L.qgemv_q2_dual(ctypes.byref(w), ctypes.byref(w1), a16, a16, a16, a16, P(0x50000),
                            a16, one, 4, None))
    # batched launch: table, count, group mix, pointers, overlaps
    def job(w_, y=0x50000, accum=None, xq=0x10000):
        return qg.qg_q2_job(w_, xq, 0x10000, 0x10000, accum, y)

    def batch(*jobs):
        arr = (qg.qg_q2_job * len(jobs))(*jobs)
        return L.qgemv_q2_batch(arr, len(jobs), None)

    w128 = qg.qg_q2_weight(0x30000, 0x40000, 128, 256, 128, 0)
    _einval(L.qgemv_q2_batch(None, 1, None))
    _einval(L.qgemv_q2_batch((qg.qg_q2_job * 1)(job(w)), 0, None))
    _einval(L.qgemv_q2_batch((qg.qg_q2_job * 17)(*[job(w, y=0x50000 + 0x1000 * i) for i in range(17)]), 17, None))
    _einval(batch(job(w), job(w128, y=0x60000)))                      # mixed group sizes
    for b in bad:
        _einval(batch(job(w), job(b, y=0x60000)))
    _einval(batch(job(w, xq=0x10004)))                                # xq misaligned
    _einval(batch(job(w, y=0)))                                       # null y
    _einval(batch(job(w, y=0x50000, accum=0x50010)))                  # accum partly over y
    _einval(batch(job(w, y=0x50000), job(w1, y=0x50100)))             # outputs overlap
    _einval(batch(job(w, y=0x50000), job(w1, y=0x60000, accum=0x50000)))  # output over a residual
    # row-batched quantiser and the batched Q2 product
    _einval(L.qquant_act_i8_rows(a16, 0, 64, a16, a16, a16, None))
    _einval(L.qquant_act_i8_rows(a16, 4, 100, a16, a16, a16, None))
    _einval(L.qquant_act_i8_rows(None, 4, 64, a16, a16, a16, None))
    _einval(L.qquant_act_i8_rows(P(0x10004), 4, 64, a16, a16, a16, None))
    w8 = qg.qg_q2_weight(0x10000, 0x20000, 128, 256, 64, 0)
    _einval(L.qgemm_q2_batched(ctypes.byref(w8), a16, a16, a16, None, a16, 0, None, 0, None))          # nb < 1
    _einval(L.qgemm_q2_batched(ctypes.byref(w8), None, a16, a16, None, a16, 4, None, 0, None))
    _einval(L.qgemm_q2_batched(ctypes.byref(w8), a16, a16, a16, None, P(0x10004), 4, None, 0, None))   # y misaligned
    _einval(L.qgemm_q2_batched(ctypes.byref(w8), a16, a16, a16, P(0x10010), a16, 4, None, 0, None))    # accum over y
    ws2 = qg.qg_q2_weight(0x10000, 0x20002, 128, 256, 64, 0)                                  # scales not 8-aligned
    _einval(L.qgemm_q2_batched(ctypes.byref(ws2), a16, a16, a16, None, a16, 4, None, 0, None))
    for b in bad:
        _einval(L.qgemm_q2_batched(ctypes.byref(b), a16, a16, a16, None, a16, 4, None, 0, None))
    wdown = qg.qg_q2_weight(0x10000, 0x20000, 5120, 17408, 128, 0)                            # splits K
    need = L.qgemm_q2_batched_ws_bytes(5120, 17408, 128, 512)
    assert need == 3 * 512 * 5120 * 4, need
    assert L.qgemm_q2_batched_ws_bytes(17408, 5120, 128, 512) == 0
    # the product's K split: the occupancy rule (about one workgroup per CU,
    # at most 16 splits, at least a group per split); shapes (M, K, group,
    # nb) -> splits
    for (Mx, Kx, gx, nbx), S_exp in {(4352, 32768, 128, 512): 4, (4352, 16384, 64, 512): 4,
                                      (4352, 24576, 128, 512): 4, (100, 5120, 128, 5): 16,
                                      (272, 65536, 128, 128): 16, (17408, 65536, 128, 512): 1,
                                      (272, 256, 128, 128): 2}.items():
        n = L.qgemm_q2_batched_ws_bytes(Mx, Kx, gx, nbx)
        S = n // (nbx * Mx * 4) if n else 1
        assert S == S_exp, ((Mx, Kx, gx, nbx), S)
    # the group sums are not read by the product: a null suma is accepted
    # (the call then fails on the workspace, as without a null)
    _einval(L.qgemm_q2_batched(ctypes.byref(wdown), a16, None, a16, None, a16, 512, None, 0, None))
    _einval(L.qgemm_q2_batched(ctypes.byref(wdown), a16, a16, a16, None, a16, 512, None, 0, None))
    _einval(L.qgemm_q2_batched(ctypes.byref(wdown), a16, a16, a16, None, a16, 512, a16, need - 16, None))
    # gate|up GEMV with the gated product and its quantiser
    wg = qg.qg_q2_weight(0x10000, 0x20000, 128, 256, 64, 0)
    wu = qg.qg_q2_weight(0x30000, 0x40000, 128, 256, 64, 0)
    wu100 = qg.qg_q2_weight(0x30000, 0x40000, 100, 256, 64, 0)
    wg100 = qg.qg_q2_weight(0x10000, 0x20000, 100, 256, 64, 0)
    ok = (a16, a16, a16)
    _einval(L.qgemv_q2_gate_up_glu(ctypes.byref(wg100), ctypes.byref(wu100), *ok, 0, P(0x50000), P(0x60000), P(0x61000), P(0x62000), None))  # M % 64
    _einval(L.qgemv_q2_gate_up_glu(ctypes.byref(wg), ctypes.byref(wu100), *ok, 0, P(0x50000), P(0x60000), P(0x61000), P(0x62000), None))   # shapes differ
    _einval(L.qgemv_q2_gate_up_glu(ctypes.byref(wg), ctypes.byref(wu), *ok, 7, P(0x50000), P(0x60000), P(0x61000), P(0x62000), None))      # kind
    _einval(L.qgemv_q2_gate_up_glu(ctypes.byref(wg), ctypes.byref(wu), *ok, 0, P(0x50008), P(0x60000), P(0x61000), P(0x62000), None))      # t misaligned
    _einval(L.qgemv_q2_gate_up_glu(ctypes.byref(wg), ctypes.byref(wu), *ok, 0, P(0x50000), P(0x50100), P(0x61000), P(0x62000), None))      # xq_out in t
    _einval(L.qgemv_q2_gate_up_glu(ctypes.byref(wg), ctypes.byref(wu), *ok, 0, None, P(0x60000), P(0x61000), P(0x62000), None))
    # gate|up pair of the batched Q2 product
    w8b = qg.qg_q2_weight(0x30000, 0x40000, 128, 256, 64, 0)
    w8c = qg.qg_q2_weight(0x30000, 0x40000, 128, 256, 128, 0)                                 # other group
    _einval(L.qgemm_q2_batched_dual(ctypes.byref(w8), ctypes.byref(w8c), a16, a16, a16, P(0x50000), P(0x60000), 4, None, 0, None))
    _einval(L.qgemm_q2_batched_dual(ctypes.byref(w8), ctypes.byref(w8b), a16, a16, a16, P(0x50000), None, 4, None, 0, None))
    _einval(L.qgemm_q2_batched_dual(ctypes.byref(w8), ctypes.byref(w8b), a16, a16, a16, P(0x50000), P(0x50100), 4, None, 0, None))  # overlap
    _einval(L.qgemm_q2_batched_dual(ctypes.byref(w8), ctypes.byref(w8b), a16, a16, a16, P(0x50000), P(0x60004), 4, None, 0, None))  # misaligned
    _einval(L.qgemm_q2_batched_dual(ctypes.byref(w8), ctypes.byref(w8b), a16, a16, a16, P(0x50000), P(0x60000), 0, None, 0, None))  # nb < 1
    assert L.qgemm_q2_batched_dual_ws_bytes(5120, 17408, 128, 512) == 2 * L.qgemm_q2_batched_ws_bytes(5120, 17408, 128, 512)
    wd0 = qg.qg_q2_weight(0x10000, 0x20000, 5120, 17408, 128, 0)
    wd1 = qg.qg_q2_weight(0x30000, 0x40000, 5120, 17408, 128, 0)
    _einval(L.qgemm_q2_batched_dual(ctypes.byref(wd0), ctypes.byref(wd1), a16, a16, a16, P(0x1000000), P(0x9000000), 512,
                                    a16, L.qgemm_q2_batched_ws_bytes(5120, 17408, 128, 512), None))     # ws holds one matrix only
    # the batched q8_row product's K limit (int32 limb sums)
    assert L.qgemm_q8row_batched_ws_bytes(4, 131068) > 0 and L.qgemm_q8row_batched_ws_bytes(4, 131072) == 0
    _einval(L.qgemm_q8row_batched(a16, a16, a16, a16, 4, 64, 131072, 0, P(0x100000), 1 << 30, None))
    # a workspace overlapping an output or an input
    w2s = qg.qg_q2_weight(0x10000, 0x20000, 5120, 17408, 128, 0)
    nws = L.qgemv_q2_ws_bytes(5120, 17408, 128, 4)
    _einval(L.qgemv_q2(ctypes.byref(w2s), a16, a16, a16, P(0x200000), P(0x200000 + 4 * 5120 - 16), nws, 4, None))
    nwb = L.qgemm_q2_batched_ws_bytes(5120, 17408, 128, 512)
    _einval(L.qgemm_q2_batched(ctypes.byref(w2s), a16, a16, a16, None, P(0x1000000), 512, P(0x1000000 + 4096), nwb, None))
    gws2 = L.qgemm_q8row_batched_ws_bytes(256, 512)
    _einval(L.qgemm_q8row_batched(a16, a16, P(0x800000), P(0x400000), 256, 64, 512, 0, P(0x800000 - 256), gws2, None))
    _einval(L.qgemm_q8row_batched(a16, a16, P(0x800000), P(0x400000), 256, 64, 512, 0, P(0x400000), gws2, None))
    # column prescale and the batched q8_row product of it
    _einval(L.qact_silu_mul_pre(None, a16, None, a16, 1, 64, None))
    _einval(L.qact_silu_mul_pre(a16, a16, None, a16, 0, 64, None))                     # rows < 1
    _einval(L.qact_silu_mul_pre(a16, a16, None, a16, 4, 0, None))                      # n < 1
    _einval(L.qact_silu_mul_pre(P(0x10002), a16, None, P(0x40000), 4, 64, None))      # g misaligned
    _einval(L.qact_silu_mul_pre(P(0x20000), P(0x30000), None, P(0x20100), 4, 64, None))  # act partly over g
    _einval(L.qact_silu_mul_pre(P(0x20000), P(0x30000), P(0x40040), P(0x40000), 4, 64, None))  # col inside act
    gws = L.qgemm_q8row_batched_ws_bytes(256, 512)
    _einval(L.qgemm_q8row_batched_silu(a16, a16, None, a16, None, a16, 256, 64, 512, 0, P(0x100000), gws, None))
    _einval(L.qgemm_q8row_batched_silu(a16, a16, a16, P(0x20004), None, a16, 256, 64, 512, 0, P(0x100000), gws, None))
    _einval(L.qgemm_q8row_batched_silu(a16, a16, a16, a16, P(0x20008), a16, 256, 64, 512, 0, P(0x100000), gws, None))
    _einval(L.qgemm_q8row_batched_silu(a16, a16, a16, a16, None, a16, 256, 64, 512, 4, P(0x100000), gws, None))
    _einval(L.qgemm_q8row_batched_silu(a16, a16, a16, a16, None, a16, 256, 64, 510, 0, P(0x100000), gws, None))
    _einval(L.qgemm_q8row_batched_silu(a16, a16, a16, a16, None, a16, 256, 64, 512, 0, P(0x100000), gws - 1, None))
    # host repacks
    z = np.zeros(64, np.uint8)
    _einval(L.qg_repack_q8row(None, 4, 4, z.ctypes.data, 64))
    _einval(L.qg_repack_q8row(z.ctypes.data, 4, 4, z.ctypes.data, 10))
    _einval(L.qg_repack_q2(z.ctypes.data, 17, 1, 64, 64, z.ctypes.data, 64, z.ctypes.data, 64))
    _einval(L.qg_repack_q2(z.ctypes.data, 18, 1, 64, 32, z.ctypes.data, 64, z.ctypes.data, 64))


def test_binding_raises_on_error():
    with pytest.raises(qg.QGError):
        qg.repack_q2(np.zeros(10, np.uint8), 1, 64, 64)


def test_c_client_builds_against_the_header(tmp_path):
    """A plain C program (no Python, no framework) compiles with -Wall -Werror
    against include/qgemv.h and links against libqgemv.so and the HIP runtime."""
    import sys
    sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "c_abi"))
    import build_client
    out = build_client.build(str(tmp_path / "qgemv_c_client"))
    assert os.path.exists(out)


def test_einval_paths_in_launch_quantiser():
    """qgemv_q2_x, qgemv_q2_dual_x, qgemv_q2_gate_up_glu_x reject bad
    arguments before any launch (the pointers are never dereferenced)."""
    L = qg.lib()
    P = ctypes.c_void_p
    F = ctypes.c_float
    a16 = P(0x10000)
    w = qg.qg_q2_weight(0x100000, 0x200000, 128, 256, 64, 0)
    w1 = qg.qg_q2_weight(0x300000, 0x400000, 128, 256, 64, 0)
    X, Y, Y1, WS = P(0x500000), P(0x600000), P(0x700000), P(0x800000)
    # workspace sizes: counters (tiles rounded up to 64 ints) then [S][Mp] f32
    assert L.qgemv_q2_x_ws_bytes(128, 256, 64, 1) == 0
    assert L.qgemv_q2_x_ws_bytes(128, 256, 64, 2) == 256 + 2 * 128 * 4
    assert L.qgemv_q2_x_ws_bytes(5120, 17408, 128, 4) == 128 * 4 + 4 * 5120 * 4   # 80 tiles -> 128 counters
    # auto split of the in-launch form: every (tile, split) workgroup in one round
    assert L.qgemv_q2_x_auto_split(5120, 17408, 128) == 3      # 80 tiles x 3 = 240 workgroups
    assert L.qgemv_q2_x_auto_split(17408, 5120, 128) == 1      # 272 tiles fill the GPU
    assert L.qgemv_q2_x_auto_split(4096, 4096, 64) == 1        # 74 KB per row tile: no split
    assert L.qgemv_q2_x_auto_split(64, 512, 64) == 1           # 8 groups: no split
    assert L.qgemv_q2_x_auto_split(64, 1024, 64) == 1          # 18 KB per row tile
    assert L.qgemv_q2_x_auto_split(64, 16384, 64) == 4         # 295 KB: 4 pieces of 74 KB
    assert L.qgemv_q2_x_auto_split(1, 65536, 64) == 16
    assert L.qgemv_q2_x_ws_bytes(5120, 17408, 128, 0) == 128 * 4 + 3 * 5120 * 4
    # qgemv_q2_x
    _einval(L.qgemv_q2_x(None, X, None, 0, None, Y, None, 0, 1, None))
    _einval(L.qgemv_q2_x(ctypes.byref(w), None, None, 0, None, Y, None, 0, 1, None))            # null x
    _einval(L.qgemv_q2_x(ctypes.byref(w), P(0x500008), None, 0, None, Y, None, 0, 1, None))     # x misaligned
    _einval(L.qgemv_q2_x(ctypes.byref(w), X, None, 0, None, None, None, 0, 1, None))            # null y
    _einval(L.qgemv_q2_x(ctypes.byref(w), X, None, 0, None, P(0x500100), None, 0, 1, None))     # y inside x
    _einval(L.qgemv_q2_x(ctypes.byref(w), X, None, 0, P(0x600004), Y, None, 0, 1, None))        # accum over y
    _einval(L.qgemv_q2_x(ctypes.byref(w), X, None, 0, None, Y, None, 0, 17, None))
    _einval(L.qgemv_q2_x(ctypes.byref(w), X, None, 0, None, Y, None, 0, 2, None))               # no workspace
    _einval(L.qgemv_q2_x(ctypes.byref(w), X, None, 0, None, Y, WS, 100, 2, None))               # too small
    _einval(L.qgemv_q2_x(ctypes.byref(w), X, None, 0, None, Y, P(0x800008), 4096, 2, None))     # ws misaligned
    _einval(L.qgemv_q2_x(ctypes.byref(w), X, None, 0, None, Y, P(0x500000), 4096, 2, None))     # ws over x
    _einval(L.qgemv_q2_x(ctypes.byref(w), X, None, 0, None, Y, P(0x600000), 4096, 2, None))     # ws over y
    _einval(L.qgemv_q2_x(ctypes.byref(w), X, None, 0, None, Y, P(0x100100), 4096, 2, None))     # ws over the codes
    _einval(L.qgemv_q2_x(ctypes.byref(w), X, None, 0, None, Y, P(0x200040), 4096, 2, None))     # ws over the scales
    # partial maxima of |x|: both or neither, 1..512 of them, aligned, apart from y
    _einval(L.qgemv_q2_x(ctypes.byref(w), X, P(0xa00000), 0, None, Y, None, 0, 1, None))
    _einval(L.qgemv_q2_x(ctypes.byref(w), X, None, 4, None, Y, None, 0, 1, None))
    _einval(L.qgemv_q2_x(ctypes.byref(w), X, P(0xa00000), 513, None, Y, None, 0, 1, None))
    _einval(L.qgemv_q2_x(ctypes.byref(w), X, P(0xa00002), 4, None, Y, None, 0, 1, None))
    _einval(L.qgemv_q2_x(ctypes.byref(w), X, P(0x600010), 4, None, Y, None, 0, 1, None))       # xmax over y
    _einval(L.qgemv_q2_x(ctypes.byref(w), X, P(0x800010), 4, None, Y, P(0x800000), 4096, 2, None))  # over ws
    big = qg.qg_q2_weight(0x100000, 0x200000, 128, 32768 + 64, 64, 0)
    _einval(L.qgemv_q2_x(ctypes.byref(big), X, None, 0, None, Y, None, 0, 1, None))             # K above 32768
    wide = qg.qg_q2_weight(0x100000, 0x200000, 16384, 16384 + 128, 128, 0)
    _einval(L.qgemv_q2_x(ctypes.byref(wide), X, None, 0, None, Y, None, 0, 1, None))            # K above 16384 at 8 waves
    _einval(L.qgemv_q2_x(ctypes.byref(wide), X, None, 0, None, Y, WS, 1 << 20, 4, None))       # whatever the split
    assert L.qgemv_q2_gate_up_glu_x_ws_bytes(130) == 256 + 2 * 192 * 4
    # qgemv_q2_dual_x
    _einval(L.qgemv_q2_dual_x(ctypes.byref(w), None, X, None, F(0), Y, Y1, None))
    other = qg.qg_q2_weight(0x300000, 0x400000, 64, 256, 64, 0)
    _einval(L.qgemv_q2_dual_x(ctypes.byref(w), ctypes.byref(other), X, None, F(0), Y, Y1, None))
    _einval(L.qgemv_q2_dual_x(ctypes.byref(w), ctypes.byref(w1), X, None, F(0), Y, None, None))
    _einval(L.qgemv_q2_dual_x(ctypes.byref(w), ctypes.byref(w1), X, None, F(0), Y, P(0x600100), None))
    _einval(L.qgemv_q2_dual_x(ctypes.byref(w), ctypes.byref(w1), X, None, F(0), Y, P(0x500000), None))
    _einval(L.qgemv_q2_dual_x(ctypes.byref(w), ctypes.byref(w1), X, P(0x900008), F(0), Y, Y1, None))
    _einval(L.qgemv_q2_dual_x(ctypes.byref(w), ctypes.byref(w1), X, P(0x900000), F(-1.0), Y, Y1, None))
    _einval(L.qgemv_q2_dual_x(ctypes.byref(w), ctypes.byref(w1), X, P(0x900000), F(float("nan")), Y, Y1, None))
    _einval(L.qgemv_q2_dual_x(ctypes.byref(w), ctypes.byref(w1), X, P(0x600000), F(0), Y, Y1, None))  # norm_w = y0
    wn = qg.qg_q2_weight(0x100000, 0x200000, 128, 16384 + 64, 64, 0)
    wn1 = qg.qg_q2_weight(0x300000, 0x400000, 128, 16384 + 64, 64, 0)
    _einval(L.qgemv_q2_dual_x(ctypes.byref(wn), ctypes.byref(wn1), X, P(0x900000), F(0), Y, Y1, None))
    # qgemv_q2_gate_up_glu_x
    _einval(L.qgemv_q2_gate_up_glu_x(ctypes.byref(w), ctypes.byref(w1), X, None, F(0), 2, Y, None, WS, 4096, None))
    _einval(L.qgemv_q2_gate_up_glu_x(ctypes.byref(w), ctypes.byref(w1), X, None, F(0), 0, None, None, WS, 4096, None))
    _einval(L.qgemv_q2_gate_up_glu_x(ctypes.byref(w), ctypes.byref(w1), X, None, F(0), 0, P(0x500010), None, WS, 4096, None))
    _einval(L.qgemv_q2_gate_up_glu_x(ctypes.byref(w), ctypes.byref(w1), X, None, F(0), 0, Y, None, None, 0, None))
    _einval(L.qgemv_q2_gate_up_glu_x(ctypes.byref(w), ctypes.byref(w1), X, None, F(0), 0, Y, None, WS, 100, None))
    _einval(L.qgemv_q2_gate_up_glu_x(ctypes.byref(w), ctypes.byref(w1), X, None, F(0), 0, Y, None, P(0x600000), 4096, None))
    # tmax: aligned, apart from t, x and the workspace
    _einval(L.qgemv_q2_gate_up_glu_x(ctypes.byref(w), ctypes.byref(w1), X, None, F(0), 0, Y, P(0xa00002), WS, 4096, None))
    _einval(L.qgemv_q2_gate_up_glu_x(ctypes.byref(w), ctypes.byref(w1), X, None, F(0), 0, Y, P(0x600008), WS, 4096, None))
    _einval(L.qgemv_q2_gate_up_glu_x(ctypes.byref(w), ctypes.byref(w1), X, None, F(0), 0, Y, P(0x500008), WS, 4096, None))
    _einval(L.qgemv_q2_gate_up_glu_x(ctypes.byref(w), ctypes.byref(w1), X, None, F(0), 0, Y, WS, WS, 4096, None))


def test_q8row_balanced_sizes_and_einval():
    L = qg.lib()
    P = ctypes.c_void_p
    # 248320 rows: 3880 tiles = 15 rounds of 256 + 40, split 7 ways
    assert L.qgemv_q8row_balanced_ws_bytes(248320, 5120) == 256 + 40 * 7 * 64 * 4
    assert L.qgemv_q8row_balanced_ws_bytes(100, 512) == 0          # under one round
    assert L.qgemv_q8row_balanced_ws_bytes(64 * 512, 512) == 0     # whole rounds
    assert L.qgemv_q8row_balanced_ws_bytes(64 * 257, 1024) == 256 + 1 * 16 * 64 * 4   # S capped at 16
    assert L.qgemv_q8row_balanced_ws_bytes(64 * 257, 96) == 256 + 1 * 6 * 64 * 4      # S at most the chunks
    a16 = P(0x10000)
    _einval(L.qgemv_q8row_balanced(None, a16, a16, a16, 64, 64, None, 0, None))
    _einval(L.qgemv_q8row_balanced(a16, a16, a16, a16, 64, 62, None, 0, None))
    M = 64 * 257
    _einval(L.qgemv_q8row_balanced(a16, P(0x200000), P(0x300000), P(0x400000), M, 1024, None, 0, None))
    _einval(L.qgemv_q8row_balanced(a16, P(0x200000), P(0x300000), P(0x400000), M, 1024, P(0x500000), 100, None))
    _einval(L.qgemv_q8row_balanced(a16, P(0x200000), P(0x300000), P(0x400000), M, 1024, P(0x500008), 1 << 20, None))
    _einval(L.qgemv_q8row_balanced(a16, P(0x200000), P(0x300000), P(0x400000), M, 1024, P(0x400100), 1 << 20, None))
    _einval(L.qgemv_q8row_balanced(P(0x1000000), P(0x200000), P(0x300000), P(0x400000), M, 1024, P(0x1000400), 1 << 20, None))


def test_probe_entry_points_einval():
    """The measurement probes validate their arguments before any launch."""
    L = qg.lib()
    P = ctypes.c_void_p
    _einval(L.qg_probe_stream_read(None, 1 << 20, 1, P(0x1000), 64, 8, None))
    _einval(L.qg_probe_stream_read(P(0x1008), 1 << 20, 1, P(0x1000), 64, 8, None))   # misaligned
    _einval(L.qg_probe_stream_read(P(0x1000), 8, 1, P(0x2000), 64, 8, None))         # under 16 bytes
    _einval(L.qg_probe_stream_read(P(0x1000), 1 << 20, 1, P(0x2000), 64, 5, None))   # loads not 4/8/16
    _einval(L.qg_probe_mfma(2, 10, 64, P(0x1000), P(0x2000), None))
    _einval(L.qg_probe_mfma(0, 0, 64, P(0x1000), P(0x2000), None))
    _einval(L.qg_probe_mfma(0, 10, 64, P(0x1000), P(0x2004), None))                 # clocks misaligned
    w = qg.qg_q2_weight(0x100000, 0x200000, 128, 256, 64, 0)
    _einval(L.qg_probe_q2_x_stamped(ctypes.byref(w), P(0x500000), None, 0, None, P(0x600000), None, 0, 1,
                                    None, None))                                      # no stamps
    _einval(L.qg_probe_q2_gate_up_glu_x_stamped(ctypes.byref(w), ctypes.byref(w), P(0x500000), None,
                                                ctypes.c_float(0.0), 0, P(0x600000), None, P(0x800000), 4096,
                                                P(0x900004), None))                  # stamps misaligned
    _einval(L.qg_probe_mfma_valu(2, 4, 10, 64, 2, P(0x1000), 64 * 512, None))    # mfma not 0/1
    _einval(L.qg_probe_mfma_valu(1, 3, 10, 64, 2, P(0x1000), 64 * 512, None))    # fmas not 0/2/4/8
    _einval(L.qg_probe_mfma_valu(0, 0, 10, 64, 2, P(0x1000), 64 * 512, None))    # nothing to run
    _einval(L.qg_probe_mfma_valu(1, 4, 10, 64, 5, P(0x1000), 64 * 1280, None))   # 5 waves per SIMD
    _einval(L.qg_probe_mfma_valu(1, 4, 10, 64, 2, P(0x1000), 64 * 512 - 1, None))  # sink too small
    _einval(L.qg_probe_lds_read(12, 10, 64, 8, P(0x1000), 64 * 512, None))       # 12 bytes per lane
    _einval(L.qg_probe_lds_read(16, 10, 64, 17, P(0x1000), 64 * 64 * 17, None))  # 17 waves
    _einval(L.qg_probe_lds_read(16, 10, 64, 8, P(0x1002), 64 * 512, None))       # sink misaligned
    _einval(L.qg_probe_lds_read(16, 10, 64, 8, P(0x1000), 64 * 512 - 1, None))   # sink too small
