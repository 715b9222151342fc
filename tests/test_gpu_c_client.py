"""The C-ABI used from plain C: the client program under tests/c_abi (built
by __graft_entry__.build()) runs a q8_row GEMV and a Q2 GEMV with its
activation quantiser and a K split (and the same GEMV with the quantiser
and the split's reduce inside one launch), in its own process, on inputs
this test writes; its outputs are held to the oracle (the quantiser bit for bit, the
GEMVs within |y - y_ref| <= 2e-5 * sum_i |w_i x_i|)."""
import os
import subprocess

import numpy as np
import pytest

import oracle
import synth
from conftest import gpu_available

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not gpu_available(), reason="needs a HIP device")]

HERE = os.path.dirname(os.path.abspath(__file__))
CLIENT = os.path.join(HERE, "c_abi", "_build", "qgemv_c_client")


@pytest.mark.parametrize("M2,K2,group,split", [(300, 1024, 128, 4), (4096, 4096, 64, 0)])
def test_c_client_matches_oracle(tmp_path, M2, K2, group, split):
    assert os.path.exists(CLIENT), "the C client is not built (run __graft_entry__.build())"
    q8, rs, xs = synth.config_inputs("q8row_256x512")
    M8, K8 = q8.shape
    blob, x2 = synth.q2_inputs(M2, K2, group, seed=81 + M2)
    inp, outp = tmp_path / "in.bin", tmp_path / "out.bin"
    with open(inp, "wb") as f:
        f.write(np.array([M8, K8, M2, K2, group, split], np.int64).tobytes())
        f.write(np.ascontiguousarray(q8, np.int8).tobytes())
        f.write(np.ascontiguousarray(rs, np.float32).tobytes())
        f.write(np.ascontiguousarray(xs, np.float32).tobytes())
        f.write(np.ascontiguousarray(blob, np.uint8).tobytes())
        f.write(np.ascontiguousarray(x2, np.float32).tobytes())
    r = subprocess.run([CLIENT, str(inp), str(outp)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, f"client failed ({r.returncode}): {r.stderr}"
    raw = outp.read_bytes()
    off = 0

    def take(n, dt):
        nonlocal off
        a = np.frombuffer(raw, dtype=dt, count=n, offset=off)
        off += n * np.dtype(dt).itemsize
        return a

    y8, y2 = take(M8, np.float32), take(M2, np.float32)
    xq, sc, suma = take(K2, np.int8), take(1, np.float32)[0], take(K2 // 64, np.int32)
    y2x = take(M2, np.float32)
    assert off == len(raw)
    rq, rsc, rsu = oracle.act_quant_i8(x2)
    assert np.array_equal(xq, rq) and sc == rsc and np.array_equal(suma, rsu)
    y8r, m8 = oracle.q8row_gemv(q8, rs, xs)
    assert np.all(np.abs(y8.astype(np.float64) - y8r) <= 2e-5 * m8), "q8_row GEMV from C outside bound"
    y2r, m2 = oracle.q2_gemv(blob, M2, K2, group, rq, rsc)
    assert np.all(np.abs(y2.astype(np.float64) - y2r) <= 2e-5 * m2), "Q2 GEMV from C outside bound"
    assert np.all(np.abs(y2x.astype(np.float64) - y2r) <= 2e-5 * m2), "qgemv_q2_x from C outside bound"
    if split:  # the same explicit split: the same bits as quantiser + qgemv_q2
        assert np.array_equal(y2x.view(np.uint32), y2.view(np.uint32)), "qgemv_q2_x from C differs from qgemv_q2"
