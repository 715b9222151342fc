"""Every plausible slip in the oracle must be caught by at least one pin.

Each case copies ``oracle/qoracle.c``, plants one mistake in the copy (a wrong
sign, index, constant, rounding mode or dropped term), builds it with gcc in a
temporary folder and runs all pins against it.  The planted mistakes live
only in this file and in the temporary copies.  CPU only.

(Dropping the zero guard of the quantiser's reciprocal is not listed: on
x86-64 the resulting NaN converts to int8 0, the same output as the guard.)
"""
import os

import pytest

import oracle
from oracle_pins import ALL_PINS

MUTANTS = {
    "f16 subnormal as 2^-14": ("ldexp((double)m, -24)", "ldexp((double)m, -14)"),
    "f16 exponent bias": ("ldexp((double)(1024 + m), e - 25)", "ldexp((double)(1024 + m), e - 24)"),
    "q8 row scale dropped": ("y[j] = (double)rs[o] * acc;\n        if (mass) mass[j] = fabs((double)rs[o]) * am;\n    }\n}\n\n/* ---- batched",
                             "y[j] = acc;\n        if (mass) mass[j] = fabs((double)rs[o]) * am;\n    }\n}\n\n/* ---- batched"),
    "q8 activation reversed": ("double t = (double)qr[i] * (double)xs[i];", "double t = (double)qr[i] * (double)xs[K - 1 - i];"),
    "q8 sign": ("            acc += t;\n            am += fabs(t);\n        }\n        y[j] = (double)rs[o] * acc;\n        if (mass) mass[j] = fabs((double)rs[o]) * am;\n    }\n}\n\n/* ---- batched",
                "            acc -= t;\n            am += fabs(t);\n        }\n        y[j] = (double)rs[o] * acc;\n        if (mass) mass[j] = fabs((double)rs[o]) * am;\n    }\n}\n\n/* ---- batched"),
    "gemm ignores batch row": ("const float *xr = xs + b * K;", "const float *xr = xs;"),
    "gemm transposed scale": ("y[j] = (double)rs[o] * acc;\n        if (mass) mass[j] = fabs((double)rs[o]) * am;\n    }\n}\n\n/* ---- Q2",
                              "y[j] = (double)rs[b % M] * acc;\n        if (mass) mass[j] = fabs((double)rs[o]) * am;\n    }\n}\n\n/* ---- Q2"),
    "quant half-to-even": ("float v = roundf(x[i] * inv);", "float v = rintf(x[i] * inv);"),
    "quant truncation": ("float v = roundf(x[i] * inv);", "float v = truncf(x[i] * inv);"),
    "quant /128": ("float sc = amax / 127.0f;", "float sc = amax / 128.0f;"),
    "quant suma index": ("for (int k = 0; k < 64; k++) s += xq[g * 64 + k];", "for (int k = 0; k < 64; k++) s += xq[k];"),
    "q2 code bit order": ("return (blk[2 + k / 4] >> (2 * (k % 4))) & 3;", "return (blk[2 + k / 4] >> (2 * (3 - k % 4))) & 3;"),
    "q2 code byte index": ("return (blk[2 + k / 4] >> (2 * (k % 4))) & 3;", "return (blk[2 + (k / 4) % 16] >> (2 * (k % 4))) & 3;"),
    "q2 value offset dropped": ("w[o * K + i] = q2_d(blk) * (double)(q2_code(blk, (int)(i % group)) - 1);",
                                "w[o * K + i] = q2_d(blk) * (double)(q2_code(blk, (int)(i % group)));"),
    "q2 scale byte order": ("return qo_f16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));",
                            "return qo_f16_to_f64((uint16_t)(blk[1] | (blk[0] << 8)));"),
    "q2 dots offset dropped": ("s += (q2_code(blk, (int)(i % group)) - 1) * (int32_t)xq[i];",
                               "s += (q2_code(blk, (int)(i % group))) * (int32_t)xq[i];"),
    "q2 gemv group index": ("const uint8_t *blk = q2_blk(blob, K, group, o, (u * 64) / group);",
                            "const uint8_t *blk = q2_blk(blob, K, group, o, u % (K / group));"),
    "q2 gemv act scale dropped": ("y[j] = (double)sc * acc;", "y[j] = acc;"),
    "accum dropped": ("y[j] += (double)accum[o];", "y[j] += 0.0;"),
    "accum sign": ("y[j] += (double)accum[o];", "y[j] -= (double)accum[o];"),
    "accum row index": ("y[j] += (double)accum[o];", "y[j] += (double)accum[j];"),
    "rms mean divisor": ("float ms = (float)(ss / (double)K);", "float ms = (float)(ss / (double)(K - 1));"),
    "rms eps dropped": ("float inv = 1.0f / sqrtf(ms + eps);", "float inv = 1.0f / sqrtf(ms);"),
    "rms sqrt dropped": ("float inv = 1.0f / sqrtf(ms + eps);", "float inv = 1.0f / (ms + eps);"),
    "rms weight dropped": ("v[i] = xi * w[i];", "v[i] = xi;"),
    "rms weight index": ("v[i] = xi * w[i];", "v[i] = xi * w[0];"),
    "glu exp sign": ("float e = exp_f32(-g[i]);", "float e = exp_f32(g[i]);"),
    "glu denominator": ("float den = 1.0f + e;\n        if (kind == 0) {", "float den = 1.0f - e;\n        if (kind == 0) {"),
    "silu_pre denominator": ("float den = 1.0f + e;\n            float s = g[k] / den;", "float den = 1.0f - e;\n            float s = g[k] / den;"),
    "glu silu as sigmoid": ("float silu = g[i] / den;", "float silu = 1.0f / den;"),
    "glu sigmoid as silu": ("float sig = 1.0f / den;", "float sig = g[i] / den;"),
    "glu up index": ("t[i] = silu * u[i];", "t[i] = silu * u[0];"),
    "silu_pre exp sign": ("float e = exp_f32(-g[k]);", "float e = exp_f32(g[k]);"),
    "silu_pre product for quotient": ("float s = g[k] / den;", "float s = g[k] * den;"),
    "silu_pre column dropped": ("                v = v * col[i];", "                v = v;"),
    "silu_pre column by row": ("                v = v * col[i];", "                v = v * col[r];"),
    "silu_pre up from row 0": ("float v = s * u[k];", "float v = s * u[i];"),
    "quant divides by the scale": ("float v = roundf(x[i] * inv);", "float v = roundf(x[i] / sc);"),
    "rms sum of squares in binary32": ("double ss = 0.0;\n    for (int64_t i = 0; i < K; i++) ss += (double)x[i] * (double)x[i];",
                                       "float ss = 0.0f;\n    for (int64_t i = 0; i < K; i++) ss += x[i] * x[i];"),
    "rms weight folded into inv": ("float xi = x[i] * inv;\n        v[i] = xi * w[i];",
                                   "float iw = inv * w[i];\n        v[i] = x[i] * iw;"),
    "q2 gemm token row ignored": ("qo_q2_gemv(blob, M, K, group, xq + b * K, sc[b], &o, 1, &yj, &mj);",
                                  "qo_q2_gemv(blob, M, K, group, xq, sc[b], &o, 1, &yj, &mj);"),
    "q2 gemm scale of token 0": ("qo_q2_gemv(blob, M, K, group, xq + b * K, sc[b], &o, 1, &yj, &mj);",
                                 "qo_q2_gemv(blob, M, K, group, xq + b * K, sc[0], &o, 1, &yj, &mj);"),
    "q2 gemm residual index": ("if (accum) yj += (double)accum[b * M + o];", "if (accum) yj += (double)accum[o * nb + b];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(os.path.join(os.path.dirname(oracle.__file__), "qoracle.c")).read()
    assert src.count(old) == 1, f"mutation anchor not unique/found: {name}"
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new))
    lib = oracle.build(str(mpath), str(tmp_path / "libmutant.so"))
    orc = oracle.Oracle(lib)
    caught = []
    for pin_name, pin in ALL_PINS.items():
        try:
            pin(orc)
        except Exception:  # a failed assertion or a crash both expose the slip
            caught.append(pin_name)
    assert caught, f"no pin catches mutant '{name}'"
