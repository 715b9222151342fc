"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module draws random numbers and lays them out in the input formats; it
holds none of the method's arithmetic (no dequantisation, no activation
quantisation, no products).  Both the HIP path and the CPU oracle consume
exactly these arrays.

Formats produced (as the pages define them):

* q8_row (cortiq-engine pages, ``q8_matvec`` shader doc): int8 weights,
  row-major ``[M][K]``, one f32 scale per row, activations ``xs`` f32 already
  prescaled by the caller.
* Q2 GGUF-style blocks (qxmx GPU engine page, ``dequant_embd`` and
  ``upload_q2``): per row, ``K/group`` blocks of ``2 + group/4`` bytes: an
  IEEE binary16 scale ``d`` (little-endian) followed by ``group/4`` bytes of
  2-bit codes.  Independent uniform codes 0..3, four per byte, make every
  code byte a uniform random byte, so the code bytes are drawn directly.

Seeds: ``numpy.random.PCG64(seed)``; the default seed of a workload is
``20260 + its seed id`` (``SEED_IDS``), plus 100 per FFN-matrix substream.
"""
from __future__ import annotations

import numpy as np

SEED_BASE = 20260

# The five workloads.  Shapes follow the pages' engine (model width 5120,
# FFN width 17408, a ~248K-row vocabulary projection).
CONFIGS = {
    "q8row_256x512": dict(kind="q8row", M=256, K=512, rs=(0.001, 0.01)),
    "q2_g64_4096x4096": dict(kind="q2", M=4096, K=4096, group=64),
    "q2_g128_gate_17408x5120": dict(kind="q2", M=17408, K=5120, group=128),
    "q2_g128_up_17408x5120": dict(kind="q2", M=17408, K=5120, group=128),
    "q2_g128_down_5120x17408": dict(kind="q2", M=5120, K=17408, group=128),
    "q8row_lm_head_248320x5120": dict(kind="q8row", M=248320, K=5120, rs=(0.0005, 0.005)),
    "q8row_gemm_512x17408x5120": dict(kind="q8gemm", nb=512, M=17408, K=5120, rs=(0.001, 0.01)),
}
# Seed id of each workload: the default seed is SEED_BASE + id, plus 100 per
# substream for the three FFN matrices, which share id 3.
SEED_IDS = {"q8row_256x512": 1, "q2_g64_4096x4096": 2,
            "q2_g128_gate_17408x5120": 3, "q2_g128_up_17408x5120": 3, "q2_g128_down_5120x17408": 3,
            "q8row_lm_head_248320x5120": 4, "q8row_gemm_512x17408x5120": 5}
# distinct streams for the three FFN matrices
_SUBSTREAM = {"q2_g128_gate_17408x5120": 0, "q2_g128_up_17408x5120": 1, "q2_g128_down_5120x17408": 2}


def rng_for(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def default_seed(name: str) -> int:
    return SEED_BASE + SEED_IDS[name] + 100 * _SUBSTREAM.get(name, 0)


def q8row_inputs(M: int, K: int, rs_range=(0.001, 0.01), seed: int = 0, *,
                 rng: np.random.Generator | None = None, chunk_rows: int = 1 << 16):
    """int8 weights U{-127..127} ``[M][K]``, f32 row scales U[lo, hi), xs f32 N(0,1)."""
    g = rng if rng is not None else rng_for(seed)
    q = np.empty((M, K), dtype=np.int8)
    for r0 in range(0, M, chunk_rows):
        r1 = min(M, r0 + chunk_rows)
        q[r0:r1] = g.integers(-127, 128, size=(r1 - r0, K), dtype=np.int8)
    rs = g.uniform(rs_range[0], rs_range[1], size=M).astype(np.float32)
    xs = g.standard_normal(K, dtype=np.float32)
    return q, rs, xs


def q8gemm_inputs(nb: int, M: int, K: int, rs_range=(0.001, 0.01), seed: int = 0):
    """Batched prefill inputs: weights and row scales as above, xs ``[nb][K]`` N(0,1)."""
    g = rng_for(seed)
    q, rs, _ = q8row_inputs(M, K, rs_range, rng=g)
    xs = g.standard_normal((nb, K), dtype=np.float32)
    return q, rs, xs


def gate_inputs(rows: int, n: int, seed: int = 0, col: bool = True):
    """Inputs of the column prescale: gate g = 2 N(0,1) (reaching the saturated
    ends of silu), up u N(0,1), both [rows][n], and a column field col U[0.5, 2)
    of n values (None when col is False)."""
    r = rng_for(seed)
    g = (2.0 * r.standard_normal((rows, n))).astype(np.float32)
    u = r.standard_normal((rows, n), dtype=np.float32)
    c = r.uniform(0.5, 2.0, n).astype(np.float32) if col else None
    return g, u, c


def q2_scales_f16(g: np.random.Generator, M: int, ngroups: int, sigma: float = 0.02):
    """f16 group scales |N(0, sigma)|, rounded to nearest-even binary16; raw bit patterns."""
    d = np.abs(g.normal(0.0, sigma, size=(M, ngroups))).astype(np.float16)
    return d.view(np.uint16)


def assemble_q2_blocks(d_bits: np.ndarray, code_bytes: np.ndarray) -> np.ndarray:
    """Lay out GGUF-style blocks: per (row, group) the 2 scale bytes (LE) then the code bytes.

    ``d_bits``: uint16 ``[M][ngroups]``; ``code_bytes``: uint8 ``[M][ngroups][group/4]``.
    Returns a flat uint8 array of ``M*ngroups*(2 + group/4)`` bytes.
    """
    M, ng = d_bits.shape
    nb = code_bytes.shape[2]
    out = np.empty((M, ng, 2 + nb), dtype=np.uint8)
    out[:, :, 0:2] = d_bits.astype("<u2").reshape(M, ng, 1).view(np.uint8)
    out[:, :, 2:] = code_bytes
    return out.reshape(-1)


def q2_inputs(M: int, K: int, group: int, seed: int = 0, sigma: float = 0.02):
    """Q2 weights as a GGUF-style block blob plus an f32 N(0,1) activation vector."""
    assert group in (64, 128) and K % group == 0
    g = rng_for(seed)
    ng = K // group
    d_bits = q2_scales_f16(g, M, ng, sigma)
    codes = g.integers(0, 256, size=(M, ng, group // 4), dtype=np.uint8)
    blob = assemble_q2_blocks(d_bits, codes)
    x = g.standard_normal(K, dtype=np.float32)
    return blob, x


def activation(K: int, seed: int) -> np.ndarray:
    return rng_for(seed).standard_normal(K, dtype=np.float32)


def config_inputs(name: str, seed: int | None = None):
    """Inputs of one named workload, with its default seed unless one is given."""
    c = CONFIGS[name]
    s = default_seed(name) if seed is None else seed
    if c["kind"] == "q8row":
        return q8row_inputs(c["M"], c["K"], c["rs"], s)
    if c["kind"] == "q2":
        return q2_inputs(c["M"], c["K"], c["group"], s)
    if c["kind"] == "q8gemm":
        return q8gemm_inputs(c["nb"], c["M"], c["K"], c["rs"], s)
    raise KeyError(name)
