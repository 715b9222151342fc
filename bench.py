#!/usr/bin/env python3
"""Benchmark of the weight-only-quantized decode hot path on one MI355X.

A step is one pass of the batch-1 decode path at the pages' model shapes,
captured once in a HIP graph and replayed, three launches:
    Q2 g128 gate and up GEMVs 17408x5120 (one launch for the pair, the f32
    activation x (K=5120) quantised inside it) -> Q2 g128 down GEMV
    5120x17408 (h, K=17408, quantised inside the launch; split-K partials
    added by the last workgroup of each row tile) -> q8_row lm_head GEMV
    248320x5120 (its last partial round of 40 row tiles split along K over
    the whole GPU).
The same step as six launches (the quantisers and the split reduce as
launches of their own, the same bits) is timed beside it.
`value` is the weight bytes the step streams (the formats' own bytes: 34 B
per 128 Q2 weights, K+4 bytes per q8_row row) divided by the step time:
batch-1 quantized GEMV weight GB/s.  Inputs are synthetic and seeded, already
resident in HBM when timing starts.  The lm_head stream (1.27 GB) evicts the
256 MB last-level cache every step, so the FFN weights also come from HBM.

Also reported: per-kernel times and roofline fractions, the dominant
kernel's roofline (HIP events on the launch stream), the CPU oracle timed
on this host over the same step (cpu_baseline), and the second half of the
metric, the batched prefill q8_row GEMM (nb=512 x 17408 x 5120, int8 MFMA
with exact activation limbs), in algorithmic TFLOP/s (`prefill_gemm`), and
the FFN block in its fused form (RMSNorm+quant, gate|up with the SiLU gate,
quant, down with the residual: two launches) next to the main step
(`fused_ffn`), each Q2 GEMV's streaming rate from HBM
over rotated weight copies launched back to back (`q2_sustained`), and the
batched prefill Q2 product over 512 token rows (`prefill_q2_gemm`).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP16_DENSE_TFLOPS = 2500.0
INT8_DENSE_TOPS = 5000.0
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "q8row_gemv_lm_head_248320x5120_traffic.txt")
KERNEL_SRC = os.path.join(ROOT, "weight_quantized_decode_q8_amd", "csrc", "q8row_gemv.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-gemm", action="store_true", help="skip the prefill GEMM leg")
    ap.add_argument("--no-breakdown", action="store_true",
                    help="skip the per-kernel timing table (for counter runs)")
    ap.add_argument("--down-split", type=int, default=0,
                    help="split of the down projection's one-launch form (0: the library's choice)")
    ap.add_argument("--timeline-only", action="store_true",
                    help="only the per-workgroup timeline of the fused FFN launches")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run a plain 1 GiB device copy (for counter calibration)")
    return ap.parse_args()


def src_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def read_traffic():
    """Bytes per lm_head launch from the committed counter summary, or None
    when the kernel source changed since the counters were taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.startswith("#"):
            k, v = line.strip().split("=", 1)
            kv[k.strip()] = v.strip()
    if kv.get("source_sha256") != src_sha(KERNEL_SRC):
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def measure_achievable(qg, torch, dev, stream, log):
    """What this GPU reaches: a streaming read of a 4 GiB buffer (16-byte
    non-temporal loads, the best of several grid sizes) and register-only
    matrix-core loops (int8 16x16x64, fp16 16x16x32), with the shader clock
    read from s_memtime against the wall clock during the loops; whether
    vector-ALU work hides behind matrix-core work; the LDS read rate."""
    out = {}
    nbytes = 4 << 30
    buf = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    best = None
    sweep = {}
    for loads in (4, 8, 16):
        for wg in (1024, 2048, 4096, 8192, 16384, 32768):
            sink = torch.zeros(wg, dtype=torch.int32, device=dev)
            qg.qg_probe_stream_read(buf, 0x5EED1E55, sink, wg, loads)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            reps = 5
            a.record(stream)
            for _ in range(reps):
                qg.qg_probe_stream_read(buf, 0x5EED1E55, sink, wg, loads)
            b.record(stream)
            torch.cuda.synchronize()
            gbs = nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9
            sweep[f"{loads}x{wg}"] = round(gbs, 1)
            if best is None or gbs > best[0]:
                best = (gbs, wg, loads)
    del buf
    out["stream_read"] = {"GB/s": round(best[0], 1), "frac_hbm_spec": round(best[0] / HBM_PEAK_GBS, 4),
                          "workgroups": best[1], "loads_in_flight": best[2], "bytes": nbytes,
                          "sweep_GB/s": sweep,
                          "note": "qg_probe_stream_read: one pass over 4 GiB, 16-byte non-temporal loads, "
                                  "4-16 in flight per lane, 512-thread workgroups, 1024-32768 of them (best)"}
    khz = qg.qg_probe_wall_clock_khz()
    wgs, iters = 2048, 400
    sink = torch.empty(wgs * 256, dtype=torch.float32, device=dev)
    clocks = torch.zeros(2, dtype=torch.int64, device=dev)
    for kind, name, ops_per, spec in ((0, "mfma_i8", 32768, INT8_DENSE_TOPS), (1, "mfma_f16", 16384, FP16_DENSE_TFLOPS)):
        qg.qg_probe_mfma(kind, iters, wgs, sink, clocks)  # the clock settles under load
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        qg.qg_probe_mfma(kind, iters, wgs, sink, clocks)
        b.record(stream)
        torch.cuda.synchronize()
        us = a.elapsed_time(b) * 1e3
        ops = wgs * 4 * 8 * iters * ops_per
        cyc, ticks = (int(v) for v in clocks.cpu())
        mhz = cyc / (ticks / khz * 1e3) if ticks else None
        rate = ops / us / 1e6
        out[name] = {"T/s": round(rate, 1), "frac_dense_spec": round(rate / spec, 4), "us": round(us, 1),
                     "shader_clock_MHz": round(mhz, 0) if mhz else None,
                     "note": f"qg_probe_mfma kind {kind}: {wgs} workgroups x 4 waves x 8 independent chains x "
                             f"{iters} rounds, register operands only"}
    # vector-ALU work beside matrix-core work: 8 int8 MFMA chains per wave,
    # 4 independent f32 FMAs after each MFMA, 2 waves per SIMD (the batched
    # products' occupancy); each kind alone, then both
    wg_mv, it_mv = 1024, 200
    sink = torch.empty(wg_mv * 512, dtype=torch.float32, device=dev)
    mv = {}
    for key, mf, nf in (("mfma", 1, 0), ("fma", 0, 4), ("both", 1, 4)):
        qg.qg_probe_mfma_valu(mf, nf, it_mv, wg_mv, 2, sink)
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        qg.qg_probe_mfma_valu(mf, nf, it_mv, wg_mv, 2, sink)
        b.record(stream)
        torch.cuda.synchronize()
        mv[key] = a.elapsed_time(b) * 1e3
    lo, hi = min(mv["mfma"], mv["fma"]), max(mv["mfma"], mv["fma"])
    out["mfma_valu"] = {"us_mfma_alone": round(mv["mfma"], 1), "us_fma_alone": round(mv["fma"], 1),
                        "us_both": round(mv["both"], 1),
                        "added_frac": round((mv["both"] - hi) / lo, 3),
                        "note": "qg_probe_mfma_valu: 8 int8 16x16x64 MFMA chains per wave, 4 independent f32 FMAs "
                                "after each MFMA, 2 waves per SIMD; added_frac 0: the faster kind hides behind the "
                                "slower, 1: their times add"}
    # LDS read rate: 16-byte reads, one workgroup of 16 waves per CU
    it_l, waves_l = 2000, 16
    sink_i = torch.empty(256 * 64 * waves_l, dtype=torch.int32, device=dev)
    qg.qg_probe_lds_read(16, it_l, 256, waves_l, sink_i)
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    qg.qg_probe_lds_read(16, it_l, 256, waves_l, sink_i)
    b.record(stream)
    torch.cuda.synchronize()
    us_l = a.elapsed_time(b) * 1e3
    per_cu = it_l * 8 * 64 * 16 * waves_l
    out["lds_read"] = {"GB/s_per_CU": round(per_cu / us_l / 1e3, 1), "us": round(us_l, 1),
                       "note": "qg_probe_lds_read: 16-byte conflict-free LDS reads, 16 waves on each of 256 CUs"}
    out["wall_clock_kHz"] = khz
    return out


def ffn_timeline(qg, torch, dev, W, Wdn, L4, xs4_d, y4, ws4, S_dn, capture, log, reps=8):
    """Where the fused decode FFN's microseconds go: the gate|up launch (RMSNorm
    + quantiser, SiLU gate, tile maxima) and the down launch (quantiser on its
    split of t, split-K reduce, residual), each workgroup stamping the device
    wall clock at its start, after its prologue, when its tile result is
    summed over its waves, and at its exit.  Timed inside a graph right after
    the lm_head, so the weights come from HBM as in the decode step."""
    import numpy as np

    khz = qg.qg_probe_wall_clock_khz()
    Wg, Wu = W["q2_g128_gate_17408x5120"], W["q2_g128_up_17408x5120"]
    F, D = Wg.M, Wg.K
    rng = np.random.Generator(np.random.PCG64(20260 + 901))
    h = torch.from_numpy(rng.standard_normal(D, dtype=np.float32)).to(dev)
    nw = torch.from_numpy((1.0 + 0.1 * rng.standard_normal(D)).astype(np.float32)).to(dev)
    t = torch.empty(F, dtype=torch.float32, device=dev)
    tmax = torch.empty((F + 63) // 64, dtype=torch.float32, device=dev)
    hout = torch.empty(D, dtype=torch.float32, device=dev)
    ws_g = qg.qgemv_q2_gate_up_glu_x_workspace(F, dev)
    ws_d = qg.qgemv_q2_x_workspace(Wdn.M, Wdn.K, Wdn.group, S_dn, dev)
    n_g = 2 * ((F + 63) // 64)
    n_d = ((Wdn.M + 63) // 64) * S_dn
    st_g = torch.zeros(4 * n_g, dtype=torch.int64, device=dev)
    st_d = torch.zeros(4 * n_d, dtype=torch.int64, device=dev)

    def fn():
        L4.gemv_balanced(xs4_d, y4, ws4)
        qg.qg_probe_q2_gate_up_glu_x_stamped(Wg, Wu, h, qg.QG_GLU_SILU, t, ws_g, st_g, norm_w=nw, eps=1e-6,
                                             tmax=tmax)
        qg.qg_probe_q2_x_stamped(Wdn, t, hout, st_d, accum=h, ws=ws_d, split_k=S_dn, xmax=tmax)

    g = capture(fn)
    runs = []
    for _ in range(reps):
        g.replay()
        torch.cuda.synchronize()
        runs.append((st_g.cpu().numpy().reshape(-1, 4).astype(np.float64),
                     st_d.cpu().numpy().reshape(-1, 4).astype(np.float64)))
    us = 1e3 / khz  # microseconds per tick

    def kernel_stats(a, t0):
        a = (a - t0) * us
        q = lambda v, p: round(float(np.percentile(v, p)), 2)
        return {"workgroups": int(a.shape[0]),
                "start_us": {"first": q(a[:, 0], 0), "median": q(a[:, 0], 50), "last": q(a[:, 0], 100)},
                "prologue_us": {"median": q(a[:, 1] - a[:, 0], 50), "max": q(a[:, 1] - a[:, 0], 100)},
                "tile_result_us": {"median": q(a[:, 2] - a[:, 0], 50), "max": q(a[:, 2] - a[:, 0], 100),
                                   "last_at": q(a[:, 2], 100)},
                "exit_last_at_us": q(a[:, 3], 100),
                "span_us": round(float(a[:, 3].max() - a[:, 0].min()), 2)}

    out = {}
    spans = []
    for i, (a, b) in enumerate(runs[2:]):  # the first replays warm the clock
        t0 = a[:, 0].min()
        kg, kd = kernel_stats(a, t0), kernel_stats(b, t0)
        gap = round(float((b[:, 0].min() - a[:, 3].max()) * us), 2)
        spans.append((kg["span_us"], kd["span_us"], gap))
        out = {"gate_up_glu_x": kg, "down_x": kd, "gap_between_us": gap}
    sp = np.array(spans)
    out["replays"] = len(spans)
    out["span_us_median"] = {"gate_up_glu_x": round(float(np.median(sp[:, 0])), 2),
                             "down_x": round(float(np.median(sp[:, 1])), 2),
                             "gap_between": round(float(np.median(sp[:, 2])), 2)}
    out["note"] = ("device wall clock (s_memrealtime) per workgroup, relative to the first gate|up workgroup's "
                   "start, last replay shown in full; spans are first start to last exit of each launch")
    log(f"FFN timeline: {out}")
    return out


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_oracle_baseline(oracle, synth, host, q4, rs4, xs4, x_gu, x_dn, step_bytes, log):
    """The fp64 C oracle on this host: whole decode steps with the rows of
    each matrix spread over the host threads this process may use (at most
    16, the host share of one GPU), plus each workload on one thread, and a
    sample of the batched GEMM's outputs.  A baseline, not a target."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    threads = max(1, min(16, avail))
    names = ("q2_g128_gate_17408x5120", "q2_g128_up_17408x5120", "q2_g128_down_5120x17408")
    cfg = {n: synth.CONFIGS[n] for n in names}

    def chunks(M):
        cuts = np.linspace(0, M, threads + 1).astype(np.int64)
        return [np.arange(a, b, dtype=np.int64) for a, b in zip(cuts[:-1], cuts[1:]) if b > a]

    pool = ThreadPoolExecutor(max_workers=threads)

    def oracle_step():  # the ctypes calls release the interpreter lock: one row range per thread
        rq, rsc, _ = oracle.act_quant_i8(x_gu)
        rd, rdsc, _ = oracle.act_quant_i8(x_dn)
        jobs = []
        for n in names:
            c = cfg[n]
            xq, sc = (rd, rdsc) if n.startswith("q2_g128_down") else (rq, rsc)
            for r in chunks(c["M"]):
                jobs.append(pool.submit(oracle.q2_gemv, host[n][0], c["M"], c["K"], c["group"], xq, sc, r))
        for r in chunks(q4.shape[0]):
            jobs.append(pool.submit(oracle.q8row_gemv, q4, rs4, xs4, r))
        for j in jobs:
            j.result()

    c0 = time.perf_counter()
    passes = 0
    while passes == 0 or time.perf_counter() - c0 < 10.0:
        oracle_step()
        passes += 1
    cpu_s = (time.perf_counter() - c0) / passes
    pool.shutdown()

    def timed(fn, budget=1.0):
        t0 = time.perf_counter()
        n = 0
        while n == 0 or time.perf_counter() - t0 < budget:
            fn()
            n += 1
        return (time.perf_counter() - t0) / n

    single = {}
    q1, rs1, xs1 = synth.config_inputs("q8row_256x512")
    s1 = timed(lambda: oracle.q8row_gemv(q1, rs1, xs1), 0.5)
    single["q8row_256x512"] = {"ms": round(s1 * 1e3, 4), "GB/s": round(q1.shape[0] * (q1.shape[1] + 4) / s1 / 1e9, 3)}
    b2, x2 = synth.config_inputs("q2_g64_4096x4096")
    s2 = timed(lambda: oracle.q2_gemv(b2, 4096, 4096, 64, *oracle.act_quant_i8(x2)[:2]), 1.0)
    single["q2_g64_4096x4096"] = {"ms": round(s2 * 1e3, 3), "GB/s": round(4096 * 64 * 18 / s2 / 1e9, 3)}
    for n in names:
        c = cfg[n]
        x = x_dn if n.startswith("q2_g128_down") else x_gu
        s3 = timed(lambda: oracle.q2_gemv(host[n][0], c["M"], c["K"], c["group"], *oracle.act_quant_i8(x)[:2]), 1.0)
        single[n] = {"ms": round(s3 * 1e3, 2),
                     "GB/s": round(c["M"] * (c["K"] // c["group"]) * (2 + c["group"] // 4) / s3 / 1e9, 3)}
    # the lm_head and the batched GEMM on samples of their rows / outputs
    rows4 = np.arange(0, q4.shape[0], 64, dtype=np.int64)
    s4 = timed(lambda: oracle.q8row_gemv(q4, rs4, xs4, rows4), 0.5)
    single["q8row_lm_head_248320x5120"] = {
        "ms_extrapolated": round(s4 * q4.shape[0] / rows4.size * 1e3, 1),
        "GB/s": round(rows4.size * (q4.shape[1] + 4) / s4 / 1e9, 3), "sample": f"{rows4.size} rows (every 64th)"}
    c5 = synth.CONFIGS["q8row_gemm_512x17408x5120"]
    rng = np.random.Generator(np.random.PCG64(20260 + 970))
    q5 = rng.integers(-127, 128, size=(256, c5["K"]), dtype=np.int8)
    rs5 = rng.uniform(0.001, 0.01, 256).astype(np.float32)
    xs5 = rng.standard_normal((64, c5["K"]), dtype=np.float32)
    bs = np.repeat(np.arange(64, dtype=np.int64), 256)
    os_ = np.tile(np.arange(256, dtype=np.int64), 64)
    s5 = timed(lambda: oracle.q8row_gemm(q5, rs5, xs5, entries=(bs, os_)), 0.5)
    gflops = 2 * bs.size * c5["K"] / s5 / 1e9
    single["q8row_gemm_512x17408x5120"] = {
        "GFLOP/s": round(gflops, 3),
        "s_extrapolated": round(2 * c5["nb"] * c5["M"] * c5["K"] / (gflops * 1e9), 1),
        "sample": "64 x 256 outputs of the same K (random rows of the workload's distributions)"}
    cpu = {"value": round(step_bytes / cpu_s / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "seconds_per_step": round(cpu_s, 4), "passes": passes,
           "sample": f"{passes} whole decode steps (all six kernels' work) by the fp64 C oracle, the rows of "
                     f"each matrix split over {threads} host threads, mean per step",
           "host_cpus_visible": avail, "os_cpu_count": os.cpu_count(), "cpu_model": _cpu_model(),
           "single_thread": single}
    log(f"cpu oracle: {cpu}")
    return cpu


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(row sharding across GPUs is a design note, not built)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import weight_quantized_decode_q8_amd as qg

    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    dev = "cuda:0"
    torch.cuda.set_device(0)

    # ---------------- inputs (seeded, synthetic; shapes of the pages' model)
    t0 = time.time()
    host = {}
    for name in ("q2_g128_gate_17408x5120", "q2_g128_up_17408x5120", "q2_g128_down_5120x17408"):
        host[name] = synth.config_inputs(name)
    q4, rs4, xs4 = synth.config_inputs("q8row_lm_head_248320x5120")
    x_dn = host["q2_g128_down_5120x17408"][1]
    x_gu = host["q2_g128_gate_17408x5120"][1]
    log(f"inputs generated in {time.time() - t0:.1f}s")

    W = {}
    for name in ("q2_g128_gate_17408x5120", "q2_g128_up_17408x5120", "q2_g128_down_5120x17408"):
        c = synth.CONFIGS[name]
        W[name] = qg.Q2Weight.from_blocks(host[name][0], c["M"], c["K"], c["group"], dev)
    L4 = qg.Q8RowWeight.from_host(q4, rs4, dev)
    M4, K4 = q4.shape
    xs4_d = torch.from_numpy(xs4).to(dev)
    xgu_d = torch.from_numpy(x_gu).to(dev)
    xdn_d = torch.from_numpy(x_dn).to(dev)
    Kgu, Kdn = x_gu.size, x_dn.size
    xq_gu = torch.empty(Kgu, dtype=torch.int8, device=dev)
    xq_dn = torch.empty(Kdn, dtype=torch.int8, device=dev)
    sc_gu = torch.empty(1, dtype=torch.float32, device=dev)
    sc_dn = torch.empty(1, dtype=torch.float32, device=dev)
    su_gu = torch.empty(Kgu // 64, dtype=torch.int32, device=dev)
    su_dn = torch.empty(Kdn // 64, dtype=torch.int32, device=dev)
    y = {n: torch.empty(W[n].M, dtype=torch.float32, device=dev) for n in W}
    y4 = torch.empty(M4, dtype=torch.float32, device=dev)
    ws = {n: torch.zeros(max(1, qg.qgemv_q2_ws_bytes(W[n].M, W[n].K, W[n].group, 0)),
                         dtype=torch.uint8, device=dev) for n in W}
    log(f"inputs resident in HBM after {time.time() - t0:.1f}s")

    def k_quant_gu():
        qg.qquant_act_i8(xgu_d, xq_gu, sc_gu, su_gu)

    def k_quant_dn():
        qg.qquant_act_i8(xdn_d, xq_dn, sc_dn, su_dn)

    def k_gate():
        qg.qgemv_q2(W["q2_g128_gate_17408x5120"], xq_gu, su_gu, sc_gu, y["q2_g128_gate_17408x5120"], ws["q2_g128_gate_17408x5120"])

    def k_up():
        qg.qgemv_q2(W["q2_g128_up_17408x5120"], xq_gu, su_gu, sc_gu, y["q2_g128_up_17408x5120"], ws["q2_g128_up_17408x5120"])

    Mgu_ = W["q2_g128_gate_17408x5120"].M
    ws_pair = torch.zeros(max(1, qg.qgemv_q2_dual_ws_bytes(Mgu_, Kgu, W["q2_g128_gate_17408x5120"].group, 0)),
                          dtype=torch.uint8, device=dev)

    def k_gate_up():
        qg.qgemv_q2_dual(W["q2_g128_gate_17408x5120"], W["q2_g128_up_17408x5120"], xq_gu, su_gu, sc_gu, y["q2_g128_gate_17408x5120"], y["q2_g128_up_17408x5120"], ws_pair)

    Wdn = W["q2_g128_down_5120x17408"]
    # the down projection's split: the in-launch form's automatic choice
    # (its partials are added inside the launch); the six-launch form is run
    # with the same split so that the two give the same bits
    S_dn = args.down_split or qg.qgemv_q2_x_auto_split(Wdn.M, Wdn.K, Wdn.group)
    ws_dn6 = torch.zeros(max(1, qg.qgemv_q2_ws_bytes(Wdn.M, Wdn.K, Wdn.group, S_dn)), dtype=torch.uint8, device=dev)
    ws_dnx = qg.qgemv_q2_x_workspace(Wdn.M, Wdn.K, Wdn.group, S_dn, dev)

    def k_down():
        qg.qgemv_q2(Wdn, xq_dn, su_dn, sc_dn, y["q2_g128_down_5120x17408"], ws_dn6, S_dn)

    def k_gate_up_x():  # the activation quantiser inside the pair launch
        qg.qgemv_q2_dual_x(W["q2_g128_gate_17408x5120"], W["q2_g128_up_17408x5120"], xgu_d,
                           y["q2_g128_gate_17408x5120"], y["q2_g128_up_17408x5120"])

    def k_down_x():  # quantiser and split-K reduce inside the launch
        qg.qgemv_q2_x(Wdn, xdn_d, y["q2_g128_down_5120x17408"], ws=ws_dnx, split_k=S_dn)

    # the lm_head's last partial round of row tiles (3880 = 15 x 256 + 40)
    # split along K over the whole GPU (qgemv_q8row_balanced)
    ws4 = L4.workspace(dev)

    def k_lm_head():
        L4.gemv_balanced(xs4_d, y4, ws4)

    def k_lm_head_plain():
        L4.gemv(xs4_d, y4)

    def step6():  # the same step as six launches: quantisers and the split reduce on their own
        k_quant_gu()
        k_gate_up()
        k_quant_dn()
        k_down()
        k_lm_head()

    def step():
        k_gate_up_x()
        k_down_x()
        k_lm_head()

    q2_bytes = {n: W[n].M * (W[n].K // W[n].group) * (2 + W[n].group // 4) for n in W}
    lm_bytes = M4 * (K4 + 4)
    step_bytes = sum(q2_bytes.values()) + lm_bytes

    # ---------------- eager reference run, then graph capture; the pair
    # launch must give the two single GEMVs' outputs bit for bit
    k_quant_gu()
    k_gate()
    k_up()
    torch.cuda.synchronize()
    single = {n: y[n].clone() for n in ("q2_g128_gate_17408x5120", "q2_g128_up_17408x5120")}
    step6()
    torch.cuda.synchronize()
    for n in single:
        assert torch.equal(y[n], single[n]), f"the pair launch's {n} output differs from the single GEMV"
    ref = {n: y[n].clone() for n in y}
    for n in y:
        y[n].fill_(float("nan"))
    step()
    torch.cuda.synchronize()
    for n in y:
        assert torch.equal(y[n], ref[n]), f"the three-launch step's {n} output differs from the six-launch step"
    ref4 = y4.clone()

    def capture(fn, n=1):
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            fn()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(n):
                fn()
        return g

    g_step = capture(step)
    for _ in range(3):
        g_step.replay()
        torch.cuda.synchronize()
        for n in y:
            assert torch.equal(y[n], ref[n]), f"graph replay of {n} differs from eager"
        assert torch.equal(y4, ref4), "graph replay of lm_head differs from eager"

    # ---------------- timed region: K steps, captured back to back in one
    # graph (as a model's decode graph holds its layers' launches back to
    # back); every step streams all its weights again.  A graph launch ends
    # with a release to the host and the next one starts with an acquire, a
    # few microseconds per launch: the same K steps as K launches of a
    # one-step graph are timed beside it.
    stream = torch.cuda.current_stream()
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)

    def time_graph(g_warm, g_main, per_replay_steps=None):
        """Microseconds per step: warmup graph, then the timed graph between
        events (per_replay_steps: the one-step graph replayed that many times)."""
        nonlocal_wall[0] = 0.0
        if g_warm is not None:
            g_warm.replay()
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        ev0.record(stream)
        if per_replay_steps is None:
            g_main.replay()
        else:
            for _ in range(per_replay_steps):
                g_main.replay()
        ev1.record(stream)
        torch.cuda.synchronize()
        nonlocal_wall[0] = time.perf_counter() - w0
        return ev0.elapsed_time(ev1) * 1e3 / args.steps

    nonlocal_wall = [0.0]
    g_steps = capture(step, args.steps)
    g_warm = capture(step, args.warmup) if args.warmup > 0 else None
    us_main = time_graph(g_warm, g_steps)
    wall = nonlocal_wall[0]
    for n in y:
        assert torch.equal(y[n], ref[n]), f"the {args.steps}-step graph's {n} differs from eager"
    assert torch.equal(y4, ref4), "the K-step graph's lm_head differs from eager"
    ms_per_step = us_main / 1e3
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    us_one_step_graphs = time_graph(None, g_step, args.steps)
    log(f"step {us_main:.1f} us, {value:.0f} GB/s (wall {wall * 1e6 / args.steps:.1f} us/step); "
        f"as {args.steps} one-step graph launches {us_one_step_graphs:.1f} us")
    del g_warm

    # the same step as six launches, timed the same way (context)
    g_step6 = capture(step6)
    for _ in range(3):
        g_step6.replay()
        torch.cuda.synchronize()
        for n in y:
            assert torch.equal(y[n], ref[n]), f"graph replay of the six-launch step's {n} differs"
    g_steps6 = capture(step6, args.steps)
    us_step6 = time_graph(None, g_steps6)
    del g_steps6
    log(f"six-launch step {us_step6:.1f} us")

    # ---------------- per-kernel times (graph of n back-to-back launches)
    def kernel_us(fn, n):
        g = capture(fn, n)
        g.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        reps = 5
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (reps * n)

    # The prefill products are MFMA work whose shader clock takes several
    # milliseconds of continuous load to settle: time them after replaying
    # the graph for at least warm_ms, and keep the figure right after capture
    # ("cold") beside it.
    def steady_us(fn, n, reps=5, warm_ms=60.0):
        g = capture(fn, n)
        g.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)

        def timed():
            a.record(stream)
            for _ in range(reps):
                g.replay()
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b)

        cold_ms = timed()
        spent = cold_ms
        while spent < warm_ms:
            spent += timed()
        return timed() * 1e3 / (reps * n), cold_ms * 1e3 / (reps * n)

    # the two small workloads: the 256 x 512 q8_row GEMV and the 4096 x 4096
    # g64 Q2 GEMV (with its quantiser), each back to back in a graph
    small = []
    if not args.no_breakdown:
        q1, rs1, xs1 = synth.config_inputs("q8row_256x512")
        W1 = qg.Q8RowWeight.from_host(q1, rs1, dev)
        xs1_d = torch.from_numpy(xs1).to(dev)
        y1 = torch.empty(q1.shape[0], dtype=torch.float32, device=dev)
        c2 = synth.CONFIGS["q2_g64_4096x4096"]
        b2s, x2s = synth.config_inputs("q2_g64_4096x4096")
        W2s = qg.Q2Weight.from_blocks(b2s, c2["M"], c2["K"], c2["group"], dev)
        x2s_d = torch.from_numpy(x2s).to(dev)
        xq2s = torch.empty(c2["K"], dtype=torch.int8, device=dev)
        sc2s = torch.empty(1, dtype=torch.float32, device=dev)
        su2s = torch.empty(c2["K"] // 64, dtype=torch.int32, device=dev)
        y2s = torch.empty(c2["M"], dtype=torch.float32, device=dev)
        qg.qquant_act_i8(x2s_d, xq2s, sc2s, su2s)
        ws2s_x = qg.qgemv_q2_x_workspace(c2["M"], c2["K"], c2["group"], 0, dev)
        small = [("q8row_256x512", lambda: W1.gemv(xs1_d, y1), q1.shape[0] * (q1.shape[1] + 4), 50),
                 ("q2_4096x4096_g64", lambda: qg.qgemv_q2(W2s, xq2s, su2s, sc2s, y2s), 4096 * 64 * 18, 50),
                 ("q2_4096x4096_g64_x", lambda: qg.qgemv_q2_x(W2s, x2s_d, y2s, ws=ws2s_x, split_k=0),
                  4096 * 64 * 18, 50),
                 ("act_quant_K4096", lambda: qg.qquant_act_i8(x2s_d, xq2s, sc2s, su2s), None, 50)]
        # the column prescale act = silu(g) u col at the down projection's K
        gp, up_, cp = (torch.from_numpy(a).to(dev) for a in synth.gate_inputs(1, 17408, seed=20260 + 960))
        actp = torch.empty_like(gp)
        small.append(("silu_mul_pre_K17408", lambda: qg.qact_silu_mul_pre(gp, up_, cp, actp), None, 50))

    kernels = {}
    for name, fn, nbytes, n in small + ([] if args.no_breakdown else [("act_quant_K5120", k_quant_gu, None, 50),
                                ("q2_gate_17408x5120_g128", k_gate, q2_bytes["q2_g128_gate_17408x5120"], 20),
                                ("q2_up_17408x5120_g128", k_up, q2_bytes["q2_g128_up_17408x5120"], 20),
                                ("q2_gate_up_pair_2x17408x5120_g128", k_gate_up,
                                 q2_bytes["q2_g128_gate_17408x5120"] + q2_bytes["q2_g128_up_17408x5120"], 20),
                                ("act_quant_K17408", k_quant_dn, None, 50),
                                ("q2_down_5120x17408_g128", k_down, q2_bytes["q2_g128_down_5120x17408"], 20),
                                ("q2_gate_up_pair_x_2x17408x5120_g128", k_gate_up_x,
                                 q2_bytes["q2_g128_gate_17408x5120"] + q2_bytes["q2_g128_up_17408x5120"], 20),
                                ("q2_down_x_5120x17408_g128", k_down_x, q2_bytes["q2_g128_down_5120x17408"], 20),
                                ("q8row_lm_head_248320x5120", k_lm_head, lm_bytes, 10),
                                ("q8row_lm_head_248320x5120_plain_launch", k_lm_head_plain, lm_bytes, 10)]):
        us = kernel_us(fn, n)
        ent = {"us": round(us, 3)}
        if nbytes:
            gbs = nbytes / us / 1e3
            ent.update({"weight_bytes": nbytes, "GB/s": round(gbs, 1),
                        "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)})
        if nbytes and nbytes < (64 << 20):
            ent["note"] = "back-to-back calls: weights cache-resident, launch-bound"
        kernels[name] = ent
        log(f"  {name}: {ent}")

    # ---------------- dominant kernel roofline: HIP events on its stream
    n_dom = 20
    k_lm_head()
    torch.cuda.synchronize()
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(n_dom):
        k_lm_head()
    b.record(stream)
    torch.cuda.synchronize()
    dom_us = a.elapsed_time(b) * 1e3 / n_dom
    achieved = lm_bytes / dom_us / 1e3
    roofline = {"bound": "hbm", "kernel": "q8row_gemv_t64 (lm_head 248320x5120, balanced launch)",
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": read_traffic(),
                "avg_launch_us": round(dom_us, 2), "algorithmic_bytes_per_launch": lm_bytes}

    timeline = None
    if not args.no_breakdown or args.timeline_only:
        timeline = ffn_timeline(qg, torch, dev, W, Wdn, L4, xs4_d, y4, ws4, S_dn, capture, log)
    if args.timeline_only:
        print(json.dumps({"ffn_timeline": timeline}), flush=True)
        return

    # ---------------- fused FFN block: the same three matrices with the fused
    # producers, gate and up in one launch and the residual in the down
    # projection's epilogue
    fused = None
    if not args.no_breakdown:
        rng = np.random.Generator(np.random.PCG64(20260 + 900))
        h_d = torch.from_numpy(rng.standard_normal(Kgu, dtype=np.float32)).to(dev)
        nw_d = torch.from_numpy((1.0 + 0.1 * rng.standard_normal(Kgu)).astype(np.float32)).to(dev)
        h_out = torch.empty(Kgu, dtype=torch.float32, device=dev)
        Mgu = W["q2_g128_gate_17408x5120"].M
        ws_gu = torch.zeros(max(1, qg.qgemv_q2_dual_ws_bytes(Mgu, Kgu, 128, 0)), dtype=torch.uint8, device=dev)
        g_buf = torch.empty(Mgu, dtype=torch.float32, device=dev)
        u_buf = torch.empty(Mgu, dtype=torch.float32, device=dev)

        Wg_, Wu_ = W["q2_g128_gate_17408x5120"], W["q2_g128_up_17408x5120"]
        ws_glu = qg.qgemv_q2_gate_up_glu_x_workspace(Mgu, dev)
        tmax_d = torch.empty((Mgu + 63) // 64, dtype=torch.float32, device=dev)

        def ffn_x():  # two launches: the producers and the split reduce inside the GEMV launches;
            # the gate|up launch hands max|t| per row tile to the down launch, whose
            # workgroups then read only their own split of t
            qg.qgemv_q2_gate_up_glu_x(Wg_, Wu_, h_d, qg.QG_GLU_SILU, g_buf, ws_glu, norm_w=nw_d, eps=1e-6,
                                      tmax=tmax_d)
            qg.qgemv_q2_x(Wdn, g_buf, h_out, accum=h_d, ws=ws_dnx, split_k=S_dn, xmax=tmax_d)

        def ffn_x_whole_max():  # the same, each down workgroup finding max|t| over all of t
            qg.qgemv_q2_gate_up_glu_x(Wg_, Wu_, h_d, qg.QG_GLU_SILU, g_buf, ws_glu, norm_w=nw_d, eps=1e-6)
            qg.qgemv_q2_x(Wdn, g_buf, h_out, accum=h_d, ws=ws_dnx, split_k=S_dn)

        def ffn_fused():  # five launches: the fused producers as launches of their own
            qg.qquant_rmsnorm_i8(h_d, nw_d, 1e-6, xq_gu, sc_gu, su_gu)
            qg.qgemv_q2_gate_up_glu(Wg_, Wu_, xq_gu, su_gu, sc_gu, qg.QG_GLU_SILU, g_buf, xq_dn, sc_dn, su_dn)
            qg.qgemv_q2_accum(Wdn, xq_dn, su_dn, sc_dn, h_d, h_out, ws_dn6, S_dn)

        def ffn_dual_then_glu():  # the gated product as its own launches too
            qg.qquant_rmsnorm_i8(h_d, nw_d, 1e-6, xq_gu, sc_gu, su_gu)
            qg.qgemv_q2_dual(Wg_, Wu_, xq_gu, su_gu, sc_gu, g_buf, u_buf, ws_gu)
            qg.qquant_glu_i8(g_buf, u_buf, qg.QG_GLU_SILU, g_buf, xq_dn, sc_dn, su_dn)
            qg.qgemv_q2_accum(Wdn, xq_dn, su_dn, sc_dn, h_d, h_out, ws_dn6, S_dn)

        def timed_step(ffn):
            def fn():
                ffn()
                k_lm_head()
            h_out.fill_(float("nan"))
            fn()
            torch.cuda.synchronize()
            if ref_h is not None:
                assert torch.equal(h_out, ref_h), f"{ffn.__name__} differs from the other FFN forms"
            g = capture(fn, 1)
            for _ in range(3):
                g.replay()
                torch.cuda.synchronize()
                assert torch.equal(h_out, ref_h if ref_h is not None else h_out), "graph replay differs from eager"
            gk = capture(fn, args.steps)
            us = time_graph(g, gk)
            assert torch.equal(h_out, ref_h if ref_h is not None else h_out), "the K-step graph differs from eager"
            del gk
            return us

        ref_h = None
        ffn_fused()
        torch.cuda.synchronize()
        ref_h = h_out.clone()
        # the forms measured in turn, three rounds, median per form (the clock drifts
        # by a microsecond or two over a run)
        rounds = {f: [] for f in (ffn_x, ffn_x_whole_max, ffn_fused, ffn_dual_then_glu)}
        for _ in range(3):
            for f in rounds:
                rounds[f].append(timed_step(f))
        med = {f: sorted(v)[1] for f, v in rounds.items()}
        us_x, us_xw, us_fs, us_dg = med[ffn_x], med[ffn_x_whole_max], med[ffn_fused], med[ffn_dual_then_glu]
        fused = {"workload": "decode step with the FFN block fused: RMSNorm+quant -> gate|up Q2 GEMV with the "
                             "SiLU gate in its epilogue -> quant -> down Q2 GEMV + residual, then the q8_row lm_head",
                 "us_per_step": round(us_x, 2), "GB/s": round(step_bytes / us_x / 1e3, 1),
                 "frac_hbm_peak": round(step_bytes / us_x / 1e3 / HBM_PEAK_GBS, 4),
                 "launches": 3,
                 "form": "qgemv_q2_gate_up_glu_x (RMSNorm + quantiser in the launch, g and u meeting in a "
                         "workspace, max|t| per row tile out) -> qgemv_q2_x (the quantiser on its split of t with "
                         "the tiles' max, split-K reduce and residual in the launch) -> lm_head",
                 "whole_vector_max_us_per_step": round(us_xw, 2),
                 "producers_as_launches_us_per_step": round(us_fs, 2), "producers_as_launches_launches": 6,
                 "gated_product_as_own_launches_us_per_step": round(us_dg, 2),
                 "main_step_us_per_step": round(ms_per_step * 1e3, 2), "main_step_launches": 3,
                 "step_weight_bytes": step_bytes,
                 "note": "timed like the main step (graph replays, the lm_head evicting the last-level cache); "
                         "all forms give the same bits"}
        log(f"fused FFN: {fused}")

    # ---------------- Q2 GEMV streaming rate from HBM: copies of one matrix
    # (>= 512 MB, twice the last-level cache) launched back to back in one
    # graph, each launch reading weights no earlier launch left in cache
    sustained = None
    if not args.no_breakdown:
        sustained = {}
        xs_by_k = {Kgu: (xq_gu, su_gu, sc_gu), Kdn: (xq_dn, su_dn, sc_dn)}
        c2 = synth.CONFIGS["q2_g64_4096x4096"]
        b2, x2 = synth.config_inputs("q2_g64_4096x4096")
        W2 = qg.Q2Weight.from_blocks(b2, c2["M"], c2["K"], c2["group"], dev)
        xq2 = torch.empty(c2["K"], dtype=torch.int8, device=dev)
        sc2 = torch.empty(1, dtype=torch.float32, device=dev)
        su2 = torch.empty(c2["K"] // 64, dtype=torch.int32, device=dev)
        qg.qquant_act_i8(torch.from_numpy(x2).to(dev), xq2, sc2, su2)
        xs_by_k[c2["K"]] = (xq2, su2, sc2)
        for label, W0, mode in [("Q2 g64 4096x4096", W2, "single"),
                                ("Q2 g64 4096x4096, 16 per launch", W2, "batch"),
                                ("gate Q2 g128 17408x5120", W["q2_g128_gate_17408x5120"], "single"),
                                ("gate|up dual Q2 g128 2x17408x5120", W["q2_g128_gate_17408x5120"], "dual"),
                                ("gate Q2 g128 17408x5120, 16 per launch", W["q2_g128_gate_17408x5120"], "batch"),
                                ("down Q2 g128 5120x17408", W["q2_g128_down_5120x17408"], "single"),
                                ("down Q2 g128 5120x17408, 16 per launch", W["q2_g128_down_5120x17408"], "batch")]:
            dual = mode == "dual"
            nb_w = W0.M * (W0.K // W0.group) * (2 + W0.group // 4)
            ncopy = max(2, -(-(512 << 20) // nb_w))
            ncopy += ncopy % 2
            if mode == "batch":  # whole launches of 16: a launch of fewer matrices streams slower
                ncopy = -(-ncopy // qg.QG_Q2_BATCH_MAX) * qg.QG_Q2_BATCH_MAX
            copies = [W0] + [qg.Q2Weight(W0.codes.clone(), W0.scales.clone(), W0.M, W0.K, W0.group)
                             for _ in range(ncopy - 1)]
            xq_c, su_c, sc_c = xs_by_k[W0.K]
            outs = [torch.empty(W0.M, dtype=torch.float32, device=dev) for _ in range(ncopy)]
            nws = (qg.qgemv_q2_dual_ws_bytes if dual else qg.qgemv_q2_ws_bytes)(W0.M, W0.K, W0.group, 0)
            ws_c = torch.zeros(max(1, nws), dtype=torch.uint8, device=dev)

            def rotate():
                if dual:
                    for i in range(0, ncopy, 2):
                        qg.qgemv_q2_dual(copies[i], copies[i + 1], xq_c, su_c, sc_c, outs[i], outs[i + 1], ws_c)
                elif mode == "batch":
                    for i in range(0, ncopy, qg.QG_Q2_BATCH_MAX):
                        qg.qgemv_q2_batch([(copies[k], xq_c, su_c, sc_c, outs[k])
                                           for k in range(i, min(ncopy, i + qg.QG_Q2_BATCH_MAX))])
                else:
                    for i in range(ncopy):
                        qg.qgemv_q2(copies[i], xq_c, su_c, sc_c, outs[i], ws_c)

            us = kernel_us(rotate, 1) / ncopy
            split = 1 if mode == "batch" else qg.qgemv_q2_auto_split(W0.M, W0.K, W0.group)
            launches = {"dual": ncopy // 2, "batch": -(-ncopy // qg.QG_Q2_BATCH_MAX)}.get(mode, ncopy)
            sustained[label] = {"us_per_matrix": round(us, 2), "GB/s": round(nb_w / us / 1e3, 1),
                                "frac_hbm_peak": round(nb_w / us / 1e3 / HBM_PEAK_GBS, 4),
                                "copies": ncopy, "weight_bytes": nb_w, "split_k": split,
                                "launches": launches}
            log(f"  sustained {label}: {sustained[label]}")
            del copies, outs
        del W2
        torch.cuda.empty_cache()

    if args.calib_copy:
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()

    # ---------------- prefill GEMM: y[b,o] = rs[o] sum_i q[o,i] xs[b,i]
    gemm = None
    if not args.no_gemm:
        del L4
        torch.cuda.empty_cache()
        c5 = synth.CONFIGS["q8row_gemm_512x17408x5120"]
        nb5, M5, K5 = c5["nb"], c5["M"], c5["K"]
        q5, rs5, xs5 = synth.config_inputs("q8row_gemm_512x17408x5120")
        W5 = qg.Q8RowWeight.from_host(q5, rs5, dev)
        del q5
        xs5_d = torch.from_numpy(xs5).to(dev)
        y5 = torch.empty((nb5, M5), dtype=torch.float32, device=dev)
        ws5 = torch.empty(qg.qgemm_q8row_batched_ws_bytes(nb5, K5), dtype=torch.uint8, device=dev)

        def k_gemm():
            qg.qgemm_q8row_batched(W5.packed, W5.rs, xs5_d, y5, nb5, M5, K5, ws5, xs_limbs=0)

        def k_gemm3():
            qg.qgemm_q8row_batched(W5.packed, W5.rs, xs5_d, y5, nb5, M5, K5, ws5, xs_limbs=3)

        k_gemm()
        # ten calls per graph, as the other prefill legs: the figure is the
        # call's own time, without a graph launch per call
        g_us, g_cold = steady_us(k_gemm, 10, reps=4)
        g3_us, _ = steady_us(k_gemm3, 10, reps=4)
        flop = 2 * nb5 * M5 * K5
        tflops = flop / g_us / 1e6
        gemm = {"workload": f"batched prefill q8_row GEMM nb={nb5} M={M5} K={K5} (xs limbs: auto)",
                "us": round(g_us, 2), "TFLOP/s": round(tflops, 1), "unit": "TFLOP/s",
                "algorithmic_flop": flop, "us_cold": round(g_cold, 2),
                "frac_fp16_dense_peak": round(tflops / FP16_DENSE_TFLOPS, 4),
                "frac_int8_dense_peak_hw": round(2 * tflops / INT8_DENSE_TOPS, 4),
                "note": "2 int8 limbs per activation on these N(0,1) rows: hardware int8 ops = 2x algorithmic",
                "accuracy": "auto picks 2 limbs here; the 2e-5 bound then rests on the rounding errors of "
                            "different elements cancelling, which holds for dense weight rows (the contract in "
                            "include/qgemv.h); with 3 limbs the bound is certain wherever condition (C) holds",
                "limbs3_us": round(g3_us, 2), "limbs3_TFLOP/s": round(flop / g3_us / 1e6, 1)}
        # The same product fed by the column prescale of the q8_row FFN: act =
        # silu(g) u col formed inside the product's prep, against the prescale
        # launch followed by the product.
        g5, u5, c5c = (torch.from_numpy(a).to(dev) for a in synth.gate_inputs(nb5, K5, seed=20260 + 961))
        act5 = torch.empty_like(g5)

        def k_gemm_silu():
            qg.qgemm_q8row_batched_silu(W5.packed, W5.rs, g5, u5, c5c, y5, nb5, M5, K5, ws5, xs_limbs=0)

        def k_two_step():
            qg.qact_silu_mul_pre(g5, u5, c5c, act5)
            qg.qgemm_q8row_batched(W5.packed, W5.rs, act5, y5, nb5, M5, K5, ws5, xs_limbs=0)

        us_f, _ = steady_us(k_gemm_silu, 10, reps=4)
        us_t, _ = steady_us(k_two_step, 10, reps=4)
        gemm["silu_fused"] = {"workload": f"the same product of act = silu(g) u col (g, u [{nb5}][{K5}])",
                              "us": round(us_f, 2), "TFLOP/s": round(flop / us_f / 1e6, 1),
                              "two_step_us": round(us_t, 2),
                              "note": "auto limbs pick the 24-bit (3-limb) form for most of these rows: a gated "
                                      "product's max/mean ratio per row is about 26 (N(0,1): about 5), beyond "
                                      "what 16-bit activations keep inside the bound"}
        del g5, u5, c5c, act5

        # Context, not this library's path: the vendor GEMMs on the same shape,
        # timed the same way -- hipBLASLt int8 with the same hardware int8 work
        # (17408 x 5120 by 5120 x 1024, i.e. two limbs of 512 rows) and torch's
        # fp16 matmul over the 512 rows (which would not meet the error bound).
        try:
            Wi = torch.randint(-127, 128, (M5, K5), dtype=torch.int8, device=dev)
            Xi = torch.randint(-127, 128, (2 * nb5, K5), dtype=torch.int8, device=dev).t()
            us_i8, _ = steady_us(lambda: torch._int_mm(Wi, Xi), 10, reps=2)
            Wh = Wi.to(torch.float16)
            Xh = torch.randn(nb5, K5, dtype=torch.float16, device=dev)
            us_h, _ = steady_us(lambda: torch.mm(Xh, Wh.t()), 10, reps=2)
            gemm["vendor_context"] = {
                "int8_mm_17408x5120x1024_us": round(us_i8, 2),
                "fp16_mm_512x5120x17408_us": round(us_h, 2),
                "note": "torch._int_mm (hipBLASLt) at this kernel's hardware int8 work; torch.mm in fp16 at the "
                        "same algorithmic work without the accuracy"}
            del Wi, Xi, Wh, Xh
        except RuntimeError as exc:  # an op missing from this torch build
            gemm["vendor_context"] = {"error": str(exc)[:120]}
        log(f"prefill GEMM: {gemm}")

    # ---------------- prefill Q2 product: 512 token rows through the FFN gate
    # matrix (17408 x 5120 g128): row-batched quantiser, then int8 MFMA
    q2gemm = None
    if not args.no_gemm:
        cg = synth.CONFIGS["q2_g128_gate_17408x5120"]
        Mg, Kg, Gg = cg["M"], cg["K"], cg["group"]
        nbq = 512
        Wq = W["q2_g128_gate_17408x5120"]
        Xq = torch.from_numpy(synth.rng_for(20260 + 950).standard_normal((nbq, Kg), dtype=np.float32)).to(dev)
        xq_r = torch.empty((nbq, Kg), dtype=torch.int8, device=dev)
        sc_r = torch.empty(nbq, dtype=torch.float32, device=dev)
        su_r = torch.empty((nbq, Kg // 64), dtype=torch.int32, device=dev)
        y_r = torch.empty((nbq, Mg), dtype=torch.float32, device=dev)
        nws_r = qg.qgemm_q2_batched_ws_bytes(Mg, Kg, Gg, nbq)
        ws_r = torch.empty(nws_r, dtype=torch.uint8, device=dev) if nws_r else None

        def k_quant_rows():
            qg.qquant_act_i8_rows(Xq, xq_r, sc_r, su_r)

        def k_q2gemm():
            qg.qgemm_q2_batched(Wq, xq_r, su_r, sc_r, y_r, ws=ws_r)

        k_quant_rows()
        us_g, us_g_cold = steady_us(k_q2gemm, 10)
        us_q = kernel_us(k_quant_rows, 10)
        flop = 2 * nbq * Mg * Kg
        tops = flop / us_g / 1e6
        q2gemm = {"workload": f"batched prefill Q2 g128 product nb={nbq} M={Mg} K={Kg} (int8 activations per token)",
                  "us": round(us_g, 2), "TOP/s": round(tops, 1), "unit": "TOP/s", "algorithmic_ops": flop,
                  "us_cold": round(us_g_cold, 2),
                  "frac_int8_dense_peak": round(tops / INT8_DENSE_TOPS, 4),
                  "frac_fp16_dense_peak": round(tops / FP16_DENSE_TFLOPS, 4),
                  "quant_rows_us": round(us_q, 2),
                  "note": "one int8 MFMA per 64-wide unit; per-group scaling in f32 on the vector ALUs"}
        log(f"prefill Q2 product: {q2gemm}")

        # the whole prefill FFN block over the same 512 tokens: RMSNorm+quant
        # rows -> gate, up products -> SiLU gate+quant rows -> down product
        # with the residual (as the qxmx page's ffn_forward_b)
        Wd = W["q2_g128_down_5120x17408"]
        Fd = Wd.K
        H = torch.from_numpy(synth.rng_for(20260 + 951).standard_normal((nbq, Kg), dtype=np.float32)).to(dev)
        Hout = torch.empty_like(H)
        nw = torch.from_numpy((1.0 + 0.1 * synth.rng_for(20260 + 952).standard_normal(Kg)).astype(np.float32)).to(dev)
        G = torch.empty((nbq, Fd), dtype=torch.float32, device=dev)
        U = torch.empty((nbq, Fd), dtype=torch.float32, device=dev)
        xq_f = torch.empty((nbq, Fd), dtype=torch.int8, device=dev)
        sc_f = torch.empty(nbq, dtype=torch.float32, device=dev)
        su_f = torch.empty((nbq, Fd // 64), dtype=torch.int32, device=dev)
        nws_d = qg.qgemm_q2_batched_ws_bytes(Wd.M, Wd.K, Wd.group, nbq)
        ws_d = torch.empty(nws_d, dtype=torch.uint8, device=dev) if nws_d else None

        nws_p = qg.qgemm_q2_batched_dual_ws_bytes(Mg, Kg, Gg, nbq)
        ws_p = torch.empty(nws_p, dtype=torch.uint8, device=dev) if nws_p else None

        def k_pair():
            qg.qgemm_q2_batched_dual(W["q2_g128_gate_17408x5120"], W["q2_g128_up_17408x5120"], xq_r, su_r, sc_r, G, U, ws=ws_p)

        def ffn_prefill():
            qg.qquant_rmsnorm_i8_rows(H, nw, 1e-6, xq_r, sc_r, su_r)
            qg.qgemm_q2_batched_dual(W["q2_g128_gate_17408x5120"], W["q2_g128_up_17408x5120"], xq_r, su_r, sc_r, G, U, ws=ws_p)
            qg.qquant_glu_i8_rows(G, U, qg.QG_GLU_SILU, G, xq_f, sc_f, su_f)
            qg.qgemm_q2_batched(Wd, xq_f, su_f, sc_f, Hout, accum=H, ws=ws_d)

        qg.qquant_rmsnorm_i8_rows(H, nw, 1e-6, xq_r, sc_r, su_r)
        us_pair, _ = steady_us(k_pair, 5)
        q2gemm["gate_up_pair_us"] = round(us_pair, 2)

        ffn_prefill()
        us_ffn, us_ffn_cold = steady_us(ffn_prefill, 5)
        ops3 = 3 * flop
        q2gemm["ffn_block"] = {
            "workload": f"prefill FFN block, {nbq} tokens: RMSNorm+quant rows -> gate|up pair -> SiLU gate+quant rows "
                        f"-> down + residual (Q2 g128 17408x5120 / 5120x17408)",
            "us": round(us_ffn, 2), "TOP/s": round(ops3 / us_ffn / 1e6, 1), "us_cold": round(us_ffn_cold, 2),
            "frac_int8_dense_peak": round(ops3 / us_ffn / 1e6 / INT8_DENSE_TOPS, 4)}
        log(f"prefill FFN block: {q2gemm['ffn_block']}")
        del Xq, xq_r, y_r, H, Hout, G, U, xq_f
        torch.cuda.empty_cache()

    # ---------------- achievable peaks of this GPU (measurement probes)
    achievable = None
    if not args.no_breakdown:
        achievable = measure_achievable(qg, torch, dev, stream, log)
        log(f"achievable: {achievable}")

    # ---------------- CPU oracle over the same step, on this host
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        cpu = cpu_oracle_baseline(oracle, synth, host, q4, rs4, xs4, x_gu, x_dn, step_bytes, log)

    out = {
        "metric": "batch-1 quantized GEMV weight GB/s (% of HBM peak); prefill GEMM TFLOP/s",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "frac_hbm_peak": round(value / HBM_PEAK_GBS, 4),
        "dtype": "f32",
        "dtype_detail": "q8_row: int8 weights x f32 activations, f32 accumulate; Q2: 2-bit codes x int8 "
                        "activations, exact int32 unit dots, f32 scale accumulate",
        "data": "synthetic",
        "config": {"workload": "decode_step_batch1: act-quant + Q2 g128 FFN (gate, up 17408x5120; "
                               "down 5120x17408) + q8_row lm_head 248320x5120",
                   "step_weight_bytes": step_bytes,
                   "graph": "hipGraph of three launches: gate|up pair with the act-quant in the launch "
                            "(qgemv_q2_dual_x), down with the act-quant and the split-K reduce in the launch "
                            "(qgemv_q2_x), lm_head (qgemv_q8row_balanced)",
                   "down_split_k": S_dn,
                   "timing": f"the {args.steps} timed steps captured back to back in one graph (a model's decode "
                             "graph holds its launches back to back); every step streams all its weights",
                   "one_step_graph_launches_us_per_step": round(us_one_step_graphs, 2),
                   "six_launch_form_us_per_step": round(us_step6, 2),
                   "six_launch_form": "act-quant, gate|up pair, act-quant, down partials, split-K reduce, "
                                      "lm_head (same bits)",
                   "parallelism": "single GPU"},
        "kernels": kernels,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "achievable": achievable,
        "context_pages": {
            "what": "the pages' own throughput figure for their Q2 GEMV (2-bit weights x int8 activations, "
                    "ESIMD/XMX DPAS, split-K) on an Intel Xe2 B70-class GPU: 240-468 GB/s of weight bytes "
                    "(qxmx qxmx_gpu.cpp page, the comment above gemv_dpas8); another machine, shapes not stated",
            "GB/s_low": 240.0, "GB/s_high": 468.0,
            "this_step_GB/s": round(value, 1)},
        "prefill_gemm": gemm,
        "prefill_q2_gemm": q2gemm,
        "fused_ffn": fused,
        "ffn_timeline": timeline,
        "q2_sustained": sustained,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
