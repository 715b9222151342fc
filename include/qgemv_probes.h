/*
 * qgemv_probes.h -- measurement probes of libqgemv.so.  They are not part
 * of the product path: the benchmark calls them to measure what this GPU
 * actually reaches (HBM read rate, matrix-core rate, shader clock), to
 * quote next to the published peaks the library's kernels are rated
 * against.  Same conventions as qgemv.h (device pointers, a hipStream_t
 * as void *, QG_EINVAL before any launch, QG_ELAUNCH on a failed launch).
 */
#ifndef QGEMV_PROBES_H
#define QGEMV_PROBES_H

#include <stddef.h>

#include "qgemv.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Device: reads the first bytes/16*16 bytes of buf once, with 16-byte
 * non-temporal loads, `loads` (4, 8 or 16) in flight per lane, over
 * `workgroups` workgroups of 512 threads (grid-stride).  Writes nothing unless a workgroup's folded
 * value equals `sentinel` (then sink[workgroup] = that value): pick a
 * sentinel the data cannot fold to, and time the launch.
 *   buf:  device, 16-byte aligned, >= 16 bytes.
 *   sink: device, unsigned[workgroups].
 * QG_EINVAL: null or misaligned pointer, bytes < 16, workgroups outside
 * 1..2^20, loads not 4, 8 or 16.                                          */
qg_status qg_probe_stream_read(const void *buf, size_t bytes,
                               unsigned sentinel, unsigned *sink,
                               int workgroups, int loads, void *stream);

/* Device: `workgroups` workgroups of 4 waves, each wave running `iters`
 * rounds of 8 independent matrix-core products on register operands:
 * kind 0 = v_mfma_i32_16x16x64_i8 (32768 int8 ops each), kind 1 =
 * v_mfma_f32_16x16x32_f16 (16384 fp16 flops each).
 *   sink:   device, f32[workgroups * 256], written (keeps the work live).
 *   clocks: device, uint64[2]: the shader-clock cycles (s_memtime) and the
 *           constant-rate wall-clock ticks (s_memrealtime, rate from
 *           qg_probe_wall_clock_khz) that wave 0 of workgroup 0 spent in
 *           its loop.
 * QG_EINVAL: bad kind, iters < 1, workgroups outside 1..65536, null or
 * misaligned pointer.                                                     */
qg_status qg_probe_mfma(int kind, int iters, int workgroups, float *sink,
                        unsigned long long *clocks, void *stream);

/* Device: whether vector-ALU work hides behind matrix-core work.
 * `workgroups` workgroups of 256 * waves_per_simd threads (waves_per_simd
 * waves on each SIMD), each wave running `iters` rounds of 8 independent
 * v_mfma_i32_16x16x64_i8 chains (mfma = 1) each followed by `fmas`
 * independent f32 FMAs (0, 2, 4 or 8), or the FMAs alone (mfma = 0,
 * fmas > 0).  Time the launch: if the two kinds overlapped, mfma + fmas
 * would take as long as the slower alone; if they add, as long as both.
 *   sink: device, f32[sink_elems], sink_elems >= workgroups * 256 *
 *         waves_per_simd; the first that many are written.
 * QG_EINVAL: mfma not 0/1, fmas not 0/2/4/8, both zero, iters < 1,
 * workgroups outside 1..65536, waves_per_simd outside 1..4, null or
 * misaligned sink, sink_elems too small.                                  */
qg_status qg_probe_mfma_valu(int mfma, int fmas, int iters, int workgroups,
                             int waves_per_simd, float *sink,
                             size_t sink_elems, void *stream);

/* Device: the LDS read rate.  `workgroups` workgroups of 64 * waves
 * threads, each wave running `iters` rounds of 8 LDS reads of
 * bytes_per_lane (4, 8 or 16) bytes per lane, consecutive lanes at
 * consecutive addresses of a 64 KiB LDS buffer (no bank conflicts); one
 * workgroup per CU when the grid is the CU count.  Bytes read per
 * workgroup: iters * 8 * 64 * bytes_per_lane * waves.
 *   sink: device, int32[sink_elems], sink_elems >= workgroups * 64 *
 *         waves; the first that many are written.
 * QG_EINVAL: bytes_per_lane not 4/8/16, iters < 1, workgroups outside
 * 1..65536, waves outside 1..16, null or misaligned sink, sink_elems too
 * small.                                                                  */
qg_status qg_probe_lds_read(int bytes_per_lane, int iters, int workgroups,
                            int waves, int *sink, size_t sink_elems,
                            void *stream);

/* Host: the current device's wall-clock counter rate in kHz (the unit of
 * qg_probe_mfma's clocks[1]).  QG_ELAUNCH if the runtime cannot say.     */
qg_status qg_probe_wall_clock_khz(int *khz);

/* Device: the timeline of one launch -- qgemv_q2_x and
 * qgemv_q2_gate_up_glu_x exactly as in qgemv.h (same kernels, same
 * results), with every workgroup recording the device wall clock
 * (s_memrealtime, qg_probe_wall_clock_khz) at four points: its start,
 * the end of its prologue (the quantised vector in LDS), the moment its
 * row tile's partial (or g / u) is summed over its waves, and its exit.
 *   stamps: device, uint64[4 * workgroups], 8-byte aligned; workgroup
 *           (x, y) of the grid writes entries 4 * (y * gx + x) + 0..3.
 *           The grid is ceil(M/64) x S (S = the split actually used) for
 *           qgemv_q2_x and 2 * ceil(M/64) x 1 for the pair (gate tiles
 *           first).
 * Arguments and errors otherwise as the product entry points.             */
qg_status qg_probe_q2_x_stamped(const qg_q2_weight *w, const float *x,
                                const float *xmax, int64_t nxmax,
                                const float *accum, float *y, void *ws,
                                size_t ws_bytes, int split_k,
                                unsigned long long *stamps, void *stream);
qg_status qg_probe_q2_gate_up_glu_x_stamped(const qg_q2_weight *w_gate,
                                            const qg_q2_weight *w_up,
                                            const float *x,
                                            const float *norm_w, float eps,
                                            int kind, float *t, float *tmax,
                                            void *ws, size_t ws_bytes,
                                            unsigned long long *stamps,
                                            void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QGEMV_PROBES_H */
