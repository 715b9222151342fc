// capi.cpp -- the C-ABI entry points: argument validation, then the launch.
// Nothing is enqueued unless every argument checks out; there is no fallback.
#include <stdarg.h>
#include <stdio.h>

#include "qg_internal.h"
#include "qgemv_probes.h"

namespace qg {

namespace {
thread_local char g_msg[512] = "";

bool aligned(const void *p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

qg_status launched(hipError_t e, const char *what) {
  if (e != hipSuccess) return fail(QG_ELAUNCH, "%s: launch failed: %s", what, hipGetErrorString(e));
  return QG_OK;
}

qg_status check_q2_weight(const qg_q2_weight *w, const char *fn) {
  if (!w) return fail(QG_EINVAL, "%s: null weight descriptor", fn);
  if (!w->codes || !w->scales) return fail(QG_EINVAL, "%s: null weight plane", fn);
  if (w->reserved != 0) return fail(QG_EINVAL, "%s: reserved field must be 0", fn);
  if (w->group != 64 && w->group != 128) return fail(QG_EINVAL, "%s: group %d is not 64 or 128", fn, w->group);
  if (w->M < 1 || w->M > (1LL << 31) - 64) return fail(QG_EINVAL, "%s: bad M=%lld", fn, (long long)w->M);
  if (w->K < w->group || w->K % w->group != 0 || w->K > (1 << 24))
    return fail(QG_EINVAL, "%s: K=%lld must be a positive multiple of group %d (at most 2^24)", fn, (long long)w->K, w->group);
  if (!aligned(w->codes, 16)) return fail(QG_EINVAL, "%s: codes plane not 16-byte aligned", fn);
  if (!aligned(w->scales, 2)) return fail(QG_EINVAL, "%s: scales plane not 2-byte aligned", fn);
  return QG_OK;
}
}  // namespace

qg_status fail(qg_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return s;
}

}  // namespace qg

using qg::aligned;
using qg::fail;

extern "C" {

const char *qg_status_string(qg_status s) {
  switch (s) {
    case QG_OK: return "QG_OK";
    case QG_EINVAL: return "QG_EINVAL";
    case QG_ELAUNCH: return "QG_ELAUNCH";
  }
  return "QG_UNKNOWN";
}

const char *qg_last_error(void) { return qg::g_msg; }

int qg_abi_version(void) { return 7; }

static bool overlap(const float *a, const float *b, int64_t n) { return a < b + n && b < a + n; }

// Byte ranges [a, a + na) and [b, b + nb) share a byte (null b: never).
static bool bytes_overlap(const void *a, size_t na, const void *b, size_t nb) {
  if (!a || !b || !na || !nb) return false;
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + nb && y < x + na;
}

static qg_status q8row_args(const char *fn, const void *qpacked, const float *rs, const float *xs, float *y,
                            int64_t M, int64_t K) {
  if (!qpacked || !rs || !xs || !y) return fail(QG_EINVAL, "%s: null pointer", fn);
  if (M < 1 || M > (1LL << 31) - 64) return fail(QG_EINVAL, "%s: bad M=%lld", fn, (long long)M);
  if (K < 4 || K % 4 != 0 || K > (1 << 30)) return fail(QG_EINVAL, "%s: K=%lld must be a positive multiple of 4", fn, (long long)K);
  if (!aligned(qpacked, 16)) return fail(QG_EINVAL, "%s: weight image not 16-byte aligned", fn);
  if (!aligned(xs, 16)) return fail(QG_EINVAL, "%s: xs not 16-byte aligned", fn);
  if (!aligned(rs, 4) || !aligned(y, 4)) return fail(QG_EINVAL, "%s: rs/y not 4-byte aligned", fn);
  return QG_OK;
}

qg_status qgemv_q8row(const void *qpacked, const float *rs, const float *xs, float *y, int64_t M,
                      int64_t K, void *stream) {
  const char *fn = "qgemv_q8row";
  qg_status st = q8row_args(fn, qpacked, rs, xs, y, M, K);
  if (st != QG_OK) return st;
  return qg::launched(qg::launch_q8row_gemv(qpacked, rs, xs, y, (int)M, (int)K, (hipStream_t)stream), fn);
}

size_t qgemv_q8row_balanced_ws_bytes(int64_t M, int64_t K) {
  if (M < 1 || M > (1LL << 31) - 64 || K < 4 || K > (1 << 30)) return 0;
  const qg::Q8TailSplit t = qg::q8row_tail_split(M, K);
  if (t.tiles_split == 0) return 0;
  return qg::q8_tail_cnt_bytes(t.tiles_split) + (size_t)t.tiles_split * t.S * 64 * sizeof(float);
}

qg_status qgemv_q8row_balanced(const void *qpacked, const float *rs, const float *xs, float *y, int64_t M,
                               int64_t K, void *ws, size_t ws_bytes, void *stream) {
  const char *fn = "qgemv_q8row_balanced";
  qg_status st = q8row_args(fn, qpacked, rs, xs, y, M, K);
  if (st != QG_OK) return st;
  const size_t need = qgemv_q8row_balanced_ws_bytes(M, K);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(QG_EINVAL, "%s: workspace %zu bytes < %zu needed", fn, ws ? ws_bytes : (size_t)0, need);
  if (need > 0 && !aligned(ws, 16)) return fail(QG_EINVAL, "%s: workspace not 16-byte aligned", fn);
  const size_t ybytes = (size_t)M * sizeof(float), xbytes = (size_t)K * sizeof(float);
  const size_t wbytes = (size_t)qg::round_up(M, 64) * (size_t)qg::round_up(K, 16);
  if (need > 0 && (bytes_overlap(ws, need, y, ybytes) || bytes_overlap(ws, need, xs, xbytes) ||
                   bytes_overlap(ws, need, rs, ybytes) || bytes_overlap(ws, need, qpacked, wbytes)))
    return fail(QG_EINVAL, "%s: workspace overlaps y, xs, rs or the weight image", fn);
  return qg::launched(
      qg::launch_q8row_gemv_balanced(qpacked, rs, xs, y, (int)M, (int)K, ws, (hipStream_t)stream), fn);
}

qg_status qquant_act_i8(const float *x, int64_t K, int8_t *xq, float *act_scale, int32_t *suma,
                        void *stream) {
  const char *fn = "qquant_act_i8";
  if (!x || !xq || !act_scale || !suma) return fail(QG_EINVAL, "%s: null pointer", fn);
  if (K < 64 || K % 64 != 0 || K > (1 << 24)) return fail(QG_EINVAL, "%s: K=%lld must be a positive multiple of 64", fn, (long long)K);
  if (!aligned(x, 16)) return fail(QG_EINVAL, "%s: x not 16-byte aligned", fn);
  if (!aligned(xq, 4) || !aligned(act_scale, 4) || !aligned(suma, 4)) return fail(QG_EINVAL, "%s: misaligned output", fn);
  return qg::launched(qg::launch_act_quant(x, 1, (int)K, xq, act_scale, suma, (hipStream_t)stream), fn);
}

qg_status qquant_act_i8_rows(const float *x, int64_t nb, int64_t K, int8_t *xq, float *act_scale, int32_t *suma,
                             void *stream) {
  const char *fn = "qquant_act_i8_rows";
  if (!x || !xq || !act_scale || !suma) return fail(QG_EINVAL, "%s: null pointer", fn);
  if (nb < 1 || nb > (1 << 24)) return fail(QG_EINVAL, "%s: bad nb=%lld", fn, (long long)nb);
  if (K < 64 || K % 64 != 0 || K > (1 << 24)) return fail(QG_EINVAL, "%s: K=%lld must be a positive multiple of 64", fn, (long long)K);
  if (nb * K > (1LL << 40)) return fail(QG_EINVAL, "%s: problem too large", fn);
  if (!aligned(x, 16)) return fail(QG_EINVAL, "%s: x not 16-byte aligned", fn);
  if (!aligned(xq, 4) || !aligned(act_scale, 4) || !aligned(suma, 4)) return fail(QG_EINVAL, "%s: misaligned output", fn);
  return qg::launched(qg::launch_act_quant(x, (int)nb, (int)K, xq, act_scale, suma, (hipStream_t)stream), fn);
}

static qg_status check_quant_outputs(const char *fn, int64_t K, const int8_t *xq, const float *act_scale,
                                     const int32_t *suma) {
  if (!xq || !act_scale || !suma) return fail(QG_EINVAL, "%s: null pointer", fn);
  if (K < 64 || K % 64 != 0 || K > (1 << 24)) return fail(QG_EINVAL, "%s: K=%lld must be a positive multiple of 64", fn, (long long)K);
  if (!aligned(xq, 4) || !aligned(act_scale, 4) || !aligned(suma, 4)) return fail(QG_EINVAL, "%s: misaligned output", fn);
  return QG_OK;
}

static qg_status rmsnorm_common(const char *fn, const float *x, const float *w, int64_t nb, int64_t K, float eps,
                                int8_t *xq, float *act_scale, int32_t *suma, void *stream) {
  qg_status st = check_quant_outputs(fn, K, xq, act_scale, suma);
  if (st != QG_OK) return st;
  if (!x || !w) return fail(QG_EINVAL, "%s: null pointer", fn);
  if (nb < 1 || nb > (1 << 24) || nb * K > (1LL << 40)) return fail(QG_EINVAL, "%s: bad nb=%lld", fn, (long long)nb);
  if (!aligned(x, 16) || !aligned(w, 16)) return fail(QG_EINVAL, "%s: x and w must be 16-byte aligned", fn);
  if (!(eps >= 0.0f) || eps > 3.4e38f) return fail(QG_EINVAL, "%s: eps must be finite and >= 0", fn);
  return qg::launched(qg::launch_rmsnorm_quant(x, w, (int)nb, (int)K, eps, xq, act_scale, suma, (hipStream_t)stream),
                      fn);
}

qg_status qquant_rmsnorm_i8(const float *x, const float *w, int64_t K, float eps, int8_t *xq, float *act_scale,
                            int32_t *suma, void *stream) {
  return rmsnorm_common("qquant_rmsnorm_i8", x, w, 1, K, eps, xq, act_scale, suma, stream);
}

qg_status qquant_rmsnorm_i8_rows(const float *x, const float *w, int64_t nb, int64_t K, float eps, int8_t *xq,
                                 float *act_scale, int32_t *suma, void *stream) {
  return rmsnorm_common("qquant_rmsnorm_i8_rows", x, w, nb, K, eps, xq, act_scale, suma, stream);
}

static qg_status glu_common(const char *fn, const float *g, const float *u, int64_t nb, int64_t K, int kind, float *t,
                            int8_t *xq, float *act_scale, int32_t *suma, void *stream) {
  qg_status st = check_quant_outputs(fn, K, xq, act_scale, suma);
  if (st != QG_OK) return st;
  if (!g || !u || !t) return fail(QG_EINVAL, "%s: null pointer", fn);
  if (nb < 1 || nb > (1 << 24) || nb * K > (1LL << 40)) return fail(QG_EINVAL, "%s: bad nb=%lld", fn, (long long)nb);
  if (kind != QG_GLU_SILU && kind != QG_GLU_SIGMOID) return fail(QG_EINVAL, "%s: kind %d is not SILU or SIGMOID", fn, kind);
  if (!aligned(g, 16) || !aligned(u, 16) || !aligned(t, 16))
    return fail(QG_EINVAL, "%s: g, u and t must be 16-byte aligned", fn);
  const int64_t n = nb * K;
  auto part_overlap = [n](const float *a, const float *b) { return a != b && a < b + n && b < a + n; };
  if (part_overlap(t, g) || part_overlap(t, u)) return fail(QG_EINVAL, "%s: t must be g, u or a separate buffer", fn);
  return qg::launched(
      qg::launch_glu_quant(g, u, (int)nb, (int)K, kind, t, xq, act_scale, suma, (hipStream_t)stream), fn);
}

qg_status qquant_glu_i8(const float *g, const float *u, int64_t K, int kind, float *t, int8_t *xq,
                        float *act_scale, int32_t *suma, void *stream) {
  return glu_common("qquant_glu_i8", g, u, 1, K, kind, t, xq, act_scale, suma, stream);
}

qg_status qquant_glu_i8_rows(const float *g, const float *u, int64_t nb, int64_t K, int kind, float *t, int8_t *xq,
                             float *act_scale, int32_t *suma, void *stream) {
  return glu_common("qquant_glu_i8_rows", g, u, nb, K, kind, t, xq, act_scale, suma, stream);
}

int qgemv_q2_auto_split(int64_t M, int64_t K, int group) {
  if (M < 1 || (group != 64 && group != 128) || K < group || K % group) return 1;
  return qg::q2_auto_split(M, K, group);
}

size_t qgemv_q2_ws_bytes(int64_t M, int64_t K, int group, int split_k) {
  if (M < 1 || (group != 64 && group != 128) || K < group || K % group) return 0;
  const int S = split_k == 0 ? qg::q2_auto_split(M, K, group) : split_k;
  if (S <= 1 || S > qg::kMaxSplit) return 0;
  return (size_t)S * (size_t)qg::round_up(M, 64) * sizeof(float);
}

static qg_status q2_common(const char *fn, const qg_q2_weight *w, const qg_q2_weight *w1, const int8_t *xq,
                           const int32_t *suma, const float *act_scale, const float *accum, float *y,
                           float *y1, int32_t *dots, void *ws, size_t ws_bytes, int split_k, void *stream) {
  qg_status st = qg::check_q2_weight(w, fn);
  if (st != QG_OK) return st;
  if (w1) {
    st = qg::check_q2_weight(w1, fn);
    if (st != QG_OK) return st;
    if (w1->M != w->M || w1->K != w->K || w1->group != w->group)
      return fail(QG_EINVAL, "%s: the two weights differ in shape (%lldx%lld g%d vs %lldx%lld g%d)", fn,
                  (long long)w->M, (long long)w->K, w->group, (long long)w1->M, (long long)w1->K, w1->group);
    if (!y1) return fail(QG_EINVAL, "%s: null pointer", fn);
    if (!aligned(y1, 4)) return fail(QG_EINVAL, "%s: misaligned pointer", fn);
    if (overlap(y, y1, w->M)) return fail(QG_EINVAL, "%s: the two outputs overlap", fn);
  }
  if (!xq || !suma || !act_scale || !y) return fail(QG_EINVAL, "%s: null pointer", fn);
  if (!aligned(xq, 16)) return fail(QG_EINVAL, "%s: xq not 16-byte aligned", fn);
  if (!aligned(suma, 4) || !aligned(act_scale, 4) || !aligned(y, 4) || (dots && !aligned(dots, 4)) ||
      (accum && !aligned(accum, 4)))
    return fail(QG_EINVAL, "%s: misaligned pointer", fn);
  if (accum && accum != y && overlap(accum, y, w->M))
    return fail(QG_EINVAL, "%s: accum must be y itself or not overlap it", fn);
  if (split_k < 0 || split_k > qg::kMaxSplit) return fail(QG_EINVAL, "%s: split_k=%d outside 0..16", fn, split_k);
  const int S = split_k == 0 ? qg::q2_auto_split(w->M, w->K, w->group) : split_k;
  const size_t need = (w1 ? 2 : 1) * qgemv_q2_ws_bytes(w->M, w->K, w->group, S);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(QG_EINVAL, "%s: workspace %zu bytes < %zu needed for split %d", fn, ws ? ws_bytes : (size_t)0, need, S);
  if (need > 0 && !aligned(ws, 4)) return fail(QG_EINVAL, "%s: workspace not 4-byte aligned", fn);
  const size_t ybytes = (size_t)w->M * sizeof(float);
  if (need > 0 && (bytes_overlap(ws, need, y, ybytes) || bytes_overlap(ws, need, y1, ybytes) ||
                   bytes_overlap(ws, need, accum, ybytes)))
    return fail(QG_EINVAL, "%s: workspace overlaps an output or the residual", fn);
  qg::Q2Call call{};
  call.codes[0] = w->codes;
  call.scales[0] = w->scales;
  call.y[0] = y;
  if (w1) {
    call.codes[1] = w1->codes;
    call.scales[1] = w1->scales;
    call.y[1] = y1;
  }
  call.M = (int)w->M;
  call.K = (int)w->K;
  call.group = w->group;
  call.xq = xq;
  call.suma = suma;
  call.act_scale = act_scale;
  call.accum = accum;
  call.dots = dots;
  call.partials = static_cast<float *>(ws);
  call.split = S;
  return qg::launched(qg::launch_q2_gemv(call, (hipStream_t)stream), fn);
}

qg_status qgemv_q2(const qg_q2_weight *w, const int8_t *xq, const int32_t *suma, const float *act_scale,
                   float *y, void *ws, size_t ws_bytes, int split_k, void *stream) {
  return q2_common("qgemv_q2", w, nullptr, xq, suma, act_scale, nullptr, y, nullptr, nullptr, ws, ws_bytes,
                   split_k, stream);
}

qg_status qgemv_q2_noalloc(const qg_q2_weight *w, const int8_t *xq, const int32_t *suma, const float *act_scale,
                           float *y, int split_k, void *stream) {
  const char *fn = "qgemv_q2_noalloc";
  qg_status st = qg::check_q2_weight(w, fn);
  if (st != QG_OK) return st;
  if (split_k < 0 || split_k > qg::kMaxSplit) return fail(QG_EINVAL, "%s: split_k=%d outside 0..16", fn, split_k);
  const size_t need = qgemv_q2_ws_bytes(w->M, w->K, w->group, split_k);
  if (need > qg::kStaticScratchBytes)
    return fail(QG_EINVAL, "%s: split %d of %lld rows needs %zu bytes of partials; the static scratch holds %zu", fn,
                split_k == 0 ? qg::q2_auto_split(w->M, w->K, w->group) : split_k, (long long)w->M, need,
                qg::kStaticScratchBytes);
  void *ws = nullptr;
  if (need > 0) {
    hipError_t e = qg::static_scratch(&ws);
    if (e != hipSuccess) return fail(QG_ELAUNCH, "%s: no device address for the static scratch: %s", fn,
                                     hipGetErrorString(e));
  }
  return q2_common(fn, w, nullptr, xq, suma, act_scale, nullptr, y, nullptr, nullptr, ws,
                   need > 0 ? qg::kStaticScratchBytes : 0, split_k, stream);
}

qg_status qgemv_q2_dots(const qg_q2_weight *w, const int8_t *xq, const int32_t *suma, const float *act_scale,
                        float *y, int32_t *dots, void *ws, size_t ws_bytes, int split_k, void *stream) {
  if (!dots) return fail(QG_EINVAL, "qgemv_q2_dots: null dots");
  return q2_common("qgemv_q2_dots", w, nullptr, xq, suma, act_scale, nullptr, y, nullptr, dots, ws, ws_bytes,
                   split_k, stream);
}

qg_status qgemv_q2_accum(const qg_q2_weight *w, const int8_t *xq, const int32_t *suma, const float *act_scale,
                         const float *accum, float *y, void *ws, size_t ws_bytes, int split_k, void *stream) {
  if (!accum) return fail(QG_EINVAL, "qgemv_q2_accum: null accum");
  return q2_common("qgemv_q2_accum", w, nullptr, xq, suma, act_scale, accum, y, nullptr, nullptr, ws, ws_bytes,
                   split_k, stream);
}

size_t qgemv_q2_dual_ws_bytes(int64_t M, int64_t K, int group, int split_k) {
  return 2 * qgemv_q2_ws_bytes(M, K, group, split_k);
}

qg_status qgemv_q2_dual(const qg_q2_weight *w0, const qg_q2_weight *w1, const int8_t *xq, const int32_t *suma,
                        const float *act_scale, float *y0, float *y1, void *ws, size_t ws_bytes, int split_k,
                        void *stream) {
  if (!w1) return fail(QG_EINVAL, "qgemv_q2_dual: null weight descriptor");
  return q2_common("qgemv_q2_dual", w0, w1, xq, suma, act_scale, nullptr, y0, y1, nullptr, ws, ws_bytes, split_k,
                   stream);
}

qg_status qgemv_q2_gate_up_glu(const qg_q2_weight *w_gate, const qg_q2_weight *w_up, const int8_t *xq,
                               const int32_t *suma, const float *act_scale, int kind, float *t, int8_t *xq_out,
                               float *act_scale_out, int32_t *suma_out, void *stream) {
  const char *fn = "qgemv_q2_gate_up_glu";
  qg_status st = qg::check_q2_weight(w_gate, fn);
  if (st != QG_OK) return st;
  st = qg::check_q2_weight(w_up, fn);
  if (st != QG_OK) return st;
  if (w_up->M != w_gate->M || w_up->K != w_gate->K || w_up->group != w_gate->group)
    return fail(QG_EINVAL, "%s: the two weights differ in shape or group", fn);
  if (!xq || !suma || !act_scale || !t || !xq_out || !act_scale_out || !suma_out)
    return fail(QG_EINVAL, "%s: null pointer", fn);
  if (kind != QG_GLU_SILU && kind != QG_GLU_SIGMOID) return fail(QG_EINVAL, "%s: kind %d is not SILU or SIGMOID", fn, kind);
  const int64_t M = w_gate->M;
  if (M % 64 != 0 || M > (1 << 24)) return fail(QG_EINVAL, "%s: M=%lld must be a multiple of 64 (the gated vector is quantised)", fn, (long long)M);
  if (!aligned(xq, 16) || !aligned(t, 16)) return fail(QG_EINVAL, "%s: xq and t must be 16-byte aligned", fn);
  if (!aligned(suma, 4) || !aligned(act_scale, 4) || !aligned(xq_out, 4) || !aligned(act_scale_out, 4) ||
      !aligned(suma_out, 4))
    return fail(QG_EINVAL, "%s: misaligned pointer", fn);
  const size_t tb = (size_t)M * sizeof(float);
  if (bytes_overlap(t, tb, xq_out, (size_t)M) || bytes_overlap(t, tb, suma_out, (size_t)(M / 64) * 4) ||
      bytes_overlap(t, tb, act_scale_out, 4) || bytes_overlap(xq_out, (size_t)M, suma_out, (size_t)(M / 64) * 4) ||
      bytes_overlap(t, tb, xq, (size_t)w_gate->K) || bytes_overlap(suma_out, (size_t)(M / 64) * 4, suma, (size_t)(w_gate->K / 64) * 4))
    return fail(QG_EINVAL, "%s: an output overlaps another output or an input", fn);
  qg::Q2Call call{};
  call.codes[0] = w_gate->codes;
  call.scales[0] = w_gate->scales;
  call.codes[1] = w_up->codes;
  call.scales[1] = w_up->scales;
  call.M = (int)M;
  call.K = (int)w_gate->K;
  call.group = w_gate->group;
  call.xq = xq;
  call.suma = suma;
  call.act_scale = act_scale;
  call.split = 1;
  return qg::launched(qg::launch_q2_gate_up_glu(call, kind, t, xq_out, act_scale_out, suma_out, (hipStream_t)stream),
                      fn);
}

size_t qgemv_q2_x_ws_bytes(int64_t M, int64_t K, int group, int split_k) {
  if (M < 1 || K < 1 || (group != 64 && group != 128)) return 0;
  const int S = split_k == 0 ? qg::q2x_auto_split(M, K, group) : split_k;
  if (S <= 1 || S > qg::kMaxSplit) return 0;
  return qg::q2x_cnt_bytes(M) + (size_t)S * (size_t)qg::round_up(M, 64) * sizeof(float);
}

// Byte range [p, p + n) overlaps one of the Q2 weight's device planes.
static bool overlaps_q2_planes(const void *p, size_t n, const qg_q2_weight *w) {
  const size_t rows = (size_t)qg::round_up(w->M, 64);
  return bytes_overlap(p, n, w->codes, rows * (size_t)(w->K / 4)) ||
         bytes_overlap(p, n, w->scales, rows * (size_t)(w->K / w->group) * 2);
}

// The f32 input vector of the in-launch quantiser: present, 16-byte
// aligned, and short enough for each workgroup to hold it.
static qg_status check_x_input(const char *fn, const qg_q2_weight *w, const float *x, const float *norm_w,
                               float eps) {
  if (!x) return fail(QG_EINVAL, "%s: null x", fn);
  if (!aligned(x, 16) || (norm_w && !aligned(norm_w, 16)))
    return fail(QG_EINVAL, "%s: x and norm_w must be 16-byte aligned", fn);
  const int64_t kmax = qg::q2x_max_k(w->M);
  if (w->K > kmax)
    return fail(QG_EINVAL, "%s: K=%lld above %lld for M=%lld", fn, (long long)w->K, (long long)kmax, (long long)w->M);
  if (norm_w && w->K > qg::kQ2XNormMaxK)
    return fail(QG_EINVAL, "%s: K=%lld above %d with the RMSNorm", fn, (long long)w->K, qg::kQ2XNormMaxK);
  if (norm_w && !(eps >= 0.0f && eps <= 3.4e38f)) return fail(QG_EINVAL, "%s: eps must be finite and >= 0", fn);
  return QG_OK;
}

static qg_status q2_x_impl(const char *fn, const qg_q2_weight *w, const float *x, const float *xmax, int64_t nxmax,
                           const float *accum, float *y, void *ws, size_t ws_bytes, int split_k,
                           unsigned long long *stamps, void *stream) {
  qg_status st = qg::check_q2_weight(w, fn);
  if (st != QG_OK) return st;
  if (split_k < 0 || split_k > qg::kMaxSplit) return fail(QG_EINVAL, "%s: split_k=%d outside 0..16", fn, split_k);
  const int S = split_k == 0 ? qg::q2x_auto_split(w->M, w->K, w->group) : split_k;
  if ((st = check_x_input(fn, w, x, nullptr, 0.0f)) != QG_OK) return st;
  if (!y) return fail(QG_EINVAL, "%s: null pointer", fn);
  if (!aligned(y, 4) || (accum && !aligned(accum, 4))) return fail(QG_EINVAL, "%s: misaligned pointer", fn);
  if (accum && accum != y && overlap(accum, y, w->M))
    return fail(QG_EINVAL, "%s: accum must be y itself or not overlap it", fn);
  const size_t xbytes = (size_t)w->K * sizeof(float), ybytes = (size_t)w->M * sizeof(float);
  if (bytes_overlap(x, xbytes, y, ybytes)) return fail(QG_EINVAL, "%s: x overlaps y", fn);
  if ((xmax == nullptr) != (nxmax == 0))
    return fail(QG_EINVAL, "%s: xmax and nxmax must be both given or NULL and 0", fn);
  if (xmax && (nxmax < 1 || nxmax > QG_Q2X_MAX_PARTS))
    return fail(QG_EINVAL, "%s: nxmax=%lld outside 1..%d", fn, (long long)nxmax, QG_Q2X_MAX_PARTS);
  if (xmax && !aligned(xmax, 4)) return fail(QG_EINVAL, "%s: misaligned xmax", fn);
  const size_t pbytes = (size_t)nxmax * sizeof(float);
  if (xmax && bytes_overlap(xmax, pbytes, y, ybytes)) return fail(QG_EINVAL, "%s: xmax overlaps y", fn);
  const size_t need = qgemv_q2_x_ws_bytes(w->M, w->K, w->group, S);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(QG_EINVAL, "%s: workspace %zu bytes < %zu needed for split %d", fn, ws ? ws_bytes : (size_t)0, need, S);
  if (need > 0 && !aligned(ws, 16)) return fail(QG_EINVAL, "%s: workspace not 16-byte aligned", fn);
  if (need > 0 && (bytes_overlap(ws, need, y, ybytes) || bytes_overlap(ws, need, accum, ybytes) ||
                   bytes_overlap(ws, need, x, xbytes) || bytes_overlap(ws, need, xmax, pbytes) ||
                   overlaps_q2_planes(ws, need, w)))
    return fail(QG_EINVAL, "%s: workspace overlaps an output, the residual, x, xmax or the weights", fn);
  qg::Q2XCall c{};
  c.codes[0] = w->codes;
  c.scales[0] = w->scales;
  c.y[0] = y;
  c.M = (int)w->M;
  c.K = (int)w->K;
  c.group = w->group;
  c.x = x;
  c.xmax = xmax;
  c.nxmax = (int)nxmax;
  c.accum = accum;
  c.ws = ws;
  c.split = S;
  c.glu = -1;
  c.stamps = stamps;
  return qg::launched(qg::launch_q2_gemv_x(c, (hipStream_t)stream), fn);
}

qg_status qgemv_q2_x(const qg_q2_weight *w, const float *x, const float *xmax, int64_t nxmax, const float *accum,
                     float *y, void *ws, size_t ws_bytes, int split_k, void *stream) {
  return q2_x_impl("qgemv_q2_x", w, x, xmax, nxmax, accum, y, ws, ws_bytes, split_k, nullptr, stream);
}

qg_status qg_probe_q2_x_stamped(const qg_q2_weight *w, const float *x, const float *xmax, int64_t nxmax,
                                const float *accum, float *y, void *ws, size_t ws_bytes, int split_k,
                                unsigned long long *stamps, void *stream) {
  if (!stamps || !aligned(stamps, 8)) return fail(QG_EINVAL, "qg_probe_q2_x_stamped: null or misaligned stamps");
  return q2_x_impl("qg_probe_q2_x_stamped", w, x, xmax, nxmax, accum, y, ws, ws_bytes, split_k, stamps, stream);
}

int qgemv_q2_x_auto_split(int64_t M, int64_t K, int group) {
  if (M < 1 || K < 1 || (group != 64 && group != 128)) return 1;
  return qg::q2x_auto_split(M, K, group);
}

size_t qgemv_q2_gate_up_glu_x_ws_bytes(int64_t M) {
  if (M < 1) return 0;
  return qg::q2x_cnt_bytes(M) + 2 * (size_t)qg::round_up(M, 64) * sizeof(float);
}

static qg_status pair_x_common(const char *fn, const qg_q2_weight *w0, const qg_q2_weight *w1, const float *x,
                               const float *norm_w, float eps, int glu, float *y0, float *y1, float *tmax,
                               void *ws, size_t ws_bytes, void *stream, unsigned long long *stamps = nullptr) {
  qg_status st = qg::check_q2_weight(w0, fn);
  if (st != QG_OK) return st;
  if ((st = qg::check_q2_weight(w1, fn)) != QG_OK) return st;
  if (w1->M != w0->M || w1->K != w0->K || w1->group != w0->group)
    return fail(QG_EINVAL, "%s: the two weights differ in shape or group", fn);
  if ((st = check_x_input(fn, w0, x, norm_w, eps)) != QG_OK) return st;
  if (!y0 || (glu < 0 && !y1)) return fail(QG_EINVAL, "%s: null pointer", fn);
  if (!aligned(y0, 4) || (y1 && !aligned(y1, 4))) return fail(QG_EINVAL, "%s: misaligned pointer", fn);
  const size_t xbytes = (size_t)w0->K * sizeof(float), ybytes = (size_t)w0->M * sizeof(float);
  if (glu < 0 && bytes_overlap(y0, ybytes, y1, ybytes)) return fail(QG_EINVAL, "%s: the two outputs overlap", fn);
  if (bytes_overlap(x, xbytes, y0, ybytes) || bytes_overlap(norm_w, xbytes, y0, ybytes) ||
      (glu < 0 && (bytes_overlap(x, xbytes, y1, ybytes) || bytes_overlap(norm_w, xbytes, y1, ybytes))))
    return fail(QG_EINVAL, "%s: an output overlaps x or norm_w", fn);
  if (glu >= 0) {
    const size_t need = qgemv_q2_gate_up_glu_x_ws_bytes(w0->M);
    if (!ws || ws_bytes < need) return fail(QG_EINVAL, "%s: workspace %zu bytes < %zu needed", fn, ws ? ws_bytes : (size_t)0, need);
    if (!aligned(ws, 16)) return fail(QG_EINVAL, "%s: workspace not 16-byte aligned", fn);
    if (bytes_overlap(ws, need, y0, ybytes) || bytes_overlap(ws, need, x, xbytes) ||
        bytes_overlap(ws, need, norm_w, xbytes) || overlaps_q2_planes(ws, need, w0) ||
        overlaps_q2_planes(ws, need, w1))
      return fail(QG_EINVAL, "%s: workspace overlaps t, x, norm_w or the weights", fn);
    if (tmax) {
      const size_t tb = (size_t)((w0->M + 63) / 64) * sizeof(float);
      if (!aligned(tmax, 4)) return fail(QG_EINVAL, "%s: misaligned tmax", fn);
      if (bytes_overlap(tmax, tb, y0, ybytes) || bytes_overlap(tmax, tb, x, xbytes) ||
          bytes_overlap(tmax, tb, norm_w, xbytes) || bytes_overlap(tmax, tb, ws, need))
        return fail(QG_EINVAL, "%s: tmax overlaps t, x, norm_w or the workspace", fn);
    }
  }
  qg::Q2XCall c{};
  c.codes[0] = w0->codes;
  c.scales[0] = w0->scales;
  c.codes[1] = w1->codes;
  c.scales[1] = w1->scales;
  c.y[0] = y0;
  c.y[1] = glu < 0 ? y1 : nullptr;
  c.M = (int)w0->M;
  c.K = (int)w0->K;
  c.group = w0->group;
  c.x = x;
  c.norm_w = norm_w;
  c.eps = eps;
  c.ws = glu >= 0 ? ws : nullptr;
  c.split = 1;
  c.glu = glu;
  c.tmax = glu >= 0 ? tmax : nullptr;
  c.stamps = stamps;
  return qg::launched(qg::launch_q2_gemv_x(c, (hipStream_t)stream), fn);
}

qg_status qgemv_q2_dual_x(const qg_q2_weight *w0, const qg_q2_weight *w1, const float *x, const float *norm_w,
                          float eps, float *y0, float *y1, void *stream) {
  return pair_x_common("qgemv_q2_dual_x", w0, w1, x, norm_w, eps, -1, y0, y1, nullptr, nullptr, 0, stream);
}

qg_status qgemv_q2_gate_up_glu_x(const qg_q2_weight *w_gate, const qg_q2_weight *w_up, const float *x,
                                 const float *norm_w, float eps, int kind, float *t, float *tmax, void *ws,
                                 size_t ws_bytes, void *stream) {
  const char *fn = "qgemv_q2_gate_up_glu_x";
  if (kind != QG_GLU_SILU && kind != QG_GLU_SIGMOID) return fail(QG_EINVAL, "%s: kind %d is not SILU or SIGMOID", fn, kind);
  return pair_x_common(fn, w_gate, w_up, x, norm_w, eps, kind, t, nullptr, tmax, ws, ws_bytes, stream);
}

qg_status qg_probe_q2_gate_up_glu_x_stamped(const qg_q2_weight *w_gate, const qg_q2_weight *w_up, const float *x,
                                            const float *norm_w, float eps, int kind, float *t, float *tmax,
                                            void *ws, size_t ws_bytes, unsigned long long *stamps, void *stream) {
  const char *fn = "qg_probe_q2_gate_up_glu_x_stamped";
  if (!stamps || !aligned(stamps, 8)) return fail(QG_EINVAL, "%s: null or misaligned stamps", fn);
  if (kind != QG_GLU_SILU && kind != QG_GLU_SIGMOID) return fail(QG_EINVAL, "%s: kind %d is not SILU or SIGMOID", fn, kind);
  return pair_x_common(fn, w_gate, w_up, x, norm_w, eps, kind, t, nullptr, tmax, ws, ws_bytes, stream, stamps);
}

qg_status qgemv_q2_batch(const qg_q2_job *jobs, int njobs, void *stream) {
  const char *fn = "qgemv_q2_batch";
  if (!jobs) return fail(QG_EINVAL, "%s: null job table", fn);
  if (njobs < 1 || njobs > QG_Q2_BATCH_MAX) return fail(QG_EINVAL, "%s: njobs=%d outside 1..%d", fn, njobs, QG_Q2_BATCH_MAX);
  qg::Q2BatchCall c[qg::kMaxQ2Jobs];
  int64_t tiles = 0;
  for (int n = 0; n < njobs; n++) {
    const qg_q2_job &j = jobs[n];
    qg_status st = qg::check_q2_weight(&j.w, fn);
    if (st != QG_OK) return st;
    if (j.w.group != jobs[0].w.group) return fail(QG_EINVAL, "%s: job %d has group %d, job 0 has %d", fn, n, j.w.group, jobs[0].w.group);
    if (!j.xq || !j.suma || !j.act_scale || !j.y) return fail(QG_EINVAL, "%s: job %d: null pointer", fn, n);
    if (!aligned(j.xq, 16)) return fail(QG_EINVAL, "%s: job %d: xq not 16-byte aligned", fn, n);
    if (!aligned(j.suma, 4) || !aligned(j.act_scale, 4) || !aligned(j.y, 4) || (j.accum && !aligned(j.accum, 4)))
      return fail(QG_EINVAL, "%s: job %d: misaligned pointer", fn, n);
    if (j.accum && j.accum != j.y && overlap(j.accum, j.y, j.w.M))
      return fail(QG_EINVAL, "%s: job %d: accum must be y itself or not overlap it", fn, n);
    for (int m = 0; m < n; m++) {
      const qg_q2_job &o = jobs[m];
      const bool yy = j.y < o.y + o.w.M && o.y < j.y + j.w.M;
      const bool ya = o.accum && j.y < o.accum + o.w.M && o.accum < j.y + j.w.M;
      const bool ay = j.accum && o.y < j.accum + j.w.M && j.accum < o.y + o.w.M;
      if (yy || ya || ay) return fail(QG_EINVAL, "%s: jobs %d and %d: an output overlaps the other's output or residual", fn, m, n);
    }
    tiles += (j.w.M + 63) / 64;
    c[n].codes = j.w.codes;
    c[n].scales = j.w.scales;
    c[n].xq = j.xq;
    c[n].suma = j.suma;
    c[n].act_scale = j.act_scale;
    c[n].accum = j.accum;
    c[n].y = j.y;
    c[n].M = (int)j.w.M;
    c[n].K = (int)j.w.K;
  }
  if (tiles > (1LL << 30)) return fail(QG_EINVAL, "%s: too many row tiles", fn);
  return qg::launched(qg::launch_q2_batch(c, njobs, jobs[0].w.group, (hipStream_t)stream), fn);
}

size_t qgemm_q2_batched_ws_bytes(int64_t M, int64_t K, int group, int64_t nb) {
  if (M < 1 || nb < 1 || (group != 64 && group != 128) || K < group || K % group) return 0;
  const int S = qg::q2_gemm_split(M, K, group, nb);
  return S > 1 ? (size_t)S * (size_t)nb * (size_t)M * sizeof(float) : 0;
}

qg_status qgemm_q2_batched(const qg_q2_weight *w, const int8_t *xq, const int32_t *suma, const float *act_scale,
                           const float *accum, float *y, int64_t nb, void *ws, size_t ws_bytes, void *stream) {
  const char *fn = "qgemm_q2_batched";
  (void)suma;  // the product forms code - 1 in its operand
  qg_status st = qg::check_q2_weight(w, fn);
  if (st != QG_OK) return st;
  if (!xq || !act_scale || !y) return fail(QG_EINVAL, "%s: null pointer", fn);
  if (nb < 1 || nb > (1 << 24)) return fail(QG_EINVAL, "%s: bad nb=%lld", fn, (long long)nb);
  if (nb * w->M > (1LL << 40) || nb * w->K > (1LL << 40)) return fail(QG_EINVAL, "%s: problem too large", fn);
  if (!aligned(w->scales, 8)) return fail(QG_EINVAL, "%s: scales plane not 8-byte aligned", fn);
  if (!aligned(xq, 16) || !aligned(y, 16)) return fail(QG_EINVAL, "%s: xq and y must be 16-byte aligned", fn);
  if (!aligned(act_scale, 4) || (accum && !aligned(accum, 4))) return fail(QG_EINVAL, "%s: misaligned pointer", fn);
  if (accum && accum != y && overlap(accum, y, nb * w->M))
    return fail(QG_EINVAL, "%s: accum must be y itself or not overlap it", fn);
  const size_t need = qgemm_q2_batched_ws_bytes(w->M, w->K, w->group, nb);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(QG_EINVAL, "%s: workspace %zu bytes < %zu needed", fn, ws ? ws_bytes : (size_t)0, need);
  if (need > 0 && !aligned(ws, 16)) return fail(QG_EINVAL, "%s: workspace not 16-byte aligned", fn);
  const size_t ybytes = (size_t)nb * w->M * sizeof(float);
  if (need > 0 && (bytes_overlap(ws, need, y, ybytes) || bytes_overlap(ws, need, accum, ybytes)))
    return fail(QG_EINVAL, "%s: workspace overlaps the output or the residual", fn);
  return qg::launched(qg::launch_q2_gemm(w->codes, w->scales, (int)w->M, (int)w->K, w->group, xq, act_scale, accum,
                                         y, (int)nb, static_cast<float *>(ws), (hipStream_t)stream),
                      fn);
}

size_t qgemm_q2_batched_dual_ws_bytes(int64_t M, int64_t K, int group, int64_t nb) {
  return 2 * qgemm_q2_batched_ws_bytes(M, K, group, nb);
}

qg_status qgemm_q2_batched_dual(const qg_q2_weight *w0, const qg_q2_weight *w1, const int8_t *xq,
                                const int32_t *suma, const float *act_scale, float *y0, float *y1, int64_t nb,
                                void *ws, size_t ws_bytes, void *stream) {
  const char *fn = "qgemm_q2_batched_dual";
  (void)suma;  // the product forms code - 1 in its operand
  qg_status st = qg::check_q2_weight(w0, fn);
  if (st != QG_OK) return st;
  st = qg::check_q2_weight(w1, fn);
  if (st != QG_OK) return st;
  if (w0->M != w1->M || w0->K != w1->K || w0->group != w1->group)
    return fail(QG_EINVAL, "%s: the two matrices differ in shape or group", fn);
  if (!xq || !act_scale || !y0 || !y1) return fail(QG_EINVAL, "%s: null pointer", fn);
  if (nb < 1 || nb > (1 << 24)) return fail(QG_EINVAL, "%s: bad nb=%lld", fn, (long long)nb);
  if (nb * w0->M > (1LL << 40) || nb * w0->K > (1LL << 40)) return fail(QG_EINVAL, "%s: problem too large", fn);
  if (!aligned(w0->scales, 8) || !aligned(w1->scales, 8)) return fail(QG_EINVAL, "%s: scales plane not 8-byte aligned", fn);
  if (!aligned(xq, 16) || !aligned(y0, 16) || !aligned(y1, 16))
    return fail(QG_EINVAL, "%s: xq, y0 and y1 must be 16-byte aligned", fn);
  if (!aligned(act_scale, 4)) return fail(QG_EINVAL, "%s: misaligned pointer", fn);
  if (overlap(y0, y1, nb * w0->M)) return fail(QG_EINVAL, "%s: the two outputs overlap", fn);
  const size_t need = qgemm_q2_batched_dual_ws_bytes(w0->M, w0->K, w0->group, nb);
  if (need > 0 && (!ws || ws_bytes < need))
    return fail(QG_EINVAL, "%s: workspace %zu bytes < %zu needed", fn, ws ? ws_bytes : (size_t)0, need);
  if (need > 0 && !aligned(ws, 16)) return fail(QG_EINVAL, "%s: workspace not 16-byte aligned", fn);
  const size_t ybytes = (size_t)nb * w0->M * sizeof(float);
  if (need > 0 && (bytes_overlap(ws, need, y0, ybytes) || bytes_overlap(ws, need, y1, ybytes)))
    return fail(QG_EINVAL, "%s: workspace overlaps an output", fn);
  return qg::launched(qg::launch_q2_gemm(w0->codes, w0->scales, (int)w0->M, (int)w0->K, w0->group, xq,
                                         act_scale, nullptr, y0, (int)nb, static_cast<float *>(ws),
                                         (hipStream_t)stream, w1->codes, w1->scales, y1),
                      fn);
}

size_t qgemm_q8row_batched_ws_bytes(int64_t nb, int64_t K) {
  if (nb < 1 || K < 4 || K % 4 != 0 || K > qg::kGemmMaxK) return 0;
  size_t a, b, c;
  return qg::gemm_ws_layout(nb, K, &a, &b, &c);
}

static qg_status gemm_common(const char *fn, const void *qpacked, const float *rs, const qg::GemmAct &act, float *y,
                             int64_t nb, int64_t M, int64_t K, int xs_limbs, void *ws, size_t ws_bytes,
                             void *stream) {
  if (!qpacked || !rs || !y || !ws) return fail(QG_EINVAL, "%s: null pointer", fn);
  if (nb < 1 || nb > (1 << 24)) return fail(QG_EINVAL, "%s: bad nb=%lld", fn, (long long)nb);
  if (M < 1 || M > (1LL << 31) - 256) return fail(QG_EINVAL, "%s: bad M=%lld", fn, (long long)M);
  if (K < 4 || K % 4 != 0) return fail(QG_EINVAL, "%s: K=%lld must be a positive multiple of 4", fn, (long long)K);
  // Each limb's int32 sum over K is at most 128 * 128 * K in magnitude.
  if (K > qg::kGemmMaxK) return fail(QG_EINVAL, "%s: K=%lld above %d (int32 limb sums)", fn, (long long)K, qg::kGemmMaxK);
  if (nb * M > (1LL << 40) || qg::round_up(nb, 128) * qg::round_up(K, 64) * 3 > (1LL << 40))
    return fail(QG_EINVAL, "%s: problem too large", fn);
  if (xs_limbs != 0 && xs_limbs != 2 && xs_limbs != 3) return fail(QG_EINVAL, "%s: xs_limbs=%d must be 0, 2 or 3", fn, xs_limbs);
  if (!aligned(qpacked, 16) || !aligned(ws, 256))
    return fail(QG_EINVAL, "%s: qpacked must be 16-byte aligned, ws 256-byte aligned", fn);
  if (!aligned(rs, 4) || !aligned(y, 4)) return fail(QG_EINVAL, "%s: rs/y not 4-byte aligned", fn);
  const size_t need = qgemm_q8row_batched_ws_bytes(nb, K);
  if (ws_bytes < need) return fail(QG_EINVAL, "%s: workspace %zu bytes < %zu needed", fn, ws_bytes, need);
  const size_t abytes = (size_t)nb * K * sizeof(float);
  if (bytes_overlap(ws, need, y, (size_t)nb * M * sizeof(float)) || bytes_overlap(ws, need, act.xs, abytes) ||
      bytes_overlap(ws, need, act.g, abytes) || bytes_overlap(ws, need, act.u, abytes) ||
      bytes_overlap(ws, need, act.col, (size_t)K * sizeof(float)))
    return fail(QG_EINVAL, "%s: workspace overlaps the output or an activation input", fn);
  return qg::launched(qg::launch_q8row_gemm(qpacked, rs, act, y, (int)nb, (int)M, (int)K, xs_limbs, ws,
                                            (hipStream_t)stream), fn);
}

qg_status qgemm_q8row_batched(const void *qpacked, const float *rs, const float *xs, float *y,
                              int64_t nb, int64_t M, int64_t K, int xs_limbs, void *ws,
                              size_t ws_bytes, void *stream) {
  const char *fn = "qgemm_q8row_batched";
  if (!xs) return fail(QG_EINVAL, "%s: null pointer", fn);
  if (!aligned(xs, 16)) return fail(QG_EINVAL, "%s: xs must be 16-byte aligned", fn);
  return gemm_common(fn, qpacked, rs, qg::GemmAct{xs, nullptr, nullptr, nullptr}, y, nb, M, K, xs_limbs, ws, ws_bytes,
                     stream);
}

qg_status qgemm_q8row_batched_silu(const void *qpacked, const float *rs, const float *g, const float *u,
                                   const float *col, float *y, int64_t nb, int64_t M, int64_t K, int xs_limbs,
                                   void *ws, size_t ws_bytes, void *stream) {
  const char *fn = "qgemm_q8row_batched_silu";
  if (!g || !u) return fail(QG_EINVAL, "%s: null pointer", fn);
  if (!aligned(g, 16) || !aligned(u, 16) || (col && !aligned(col, 16)))
    return fail(QG_EINVAL, "%s: g, u and col must be 16-byte aligned", fn);
  return gemm_common(fn, qpacked, rs, qg::GemmAct{nullptr, g, u, col}, y, nb, M, K, xs_limbs, ws, ws_bytes, stream);
}

static bool spans_overlap(const float *a, int64_t na, const float *b, int64_t nb) { return a < b + nb && b < a + na; }

qg_status qact_silu_mul_pre(const float *g, const float *u, const float *col, float *act, int64_t rows, int64_t n,
                            void *stream) {
  const char *fn = "qact_silu_mul_pre";
  if (!g || !u || !act) return fail(QG_EINVAL, "%s: null pointer", fn);
  if (rows < 1 || n < 1 || n > (1 << 30) || rows > (1LL << 40) / n)
    return fail(QG_EINVAL, "%s: bad shape rows=%lld n=%lld", fn, (long long)rows, (long long)n);
  if (!aligned(g, 4) || !aligned(u, 4) || !aligned(act, 4) || (col && !aligned(col, 4)))
    return fail(QG_EINVAL, "%s: misaligned pointer", fn);
  const int64_t total = rows * n;
  if ((act != g && spans_overlap(act, total, g, total)) || (act != u && spans_overlap(act, total, u, total)))
    return fail(QG_EINVAL, "%s: act must be g, u or a separate buffer", fn);
  if (col && spans_overlap(act, total, col, n)) return fail(QG_EINVAL, "%s: act overlaps col", fn);
  const bool vec = n % 4 == 0 && aligned(g, 16) && aligned(u, 16) && aligned(act, 16) && (!col || aligned(col, 16));
  return qg::launched(qg::launch_silu_mul_pre(g, u, col, act, rows, (int)n, vec, (hipStream_t)stream), fn);
}

}  // extern "C"
