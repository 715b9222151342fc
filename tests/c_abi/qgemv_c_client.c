/*
 * qgemv_c_client.c -- a plain C consumer of the library's C-ABI, with no
 * Python or framework in the process: it allocates device memory with the
 * HIP runtime, repacks and uploads the weights with the library's host
 * routines, runs a q8_row GEMV and a Q2 GEMV (activation quantiser, split-K)
 * through the device entry points on a stream of its own, and writes the
 * outputs.  The test that drives it writes the inputs and compares the
 * outputs with the oracle.
 *
 * Input file (little-endian): int64 M8, K8, M2, K2, group, split; then
 * q8 int8[M8][K8], rs f32[M8], xs f32[K8], the Q2 block blob
 * (qg_q2_blocks_bytes(M2, K2, group) bytes), x f32[K2].
 * Output file: y8 f32[M8], y2 f32[M2], xq int8[K2], act_scale f32,
 * suma int32[K2/64], y2x f32[M2] (the same Q2 GEMV by qgemv_q2_x: the
 * quantiser and the split's reduce inside one launch, its workspace
 * cleared once with hipMemset as the header asks).
 * Exit status 0 on success; otherwise a message names the failing call.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

#include <hip/hip_runtime_api.h>

#include "qgemv.h"

#define HIP_OK(call)                                                        \
  do {                                                                      \
    hipError_t e_ = (call);                                                 \
    if (e_ != hipSuccess) {                                                 \
      fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));    \
      return 2;                                                             \
    }                                                                       \
  } while (0)

#define QG_OK_(call)                                                        \
  do {                                                                      \
    qg_status s_ = (call);                                                  \
    if (s_ != QG_OK) {                                                      \
      fprintf(stderr, "%s failed: %s (%s)\n", #call, qg_status_string(s_), \
              qg_last_error());                                             \
      return 3;                                                             \
    }                                                                       \
  } while (0)

static void *read_n(FILE *f, size_t n) {
  void *p = malloc(n ? n : 1);
  if (p && n && fread(p, 1, n, f) != n) {
    free(p);
    return NULL;
  }
  return p;
}

int main(int argc, char **argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s input.bin output.bin\n", argv[0]);
    return 1;
  }
  FILE *in = fopen(argv[1], "rb");
  if (!in) return 1;
  int64_t hdr[6];
  if (fread(hdr, sizeof(int64_t), 6, in) != 6) return 1;
  const int64_t M8 = hdr[0], K8 = hdr[1], M2 = hdr[2], K2 = hdr[3];
  const int group = (int)hdr[4], split = (int)hdr[5];
  const size_t blob_bytes = qg_q2_blocks_bytes(M2, K2, group);
  int8_t *q8 = read_n(in, (size_t)(M8 * K8));
  float *rs = read_n(in, (size_t)M8 * 4);
  float *xs = read_n(in, (size_t)K8 * 4);
  void *blob = read_n(in, blob_bytes);
  float *x2 = read_n(in, (size_t)K2 * 4);
  fclose(in);
  if (!q8 || !rs || !xs || !blob || !x2) {
    fprintf(stderr, "short input file\n");
    return 1;
  }

  /* host repacks */
  const size_t p8 = qg_q8row_packed_bytes(M8, K8);
  void *q8p = malloc(p8);
  QG_OK_(qg_repack_q8row(q8, M8, K8, q8p, p8));
  const size_t cb = qg_q2_codes_bytes(M2, K2), sb = qg_q2_scales_bytes(M2, K2, group);
  void *codes = malloc(cb), *scales = malloc(sb);
  QG_OK_(qg_repack_q2(blob, blob_bytes, M2, K2, group, codes, cb, scales, sb));

  /* device buffers, owned here */
  void *d_q8p, *d_codes, *d_scales, *d_ws = NULL;
  float *d_rs, *d_xs, *d_y8, *d_x2, *d_y2, *d_sc;
  int8_t *d_xq;
  int32_t *d_suma;
  HIP_OK(hipMalloc(&d_q8p, p8));
  HIP_OK(hipMalloc((void **)&d_rs, (size_t)M8 * 4));
  HIP_OK(hipMalloc((void **)&d_xs, (size_t)K8 * 4));
  HIP_OK(hipMalloc((void **)&d_y8, (size_t)M8 * 4));
  HIP_OK(hipMalloc(&d_codes, cb));
  HIP_OK(hipMalloc(&d_scales, sb));
  HIP_OK(hipMalloc((void **)&d_x2, (size_t)K2 * 4));
  HIP_OK(hipMalloc((void **)&d_y2, (size_t)M2 * 4));
  HIP_OK(hipMalloc((void **)&d_xq, (size_t)K2));
  HIP_OK(hipMalloc((void **)&d_sc, 4));
  HIP_OK(hipMalloc((void **)&d_suma, (size_t)(K2 / 64) * 4));
  const size_t ws_bytes = qgemv_q2_ws_bytes(M2, K2, group, split);
  if (ws_bytes) HIP_OK(hipMalloc(&d_ws, ws_bytes));
  HIP_OK(hipMemcpy(d_q8p, q8p, p8, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_rs, rs, (size_t)M8 * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_xs, xs, (size_t)K8 * 4, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_codes, codes, cb, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_scales, scales, sb, hipMemcpyHostToDevice));
  HIP_OK(hipMemcpy(d_x2, x2, (size_t)K2 * 4, hipMemcpyHostToDevice));

  hipStream_t stream;
  HIP_OK(hipStreamCreate(&stream));
  QG_OK_(qgemv_q8row(d_q8p, d_rs, d_xs, d_y8, M8, K8, (void *)stream));
  qg_q2_weight w;
  w.codes = d_codes;
  w.scales = d_scales;
  w.M = M2;
  w.K = K2;
  w.group = group;
  w.reserved = 0;
  QG_OK_(qquant_act_i8(d_x2, K2, d_xq, d_sc, d_suma, (void *)stream));
  QG_OK_(qgemv_q2(&w, d_xq, d_suma, d_sc, d_y2, d_ws, ws_bytes, split, (void *)stream));
  float *d_y2x = NULL;
  void *d_wsx = NULL;
  HIP_OK(hipMalloc((void **)&d_y2x, (size_t)M2 * 4));
  const size_t wsx_bytes = qgemv_q2_x_ws_bytes(M2, K2, group, split);
  if (wsx_bytes) {
    HIP_OK(hipMalloc(&d_wsx, wsx_bytes));
    HIP_OK(hipMemset(d_wsx, 0, wsx_bytes));
  }
  QG_OK_(qgemv_q2_x(&w, d_x2, NULL, 0, NULL, d_y2x, d_wsx, wsx_bytes, split, (void *)stream));
  HIP_OK(hipStreamSynchronize(stream));

  float *y8 = malloc((size_t)M8 * 4), *y2 = malloc((size_t)M2 * 4), sc;
  int8_t *xq = malloc((size_t)K2);
  int32_t *suma = malloc((size_t)(K2 / 64) * 4);
  HIP_OK(hipMemcpy(y8, d_y8, (size_t)M8 * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(y2, d_y2, (size_t)M2 * 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(xq, d_xq, (size_t)K2, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(&sc, d_sc, 4, hipMemcpyDeviceToHost));
  HIP_OK(hipMemcpy(suma, d_suma, (size_t)(K2 / 64) * 4, hipMemcpyDeviceToHost));
  float *y2x = malloc((size_t)M2 * 4);
  HIP_OK(hipMemcpy(y2x, d_y2x, (size_t)M2 * 4, hipMemcpyDeviceToHost));
  FILE *out = fopen(argv[2], "wb");
  if (!out) return 1;
  fwrite(y8, 4, (size_t)M8, out);
  fwrite(y2, 4, (size_t)M2, out);
  fwrite(xq, 1, (size_t)K2, out);
  fwrite(&sc, 4, 1, out);
  fwrite(suma, 4, (size_t)(K2 / 64), out);
  fwrite(y2x, 4, (size_t)M2, out);
  fclose(out);
  HIP_OK(hipStreamDestroy(stream));
  printf("qgemv C client: ok (q8_row %lldx%lld, Q2 g%d %lldx%lld split %d)\n", (long long)M8, (long long)K8, group,
         (long long)M2, (long long)K2, split);
  return 0;
}
