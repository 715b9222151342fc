// producers.hip -- fused activation producers: the vector the next Q2 GEMV
// consumes is formed and quantised in one launch.
//
// What is computed (qxmx qxmx_gpu.cpp page, gpu_rmsnorm_quant,
// gpu_swiglu_quant, gpu_silu_mul_quant, gpu_sigmoid_mul_quant), every
// element step one IEEE binary32 operation, correctly rounded:
//   rmsnorm:  ms  = f32(sum_i x_i^2 / K), the sum of the (exact) binary64
//                   squares in binary64;
//             inv = 1 / sqrt(ms + eps);   v_i = (x_i * inv) * w_i
//   silu:     e = exp(-g_i);  t_i = (g_i / (1 + e)) * u_i
//   sigmoid:  e = exp(-g_i);  t_i = u_i * (1 / (1 + e))
// then the int8 rule of quant_rule.h on v or t.  exp is the correctly
// rounded binary32 exponential, evaluated in binary64 and rounded once (the
// page calls its runtime's single-precision exp, whose accuracy the pages do
// not fix; a correctly rounded one makes the result independent of the
// math library).  The binary64 sum of squares is reduced as a tree, whose
// rounding to binary32 equals a left-to-right sum's unless the two binary64
// sums fall on opposite sides of a binary32 rounding boundary.
//
// The column prescale (cortiq pages, silu_mul_pre) forms the q8_row down
// projection's f32 input act = silu(g) * u * col without quantising it:
// one element-wise launch over [rows][n] values, col shared by the rows.
//
// Batches of token rows (the prefill form: the page's n_tok) run one
// workgroup per row for the norm and the quantising step.
// RMSNorm + quantiser is one workgroup of 1024 threads per vector, as the
// quantiser: its passes re-read x and w from L2 (a few tens of KiB) instead
// of holding them, so any K the quantiser takes works.  The gated product
// spends about a hundred binary64 operations per element on exp, too much
// for one CU at K = 17408, so for one vector it is two launches: the product
// over the whole GPU (with per-workgroup maxima), then one workgroup
// quantising t.  A batch of 64 or more rows runs one workgroup per row in
// one launch, each holding its row of t in LDS between the product and the
// quantiser.
#include "qg_internal.h"
#include "gate_rule.h"
#include "quant_rule.h"

namespace qg {
namespace {

// HELD: rows of at most 2 * kQuantThreads quads, each thread's quads of x
// and w read once into registers for all three passes (the same arithmetic
// in the same order as re-reading them).
template <bool HELD>
__global__ __launch_bounds__(kQuantThreads) void rmsnorm_quant_kernel(
    const float4 *__restrict__ x4, const float4 *__restrict__ w4, int n4, float eps,
    int *__restrict__ xq4, float *__restrict__ act_scale, int *__restrict__ suma) {
  __shared__ double red_ss[kQuantThreads / 64];
  __shared__ float red_max[kQuantThreads / 64];
  const int tid = threadIdx.x;
  const size_t row = blockIdx.x;  // one workgroup per token row; w is shared
  x4 += row * n4;
  xq4 += row * n4;
  suma += row * (n4 / 16);
  act_scale += row;

  float4 xh[2], wh[2];
  if (HELD) {
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const int i = min(tid + h * kQuantThreads, n4 - 1);
      xh[h] = x4[i];
      wh[h] = w4[i];
    }
  }
  // f(i, x4[i], w4[i]) for this thread's quads i = tid, tid + kQuantThreads, ...
  auto each = [&](auto f) {
    if (HELD) {
#pragma unroll
      for (int h = 0; h < 2; h++)
        if (tid + h * kQuantThreads < n4) f(tid + h * kQuantThreads, xh[h], wh[h]);
    } else {
      for (int i = tid; i < n4; i += kQuantThreads) f(i, x4[i], w4[i]);
    }
  };

  double ss = 0.0;
  each([&](int, float4 v, float4) {
    ss += ((double)v.x * (double)v.x + (double)v.y * (double)v.y) +
          ((double)v.z * (double)v.z + (double)v.w * (double)v.w);
  });
  for (int off = 32; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  if ((tid & 63) == 0) red_ss[tid >> 6] = ss;
  __syncthreads();
  ss = 0.0;
#pragma unroll
  for (int w = 0; w < kQuantThreads / 64; w++) ss += red_ss[w];
  const float ms = (float)(ss / (double)(4 * n4));
  const float inv = __fdiv_rn(1.0f, sqrt_rn(__fadd_rn(ms, eps)));

  float m = 0.0f;
  each([&](int, float4 v, float4 w) { m = fmaxf(m, abs_max4(mul4(scale4(v, inv), w))); });
  const float qinv = scale_and_inverse(block_max(m, red_max), act_scale);
  each([&](int i, float4 v, float4 w) { quant_quad(i, mul4(scale4(v, inv), w), qinv, xq4, suma); });
}

template <int KIND>
__device__ inline float4 glu4(float4 g, float4 u) {
  return make_float4(glu1<KIND>(g.x, u.x), glu1<KIND>(g.y, u.y), glu1<KIND>(g.z, u.z), glu1<KIND>(g.w, u.w));
}

// Gated product, step 1 of 2, over the whole GPU: quad i of t (one per
// thread) and, per workgroup, the largest |t| of its quads, stored as float
// bits in part[blockIdx.x] of the token row's suma (which has room: at most
// K/1024 workgroups against K/64 entries).  t may be g or u itself: every
// quad is read and then written by one thread.
constexpr int kGluThreads = 256;

template <int KIND>
__global__ __launch_bounds__(kGluThreads) void glu_kernel(const float4 *g4, const float4 *u4, float4 *t4, int n4,
                                                          int *__restrict__ part) {
  __shared__ float red[kGluThreads / 64];
  const size_t row = blockIdx.y;  // token row; its partial maxima go to its own suma row
  g4 += row * n4;
  u4 += row * n4;
  t4 += row * n4;
  part += row * (n4 / 16);
  const int i = blockIdx.x * kGluThreads + threadIdx.x;
  float m = 0.0f;
  if (i < n4) {
    const float4 t = glu4<KIND>(g4[i], u4[i]);
    t4[i] = t;
    m = abs_max4(t);
  }
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  if (threadIdx.x == 0) {
    float r = red[0];
#pragma unroll
    for (int w = 1; w < kGluThreads / 64; w++) r = fmaxf(r, red[w]);
    part[blockIdx.x] = __float_as_int(r);
  }
}

// Step 2 of 2, one workgroup per token row: max|t| from the row's nparts
// partial maxima (all read before any group sum overwrites them), then the
// quantiser over t.
__global__ __launch_bounds__(kQuantThreads) void quant_from_parts_kernel(const float4 *__restrict__ t4, int n4,
                                                                         int nparts, int *__restrict__ xq4,
                                                                         float *__restrict__ act_scale,
                                                                         int *__restrict__ suma) {
  __shared__ float red_max[kQuantThreads / 64];
  const size_t row = blockIdx.x;  // one workgroup per token row
  t4 += row * n4;
  xq4 += row * n4;
  suma += row * (n4 / 16);
  act_scale += row;
  float m = 0.0f;
  for (int j = threadIdx.x; j < nparts; j += kQuantThreads) m = fmaxf(m, __int_as_float(suma[j]));
  const float qinv = scale_and_inverse(block_max(m, red_max), act_scale);
  for (int i = threadIdx.x; i < n4; i += kQuantThreads) quant_quad(i, t4[i], qinv, xq4, suma);
}

// The gated product and its quantiser for a batch of token rows in one
// launch: one workgroup per row computes the row's t (written out, and kept
// in LDS), its max|t|, then quantises t from LDS.  A batch of rows fills the
// GPU with the product's exponentials, so the single-row form's split over
// the whole GPU is not needed; t is not read back from memory.  Rows of up to
// kGluRowMaxQuads quads.
constexpr int kGluRowMaxQuads = 4608;  // K <= 18432: 72 KiB of LDS

template <int KIND>
__global__ __launch_bounds__(kQuantThreads) void glu_quant_rows_kernel(const float4 *g4, const float4 *u4, float4 *t4,
                                                                       int n4, int *__restrict__ xq4,
                                                                       float *__restrict__ act_scale,
                                                                       int *__restrict__ suma) {
  __shared__ float4 tl[kGluRowMaxQuads];
  __shared__ float red_max[kQuantThreads / 64];
  const size_t row = blockIdx.x;
  g4 += row * n4;
  u4 += row * n4;
  t4 += row * n4;
  xq4 += row * n4;
  suma += row * (n4 / 16);
  act_scale += row;
  float m = 0.0f;
  for (int i = threadIdx.x; i < n4; i += kQuantThreads) {
    const float4 t = glu4<KIND>(g4[i], u4[i]);  // t may be g or u: each quad read, then written, by one thread
    t4[i] = t;
    tl[i] = t;
    m = fmaxf(m, abs_max4(t));
  }
  // block_max's barrier also makes every thread's tl writes visible
  const float qinv = scale_and_inverse(block_max(m, red_max), act_scale);
  for (int i = threadIdx.x; i < n4; i += kQuantThreads) quant_quad(i, tl[i], qinv, xq4, suma);
}

// Column prescale: act[r][i] = silu(g[r][i]) * u[r][i] * col[i] (col null:
// 1).  Workgroup `blk` of the grid-stride loop takes chunk blk % nck of row
// blk / nck, 256 consecutive elements (VEC: quads) of that row; act may be g
// or u itself (each element is read and written by one thread).
constexpr int kPreThreads = 256;

template <bool VEC>
__global__ __launch_bounds__(kPreThreads) void silu_mul_pre_kernel(const float *g, const float *u,
                                                                   const float *__restrict__ col, float *act,
                                                                   int64_t rows, int n, int nck) {
  const int64_t nblk = rows * nck;
  for (int64_t blk = blockIdx.x; blk < nblk; blk += gridDim.x) {
    const int64_t r = blk / nck;
    const int i = (int)(blk % nck) * kPreThreads + threadIdx.x;  // element (quad) index in the row
    if (VEC) {
      const int n4 = n / 4;
      if (i >= n4) continue;
      const size_t k = (size_t)r * n4 + i;
      const float4 gv = reinterpret_cast<const float4 *>(g)[k];
      const float4 uv = reinterpret_cast<const float4 *>(u)[k];
      const float4 cv = col ? reinterpret_cast<const float4 *>(col)[i] : make_float4(1.0f, 1.0f, 1.0f, 1.0f);
      reinterpret_cast<float4 *>(act)[k] = make_float4(silu_pre1(gv.x, uv.x, cv.x), silu_pre1(gv.y, uv.y, cv.y),
                                                       silu_pre1(gv.z, uv.z, cv.z), silu_pre1(gv.w, uv.w, cv.w));
    } else {
      if (i >= n) continue;
      const size_t k = (size_t)r * n + i;
      act[k] = silu_pre1(g[k], u[k], col ? col[i] : 1.0f);
    }
  }
}

}  // namespace

hipError_t launch_silu_mul_pre(const float *g, const float *u, const float *col, float *act, int64_t rows, int n,
                               bool vec, hipStream_t stream) {
  const int per = vec ? n / 4 : n;
  const int nck = (per + kPreThreads - 1) / kPreThreads;
  const int64_t nblk = rows * nck;
  const int grid = (int)(nblk < 65536 ? nblk : 65536);
  if (vec)
    silu_mul_pre_kernel<true><<<grid, kPreThreads, 0, stream>>>(g, u, col, act, rows, n, nck);
  else
    silu_mul_pre_kernel<false><<<grid, kPreThreads, 0, stream>>>(g, u, col, act, rows, n, nck);
  return hipGetLastError();
}

hipError_t launch_quant_from_parts(const float *t, int rows, int K, int nparts, int8_t *xq, float *act_scale,
                                   int32_t *suma, hipStream_t stream) {
  quant_from_parts_kernel<<<rows, kQuantThreads, 0, stream>>>(reinterpret_cast<const float4 *>(t), K / 4, nparts,
                                                              reinterpret_cast<int *>(xq), act_scale,
                                                              reinterpret_cast<int *>(suma));
  return hipGetLastError();
}

hipError_t launch_rmsnorm_quant(const float *x, const float *w, int rows, int K, float eps, int8_t *xq,
                                float *act_scale, int32_t *suma, hipStream_t stream) {
  if (K / 4 <= 2 * kQuantThreads)
    rmsnorm_quant_kernel<true><<<rows, kQuantThreads, 0, stream>>>(
        reinterpret_cast<const float4 *>(x), reinterpret_cast<const float4 *>(w), K / 4, eps,
        reinterpret_cast<int *>(xq), act_scale, reinterpret_cast<int *>(suma));
  else
    rmsnorm_quant_kernel<false><<<rows, kQuantThreads, 0, stream>>>(
        reinterpret_cast<const float4 *>(x), reinterpret_cast<const float4 *>(w), K / 4, eps,
        reinterpret_cast<int *>(xq), act_scale, reinterpret_cast<int *>(suma));
  return hipGetLastError();
}

hipError_t launch_glu_quant(const float *g, const float *u, int rows, int K, int kind, float *t, int8_t *xq,
                            float *act_scale, int32_t *suma, hipStream_t stream) {
  const float4 *g4 = reinterpret_cast<const float4 *>(g);
  const float4 *u4 = reinterpret_cast<const float4 *>(u);
  float4 *t4 = reinterpret_cast<float4 *>(t);
  int *s = reinterpret_cast<int *>(suma);
  const int n4 = K / 4;
  if (rows >= 64 && n4 <= kGluRowMaxQuads) {  // a batch of rows: one launch
    if (kind == 0)
      glu_quant_rows_kernel<0><<<rows, kQuantThreads, 0, stream>>>(g4, u4, t4, n4, reinterpret_cast<int *>(xq),
                                                                    act_scale, s);
    else
      glu_quant_rows_kernel<1><<<rows, kQuantThreads, 0, stream>>>(g4, u4, t4, n4, reinterpret_cast<int *>(xq),
                                                                    act_scale, s);
    return hipGetLastError();
  }
  const int nparts = (n4 + kGluThreads - 1) / kGluThreads;
  const dim3 grid(nparts, rows);
  if (kind == 0)
    glu_kernel<0><<<grid, kGluThreads, 0, stream>>>(g4, u4, t4, n4, s);
  else
    glu_kernel<1><<<grid, kGluThreads, 0, stream>>>(g4, u4, t4, n4, s);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  quant_from_parts_kernel<<<rows, kQuantThreads, 0, stream>>>(t4, n4, nparts, reinterpret_cast<int *>(xq), act_scale,
                                                              s);
  return hipGetLastError();
}

}  // namespace qg
