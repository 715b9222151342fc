// quant_rule.h -- the per-vector int8 quantisation rule as device helpers
// for one workgroup of kQuantThreads threads that owns a whole vector.
//
// The rule (qxmx qxmx_gpu.cpp page, gpu_rmsnorm_quant and its siblings
// gpu_swiglu_quant, gpu_silu_mul_quant, gpu_sigmoid_mul_quant):
// act_scale = max|v| / 127, inv = 1/act_scale (0 when act_scale is 0),
// xq = clamp(round(v * inv), -128, 127) with round-half-away-from-zero, and
// suma[g] = sum of xq over each 64-wide group.  Every step is one IEEE
// binary32 operation, correctly rounded, so the integers equal those of any
// other binary32 evaluation of the rule.
//
// The vector is handled as float4 quads: thread t takes quads t, t + 1024,
// ...; the 16 consecutive threads of one 16-lane row cover one 64-wide group
// (the quad count and kQuantThreads are multiples of 16, so a group's
// threads are active or idle together).
#pragma once

#include <hip/hip_runtime.h>

namespace qg {

constexpr int kQuantThreads = 1024;

__device__ inline int quant1(float v, float inv) {
  float r = roundf(__fmul_rn(v, inv));
  r = fminf(fmaxf(r, -128.0f), 127.0f);
  return (int)r;
}

__device__ inline float abs_max4(float4 v) {
  return fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
}

// Largest of every thread's m (exact, order-independent).  `red` holds
// kQuantThreads / 64 floats of LDS; ends with a barrier-free read.
__device__ inline float block_max(float m, float *red) {
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  __syncthreads();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < kQuantThreads / 64; w++) r = fmaxf(r, red[w]);
  return r;
}

// act_scale and its reciprocal from max|v|; thread 0 stores act_scale.
__device__ inline float scale_and_inverse(float amax, float *act_scale) {
  const float sc = __fdiv_rn(amax, 127.0f);
  if (threadIdx.x == 0) *act_scale = sc;
  return sc > 0.0f ? __fdiv_rn(1.0f, sc) : 0.0f;
}

// Running sum of s over the lanes of this lane's 16-lane row up to this
// lane (DPP row shifts, no LDS traffic): the row's last lane holds the sum
// of all 16.  Every lane of the row must be active.
__device__ inline int row16_prefix_sum(int s) {
  s += __builtin_amdgcn_update_dpp(0, s, 0x111, 0xF, 0xF, true);  // row_shr:1
  s += __builtin_amdgcn_update_dpp(0, s, 0x112, 0xF, 0xF, true);  // row_shr:2
  s += __builtin_amdgcn_update_dpp(0, s, 0x114, 0xF, 0xF, true);  // row_shr:4
  s += __builtin_amdgcn_update_dpp(0, s, 0x118, 0xF, 0xF, true);  // row_shr:8
  return s;
}

// Quantise quad i (values v) into xq4[i]; the 16 threads of a group (one
// 16-lane row, since i and the thread index advance together in multiples
// of 16) combine their sums into suma[i / 16].
__device__ inline void quant_quad(int i, float4 v, float inv, int *__restrict__ xq4, int *__restrict__ suma) {
  const int a = quant1(v.x, inv), b = quant1(v.y, inv), c = quant1(v.z, inv), d = quant1(v.w, inv);
  xq4[i] = (a & 0xff) | ((b & 0xff) << 8) | ((c & 0xff) << 16) | ((unsigned)(d & 0xff) << 24);
  const int s = row16_prefix_sum(a + b + c + d);
  if ((i & 15) == 15) suma[i >> 4] = s;
}

// Element-wise binary32 products of a quad (each one rounding), for the
// RMSNorm producers: v = (x * inv) * w.
__device__ inline float4 mul4(float4 a, float4 b) {
  return make_float4(__fmul_rn(a.x, b.x), __fmul_rn(a.y, b.y), __fmul_rn(a.z, b.z), __fmul_rn(a.w, b.w));
}

__device__ inline float4 scale4(float4 a, float s) {
  return make_float4(__fmul_rn(a.x, s), __fmul_rn(a.y, s), __fmul_rn(a.z, s), __fmul_rn(a.w, s));
}

// Correctly rounded binary32 square root: the binary64 root (correctly
// rounded) rounded once more to binary32, which for sqrt gives the correctly
// rounded binary32 result (53 >= 2 * 24 + 2).  The single-precision
// hardware root is not correctly rounded.
__device__ inline float sqrt_rn(float a) { return (float)sqrt((double)a); }

}  // namespace qg
