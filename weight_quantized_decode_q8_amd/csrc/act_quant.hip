// act_quant.hip -- per-vector int8 activation quantisation for the Q2 GEMV.
//
// What is computed (qxmx qxmx_gpu.cpp page, gpu_rmsnorm_quant, quantisation
// part): act_scale = max|x| / 127, inv = 1/act_scale (0 when act_scale is 0),
// xq = clamp(round(x * inv), -128, 127) with round-half-away-from-zero, and
// suma[g] = sum of xq over each 64-wide group.  Every step is IEEE binary32:
// the division and the reciprocal are correctly rounded (HIP's default for
// '/'), the product is a single multiply, so the integers are bit-identical
// to any other binary32 evaluation of the same rule.
//
// One workgroup of 1024 threads per vector: the vector is at most a few
// tens of KiB (the pages' widths are 5120 and 17408), so a single pass over
// L2-resident data is all it needs; the launch, not bandwidth, is its cost.
#include "qg_internal.h"

namespace qg {
namespace {

constexpr int kThreads = 1024;

__device__ inline int quant1(float v, float inv) {
  float r = roundf(v * inv);
  r = fminf(fmaxf(r, -128.0f), 127.0f);
  return (int)r;
}

__global__ __launch_bounds__(kThreads) void act_quant_i8_kernel(
    const float4 *__restrict__ x4, int n4, int *__restrict__ xq4,
    float *__restrict__ act_scale, int *__restrict__ suma) {
  __shared__ float wave_max[kThreads / 64];
  const int tid = threadIdx.x;

  // Pass 1: exact max |x| (order-independent).
  float m = 0.0f;
  for (int i = tid; i < n4; i += kThreads) {
    float4 v = x4[i];
    m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
  }
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((tid & 63) == 0) wave_max[tid >> 6] = m;
  __syncthreads();
  float amax = wave_max[0];
#pragma unroll
  for (int w = 1; w < kThreads / 64; w++) amax = fmaxf(amax, wave_max[w]);

  const float sc = amax / 127.0f;
  const float inv = sc > 0.0f ? 1.0f / sc : 0.0f;
  if (tid == 0) *act_scale = sc;

  // Pass 2: quantise four values per thread; 16 consecutive threads cover
  // one 64-wide group (n4 and kThreads are multiples of 16, so a group's
  // threads are all active or all idle together).
  for (int i = tid; i < n4; i += kThreads) {
    float4 v = x4[i];
    int a = quant1(v.x, inv), b = quant1(v.y, inv), c = quant1(v.z, inv), d = quant1(v.w, inv);
    xq4[i] = (a & 0xff) | ((b & 0xff) << 8) | ((c & 0xff) << 16) | ((unsigned)(d & 0xff) << 24);
    int s = a + b + c + d;
    s += __shfl_xor(s, 1);
    s += __shfl_xor(s, 2);
    s += __shfl_xor(s, 4);
    s += __shfl_xor(s, 8);
    if ((i & 15) == 0) suma[i >> 4] = s;
  }
}

}  // namespace

hipError_t launch_act_quant(const float *x, int K, int8_t *xq, float *act_scale,
                            int32_t *suma, hipStream_t stream) {
  act_quant_i8_kernel<<<1, kThreads, 0, stream>>>(
      reinterpret_cast<const float4 *>(x), K / 4, reinterpret_cast<int *>(xq), act_scale,
      reinterpret_cast<int *>(suma));
  return hipGetLastError();
}

}  // namespace qg
