// act_quant.hip -- per-vector int8 activation quantisation for the Q2 GEMV.
//
// What is computed (qxmx qxmx_gpu.cpp page, gpu_rmsnorm_quant, quantisation
// part): act_scale = max|x| / 127, inv = 1/act_scale (0 when act_scale is 0),
// xq = clamp(round(x * inv), -128, 127) with round-half-away-from-zero, and
// suma[g] = sum of xq over each 64-wide group.  Every step is IEEE binary32:
// the division and the reciprocal are correctly rounded, the product is a
// single multiply, so the integers are bit-identical to any other binary32
// evaluation of the same rule (the helpers are in quant_rule.h).
//
// One workgroup of 1024 threads per vector: the vector is at most a few
// tens of KiB (the pages' widths are 5120 and 17408), so a single pass over
// L2-resident data is all it needs; the launch, not bandwidth, is its cost.
// A batch of token rows (the prefill form, gpu_rmsnorm_quant's n_tok on the
// same page) is one workgroup per row, each row with its own act_scale.
#include "qg_internal.h"
#include "quant_rule.h"

namespace qg {
namespace {

// One workgroup per vector: row blockIdx.x of a [rows][K] batch, each row
// with its own act_scale and group sums (rows = 1 for a single vector).
__global__ __launch_bounds__(kQuantThreads) void act_quant_i8_kernel(
    const float4 *__restrict__ x4, int n4, int *__restrict__ xq4,
    float *__restrict__ act_scale, int *__restrict__ suma) {
  __shared__ float red[kQuantThreads / 64];
  const int tid = threadIdx.x;
  const size_t row = blockIdx.x;
  x4 += row * n4;
  xq4 += row * n4;
  suma += row * (n4 / 16);
  act_scale += row;

  // Pass 1: exact max |x| (order-independent).
  float m = 0.0f;
  for (int i = tid; i < n4; i += kQuantThreads) m = fmaxf(m, abs_max4(x4[i]));
  const float inv = scale_and_inverse(block_max(m, red), act_scale);

  // Pass 2: quantise four values per thread.
  for (int i = tid; i < n4; i += kQuantThreads) quant_quad(i, x4[i], inv, xq4, suma);
}

}  // namespace

hipError_t launch_act_quant(const float *x, int rows, int K, int8_t *xq, float *act_scale,
                            int32_t *suma, hipStream_t stream) {
  act_quant_i8_kernel<<<rows, kQuantThreads, 0, stream>>>(
      reinterpret_cast<const float4 *>(x), K / 4, reinterpret_cast<int *>(xq), act_scale,
      reinterpret_cast<int *>(suma));
  return hipGetLastError();
}

}  // namespace qg
