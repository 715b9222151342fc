// gate_rule.h -- the gated products in IEEE binary32, shared by the
// producers and by the batched q8_row product's activation prep.
//
// What is computed (qxmx qxmx_gpu.cpp page, gpu_swiglu_quant /
// gpu_silu_mul_quant / gpu_sigmoid_mul_quant; cortiq-engine 0.5.43
// gpu_wgpu.rs page, silu_mul_pre; cortiq-engine 0.3.7 gpu_metal.rs page,
// silu_mul_pre and q8_mul_mm_silu), one correctly rounded binary32
// operation per step:
//   e = exp(-g);  silu:    (g / (1 + e)) * u
//                 sigmoid: u * (1 / (1 + e))
//   column prescale of the silu product: ((g / (1 + e)) * u) * col
// exp is the binary64 exponential rounded once to binary32 (correctly
// rounded unless the binary64 value lies within an ulp of a binary32
// rounding boundary), so the result does not depend on a math library's
// single-precision exp.
#pragma once

#include <hip/hip_runtime.h>

namespace qg {

__device__ inline float exp_neg(float g) { return (float)exp(-(double)g); }

template <int KIND>
__device__ inline float glu1(float g, float u) {
  const float den = __fadd_rn(1.0f, exp_neg(g));
  if (KIND == 0) return __fmul_rn(__fdiv_rn(g, den), u);
  return __fmul_rn(u, __fdiv_rn(1.0f, den));
}

// silu(g) * u * c; c = 1 (no column field) leaves the product unchanged.
__device__ inline float silu_pre1(float g, float u, float c) { return __fmul_rn(glu1<0>(g, u), c); }

}  // namespace qg
