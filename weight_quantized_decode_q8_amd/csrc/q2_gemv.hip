// q2_gemv.hip -- batch-1 Q2 x int8 GEMV on the T64 tiled image, split-K.
//
// What is computed (qxmx qxmx_gpu.cpp page, gemv_dpas8 and gemv_reduce):
//   for each row o and 64-wide unit u
//       dot[o,u] = sum_{i in u} (code_i - 1) * xq_i            (exact int32)
//   and y[o] = act_scale * sum_u d(o,u) * dot[o,u].
// The page forms the integer dot as sum code*xq minus suma[u] (the sum of the
// unit's activations), which is what is done here too: the 2-bit codes are
// used as unsigned bytes 0..3 and the correction is one subtract per unit.
// A 128-wide group is two units sharing d (repack_q2_g128 on the same page);
// its two corrected dots are added as integers before the single scale FMA.
//
// gfx950 design (the page's is an Intel DPAS kernel with SLM staging):
//  - one lane per row, a 64-row tile per wavefront, so there is no
//    cross-lane reduction; the T64 code plane makes each wavefront load of
//    a unit 1 KiB contiguous, and the scale plane 128 B contiguous;
//  - the codes' bit order inside a unit (fixed by the repack) makes
//    (word >> 2a) & 0x03030303 four code bytes that line up with one
//    natural-order int8 activation word: 7 bit ops + 4 v_dot4_i32_i8 per
//    16 weights, no shuffles and no lookup tables;
//  - the activation words and suma are wave-uniform: scalar loads into
//    SGPRs, used directly as the dot4 operand;
//  - K is split over the workgroup's 8 or 16 waves (LDS combine) and, for
//    large matrices whose row tiles cannot fill 256 CUs, over blockIdx.y
//    splits whose f32 partials [split][Mp] are summed in fixed order by a
//    second kernel.
#include "qg_internal.h"

namespace qg {
namespace {

constexpr unsigned kCodeMask = 0x03030303u;

typedef int i32x4 __attribute__((ext_vector_type(4)));
// Wave-uniform reads (activation words, suma) through the constant address
// space become scalar loads; neither buffer is written during the kernel.
typedef const __attribute__((address_space(4))) i32x4 uniform_i32x4;
typedef const __attribute__((address_space(4))) int uniform_i32;

// Corrected dot of one unit: sum_{64 weights} code*xq - suma.
__device__ inline int unit_dot(const i32x4 c, const uniform_i32x4 *xw, int sa) {
  const i32x4 x0 = xw[0], x1 = xw[1], x2 = xw[2], x3 = xw[3];
  int p = 0;
  p = __builtin_amdgcn_sdot4((int)((unsigned)c.x & kCodeMask), x0.x, p, false);
  p = __builtin_amdgcn_sdot4((int)(((unsigned)c.x >> 2) & kCodeMask), x0.y, p, false);
  p = __builtin_amdgcn_sdot4((int)(((unsigned)c.x >> 4) & kCodeMask), x0.z, p, false);
  p = __builtin_amdgcn_sdot4((int)(((unsigned)c.x >> 6) & kCodeMask), x0.w, p, false);
  p = __builtin_amdgcn_sdot4((int)((unsigned)c.y & kCodeMask), x1.x, p, false);
  p = __builtin_amdgcn_sdot4((int)(((unsigned)c.y >> 2) & kCodeMask), x1.y, p, false);
  p = __builtin_amdgcn_sdot4((int)(((unsigned)c.y >> 4) & kCodeMask), x1.z, p, false);
  p = __builtin_amdgcn_sdot4((int)(((unsigned)c.y >> 6) & kCodeMask), x1.w, p, false);
  p = __builtin_amdgcn_sdot4((int)((unsigned)c.z & kCodeMask), x2.x, p, false);
  p = __builtin_amdgcn_sdot4((int)(((unsigned)c.z >> 2) & kCodeMask), x2.y, p, false);
  p = __builtin_amdgcn_sdot4((int)(((unsigned)c.z >> 4) & kCodeMask), x2.z, p, false);
  p = __builtin_amdgcn_sdot4((int)(((unsigned)c.z >> 6) & kCodeMask), x2.w, p, false);
  p = __builtin_amdgcn_sdot4((int)((unsigned)c.w & kCodeMask), x3.x, p, false);
  p = __builtin_amdgcn_sdot4((int)(((unsigned)c.w >> 2) & kCodeMask), x3.y, p, false);
  p = __builtin_amdgcn_sdot4((int)(((unsigned)c.w >> 4) & kCodeMask), x3.z, p, false);
  p = __builtin_amdgcn_sdot4((int)(((unsigned)c.w >> 6) & kCodeMask), x3.w, p, false);
  return p - sa;
}

// IEEE binary16 -> f32 by the hardware convert (exact, subnormals included).
__device__ inline float half_bits_to_f32(unsigned short h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// grid = (row tiles, splits); block = kWaves wavefronts sharing one tile.
// UPG = units (of 64 weights) per scale group: 1 for g64, 2 for g128.
// GPB = groups handled per unrolled step (GPB*UPG code loads in flight).
template <int UPG, int GPB, bool kDots, int kWaves>
__global__ __launch_bounds__(64 * kWaves) void q2_gemv_t64_kernel(
    const i32x4 *__restrict__ codes, const unsigned short *__restrict__ scales,
    const int8_t *__restrict__ xq, const int *__restrict__ suma,
    const float *__restrict__ act_scale, float *__restrict__ out, int *__restrict__ dots, int M,
    int Mp, int K, int S) {
  __shared__ float red[kWaves - 1][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tile = blockIdx.x;
  const int split = blockIdx.y;
  const int nunits = K / 64;
  const int ngroups = nunits / UPG;

  // Groups of this split, then of this wave: contiguous ranges.
  const int gps = (ngroups + S - 1) / S;
  const int gs0 = min(ngroups, split * gps);
  const int gs1 = min(ngroups, gs0 + gps);
  const int per = (gs1 - gs0 + kWaves - 1) / kWaves;
  const int g0 = min(gs1, gs0 + wave * per);
  const int g1 = min(gs1, g0 + per);

  const i32x4 *cp = codes + (size_t)tile * nunits * 64 + lane;
  const unsigned short *sp = scales + (size_t)tile * ngroups * 64 + lane;
  const uniform_i32x4 *xw = (const uniform_i32x4 *)xq;
  const uniform_i32 *sa = (const uniform_i32 *)suma;
  const int o = tile * 64 + lane;

  float acc = 0.0f;
  int g = g0;
  for (; g + GPB <= g1; g += GPB) {
    i32x4 c[GPB * UPG];
    unsigned short dh[GPB];
#pragma unroll
    for (int v = 0; v < GPB * UPG; v++)
      c[v] = __builtin_nontemporal_load(cp + (size_t)(g * UPG + v) * 64);
#pragma unroll
    for (int j = 0; j < GPB; j++) dh[j] = __builtin_nontemporal_load(sp + (size_t)(g + j) * 64);
#pragma unroll
    for (int j = 0; j < GPB; j++) {
      int p = 0;
#pragma unroll
      for (int v = 0; v < UPG; v++) {
        const int u = (g + j) * UPG + v;
        const int cd = unit_dot(c[j * UPG + v], xw + (size_t)u * 4, sa[u]);
        if (kDots && o < M) dots[(size_t)o * nunits + u] = cd;
        p += cd;
      }
      acc = fmaf(half_bits_to_f32(dh[j]), (float)p, acc);
    }
  }
  for (; g < g1; g++) {
    const unsigned short dh = __builtin_nontemporal_load(sp + (size_t)g * 64);
    int p = 0;
#pragma unroll
    for (int v = 0; v < UPG; v++) {
      const int u = g * UPG + v;
      const int cd = unit_dot(__builtin_nontemporal_load(cp + (size_t)u * 64), xw + (size_t)u * 4, sa[u]);
      if (kDots && o < M) dots[(size_t)o * nunits + u] = cd;
      p += cd;
    }
    acc = fmaf(half_bits_to_f32(dh), (float)p, acc);
  }

  if (wave > 0) red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < kWaves - 1; w++) acc += red[w][lane];
    if (S == 1) {
      if (o < M) out[o] = acc * act_scale[0];
    } else {
      out[(size_t)split * Mp + o] = acc;
    }
  }
}

// y[o] = act_scale * sum_s part[s][o], the splits added in fixed order
// (gemv_reduce on the qxmx page).
__global__ __launch_bounds__(256) void q2_splitk_reduce_kernel(const float *__restrict__ part, int S,
                                                               int Mp, int M,
                                                               const float *__restrict__ act_scale,
                                                               float *__restrict__ y) {
  const int o = blockIdx.x * 256 + threadIdx.x;
  if (o >= M) return;
  float s = 0.0f;
  for (int k = 0; k < S; k++) s += part[(size_t)k * Mp + o];
  y[o] = s * act_scale[0];
}

template <int UPG, int GPB, int W>
hipError_t launch_main(const i32x4 *c, const unsigned short *s, int M, int K, const int8_t *xq,
                       const int32_t *suma, const float *act_scale, float *out, int32_t *dots,
                       int S, hipStream_t stream) {
  const int tiles = (M + 63) / 64;
  const dim3 grid(tiles, S);
  if (dots)
    q2_gemv_t64_kernel<UPG, GPB, true, W><<<grid, 64 * W, 0, stream>>>(
        c, s, xq, suma, act_scale, out, dots, M, tiles * 64, K, S);
  else
    q2_gemv_t64_kernel<UPG, GPB, false, W><<<grid, 64 * W, 0, stream>>>(
        c, s, xq, suma, act_scale, out, nullptr, M, tiles * 64, K, S);
  return hipGetLastError();
}

// Waves per tile: 8 when the row tiles alone fill the CUs, else 16 so that
// each of the fewer workgroups keeps more loads in flight.
template <int UPG, int GPB>
hipError_t launch_typed(const void *codes, const void *scales, int M, int K, const int8_t *xq,
                        const int32_t *suma, const float *act_scale, float *y, int32_t *dots,
                        float *partials, int S, hipStream_t stream) {
  const int tiles = (M + 63) / 64;
  const int Mp = tiles * 64;
  float *out = S == 1 ? y : partials;
  const i32x4 *c = reinterpret_cast<const i32x4 *>(codes);
  const unsigned short *s = reinterpret_cast<const unsigned short *>(scales);
  hipError_t e = tiles >= 256 ? launch_main<UPG, GPB, 8>(c, s, M, K, xq, suma, act_scale, out, dots, S, stream)
                              : launch_main<UPG, GPB, 16>(c, s, M, K, xq, suma, act_scale, out, dots, S, stream);
  if (e != hipSuccess || S == 1) return e;
  q2_splitk_reduce_kernel<<<(M + 255) / 256, 256, 0, stream>>>(partials, S, Mp, M, act_scale, y);
  return hipGetLastError();
}

}  // namespace

int q2_auto_split(int64_t M, int64_t K, int group) {
  // A second (reduce) launch costs about as much as streaming several MB, so
  // K is split only for large matrices whose row tiles cannot fill the 256
  // CUs: then into the fewest power-of-two ranges giving >= 256 workgroups
  // (and at least one scale group per wave).
  const int64_t tiles = (M + 63) / 64;
  const int64_t ngroups = K / group;
  const int64_t bytes = M * ngroups * (2 + group / 4);
  if (tiles >= 256 || bytes < (16LL << 20)) return 1;
  int S = 1;
  while (S < kMaxSplit && tiles * S < 256 && ngroups / (2 * S) >= 16) S *= 2;
  return S;
}

hipError_t launch_q2_gemv(const void *codes, const void *scales, int M, int K, int group,
                          const int8_t *xq, const int32_t *suma, const float *act_scale,
                          float *y, int32_t *dots, float *partials, int split,
                          hipStream_t stream) {
  if (group == 64)
    return launch_typed<1, 4>(codes, scales, M, K, xq, suma, act_scale, y, dots, partials, split,
                              stream);
  return launch_typed<2, 2>(codes, scales, M, K, xq, suma, act_scale, y, dots, partials, split,
                            stream);
}

}  // namespace qg
