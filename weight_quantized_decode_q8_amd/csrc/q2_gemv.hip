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
//    natural-order int8 activation word; fields 1 and 3 are used in place
//    as 4 x code (q2_unit.h): 5 bit ops + 4 v_dot4_i32_i8 per 16 weights,
//    no shuffles and no lookup tables;
//  - the activation words and suma are wave-uniform: scalar loads into
//    SGPRs, used directly as the dot4 operand;
//  - K is split over the workgroup's 8 or 16 waves (LDS combine) and, for
//    large matrices whose row tiles cannot fill 256 CUs, over blockIdx.y
//    splits whose f32 partials [split][Mp] are summed in fixed order by a
//    second kernel.
//
// Every launch runs a table of matrices (one Q2Job each), whose row tiles
// follow one another in the grid.  That serves three extensions: the FFN
// gate and up matrices against one shared quantized activation in one
// launch (gemv_dpas8_dual on the same page), a residual added in the
// epilogue (the accum argument of gemv_dpas8): y = (acc * act_scale) + accum
// as two f32 roundings, the order of an unfused GEMV followed by a separate
// residual add, and up to 16 independent GEMVs in one launch against the
// fixed cost of each launch (matvec_pair on the cortiq-engine 0.5.43
// gpu_wgpu.rs page lays two jobs end to end in one row space the same way;
// matvec_batch on the 0.3.7 gpu_metal.rs page groups several per command
// buffer).  The gate/up and residual forms
// equal the unfused calls bit for bit when the split is the same, which the
// launchers guarantee: waves per tile and the automatic split depend only on
// one matrix's shape.
#include "gate_rule.h"
#include "q2_unit.h"
#include "qg_internal.h"

namespace qg {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
// Wave-uniform reads (activation words, suma) through the constant address
// space become scalar loads; neither buffer is written during the kernel.
typedef const __attribute__((address_space(4))) i32x4 uniform_i32x4;
typedef const __attribute__((address_space(4))) int uniform_i32;

// Corrected dot of one unit: sum_{64 weights} code*xq - suma.
__device__ inline int unit_dot(const i32x4 c, const uniform_i32x4 *xw, int sa) {
  return q2_unit_dot(c, xw[0], xw[1], xw[2], xw[3], sa);
}

// IEEE binary16 -> f32 by the hardware convert (exact, subnormals included).
__device__ inline float half_bits_to_f32(unsigned short h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

// One matrix of a launch: its planes and activation, where its result goes
// (y when S = 1, else the partials [S][Mp]) and the optional residual (S = 1
// only; with splits the reduce kernel adds it).
struct Q2Job {
  const i32x4 *codes;
  const unsigned short *scales;
  const int8_t *xq;
  const int *suma;
  const float *act_scale;
  float *out;
  const float *accum;
  int M, K;
};

// The matrices of one launch, passed by value in the kernel arguments: job
// j owns the row tiles [tile_end[j-1], tile_end[j]) of the grid.
struct Q2Batch {
  Q2Job job[kMaxQ2Jobs];
  int tile_end[kMaxQ2Jobs];
  int njobs;
};

// This workgroup's job, selected with constant indices only, so the table
// is read from the kernel-argument segment (scalar loads, no private copy).
__device__ inline void pick_job(const Q2Batch &b, int block, Q2Job &job, int &tile) {
  int j = 0;
#pragma unroll
  for (int i = 0; i < kMaxQ2Jobs - 1; i++) j += (i + 1 < b.njobs && block >= b.tile_end[i]) ? 1 : 0;
  job = b.job[0];
  int first = 0;
#pragma unroll
  for (int i = 1; i < kMaxQ2Jobs; i++)
    if (i == j) {
      job = b.job[i];
      first = b.tile_end[i - 1];
    }
  tile = block - first;
}

// f32 multiply and add, each rounded once (never contracted to an FMA).
__device__ inline float scale_add(float acc, float sc, const float *accum, int o) {
  const float y = __fmul_rn(acc, sc);
  return accum ? __fadd_rn(y, accum[o]) : y;
}

// grid = (row tiles of all jobs, splits); block = kWaves wavefronts sharing
// one tile.  UPG = units (of 64 weights) per scale group: 1 for g64, 2 for
// g128.  GPB = groups handled per unrolled step (GPB*UPG code loads in
// flight).  dots (kDots, one-job launches only) receives [M][K/64] int32.
template <int UPG, int GPB, bool kDots, int kWaves>
__global__ __launch_bounds__(64 * kWaves) void q2_gemv_t64_kernel(Q2Batch batch, int *__restrict__ dots, int S) {
  __shared__ float red[kWaves - 1][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  Q2Job job;
  int tile;
  pick_job(batch, blockIdx.x, job, tile);
  const i32x4 *__restrict__ codes = job.codes;
  const unsigned short *__restrict__ scales = job.scales;
  float *__restrict__ out = job.out;
  const int M = job.M, K = job.K;
  const int Mp = (M + 63) / 64 * 64;
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
  const uniform_i32x4 *xw = (const uniform_i32x4 *)job.xq;
  const uniform_i32 *sa = (const uniform_i32 *)job.suma;
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
      if (o < M) out[o] = scale_add(acc, job.act_scale[0], job.accum, o);
    } else {
      out[(size_t)split * Mp + o] = acc;
    }
  }
}

// y[o] = act_scale * sum_s part[s][o] (+ accum[o]), the splits added in
// fixed order (gemv_reduce on the qxmx page).  blockIdx.y picks job 0 or 1
// (one matrix, or the gate/up pair); job j's partials are job.out[s*Mp+o].
__global__ __launch_bounds__(256) void q2_splitk_reduce_kernel(Q2Batch batch, float *y0, float *y1,
                                                               const float *accum, int S) {
  const bool second = blockIdx.y != 0;
  const Q2Job job = second ? batch.job[1] : batch.job[0];
  const int M = job.M, Mp = (M + 63) / 64 * 64;
  const int o = blockIdx.x * 256 + threadIdx.x;
  if (o >= M) return;
  float *y = second ? y1 : y0;
  float s = 0.0f;
  for (int k = 0; k < S; k++) s += job.out[(size_t)k * Mp + o];
  y[o] = scale_add(s, job.act_scale[0], accum, o);
}

// Gate and up rows of one tile in one workgroup, then the gated product
// (cortiq-engine 0.5.43 gpu_wgpu.rs page, moe_gate_up: one workgroup does
// both row dots of a row and writes silu(g) * u).  Each matrix's dot is
// accumulated exactly as q2_gemv_t64_kernel accumulates it (same groups per
// wave, same order, same wave combine), g and u are each rounded once as
// fl(acc * act_scale), and t = glu(g, u) follows the producers' rule, so t
// equals the dual GEMV followed by the gated product bit for bit.  Lane 0
// of wave 0 then stores the tile's largest |t| as float bits in part[tile]
// for the quantiser's second step (quant_from_parts_kernel).
template <int UPG, int GPB, int kWaves, int KIND>
__global__ __launch_bounds__(64 * kWaves) void q2_gate_up_glu_kernel(Q2Job gate, Q2Job up, float *__restrict__ t,
                                                                     int *__restrict__ part) {
  __shared__ float red[2][kWaves - 1][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tile = blockIdx.x;
  const int M = gate.M, K = gate.K;
  const int nunits = K / 64;
  const int ngroups = nunits / UPG;
  const int per = (ngroups + kWaves - 1) / kWaves;
  const int g0 = min(ngroups, wave * per);
  const int g1 = min(ngroups, g0 + per);
  const i32x4 *cg = gate.codes + (size_t)tile * nunits * 64 + lane;
  const i32x4 *cu = up.codes + (size_t)tile * nunits * 64 + lane;
  const unsigned short *sg = gate.scales + (size_t)tile * ngroups * 64 + lane;
  const unsigned short *su = up.scales + (size_t)tile * ngroups * 64 + lane;
  const uniform_i32x4 *xw = (const uniform_i32x4 *)gate.xq;
  const uniform_i32 *sa = (const uniform_i32 *)gate.suma;
  const int o = tile * 64 + lane;

  float ag = 0.0f, au = 0.0f;
  int g = g0;
  for (; g + GPB <= g1; g += GPB) {
    i32x4 c0[GPB * UPG], c1[GPB * UPG];
    unsigned short d0[GPB], d1[GPB];
#pragma unroll
    for (int v = 0; v < GPB * UPG; v++) {
      c0[v] = __builtin_nontemporal_load(cg + (size_t)(g * UPG + v) * 64);
      c1[v] = __builtin_nontemporal_load(cu + (size_t)(g * UPG + v) * 64);
    }
#pragma unroll
    for (int j = 0; j < GPB; j++) {
      d0[j] = __builtin_nontemporal_load(sg + (size_t)(g + j) * 64);
      d1[j] = __builtin_nontemporal_load(su + (size_t)(g + j) * 64);
    }
#pragma unroll
    for (int j = 0; j < GPB; j++) {
      int p0 = 0, p1 = 0;
#pragma unroll
      for (int v = 0; v < UPG; v++) {
        const int u = (g + j) * UPG + v;
        p0 += unit_dot(c0[j * UPG + v], xw + (size_t)u * 4, sa[u]);
        p1 += unit_dot(c1[j * UPG + v], xw + (size_t)u * 4, sa[u]);
      }
      ag = fmaf(half_bits_to_f32(d0[j]), (float)p0, ag);
      au = fmaf(half_bits_to_f32(d1[j]), (float)p1, au);
    }
  }
  for (; g < g1; g++) {
    int p0 = 0, p1 = 0;
#pragma unroll
    for (int v = 0; v < UPG; v++) {
      const int u = g * UPG + v;
      p0 += unit_dot(__builtin_nontemporal_load(cg + (size_t)u * 64), xw + (size_t)u * 4, sa[u]);
      p1 += unit_dot(__builtin_nontemporal_load(cu + (size_t)u * 64), xw + (size_t)u * 4, sa[u]);
    }
    ag = fmaf(half_bits_to_f32(__builtin_nontemporal_load(sg + (size_t)g * 64)), (float)p0, ag);
    au = fmaf(half_bits_to_f32(__builtin_nontemporal_load(su + (size_t)g * 64)), (float)p1, au);
  }

  if (wave > 0) {
    red[0][wave - 1][lane] = ag;
    red[1][wave - 1][lane] = au;
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < kWaves - 1; w++) {
      ag += red[0][w][lane];
      au += red[1][w][lane];
    }
    const float sc = gate.act_scale[0];
    float m = 0.0f;
    if (o < M) {
      const float tv = glu1<KIND>(__fmul_rn(ag, sc), __fmul_rn(au, sc));
      t[o] = tv;
      m = fabsf(tv);
    }
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if (lane == 0) part[tile] = __float_as_int(m);
  }
}

// The same with the two matrices on the two halves of a 2W-wave workgroup:
// waves 0..W-1 accumulate the gate tile and waves W..2W-1 the up tile, each
// half exactly as a W-wave q2_gemv_t64_kernel workgroup does (same groups per
// wave, same combine order), so the loads in flight match the dual GEMV's.
template <int UPG, int GPB, int W, int KIND>
__global__ __launch_bounds__(128 * W) void q2_gate_up_glu_halves_kernel(Q2Job gate, Q2Job up,
                                                                        float *__restrict__ t,
                                                                        int *__restrict__ part) {
  __shared__ float red[2][W - 1][64];
  __shared__ float fin[64];
  const int lane = threadIdx.x & 63;
  const int wave2 = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int mat = wave2 / W;        // 0 gate, 1 up
  const int wave = wave2 % W;       // wave within the matrix's half
  const Q2Job &job = mat ? up : gate;
  const int tile = blockIdx.x;
  const int M = gate.M, K = gate.K;
  const int nunits = K / 64;
  const int ngroups = nunits / UPG;
  const int per = (ngroups + W - 1) / W;
  const int g0 = min(ngroups, wave * per);
  const int g1 = min(ngroups, g0 + per);
  const i32x4 *cp = (mat ? up.codes : gate.codes) + (size_t)tile * nunits * 64 + lane;
  const unsigned short *sp = (mat ? up.scales : gate.scales) + (size_t)tile * ngroups * 64 + lane;
  const uniform_i32x4 *xw = (const uniform_i32x4 *)job.xq;
  const uniform_i32 *sa = (const uniform_i32 *)job.suma;
  const int o = tile * 64 + lane;

  float acc = 0.0f;
  int g = g0;
  for (; g + GPB <= g1; g += GPB) {
    i32x4 c[GPB * UPG];
    unsigned short dh[GPB];
#pragma unroll
    for (int v = 0; v < GPB * UPG; v++) c[v] = __builtin_nontemporal_load(cp + (size_t)(g * UPG + v) * 64);
#pragma unroll
    for (int j = 0; j < GPB; j++) dh[j] = __builtin_nontemporal_load(sp + (size_t)(g + j) * 64);
#pragma unroll
    for (int j = 0; j < GPB; j++) {
      int p = 0;
#pragma unroll
      for (int v = 0; v < UPG; v++) {
        const int u = (g + j) * UPG + v;
        p += unit_dot(c[j * UPG + v], xw + (size_t)u * 4, sa[u]);
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
      p += unit_dot(__builtin_nontemporal_load(cp + (size_t)u * 64), xw + (size_t)u * 4, sa[u]);
    }
    acc = fmaf(half_bits_to_f32(dh), (float)p, acc);
  }

  if (wave > 0) red[mat][wave - 1][lane] = acc;
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 0; w < W - 1; w++) acc += red[mat][w][lane];
    if (mat == 1) fin[lane] = acc;
  }
  __syncthreads();
  if (wave2 == 0) {
    const float sc = gate.act_scale[0];
    float m = 0.0f;
    if (o < M) {
      const float tv = glu1<KIND>(__fmul_rn(acc, sc), __fmul_rn(fin[lane], sc));
      t[o] = tv;
      m = fabsf(tv);
    }
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    if (lane == 0) part[tile] = __float_as_int(m);
  }
}

template <int UPG, int GPB>
hipError_t launch_typed(const Q2Batch &b, int waves, int S, int *dots, float *y0, float *y1, const float *accum,
                        hipStream_t stream) {
  const dim3 grid(b.tile_end[b.njobs - 1], S);
#define QG_LAUNCH(W, D) q2_gemv_t64_kernel<UPG, GPB, D, W><<<grid, 64 * W, 0, stream>>>(b, dots, S)
  if (waves == 8) {
    if (dots) QG_LAUNCH(8, true); else QG_LAUNCH(8, false);
  } else {
    if (dots) QG_LAUNCH(16, true); else QG_LAUNCH(16, false);
  }
#undef QG_LAUNCH
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  const int M = b.job[0].M;
  q2_splitk_reduce_kernel<<<dim3((M + 255) / 256, b.njobs), 256, 0, stream>>>(b, y0, y1, accum, S);
  return hipGetLastError();
}

hipError_t launch_batch(const Q2Batch &b, int group, int waves, int S, int *dots, float *y0, float *y1,
                        const float *accum, hipStream_t stream) {
  if (group == 64) return launch_typed<1, 4>(b, waves, S, dots, y0, y1, accum, stream);
  return launch_typed<2, 2>(b, waves, S, dots, y0, y1, accum, stream);
}

}  // namespace

int q2_auto_split(int64_t M, int64_t K, int group) {
  // A second (reduce) launch costs about as much as streaming several MB, so
  // K is split only for large matrices whose row tiles cannot half-fill the
  // 256 CUs: then into the fewest power-of-two ranges giving >= 128
  // workgroups of 16 waves (and at least 16 scale groups per range).
  // Measured on HBM-cold 5120 x 17408 g128 weights: S = 2 streams at 2.45
  // TB/s, S = 1 at 2.10, S = 4 at 2.14, S = 8 at 2.01.
  const int64_t tiles = (M + 63) / 64;
  const int64_t ngroups = K / group;
  const int64_t bytes = M * ngroups * (2 + group / 4);
  if (tiles >= 128 || bytes < (16LL << 20)) return 1;
  int S = 1;
  while (S < kMaxSplit && tiles * S < 128 && ngroups / (2 * S) >= 16) S *= 2;
  return S;
}

// One matrix or the gate/up pair.  Waves per tile: 8 when one matrix's row
// tiles alone fill the CUs, else 16 so that each of the fewer workgroups
// keeps more loads in flight.
hipError_t launch_q2_gemv(const Q2Call &call, hipStream_t stream) {
  const int M = call.M, S = call.split;
  const int tiles = (M + 63) / 64;
  const int Mp = tiles * 64;
  const int njobs = call.codes[1] ? 2 : 1;
  Q2Batch b{};
  b.njobs = njobs;
  for (int n = 0; n < njobs; n++) {
    Q2Job &j = b.job[n];
    j.codes = reinterpret_cast<const i32x4 *>(call.codes[n]);
    j.scales = reinterpret_cast<const unsigned short *>(call.scales[n]);
    j.xq = call.xq;
    j.suma = call.suma;
    j.act_scale = call.act_scale;
    j.out = S == 1 ? call.y[n] : call.partials + (size_t)n * S * Mp;
    j.accum = S == 1 ? call.accum : nullptr;
    j.M = M;
    j.K = call.K;
    b.tile_end[n] = tiles * (n + 1);
  }
  return launch_batch(b, call.group, tiles >= 256 ? 8 : 16, S, call.dots, call.y[0], call.y[1], call.accum,
                      stream);
}

// Independent GEMVs of one group size in one launch, no split; 8 waves per
// tile when the launch's row tiles fill the CUs, else 16.
hipError_t launch_q2_batch(const Q2BatchCall *jobs, int njobs, int group, hipStream_t stream) {
  Q2Batch b{};
  b.njobs = njobs;
  int tiles = 0;
  for (int n = 0; n < njobs; n++) {
    const Q2BatchCall &c = jobs[n];
    Q2Job &j = b.job[n];
    j.codes = reinterpret_cast<const i32x4 *>(c.codes);
    j.scales = reinterpret_cast<const unsigned short *>(c.scales);
    j.xq = c.xq;
    j.suma = c.suma;
    j.act_scale = c.act_scale;
    j.out = c.y;
    j.accum = c.accum;
    j.M = c.M;
    j.K = c.K;
    tiles += (c.M + 63) / 64;
    b.tile_end[n] = tiles;
  }
  return launch_batch(b, group, tiles >= 256 ? 8 : 16, 1, nullptr, nullptr, nullptr, nullptr, stream);
}


// The gate|up GEMV with the gated product in its epilogue (one launch), then
// the quantiser's second step over t (one workgroup).  Same waves per tile
// as the dual GEMV of this shape, and no K split.
hipError_t launch_q2_gate_up_glu(const Q2Call &call, int kind, float *t, int8_t *xq_out, float *act_scale_out,
                                 int32_t *suma_out, hipStream_t stream) {
  Q2Job gate{}, up{};
  gate.codes = reinterpret_cast<const i32x4 *>(call.codes[0]);
  gate.scales = reinterpret_cast<const unsigned short *>(call.scales[0]);
  up.codes = reinterpret_cast<const i32x4 *>(call.codes[1]);
  up.scales = reinterpret_cast<const unsigned short *>(call.scales[1]);
  gate.xq = up.xq = call.xq;
  gate.suma = up.suma = call.suma;
  gate.act_scale = up.act_scale = call.act_scale;
  gate.M = up.M = call.M;
  gate.K = up.K = call.K;
  const int tiles = (call.M + 63) / 64;
  const bool w8 = tiles >= 256;
  int *part = reinterpret_cast<int *>(suma_out);
#define QG_GLU(UPG, GPB, W, KD) \
  q2_gate_up_glu_kernel<UPG, GPB, W, KD><<<tiles, 64 * W, 0, stream>>>(gate, up, t, part)
#define QG_GLU_H(UPG, GPB, KD) \
  q2_gate_up_glu_halves_kernel<UPG, GPB, 8, KD><<<tiles, 128 * 8, 0, stream>>>(gate, up, t, part)
  // 8 waves per matrix (the dual GEMV's choice at >= 256 tiles): the two
  // matrices on the halves of a 16-wave workgroup; 16 waves per matrix
  // (fewer tiles): both matrices on the same 16 waves, one after the other
  // in each group step.
  if (call.group == 64) {
    if (w8) { if (kind == 0) QG_GLU_H(1, 4, 0); else QG_GLU_H(1, 4, 1); }
    else { if (kind == 0) QG_GLU(1, 4, 16, 0); else QG_GLU(1, 4, 16, 1); }
  } else {
    if (w8) { if (kind == 0) QG_GLU_H(2, 2, 0); else QG_GLU_H(2, 2, 1); }
    else { if (kind == 0) QG_GLU(2, 2, 16, 0); else QG_GLU(2, 2, 16, 1); }
  }
#undef QG_GLU
#undef QG_GLU_H
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_quant_from_parts(t, 1, call.M, tiles, xq_out, act_scale_out, suma_out, stream);
}
}  // namespace qg
