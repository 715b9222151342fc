// q8row_gemm.hip -- batched prefill q8_row product on int8 MFMA.
//
// What is computed (cortiq-engine 0.5.43 gpu_wgpu.rs page, q8_matmat and
// q8_mul_mm; cortiq-engine 0.3.7 gpu_metal.rs page, q8_matmat / q8_mul_mm):
//     y[b, o] = rs[o] * sum_i q[o, i] * xs[b, i]
// with xs [nb][K] and y [nb][M] row-major and the weights in the T64 image.
// The silu form takes g, u [nb][K] and a column field col [K] instead of xs
// and forms xs = silu(g) * u * col in the prep kernel by the rule of
// gate_rule.h (cortiq pages, silu_mul_pre; the Metal page's q8_mul_mm_silu
// forms silu(g) * u in its activation load the same way).
//
// Precision scheme (differs from the Metal page, whose fast kernel rounds
// w*rs and xs to half): the weights stay exact int8 and the f32 activations
// are split exactly into int8 limbs of a per-row fixed-point value:
//     xs[b, i] ~= 2^e_b * (h * 65536 + m * 256 + l),  h, m, l in [-128, 127]
// where 2^e_b is the smallest power of two that brings max_i |xs[b, i]| to
// at most 126 * 65536 (a 24-bit value rounded to nearest).  Each limb is a
// separate exact int8 x int8 -> int32 MFMA product; the limbs' int32 sums
// are combined in f32 and scaled by rs[o] and 2^e_b at the end.  Dropping
// the lowest limb gives the 2-limb (16-bit) form at 2/3 of the MFMA work;
// its rounding is then 0.5 * 2^(e_b + 8) per element.
//
// The limb count is 3, 2, or chosen per 64-row tile of xs ("auto"): a tile
// uses 2 limbs only when, for every row, 2^(e_b + 8) <= 0.9e-5 * sum|xs_b| /
// sqrt(K).  With weights of the q8_row distribution (E|q| / sqrt(E q^2) >=
// 0.8) this keeps the 16-bit rounding error of every output below 1/6 of
// 2e-5 * sum_i |w_i x_i| at six standard deviations; rows with a large
// max/mean ratio (activation outliers) get the 24-bit form.
//
// gfx950 kernels: one prep launch (exponents, limb-count flags and limbs of
// every xs row), then the product on v_mfma_i32_16x16x64_i8 (A row and B
// column = lane % 16, the 16-byte k chunk = lane / 16, D[4 * (lane / 16) + v]
// [lane % 16]): a 272 x 128 output tile per 12-wave workgroup (one tile per
// CU at the FFN width), operands moved global -> LDS directly through a
// 4-stage ring, and a block order that puts the workgroups sharing one weight
// tile on the same XCD (the same L2) at the same time.
#include "gate_rule.h"
#include "qg_internal.h"

namespace qg {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kKS = 64;        // K bytes per pipeline stage (one MFMA depth)
constexpr int kCPS = kKS / 16; // 16-byte chunks per stage
constexpr int kLimbMax = 3;
constexpr int kR3 = 126 * 65536;  // largest |fixed-point value|, 3 limbs

// ------------------------------------------------------------- prep kernel
// One workgroup per row b of xs (rows past nb included, as zeros; the grid
// is nbp workgroups, nbp a multiple of 128), thread t taking the 16-float
// chunks t, t + 256, ...  It finds max|x| and sum|x| of the row, hence the
// exponent e_b (the smallest e with max|x| <= kR3 * 2^e) and whether the row
// needs the third limb, then writes the row's limbs in the weights' tiled
// form: limb l, row b, 16-byte chunk c at
//     ((l * nbt + b / 64) * nchunk + c) * 64 + b % 64        (16-byte units)
// Rows of up to kPrepHeld chunks per thread stay in registers between the
// two steps; longer rows are read a second time (from L2).  Chunks past K
// are written as zeros.
constexpr int kPrepThreads = 256;
// Chunks per thread held in registers: 2 for rows up to 8192 values, 5 up
// to 20480 (measured: 5 is 14 % faster at K = 17408 and 25 % slower at
// K = 5120, where its idle unrolled slots cost more than the second read saves).
constexpr int kPrepHeldShort = 2, kPrepHeldLong = 5;

// The activation row a prep workgroup reads: xs row b, or (kSilu) the rows
// b of g and u with the shared column field col (null: none), from which
// act = silu(g) * u * col is formed by the rule of gate_rule.h.
struct PrepRow {
  const float *x;    // xs row, or g row
  const float *u;    // u row (kSilu)
  const float *col;  // column field or null (kSilu)
};

template <bool kSilu>
__device__ __forceinline__ float act1(const PrepRow &r, int i) {
  if (!kSilu) return r.x[i];
  return silu_pre1(r.x[i], r.u[i], r.col ? r.col[i] : 1.0f);
}

template <bool kSilu>
__device__ __forceinline__ void load_chunk(const PrepRow &r, int c, int K, bool live, float (&xv)[16]) {
  if (live && c * 16 + 16 <= K) {
#pragma unroll
    for (int q = 0; q < 4; q++) {
      const int i = c * 16 + 4 * q;
      const float4 v = *reinterpret_cast<const float4 *>(r.x + i);
      if (kSilu) {
        const float4 uv = *reinterpret_cast<const float4 *>(r.u + i);
        const float4 cv = r.col ? *reinterpret_cast<const float4 *>(r.col + i) : make_float4(1.0f, 1.0f, 1.0f, 1.0f);
        xv[4 * q] = silu_pre1(v.x, uv.x, cv.x), xv[4 * q + 1] = silu_pre1(v.y, uv.y, cv.y);
        xv[4 * q + 2] = silu_pre1(v.z, uv.z, cv.z), xv[4 * q + 3] = silu_pre1(v.w, uv.w, cv.w);
      } else {
        xv[4 * q] = v.x, xv[4 * q + 1] = v.y, xv[4 * q + 2] = v.z, xv[4 * q + 3] = v.w;
      }
    }
  } else {
#pragma unroll
    for (int j = 0; j < 16; j++) xv[j] = (live && c * 16 + j < K) ? act1<kSilu>(r, c * 16 + j) : 0.0f;
  }
}

__device__ __forceinline__ void store_limbs(const float (&xv)[16], int e, i32x4 *__restrict__ dst, size_t limb_stride) {
  int lim[kLimbMax][4];
#pragma unroll
  for (int w = 0; w < 4; w++) {
    lim[0][w] = lim[1][w] = lim[2][w] = 0;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const float xs = ldexpf(xv[w * 4 + j], -e);  // exact scaling
      int v = isfinite(xs) ? (int)rintf(xs) : 0;     // nearest (a non-finite row is flagged)
      const int lo = ((v + 128) & 255) - 128;
      v = (v - lo) >> 8;
      const int mi = ((v + 128) & 255) - 128;
      const int hi = (v - mi) >> 8;
      lim[0][w] |= (hi & 255) << (8 * j);
      lim[1][w] |= (mi & 255) << (8 * j);
      lim[2][w] |= (lo & 255) << (8 * j);
    }
  }
#pragma unroll
  for (int l = 0; l < kLimbMax; l++) dst[l * limb_stride] = i32x4{lim[l][0], lim[l][1], lim[l][2], lim[l][3]};
}

template <bool kSilu, int kPrepHeld>
__global__ __launch_bounds__(kPrepThreads) void gemm_prep_kernel(const float *__restrict__ xs,
                                                                 const float *__restrict__ u,
                                                                 const float *__restrict__ col, int nb, int K,
                                                                 int nchunk, int nbt, int *__restrict__ xexp,
                                                                 int *__restrict__ need3, i32x4 *__restrict__ xl,
                                                                 i32x4 *__restrict__ zero_blk) {
  __shared__ float red_max[kPrepThreads / 64], red_sum[kPrepThreads / 64];
  __shared__ int sh_e;
  const int tid = threadIdx.x;
  // Consecutive workgroups go to the 8 XCDs in turn; XCD x gets the rows
  // x * nbp / 8 ... so the 8 rows that share a 128-byte line of limbs are
  // written through one L2 (no partial lines written back from several).
  const int b = (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;
  if (blockIdx.x == 0 && tid < 64) zero_blk[tid] = i32x4{0, 0, 0, 0};
  const bool live = b < nb;
  const size_t roff = (size_t)(live ? b : 0) * K;
  const PrepRow row{xs + roff, kSilu ? u + roff : nullptr, col};
  const int nchunk_k = (K + 15) / 16;  // chunks holding any of the row
  const bool held = nchunk_k <= kPrepHeld * kPrepThreads;

  float xh[kPrepHeld][16];
  float amax = 0.0f, asum = 0.0f;
  bool bad = false;  // an infinity or NaN in the row
  if (held) {
#pragma unroll
    for (int h = 0; h < kPrepHeld; h++) load_chunk<kSilu>(row, tid + h * kPrepThreads, K, live, xh[h]);
#pragma unroll
    for (int h = 0; h < kPrepHeld; h++)
#pragma unroll
      for (int j = 0; j < 16; j++) {
        amax = fmaxf(amax, fabsf(xh[h][j]));
        asum += fabsf(xh[h][j]);
        bad |= !isfinite(xh[h][j]);
      }
  } else {
    for (int c = tid; c < nchunk_k; c += kPrepThreads) {
      float xv[16];
      load_chunk<kSilu>(row, c, K, live, xv);
#pragma unroll
      for (int j = 0; j < 16; j++) {
        amax = fmaxf(amax, fabsf(xv[j]));
        asum += fabsf(xv[j]);
        bad |= !isfinite(xv[j]);
      }
    }
  }
  bad = __syncthreads_or(bad) != 0;
  for (int off = 32; off > 0; off >>= 1) {
    amax = fmaxf(amax, __shfl_xor(amax, off));
    asum += __shfl_xor(asum, off);
  }
  if ((tid & 63) == 0) {
    red_max[tid >> 6] = amax;
    red_sum[tid >> 6] = asum;
  }
  __syncthreads();
  if (tid == 0) {
    amax = fmaxf(fmaxf(red_max[0], red_max[1]), fmaxf(red_max[2], red_max[3]));
    asum = (red_sum[0] + red_sum[1]) + (red_sum[2] + red_sum[3]);
    int e = 0;
    if (!bad && amax > 0.0f) {  // amax finite: e within a few steps of ilogb(amax) - 22
      e = ilogbf(amax) - 22;
      while (amax > ldexpf((float)kR3, e)) e++;
      while (amax <= ldexpf((float)kR3, e - 1)) e--;
    }
    xexp[b] = e;
    const float thresh = 0.9e-5f * asum / sqrtf((float)K);
    // bit 0: the row needs the third limb; bit 1: the row is not finite (its
    // limbs are meaningless and the epilogue writes NaN for its outputs)
    need3[b] = bad ? 3 : (amax > 0.0f && ldexpf(1.0f, e + 8) > thresh) ? 1 : 0;
    sh_e = e;
  }
  __syncthreads();
  const int e = sh_e;

  const size_t limb_stride = (size_t)nbt * nchunk * 64;
  i32x4 *dst = xl + (size_t)(b / 64) * nchunk * 64 + (b & 63);
  if (held) {
#pragma unroll
    for (int h = 0; h < kPrepHeld; h++) {
      const int c = tid + h * kPrepThreads;
      if (c < nchunk) store_limbs(xh[h], e, dst + (size_t)c * 64, limb_stride);
    }
    for (int c = tid + kPrepHeld * kPrepThreads; c < nchunk; c += kPrepThreads) {
      const float zero[16] = {};
      store_limbs(zero, e, dst + (size_t)c * 64, limb_stride);
    }
  } else {
    for (int c = tid; c < nchunk; c += kPrepThreads) {
      float xv[16];
      load_chunk<kSilu>(row, c, K, live, xv);
      store_limbs(xv, e, dst + (size_t)c * 64, limb_stride);
    }
  }
}

// ------------------------------------------------------------- GEMM kernel
// One workgroup of 12 waves (3 per SIMD) computes a kTM x TN block of y^T:
// kTM = 272 weight rows (17 MFMA row blocks; 17408 = 64 * 272, so the pages'
// FFN width gives exactly 256 blocks per 128 xs rows, one per CU) by TN rows
// of xs.  Waves are 3 (weight rows: blocks 0-5, 6-11, 12-16) x 4 (xs rows),
// so a wave holds at most 6 x (TN/64) x L accumulator tiles, and three waves
// per SIMD hide each other's LDS and barrier waits behind MFMA work (measured
// 2-4 % faster than two waves per SIMD with 9 blocks each).
constexpr int kOB = 17;
constexpr int kOBW = 6;        // row blocks per wave group: 6, 6 and 5
constexpr int kTM = 16 * kOB;  // 272
constexpr int kWC = 4;         // wave groups along xs rows
constexpr int kWR = 3;         // wave groups along weight rows
constexpr int kWaves = kWR * kWC;
constexpr int kThreads = 64 * kWaves;

// s_waitcnt immediate for vmcnt(n) (gfx9 encoding: vmcnt in bits 3:0 and
// 15:14; expcnt and lgkmcnt left at their maxima, i.e. not waited for).
constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void global_void;

// A workgroup barrier for LDS traffic only: waits for this wave's LDS
// accesses (lgkmcnt(0)), not for its global stores, which __syncthreads()
// would also wait for.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("s_barrier" ::: "memory");
}

template <int L, int TN>
struct GemmShape {
  static constexpr int kWB = TN / kWC;                // xs rows per wave
  static constexpr int kBB = kWB / 16;                // 16-column MFMA blocks per wave
  static constexpr int kAPieces = kTM * kCPS;         // 16-byte pieces of A per stage
  static constexpr int kBPieces = L * TN * kCPS;      // 16-byte pieces of B per stage
  static constexpr int kAWaveLoads = kAPieces / 64;   // 1 KiB wave loads of A (17)
  static constexpr int kBWaveLoads = kBPieces / 64;
  static constexpr int kAPerWave = (kAWaveLoads + kWaves - 1) / kWaves;  // at most, per wave
  static constexpr int kBPerWave = (kBWaveLoads + kWaves - 1) / kWaves;
  static constexpr int kStages = 4;                   // LDS ring depth
  static constexpr int kStageBytes = (kAPieces + kBPieces) * 16;
  static constexpr int kRowStride = kTM + 4;          // epilogue row stride (floats)
  static constexpr int kEpiRows = 16 * kWC;          // xs rows per epilogue group
  static constexpr int kEpiBytes = kEpiRows * kRowStride * 4;
  static constexpr int kLdsBytes =
      kStages * kStageBytes > kEpiBytes ? kStages * kStageBytes : kEpiBytes;
};

// LDS of the ring or the epilogue's transpose, whichever is larger, for
// either pass shape; then the epilogue's row scales rs[o0 .. o0 + 272) and
// the exponents and flags of the pass's xs rows, moved into LDS at the start
// of the pass.
constexpr int kGemmMain = GemmShape<2, 128>::kLdsBytes > GemmShape<3, 64>::kLdsBytes
                              ? GemmShape<2, 128>::kLdsBytes
                              : GemmShape<3, 64>::kLdsBytes;
constexpr int kEpiConstBytes = (kTM + 2 * 128) * 4;

// One pass of the K loop plus the epilogue for weight block `ot` and the TN
// xs rows starting at b0, with L limbs.  `lds` is the workgroup's buffer.
template <int L, int TN>
__device__ __forceinline__ void gemm_pass(char *lds, const i32x4 *__restrict__ w, const float *__restrict__ rs,
                                          const i32x4 *__restrict__ xl, const i32x4 *__restrict__ zero_blk,
                                          const int *__restrict__ xexp, const int *__restrict__ need3,
                                          float *__restrict__ y, int nb, int M,
                                          int nchunk_w, int nchunk, int nbt64, int ot, int b0) {
  using S = GemmShape<L, TN>;
  float *rs_l = reinterpret_cast<float *>(lds + kGemmMain);  // [kTM]
  int *exp_l = reinterpret_cast<int *>(rs_l + kTM);      // [TN]
  int *need_l = exp_l + TN;                              // [TN]
  // Stage buffer `buf` holds the A pieces, then the B pieces.
  auto As = [&](int buf) { return reinterpret_cast<i32x4 *>(lds + buf * S::kStageBytes); };
  auto Bs = [&](int buf) { return As(buf) + S::kAPieces; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wq = wave % kWC;       // xs-row group
  const int wh = wave / kWC;       // weight-row group
  const int ob0 = wh * kOBW;       // first row block of this wave
  const int nob = wh < kWR - 1 ? kOBW : kOB - (kWR - 1) * kOBW;

  const int o0 = ot * kTM;
  const int m_tiles = (M + 63) / 64;
  const int b_tile0 = b0 / 64;

  // One stage = wave loads of 1 KiB that go straight from global memory into
  // LDS (lane i's 16 bytes land at base + 16 i); wave w issues wave loads
  // w, w + 8, ...  Each lane's source address is formed once; a stage moves
  // every source by 4 chunks (256 pieces).  Rows past the weight image, and
  // chunks past K in the last stage, read the zero block instead.
  const i32x4 *a_src[S::kAPerWave];
  int a_kc[S::kAPerWave];
#pragma unroll
  for (int i = 0; i < S::kAPerWave; i++) {
    const int j = min(wave + kWaves * i, S::kAWaveLoads - 1);
    const int p = 64 * j + lane;
    const int kc = p / kTM, row = p % kTM;
    const int o = o0 + row, t = o >> 6;
    a_kc[i] = kc;
    a_src[i] = t < m_tiles ? w + ((size_t)t * nchunk_w + kc) * 64 + (o & 63) : nullptr;
  }
  const i32x4 *b_src[S::kBPerWave];
#pragma unroll
  for (int i = 0; i < S::kBPerWave; i++) {
    const int j = min(wave + kWaves * i, S::kBWaveLoads - 1);
    const int l = j / ((TN / 64) * kCPS);
    const int q = j % ((TN / 64) * kCPS);
    const int bt64 = q / kCPS, kc = q % kCPS;
    b_src[i] = xl + ((size_t)(l * nbt64 + b_tile0 + bt64) * nchunk + kc) * 64 + lane;
  }
  auto issue_stage = [&](int step) {
    const int buf = step % S::kStages;
    const int c0 = step * kCPS;
#pragma unroll
    for (int i = 0; i < S::kAPerWave; i++) {
      const int j = wave + kWaves * i;
      if (j < S::kAWaveLoads) {
        const i32x4 *src = (a_src[i] != nullptr && c0 + a_kc[i] < nchunk_w)
                               ? a_src[i] + (size_t)step * (kCPS * 64) : zero_blk + lane;
        __builtin_amdgcn_global_load_lds((global_void *)src, (lds_void *)(As(buf) + 64 * j), 16, 0, 0);
      }
    }
#pragma unroll
    for (int i = 0; i < S::kBPerWave; i++) {
      const int j = wave + kWaves * i;
      if (j < S::kBWaveLoads)
        __builtin_amdgcn_global_load_lds((global_void *)(b_src[i] + (size_t)step * (kCPS * 64)),
                                         (lds_void *)(Bs(buf) + 64 * j), 16, 0, 0);
    }
  };

  i32x4 acc[kOBW][S::kBB][L];
#pragma unroll
  for (int a = 0; a < kOBW; a++)
#pragma unroll
    for (int c = 0; c < S::kBB; c++)
#pragma unroll
      for (int l = 0; l < L; l++) acc[a][c][l] = i32x4{0, 0, 0, 0};

  const int kc = lane >> 4, r16 = lane & 15;
  auto read_b = [&](int buf, i32x4 (&bf)[S::kBB][L]) {
#pragma unroll
    for (int c = 0; c < S::kBB; c++) {
      const int bcol = wq * S::kWB + c * 16 + r16;  // 0 .. TN-1
#pragma unroll
      for (int l = 0; l < L; l++)
        bf[c][l] = Bs(buf)[((l * (TN / 64) + bcol / 64) * kCPS + kc) * 64 + (bcol & 63)];
    }
  };
  auto read_a = [&](int buf, int a) { return As(buf)[kc * kTM + (ob0 + a) * 16 + r16]; };
  auto mfma_block = [&](int a, const i32x4 &af, const i32x4 (&bf)[S::kBB][L]) {
#pragma unroll
    for (int c = 0; c < S::kBB; c++)
#pragma unroll
      for (int l = 0; l < L; l++)
        acc[a][c][l] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, bf[c][l], acc[a][c][l], 0, 0, 0);
  };
  // Two K-steps (stage buffers buf0, buf1) as one software pipeline: the LDS
  // reads of the next pair of A fragments -- and at the step boundary the next
  // step's B fragments -- are issued before the MFMAs of the current pair, so
  // their latency hides behind MFMA work.
  auto compute2 = [&](int buf0, int buf1, bool has1) {
    i32x4 bf0[S::kBB][L], bf1[S::kBB][L];
    read_b(buf0, bf0);
    i32x4 c0 = read_a(buf0, 0), c1 = read_a(buf0, 1);
#pragma unroll
    for (int a = 0; a < kOBW; a += 2) {
      i32x4 n0 = c0, n1 = c1;
      if (a + 2 < kOBW) {
        if (a + 2 < nob) n0 = read_a(buf0, a + 2);
        if (a + 3 < kOBW && a + 3 < nob) n1 = read_a(buf0, a + 3);
      } else if (has1) {
        read_b(buf1, bf1);
        n0 = read_a(buf1, 0);
        n1 = read_a(buf1, 1);
      }
      if (a < nob) mfma_block(a, c0, bf0);
      if (a + 1 < kOBW && a + 1 < nob) mfma_block(a + 1, c1, bf0);
      c0 = n0;
      c1 = n1;
    }
    if (!has1) return;
#pragma unroll
    for (int a = 0; a < kOBW; a += 2) {
      i32x4 n0 = c0, n1 = c1;
      if (a + 2 < kOBW && a + 2 < nob) n0 = read_a(buf1, a + 2);
      if (a + 3 < kOBW && a + 3 < nob) n1 = read_a(buf1, a + 3);
      if (a < nob) mfma_block(a, c0, bf1);
      if (a + 1 < kOBW && a + 1 < nob) mfma_block(a + 1, c1, bf1);
      c0 = n0;
      c1 = n1;
    }
  };

  // K loop over an LDS ring of 4 stage buffers, two steps per barrier: while
  // steps s, s+1 are multiplied, the loads of steps s+2, s+3 are in flight
  // into the two buffers that steps s-2, s-1 used.
  const int nsteps = nchunk / kCPS;
  static_assert(S::kStages == 4, "the ring below holds two pairs of stages");
  // The epilogue's constants go to LDS by DMA ahead of the ring's loads (the
  // loop's first wait covers them), so that its stores are never followed by
  // a wait for a load: rs by waves 0-4, the exponents and flags by the next.
  {
    constexpr int kRsWaves = (kTM + 63) / 64;
    constexpr int kBW = TN / 64;
    if (wave < kRsWaves) {
      const int i = 64 * wave + lane;
      if (i < kTM)
        __builtin_amdgcn_global_load_lds((global_void *)(rs + min(o0 + i, M - 1)),
                                         (lds_void *)(rs_l + 64 * wave), 4, 0, 0);
    } else if (wave < kRsWaves + kBW) {
      const int j = wave - kRsWaves;
      __builtin_amdgcn_global_load_lds((global_void *)(xexp + b0 + 64 * j + lane), (lds_void *)(exp_l + 64 * j), 4, 0, 0);
    } else if (wave < kRsWaves + 2 * kBW) {
      const int j = wave - kRsWaves - kBW;
      __builtin_amdgcn_global_load_lds((global_void *)(need3 + b0 + 64 * j + lane), (lds_void *)(need_l + 64 * j), 4, 0, 0);
    }
  }
  if (0 < nsteps) issue_stage(0);
  if (1 < nsteps) issue_stage(1);
  for (int step = 0; step < nsteps; step += 2) {
    // Steps `step` and `step+1` are the oldest loads in flight.
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
    // A bare barrier: __syncthreads() would add a workgroup fence around it;
    // the wait above already covers this wave's loads, and after the barrier
    // all waves' are in LDS and every wave has finished reading the two
    // buffers refilled next.  The memory clobber keeps the compiler from
    // moving LDS accesses across it.
    asm volatile("s_barrier" ::: "memory");
    if (step + 2 < nsteps) issue_stage(step + 2);
    if (step + 3 < nsteps) issue_stage(step + 3);
    compute2(step % S::kStages, (step + 1) % S::kStages, step + 1 < nsteps);
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __syncthreads();

  // Epilogue: limbs combined in f32 per output, transposed through LDS in
  // groups of 64 xs rows, then written as whole rows of y (272 consecutive
  // outputs each) with rs[o] and 2^e_b applied on the way out.
  float *ep = reinterpret_cast<float *>(lds);
  const bool vec = (M & 3) == 0;
#pragma unroll
  for (int c = 0; c < S::kBB; c++) {
    const int row = wq * 16 + r16;  // within the group of kEpiRows
#pragma unroll
    for (int a = 0; a < kOBW; a++) {
      if (a < nob) {
        float vv[4];
#pragma unroll
        for (int v = 0; v < 4; v++) {
          if (L == 2)
            vv[v] = (float)acc[a][c][0][v] * 256.0f + (float)acc[a][c][1][v];
          else
            vv[v] = ((float)acc[a][c][0][v] * 65536.0f + (float)acc[a][c][1][v] * 256.0f) +
                    (float)acc[a][c][L - 1][v];
        }
        *reinterpret_cast<float4 *>(ep + row * S::kRowStride + (ob0 + a) * 16 + 4 * kc) =
            make_float4(vv[0], vv[1], vv[2], vv[3]);
      }
    }
    lds_barrier();
    for (int f = tid; f < S::kEpiRows * (kTM / 4); f += kThreads) {
      const int gr = f / (kTM / 4), col = (f % (kTM / 4)) * 4;
      const int b = b0 + (gr / 16) * S::kWB + c * 16 + (gr % 16);
      const int o = o0 + col;
      if (b >= nb || o >= M) continue;
      const float4 v4 = *reinterpret_cast<const float4 *>(ep + gr * S::kRowStride + col);
      const int bl = b - b0;
      const int e = exp_l[bl] + (L == 2 ? 8 : 0);
      float *dst = y + (size_t)b * M + o;
      if (need_l[bl] & 2) {  // an infinity or NaN in this xs row
        const float nan = __builtin_nanf("");
#pragma unroll
        for (int k = 0; k < 4; k++)
          if (o + k < M) dst[k] = nan;
      } else if (vec && o + 3 < M) {
        const float4 r4 = *reinterpret_cast<const float4 *>(rs_l + col);
        // streamed out: every workgroup stores its rows at once, at the end
        __builtin_nontemporal_store(f32x4{ldexpf(v4.x * r4.x, e), ldexpf(v4.y * r4.y, e),
                                          ldexpf(v4.z * r4.z, e), ldexpf(v4.w * r4.w, e)},
                                    reinterpret_cast<f32x4 *>(dst));
      } else {
        if (o < M) dst[0] = ldexpf(v4.x * rs_l[col], e);
        if (o + 1 < M) dst[1] = ldexpf(v4.y * rs_l[col + 1], e);
        if (o + 2 < M) dst[2] = ldexpf(v4.z * rs_l[col + 2], e);
        if (o + 3 < M) dst[3] = ldexpf(v4.w * rs_l[col + 3], e);
      }
    }
    lds_barrier();
  }
}

constexpr int kGemmLds = kGemmMain + kEpiConstBytes;

// One workgroup per (weight block of 272 rows, group of 128 xs rows).  The
// group is computed with 2 limbs in one pass of 128 rows, or with 3 limbs in
// two passes of 64 rows.  limbs: 2 or 3 for all groups, 0 = per group from
// the rows' need3 flags (auto).
__global__ __launch_bounds__(kThreads, 1) void q8row_gemm_kernel(
    const i32x4 *__restrict__ w, const float *__restrict__ rs, const i32x4 *__restrict__ xl,
    const i32x4 *__restrict__ zero_blk, const int *__restrict__ xexp,
    const int *__restrict__ need3, float *__restrict__ y, int nb, int M, int nchunk_w, int nchunk,
    int nbt64, int n_ot, int n_bt, int limbs) {
  __shared__ __attribute__((aligned(16))) char lds[kGemmLds];

  // Block order: the n_bt workgroups of one weight block get ids 8 apart, so
  // the round-robin dispatch over the 8 XCDs puts them on one XCD together.
  const int id = blockIdx.x;
  const int per_grp = 8 * n_bt;
  const int ot = (id / per_grp) * 8 + (id % per_grp) % 8;
  const int bt = (id % per_grp) / 8;
  if (ot >= n_ot) return;
  const int g0 = bt * 128;

  bool three = limbs == 3;
  if (limbs == 0) {
    const int lane = threadIdx.x & 63;
    const int f = (need3[g0 + lane] | need3[g0 + 64 + lane]) & 1;
    three = __builtin_amdgcn_ballot_w64(f != 0) != 0;
  }
  if (three) {
    gemm_pass<3, 64>(lds, w, rs, xl, zero_blk, xexp, need3, y, nb, M, nchunk_w, nchunk, nbt64, ot, g0);
    gemm_pass<3, 64>(lds, w, rs, xl, zero_blk, xexp, need3, y, nb, M, nchunk_w, nchunk, nbt64, ot, g0 + 64);
  } else {
    gemm_pass<2, 128>(lds, w, rs, xl, zero_blk, xexp, need3, y, nb, M, nchunk_w, nchunk, nbt64, ot, g0);
  }
}

}  // namespace

// Workspace: limbs [3][nbp/64][Kp/16][64][16 B], then e_b [nbp], need3
// [nbp], then a 1 KiB block of zeros (the source of out-of-range pieces).
size_t gemm_ws_layout(int64_t nb, int64_t K, size_t *off_exp, size_t *off_need, size_t *off_zero) {
  const int64_t nbp = round_up(nb, 128);
  const int64_t kp = round_up(K, kKS);
  const size_t limbs = (size_t)kLimbMax * nbp * kp;
  *off_exp = (size_t)round_up(limbs, 256);
  *off_need = *off_exp + (size_t)round_up(nbp * 4, 256);
  *off_zero = *off_need + (size_t)round_up(nbp * 4, 256);
  return *off_zero + 1024;
}

hipError_t launch_q8row_gemm(const void *w, const float *rs, const GemmAct &act, float *y, int nb,
                             int M, int K, int limbs, void *ws, hipStream_t stream) {
  size_t off_exp, off_need, off_zero;
  gemm_ws_layout(nb, K, &off_exp, &off_need, &off_zero);
  const int nbp = (int)round_up(nb, 128);
  const int nchunk = (int)(round_up(K, kKS) / 16);
  const int nchunk_w = (int)(round_up(K, 16) / 16);
  char *base = static_cast<char *>(ws);
  i32x4 *xl = reinterpret_cast<i32x4 *>(base);
  int *xexp = reinterpret_cast<int *>(base + off_exp);
  int *need3 = reinterpret_cast<int *>(base + off_need);
  i32x4 *zero_blk = reinterpret_cast<i32x4 *>(base + off_zero);

  const bool long_rows = (K + 15) / 16 > kPrepHeldShort * kPrepThreads;
#define QG_PREP(S, H, X, U, C) \
  gemm_prep_kernel<S, H><<<nbp, kPrepThreads, 0, stream>>>(X, U, C, nb, K, nchunk, nbp / 64, xexp, need3, xl, zero_blk)
  if (act.g) {
    if (long_rows) QG_PREP(true, kPrepHeldLong, act.g, act.u, act.col);
    else QG_PREP(true, kPrepHeldShort, act.g, act.u, act.col);
  } else {
    if (long_rows) QG_PREP(false, kPrepHeldLong, act.xs, nullptr, nullptr);
    else QG_PREP(false, kPrepHeldShort, act.xs, nullptr, nullptr);
  }
#undef QG_PREP
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  const int n_ot = (M + kTM - 1) / kTM;
  const int n_bt = nbp / 128;
  const int grid = (n_ot + 7) / 8 * 8 * n_bt;
  q8row_gemm_kernel<<<grid, kThreads, 0, stream>>>(reinterpret_cast<const i32x4 *>(w), rs, xl, zero_blk, xexp,
                                                   need3, y, nb, M, nchunk_w, nchunk, nbp / 64, n_ot, n_bt,
                                                   limbs);
  err = hipGetLastError();
  return err;
}

}  // namespace qg
