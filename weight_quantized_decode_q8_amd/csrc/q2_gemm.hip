// q2_gemm.hip -- batched (prefill) Q2 x int8 product on int8 MFMA.
//
// What is computed (qxmx qxmx_gpu.cpp page, ffn_forward_b: gemm_gpu_v4 on
// the token rows' int8 activations from the batched producers, output
// token-major as its transpose_out form, residual folded as its accum):
//   y[b, o] = act_scale[b] * sum_g d(o, g) * sum_{i in g} (code(o, i) - 1) * xq[b, i]
//             (+ accum[b, o])
// The page does not show gemm_gpu_v4's source; this kernel is designed from
// the Q2 definition and the GEMV's int32-dot-per-group arithmetic.
//
// gfx950 design:
//  - v_mfma_i32_16x16x64_i8, one MFMA depth = one 64-wide unit.  The A
//    operand is the weights' codes as signed bytes code - 1 (-1..2): a lane
//    (row lane % 16, k chunk lane / 16) needs word (lane / 16) of its row's
//    unit; (word >> 2a) & 0x03030303 holds the 4 codes of dword a of its
//    16-byte fragment in natural k order (the T64 code order), and one
//    v_perm_b32 with those codes as byte selectors into 0x020100ff turns them
//    into code - 1.  A costs 4 bytes per lane per 16 x 64 block: a quarter
//    of an int8 weight operand.  B is xq as stored, [nb][K].
//  - int32 accumulation over a scale group's units: exactly
//    sum (code - 1) * xq, the GEMV's corrected group dot (its sum code * xq
//    minus suma), so closing the group is one convert and one f32 FMA per
//    output with d(o, g), as the GEMV does per group.  On gfx950 the vector
//    ALU's time adds to the matrix pipe's instead of hiding behind it, so the
//    design counts vector instructions: per wave and g128 group, 136 for the
//    closes, 66 for the code unpack, about 10 for addresses, beside 34 MFMAs.
//  - tile 272 weight rows x 128 tokens per 8-wave workgroup (17408 = 64 x
//    272: 256 workgroups at the FFN width and 512 tokens).  Wave w owns row
//    blocks 2w and 2w + 1 across all 8 token blocks, plus row block 16 by
//    token block w (17 MFMA tiles per wave, every SIMD the same work), so
//    each code word is unpacked by one wave and feeds 8 MFMAs.
//  - a group is closed during the next group's first unit, tile by tile
//    just before the tile's accumulator restarts; its scales are read into
//    registers at the end of its last unit.
//  - operands go global -> LDS directly (global_load_lds) through a 4-stage
//    ring, two units per barrier, each stage also carrying the unit's group
//    scales, so the loop issues no other global load; the token pieces are
//    stored with an XOR swizzle so the 128-bit fragment reads hit distinct
//    LDS banks; workgroups sharing a weight tile are dispatched to one XCD.
//  - a pair launch (the page's gemm_gpu_v4_dual: gate and up against the same
//    token rows) runs both matrices' workgroups in one grid, blockIdx.y
//    choosing the matrix; every output is computed exactly as in a
//    one-matrix launch (same tiles, same K split);
//  - shapes whose tiles cannot fill the CUs (the 5120-row down projection:
//    76 tiles) split K into f32 partials [S][nb][M], added in fixed order by
//    a second kernel; (row tile, split) pairs are spread evenly over XCDs.
#include "qg_internal.h"

namespace qg {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void global_void;

constexpr int kOB = 17;        // 16-row MFMA blocks per tile
constexpr int kTM = 16 * kOB;  // 272 weight rows per tile
constexpr int kTN = 128;       // tokens per tile
constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;
constexpr int kBB = kTN / 16;  // 16-token blocks per tile (8)
constexpr int kOBW = 2;        // row blocks of one wave (2w, 2w+1), besides its tile of block 16
constexpr int kStages = 4;     // LDS ring depth in units (two per barrier)
constexpr int kABytes = kTM * 16;    // one unit of codes for the tile's rows (4352)
constexpr int kBBytes = kTN * 64;    // one unit of xq for the tile's tokens (8192)
constexpr int kDBytes = kTM * 2;     // the unit's group scales for the tile's rows (544)
constexpr int kStageBytes = kABytes + kBBytes + kDBytes;
constexpr int kAWaveLoads = (kTM + 63) / 64;  // 5, the last one 16 lanes wide
constexpr int kDDwords = kDBytes / 4;         // 136: waves 5, 6 and 8 lanes of wave 7
constexpr int kLdsBytes = kStages * kStageBytes;

__device__ inline float half_bits_to_f32(unsigned short h) { return (float)__builtin_bit_cast(_Float16, h); }

template <bool B>
struct BC {
  static constexpr bool value = B;
};

// The two weight matrices of a pair launch (gate and up against one set of
// token rows); a one-matrix launch uses entry 0 only.
struct Q2Pair {
  const i32x4 *codes[2];
  const unsigned short *scales[2];
  float *y[2];
};

template <int UPG>
__global__ __launch_bounds__(kThreads, 1) void q2_gemm_kernel(
    Q2Pair pair_args, const int8_t *__restrict__ xq,
    const float *__restrict__ act_scale, const float *accum, int nb, int M, int K, int n_ot, int n_bt, int n_split,
    float *__restrict__ part) {
  __shared__ __attribute__((aligned(16))) char lds[kLdsBytes];
  // Matrix of this workgroup (blockIdx.y); its partials follow the first
  // matrix's [S][nb][M] block.
  const int job = blockIdx.y;
  const i32x4 *__restrict__ codes = job ? pair_args.codes[1] : pair_args.codes[0];
  const unsigned short *__restrict__ scales = job ? pair_args.scales[1] : pair_args.scales[0];
  float *y = job ? pair_args.y[1] : pair_args.y[0];
  part += (size_t)job * n_split * nb * M;

  // Block order: a weight tile is a (row tile, K split) pair; its n_bt
  // workgroups get ids 8 apart, so the round-robin dispatch over the 8 XCDs
  // puts them on one XCD together, and the pairs spread evenly over XCDs.
  const int S = n_split;
  const int id = blockIdx.x;
  const int per_grp = 8 * n_bt;
  const int pair = (id / per_grp) * 8 + (id % per_grp) % 8;
  const int bt = (id % per_grp) / 8;
  if (pair >= n_ot * S) return;
  const int ot = pair / S, split = pair % S;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int o0 = ot * kTM, b0 = bt * kTN;
  const int m_tiles = (M + 63) / 64;
  const int nunits = K / 64;
  const int ngroups = nunits / UPG;
  // K split into S ranges of contiguous scale groups: this workgroup's
  // groups are [g_lo, g_hi), its units [u_lo, u_hi).
  const int gps = (ngroups + S - 1) / S;
  const int g_lo = min(ngroups, split * gps), g_hi = min(ngroups, split * gps + gps);
  const int u_lo = g_lo * UPG, u_hi = g_hi * UPG;
  const int kc = lane >> 4, r16 = lane & 15;

  // Load sources: a uniform base plus a 32-bit per-lane byte offset, formed
  // once; a unit step moves the base by 1024 bytes (codes) or 64 bytes (xq).
  // Rows past the image and tokens past nb read the last valid row or token:
  // their results are never stored.
  unsigned a_vo = 0, b_vo = 0, d_vo = 0;
  {
    const int p = min(64 * wave + lane, kTM - 1);
    const int o = min(o0 + p, m_tiles * 64 - 1);
    a_vo = (unsigned)(((o >> 6) * nunits * 64 + (o & 63)) * 16);
  }
  {
    const int p = 64 * wave + lane;  // slot 0..511
    const int t = p >> 2, s = p & 3;
    const int k = s ^ ((t >> 2) & 3);
    const int b = min(b0 + t, nb - 1);
    b_vo = (unsigned)(b * K + k * 16);
  }
  // The scales of the unit's group for rows 2j, 2j+1 of the tile in dword j
  // (waves 5-7), also moved by DMA, so the loop has no global loads of its own.
  if (wave >= 5) {
    const int j = min(64 * (wave - 5) + lane, kDDwords - 1);
    const int o = min(o0 + 2 * j, m_tiles * 64 - 2);
    d_vo = (unsigned)(((o >> 6) * ngroups * 64 + (o & 63)) * 2);
  }
  const char *a_base = reinterpret_cast<const char *>(codes);
  const char *b_base = reinterpret_cast<const char *>(xq);
  const char *d_base = reinterpret_cast<const char *>(scales);
  // A unit's uniform byte offset, opaque to the loop optimiser so that the
  // addresses stay uniform base + 32-bit lane offset (no per-lane pointers).
  auto uoff = [](int x) { return (size_t)(unsigned)__builtin_amdgcn_readfirstlane(x); };
  auto issue_stage = [&](int u, int buf) {
    char *st = lds + buf * kStageBytes;
    if (wave < kAWaveLoads && (wave < kAWaveLoads - 1 || lane < kTM - 64 * (kAWaveLoads - 1)))
      __builtin_amdgcn_global_load_lds((global_void *)(a_base + uoff(u * 1024) + a_vo),
                                       (lds_void *)(st + 1024 * wave), 16, 0, 0);
    __builtin_amdgcn_global_load_lds((global_void *)(b_base + uoff(u * 64) + b_vo),
                                     (lds_void *)(st + kABytes + 1024 * wave), 16, 0, 0);
    if (wave >= 5 && (wave < 7 || lane < kDDwords - 128))
      __builtin_amdgcn_global_load_lds((global_void *)(d_base + uoff((u / UPG) * 128) + d_vo),
                                       (lds_void *)(st + kABytes + kBBytes + 256 * (wave - 5)), 4, 0, 0);
  };
  // The first two units' loads.
  if (u_lo < u_hi) issue_stage(u_lo, 0);
  if (u_lo + 1 < u_hi) issue_stage(u_lo + 1, 1);

  // Tiles of a wave: row blocks 2w and 2w + 1 by the 8 token blocks
  // (tile 8 a + c), and row block 16 by token block w (tile 16): 17 MFMA
  // tiles per wave, each code word unpacked by one wave.
  const int a_off = ((2 * wave) * 16 + r16) * 16 + kc * 4;  // + 256 for row block 2w + 1
  const int a16_off = (16 * 16 + r16) * 16 + kc * 4;
  // token t's 16-byte chunk k of a stage's xq sits in slot t * 4 + (k ^ ((t >> 2) & 3))
  const int b_off = kABytes + (r16 * 4 + (kc ^ ((r16 >> 2) & 3))) * 16;  // + 1024 per token block
  const int d_off = kABytes + kBBytes + 2 * ((2 * wave) * 16 + 4 * kc);  // + 32 for row block 2w + 1
  const int d16_off = kABytes + kBBytes + 2 * (16 * 16 + 4 * kc);

  // Per tile an exact int32 accumulator for the current scale group and the
  // f32 sum over closed groups.  A group's first MFMA starts from 0; closing
  // the group is one convert and one FMA per output.  A group is closed
  // during the next group's first unit, tile by tile just before the tile's
  // accumulator restarts; its scales are read into registers at the end of
  // its last unit, before the ring reuses the stage.
  constexpr int kTiles = kOBW * kBB + 1;
  i32x4 acc[kTiles];
  float facc[kTiles][4];
  uint2 dq[kOBW + 1];
#pragma unroll
  for (int j = 0; j < kTiles; j++) {
    acc[j] = i32x4{0, 0, 0, 0};
#pragma unroll
    for (int v = 0; v < 4; v++) facc[j][v] = 0.0f;
  }
#pragma unroll
  for (int a = 0; a <= kOBW; a++) dq[a] = make_uint2(0u, 0u);

  // facc += d * acc for tile j, whose rows' scales are in dq[a].
  auto close_tile = [&](int j, int a) {
    const float d0 = half_bits_to_f32(dq[a].x & 0xffff), d1 = half_bits_to_f32(dq[a].x >> 16);
    const float d2 = half_bits_to_f32(dq[a].y & 0xffff), d3 = half_bits_to_f32(dq[a].y >> 16);
    facc[j][0] = fmaf(d0, (float)acc[j].x, facc[j][0]);
    facc[j][1] = fmaf(d1, (float)acc[j].y, facc[j][1]);
    facc[j][2] = fmaf(d2, (float)acc[j].z, facc[j][2]);
    facc[j][3] = fmaf(d3, (float)acc[j].w, facc[j][3]);
  };
  // code - 1 as a signed byte: byte j of 0x020100ff is code j - 1 (v_perm_b32
  // with the codes as selectors 0..3 picks it)
  auto unpack = [](unsigned w) {
    constexpr unsigned lut = 0x020100ffu;
    return i32x4{(int)__builtin_amdgcn_perm(0u, lut, w & 0x03030303u),
                 (int)__builtin_amdgcn_perm(0u, lut, (w >> 2) & 0x03030303u),
                 (int)__builtin_amdgcn_perm(0u, lut, (w >> 4) & 0x03030303u),
                 (int)__builtin_amdgcn_perm(0u, lut, (w >> 6) & 0x03030303u)};
  };
  // One unit in stage buffer buf of group g (relative to g_lo).  FIRST: the
  // group's first unit (the previous group closes, the accumulators restart
  // from 0); LAST: the group's last unit (its scales are kept).
  auto unit = [&](int buf, int g, auto first_c, auto last_c) {
    constexpr bool FIRST = decltype(first_c)::value;
    constexpr bool LAST = decltype(last_c)::value;
    const char *st = lds + buf * kStageBytes;
    const i32x4 af0 = unpack(*reinterpret_cast<const unsigned *>(st + a_off));
    const i32x4 af1 = unpack(*reinterpret_cast<const unsigned *>(st + a_off + 256));
#pragma unroll
    for (int c = 0; c < kBB; c++) {
      const i32x4 bf = *reinterpret_cast<const i32x4 *>(st + b_off + 1024 * c);
      if constexpr (FIRST) {
        const i32x4 n = i32x4{0, 0, 0, 0};
        close_tile(c, 0);
        close_tile(kBB + c, 1);
        acc[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af0, bf, n, 0, 0, 0);
        acc[kBB + c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af1, bf, n, 0, 0, 0);
      } else {
        acc[c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af0, bf, acc[c], 0, 0, 0);
        acc[kBB + c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af1, bf, acc[kBB + c], 0, 0, 0);
      }
    }
    {
      const i32x4 af = unpack(*reinterpret_cast<const unsigned *>(st + a16_off));
      const i32x4 bf = *reinterpret_cast<const i32x4 *>(st + b_off + 1024 * wave);
      if constexpr (FIRST) {
        const i32x4 n = i32x4{0, 0, 0, 0};
        close_tile(kTiles - 1, kOBW);
        acc[kTiles - 1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, bf, n, 0, 0, 0);
      } else {
        acc[kTiles - 1] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, bf, acc[kTiles - 1], 0, 0, 0);
      }
    }
    if constexpr (LAST) {
      dq[0] = *reinterpret_cast<const uint2 *>(st + d_off);
      dq[1] = *reinterpret_cast<const uint2 *>(st + d_off + 32);
      dq[2] = *reinterpret_cast<const uint2 *>(st + d16_off);
    }
  };

  // K loop over the ring, one window of two units per barrier: after the
  // barrier that makes the loads of units u, u + 1 (stage buffers B0,
  // B0 + 1) visible, the loads of u + 2, u + 3 go out into the buffers the
  // previous window used, and u, u + 1 are multiplied.
  for (int u = u_lo; u < u_hi; u += 2) {
    const int B0 = (u - u_lo) & 2;
    __builtin_amdgcn_s_waitcnt(0x0070);
    asm volatile("s_barrier" ::: "memory");
    if (u + 2 < u_hi) issue_stage(u + 2, B0 ^ 2);
    if (u + 3 < u_hi) issue_stage(u + 3, (B0 ^ 2) + 1);
    const int g = (u - u_lo) / UPG;
    if constexpr (UPG == 2) {  // one g128 group: units u, u + 1 (K is a multiple of 128)
      unit(B0, g, BC<true>{}, BC<false>{});
      unit(B0 + 1, g, BC<false>{}, BC<true>{});
    } else {  // two g64 groups
      unit(B0, g, BC<true>{}, BC<true>{});
      if (u + 1 < u_hi) unit(B0 + 1, g + 1, BC<true>{}, BC<true>{});
    }
  }
  close_tile(kTiles - 1, kOBW);
#pragma unroll
  for (int c = 0; c < kBB; c++) {
    close_tile(c, 0);
    close_tile(kBB + c, 1);
  }

  // Epilogue: y[b, o] = act_scale[b] * acc (+ accum[b, o]), two roundings;
  // with a K split, the f32 partial sums go to part[split][b][o] instead.
  // Every tile's act_scale and residual values are read before the first
  // store (a wait for a load also waits for the stores before it); each
  // output's residual is read by the lane that writes it, so y may be accum.
  const bool vec = (M & 3) == 0;
  float scl[kBB + 1];
  float res[kTiles][4];
  if (S == 1) {
#pragma unroll
    for (int c = 0; c <= kBB; c++) scl[c] = act_scale[min(b0 + (c < kBB ? c : wave) * 16 + r16, nb - 1)];
#pragma unroll
    for (int j = 0; j < kTiles; j++) {
      const int blk = j < kTiles - 1 ? 2 * wave + j / kBB : 16;
      const int c = j < kTiles - 1 ? j % kBB : wave;
      const int b = b0 + c * 16 + r16;
      const int o = o0 + blk * 16 + 4 * kc;
#pragma unroll
      for (int v = 0; v < 4; v++)
        res[j][v] = (accum && b < nb && o + v < M) ? accum[(size_t)b * M + o + v] : 0.0f;
    }
  }
#pragma unroll
  for (int j = 0; j < kTiles; j++) {
    const int blk = j < kTiles - 1 ? 2 * wave + j / kBB : 16;
    const int c = j < kTiles - 1 ? j % kBB : wave;
    const int b = b0 + c * 16 + r16;
    const int o = o0 + blk * 16 + 4 * kc;
    if (b >= nb || o >= M) continue;
    float r[4];
    if (S > 1) {
#pragma unroll
      for (int v = 0; v < 4; v++) r[v] = facc[j][v];
    } else {
      const float sc = scl[j < kTiles - 1 ? c : kBB];
#pragma unroll
      for (int v = 0; v < 4; v++) {
        r[v] = __fmul_rn(facc[j][v], sc);
        if (accum) r[v] = __fadd_rn(r[v], res[j][v]);
      }
    }
    float *dst = S > 1 ? part + ((size_t)split * nb + b) * M + o : y + (size_t)b * M + o;
    if (vec && o + 3 < M) {
      if (S > 1)  // partials: read back at once by the reduce kernel, kept in the caches
        *reinterpret_cast<float4 *>(dst) = make_float4(r[0], r[1], r[2], r[3]);
      else  // the output: streamed out (every workgroup stores at once, at the end)
        __builtin_nontemporal_store(f32x4{r[0], r[1], r[2], r[3]}, reinterpret_cast<f32x4 *>(dst));
    } else {
#pragma unroll
      for (int v = 0; v < 4; v++)
        if (o + v < M) dst[v] = r[v];
    }
  }
}


// y[b, o] = act_scale[b] * sum_s part[s][b][o] (+ accum[b, o]), the splits
// added in fixed order.  V4: four consecutive outputs of one row per thread
// (M a multiple of 4, accum 16-byte aligned), as 16-byte loads and a
// streaming store; the same arithmetic per output.
// blockIdx.y selects the matrix of a pair launch: its partials start at
// part + y * S * n and its output is y0 or y1.
template <bool V4>
__global__ __launch_bounds__(256) void q2_gemm_reduce_kernel(const float *__restrict__ part, int S, size_t n, int M,
                                                            const float *__restrict__ act_scale, const float *accum,
                                                            float *y0, float *y1) {
  float *y = blockIdx.y ? y1 : y0;
  part += (size_t)blockIdx.y * S * n;
  if (V4) {
    const size_t i = ((size_t)blockIdx.x * 256 + threadIdx.x) * 4;
    if (i >= n) return;
    float s[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int k = 0; k < S; k++) {
      const f32x4 p = *reinterpret_cast<const f32x4 *>(part + (size_t)k * n + i);
      s[0] += p.x, s[1] += p.y, s[2] += p.z, s[3] += p.w;
    }
    const float sc = act_scale[i / M];
    float r[4];
#pragma unroll
    for (int v = 0; v < 4; v++) r[v] = __fmul_rn(s[v], sc);
    if (accum) {
      const f32x4 a = *reinterpret_cast<const f32x4 *>(accum + i);
      r[0] = __fadd_rn(r[0], a.x), r[1] = __fadd_rn(r[1], a.y), r[2] = __fadd_rn(r[2], a.z), r[3] = __fadd_rn(r[3], a.w);
    }
    __builtin_nontemporal_store(f32x4{r[0], r[1], r[2], r[3]}, reinterpret_cast<f32x4 *>(y + i));
    return;
  }
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  float s = 0.0f;
  for (int k = 0; k < S; k++) s += part[(size_t)k * n + i];
  float r = __fmul_rn(s, act_scale[i / M]);
  if (accum) r = __fadd_rn(r, accum[i]);
  y[i] = r;
}

}  // namespace

// K splits: enough to give about one workgroup per CU when the (row tile,
// token tile) pairs alone cannot (at least one scale group per split).
int q2_gemm_split(int64_t M, int64_t K, int group, int64_t nb) {
  const int64_t tiles = (M + kTM - 1) / kTM * ((nb + kTN - 1) / kTN);
  const int64_t ngroups = K / group;
  int64_t S = 256 / tiles;
  if (S > ngroups) S = ngroups;
  if (S > 16) S = 16;
  if (S < 1) S = 1;
  return (int)S;
}

hipError_t launch_q2_gemm(const void *codes, const void *scales, int M, int K, int group, const int8_t *xq,
                          const float *act_scale, const float *accum, float *y, int nb,
                          float *part, hipStream_t stream, const void *codes1, const void *scales1, float *y1) {
  const int n_ot = (M + kTM - 1) / kTM;
  const int n_bt = (nb + kTN - 1) / kTN;
  const int S = q2_gemm_split(M, K, group, nb);
  const int njobs = codes1 ? 2 : 1;
  const dim3 grid((n_ot * S + 7) / 8 * 8 * n_bt, njobs);
  Q2Pair pa{};
  pa.codes[0] = reinterpret_cast<const i32x4 *>(codes);
  pa.scales[0] = reinterpret_cast<const unsigned short *>(scales);
  pa.y[0] = y;
  pa.codes[1] = codes1 ? reinterpret_cast<const i32x4 *>(codes1) : pa.codes[0];
  pa.scales[1] = scales1 ? reinterpret_cast<const unsigned short *>(scales1) : pa.scales[0];
  pa.y[1] = y1 ? y1 : y;
  if (group == 64)
    q2_gemm_kernel<1><<<grid, kThreads, 0, stream>>>(pa, xq, act_scale, accum, nb, M, K, n_ot, n_bt, S, part);
  else
    q2_gemm_kernel<2><<<grid, kThreads, 0, stream>>>(pa, xq, act_scale, accum, nb, M, K, n_ot, n_bt, S, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  const size_t n = (size_t)nb * M;
  if (M % 4 == 0 && (reinterpret_cast<uintptr_t>(accum) & 15) == 0) {
    const dim3 rgrid((unsigned)((n / 4 + 255) / 256), njobs);
    q2_gemm_reduce_kernel<true><<<rgrid, 256, 0, stream>>>(part, S, n, M, act_scale, accum, pa.y[0], pa.y[1]);
  } else {
    const dim3 rgrid((unsigned)((n + 255) / 256), njobs);
    q2_gemm_reduce_kernel<false><<<rgrid, 256, 0, stream>>>(part, S, n, M, act_scale, accum, pa.y[0], pa.y[1]);
  }
  return hipGetLastError();
}

}  // namespace qg
