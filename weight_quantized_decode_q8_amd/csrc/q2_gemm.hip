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
//    operand is the weights' 2-bit codes used as unsigned bytes 0..3: a lane
//    (row lane % 16, k chunk lane / 16) needs word (lane / 16) of its row's
//    unit, and (word >> 2a) & 0x03030303 is dword a of its 16-byte fragment
//    in natural k order (the T64 code order), so A costs 4 bytes per lane
//    per 16 x 64 block: a quarter of an int8 weight operand.
//  - B is xq as stored, [nb][K]; the "- 1" is the group's suma[b] subtracted
//    per token column, as in the GEMV (sum code*xq - sum xq).
//  - int32 accumulation over a scale group's units (exact), started from
//    -suma so that closing the group is one convert and one f32 FMA per
//    output with d(o, g), as the GEMV does per group; this per-group VALU
//    work, not the MFMA, is what the kernel's time is made of.
//  - tile 272 weight rows x 128 tokens per 8-wave workgroup (17408 = 64 x
//    272: 256 workgroups at the FFN width and 512 tokens), waves 4 (rows) x
//    2 (tokens), so each code word is unpacked by two waves rather than
//    four; operands go global -> LDS directly (global_load_lds) through
//    a 4-stage ring, two units per barrier, each stage also carrying the
//    unit's group scales and suma, so the loop issues no other global load;
//    the token pieces are stored with an XOR swizzle so the 128-bit fragment
//    reads hit distinct LDS banks; workgroups sharing a weight tile are
//    dispatched to one XCD.
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
typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void global_void;

constexpr int kOB = 17;        // 16-row MFMA blocks per tile
constexpr int kTM = 16 * kOB;  // 272 weight rows per tile
constexpr int kTN = 128;       // tokens per tile
constexpr int kWR = 4;         // wave groups along rows: blocks 0-4, 5-8, 9-12, 13-16
constexpr int kOBW = 5;        // most row blocks of one wave
constexpr int kWC = 2;         // wave groups along tokens
constexpr int kWaves = kWR * kWC;
constexpr int kThreads = 64 * kWaves;
constexpr int kBB = kTN / kWC / 16;  // 16-token blocks per wave (4)
// LDS ring depth in units: the loads of units u + kStages - 2 and
// u + kStages - 1 go out while units u and u + 1 are multiplied.
#ifndef QG_Q2GEMM_STAGES
#define QG_Q2GEMM_STAGES 4
#endif
constexpr int kStages = QG_Q2GEMM_STAGES;
static_assert(kStages % 2 == 0 && kStages >= 4, "two units per barrier");
constexpr int kABytes = kTM * 16;    // one unit of codes for the tile's rows (4352)
constexpr int kBBytes = kTN * 64;    // one unit of xq for the tile's tokens (8192)
constexpr int kDBytes = kTM * 2;     // the unit's group scales for the tile's rows (544)
constexpr int kSBytes = kTN * 4;     // the unit's suma for the tile's tokens (512)
constexpr int kStageBytes = kABytes + kBBytes + kDBytes + kSBytes;
constexpr int kAWaveLoads = (kTM + 63) / 64;  // 5, the last one 16 lanes wide
constexpr int kDDwords = kDBytes / 4;         // 136: waves 5, 6 and 8 lanes of wave 7

constexpr int vmcnt_imm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// Waits until at most n of this wave's vector memory operations are
// outstanding (n uniform; s_waitcnt takes an immediate).
__device__ inline void wait_vm_at_most(int n) {
  switch (n) {
#define QG_VM(k) \
  case k: __builtin_amdgcn_s_waitcnt(vmcnt_imm(k)); break;
    QG_VM(1) QG_VM(2) QG_VM(3) QG_VM(4) QG_VM(5) QG_VM(6) QG_VM(7) QG_VM(8) QG_VM(9) QG_VM(10) QG_VM(11)
    QG_VM(12) QG_VM(13) QG_VM(14) QG_VM(15) QG_VM(16) QG_VM(17) QG_VM(18) QG_VM(19) QG_VM(20) QG_VM(21)
#undef QG_VM
    default: __builtin_amdgcn_s_waitcnt(vmcnt_imm(0)); break;
  }
}

// LDS slot of token t's 16-byte chunk k within a stage's xq part.
__device__ inline int b_slot(int t, int k) { return t * 4 + (k ^ ((t >> 2) & 3)); }

__device__ inline float half_bits_to_f32(unsigned short h) { return (float)__builtin_bit_cast(_Float16, h); }

// The two weight matrices of a pair launch (gate and up against one set of
// token rows); a one-matrix launch uses entry 0 only.
struct Q2Pair {
  const i32x4 *codes[2];
  const unsigned short *scales[2];
  float *y[2];
};

template <int UPG>
__global__ __launch_bounds__(kThreads, 1) void q2_gemm_kernel(
    Q2Pair pair_args, const int8_t *__restrict__ xq, const int *__restrict__ suma,
    const float *__restrict__ act_scale, const float *accum, int nb, int M, int K, int n_ot, int n_bt, int n_split,
    float *__restrict__ part) {
  __shared__ __attribute__((aligned(16))) char lds[kStages * kStageBytes];
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
  const int wq = wave % kWC, wh = wave / kWC;
  const int ob0 = wh == 0 ? 0 : 1 + 4 * wh;  // first row block of this wave
  const int nob = wh == 0 ? kOBW : 4;
  const int o0 = ot * kTM, b0 = bt * kTN;
  const int m_tiles = (M + 63) / 64;
  const int nunits = K / 64;
  const int ngroups = nunits / UPG;
  // K split into S ranges of contiguous scale groups: this workgroup's
  // units are [u_lo, u_hi).
  const int gps = (ngroups + S - 1) / S;
  const int u_lo = min(ngroups, split * gps) * UPG;
  const int u_hi = min(ngroups, split * gps + gps) * UPG;
  const int kc = lane >> 4, r16 = lane & 15;

  // Load sources, formed once; a unit step moves each by 64 (codes, in
  // 16-byte units) or 64 bytes (xq).  Rows past the image and tokens past nb
  // read the last valid row or token: their results are never stored.
  const i32x4 *a_src = nullptr;
  {
    const int p = min(64 * wave + lane, kTM - 1);
    const int o = min(o0 + p, m_tiles * 64 - 1);
    a_src = codes + (size_t)(o >> 6) * nunits * 64 + (o & 63);
  }
  const int8_t *b_src;
  {
    const int p = 64 * wave + lane;  // slot 0..511
    const int t = p >> 2, s = p & 3;
    const int k = s ^ ((t >> 2) & 3);
    const int b = min(b0 + t, nb - 1);
    b_src = xq + (size_t)b * K + k * 16;
  }
  // Per-unit group data, also moved by DMA (4 bytes per lane) so that the
  // loop has no global loads of its own: the scales of the unit's group for
  // rows 2j, 2j+1 of the tile in dword j (waves 5-7), and the unit's suma for
  // each token (waves 3-4).
  const unsigned short *d_src = nullptr;
  if (wave >= 5) {
    const int j = min(64 * (wave - 5) + lane, kDDwords - 1);
    const int o = min(o0 + 2 * j, m_tiles * 64 - 2);
    d_src = scales + (size_t)(o >> 6) * ngroups * 64 + (o & 63);
  }
  const int *s_src = nullptr;
  if (wave == 3 || wave == 4) {
    const int t = 64 * (wave - 3) + lane;
    s_src = suma + (size_t)min(b0 + t, nb - 1) * nunits;
  }
  auto stage_a = [&](int buf) { return lds + buf * kStageBytes; };
  auto stage_b = [&](int buf) { return lds + buf * kStageBytes + kABytes; };
  auto stage_d = [&](int buf) { return lds + buf * kStageBytes + kABytes + kBBytes; };
  auto stage_s = [&](int buf) { return lds + buf * kStageBytes + kABytes + kBBytes + kDBytes; };
  auto issue_stage = [&](int u) {
    const int buf = u % kStages;
    if (wave < kAWaveLoads && (wave < kAWaveLoads - 1 || lane < kTM - 64 * (kAWaveLoads - 1)))
      __builtin_amdgcn_global_load_lds((global_void *)(a_src + (size_t)u * 64), (lds_void *)(stage_a(buf) + 1024 * wave),
                                       16, 0, 0);
    __builtin_amdgcn_global_load_lds((global_void *)(b_src + (size_t)u * 64), (lds_void *)(stage_b(buf) + 1024 * wave),
                                     16, 0, 0);
    if (wave >= 5 && (wave < 7 || lane < kDDwords - 128))
      __builtin_amdgcn_global_load_lds((global_void *)(d_src + (size_t)(u / UPG) * 64),
                                       (lds_void *)(stage_d(buf) + 256 * (wave - 5)), 4, 0, 0);
    if (wave == 3 || wave == 4)
      __builtin_amdgcn_global_load_lds((global_void *)(s_src + u), (lds_void *)(stage_s(buf) + 256 * (wave - 3)), 4, 0,
                                       0);
  };

  // Per tile an exact int32 accumulator for the current scale group and the
  // f32 sum over closed groups.  A group's first MFMA starts from -suma of
  // the group's tokens instead of 0, so the int32 result is already
  // sum (code - 1) * xq and closing the group is one convert and one FMA.
  i32x4 acc[kOBW][kBB];
  float facc[kOBW][kBB][4];
#pragma unroll
  for (int a = 0; a < kOBW; a++)
#pragma unroll
    for (int c = 0; c < kBB; c++) {
      acc[a][c] = i32x4{0, 0, 0, 0};
#pragma unroll
      for (int v = 0; v < 4; v++) facc[a][c][v] = 0.0f;
    }

  // -suma of a group for this lane's token in each token block; the group's
  // units sit in stage buffers buf0 and (g128) buf1.
  auto group_start = [&](int buf0, int buf1, i32x4 (&nc)[kBB]) {
#pragma unroll
    for (int c = 0; c < kBB; c++) {
      const int t = wq * (kTN / kWC) + c * 16 + r16;
      int sum = *reinterpret_cast<const int *>(stage_s(buf0) + 4 * t);
      if (UPG == 2) sum += *reinterpret_cast<const int *>(stage_s(buf1) + 4 * t);
      nc[c] = i32x4{-sum, -sum, -sum, -sum};
    }
  };
  // Close a group whose scales sit in stage buffer buf: facc += d * acc.
  auto close_group = [&](int buf) {
#pragma unroll
    for (int a = 0; a < kOBW; a++) {
      if (a < nob) {
        const uint2 dq = *reinterpret_cast<const uint2 *>(stage_d(buf) + 2 * ((ob0 + a) * 16 + 4 * kc));
        const float d[4] = {half_bits_to_f32(dq.x & 0xffff), half_bits_to_f32(dq.x >> 16),
                            half_bits_to_f32(dq.y & 0xffff), half_bits_to_f32(dq.y >> 16)};
#pragma unroll
        for (int c = 0; c < kBB; c++) {
          facc[a][c][0] = fmaf(d[0], (float)acc[a][c].x, facc[a][c][0]);
          facc[a][c][1] = fmaf(d[1], (float)acc[a][c].y, facc[a][c][1]);
          facc[a][c][2] = fmaf(d[2], (float)acc[a][c].z, facc[a][c][2]);
          facc[a][c][3] = fmaf(d[3], (float)acc[a][c].w, facc[a][c][3]);
        }
      }
    }
  };

  // One unit: B fragments of the wave's token blocks, then per row block the
  // code word unpacked into an A fragment and one MFMA per token block; the
  // group's first unit starts each accumulator from nc.
  auto compute_unit = [&](int buf, bool first, const i32x4 (&nc)[kBB]) {
    i32x4 bf[kBB];
#pragma unroll
    for (int c = 0; c < kBB; c++) {
      const int t = wq * (kTN / kWC) + c * 16 + r16;
      bf[c] = *reinterpret_cast<const i32x4 *>(stage_b(buf) + b_slot(t, kc) * 16);
    }
#pragma unroll
    for (int a = 0; a < kOBW; a++) {
      if (a < nob) {
        const unsigned w = *reinterpret_cast<const unsigned *>(stage_a(buf) + ((ob0 + a) * 16 + r16) * 16 + kc * 4);
        const i32x4 af = {(int)(w & 0x03030303u), (int)((w >> 2) & 0x03030303u), (int)((w >> 4) & 0x03030303u),
                          (int)((w >> 6) & 0x03030303u)};
#pragma unroll
        for (int c = 0; c < kBB; c++)
          acc[a][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af, bf[c], first ? nc[c] : acc[a][c], 0, 0, 0);
      }
    }
  };

  // K loop over the ring, two units per barrier: while units u, u+1 are
  // multiplied, the loads of u+2 ... u+kStages-1 are in flight, the last two
  // of them into the buffers that u-2, u-1 used.  A wave's loads complete in
  // order, so it waits until only the stages after u+1 are outstanding
  // (this wave's loads per stage: the token pieces, plus the codes for
  // waves 0-4, the scales for waves 5-7 and the sums for waves 3-4).
  const int nl = 1 + (wave < kAWaveLoads ? 1 : 0) + (wave >= 5 ? 1 : 0) + ((wave == 3 || wave == 4) ? 1 : 0);
#pragma unroll
  for (int k = 0; k < kStages - 2; k++)
    if (u_lo + k < u_hi) issue_stage(u_lo + k);
  for (int u = u_lo; u < u_hi; u += 2) {
    const int after = max(0, min(kStages - 4, u_hi - (u + 2)));  // stages issued after u + 1
    wait_vm_at_most(after * nl);
    asm volatile("s_barrier" ::: "memory");  // every wave's loads of u, u+1 are in LDS
    if (u + kStages - 2 < u_hi) issue_stage(u + kStages - 2);
    if (u + kStages - 1 < u_hi) issue_stage(u + kStages - 1);
    const int b0u = u % kStages, b1u = (u + 1) % kStages;
    i32x4 nc[kBB];
    if (UPG == 2) {  // one g128 group: units u, u+1 (K is a multiple of 128)
      group_start(b0u, b1u, nc);
      compute_unit(b0u, true, nc);
      compute_unit(b1u, false, nc);
      close_group(b1u);
    } else {  // two g64 groups
      group_start(b0u, b0u, nc);
      compute_unit(b0u, true, nc);
      close_group(b0u);
      if (u + 1 < u_hi) {
        group_start(b1u, b1u, nc);
        compute_unit(b1u, true, nc);
        close_group(b1u);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));

  // Epilogue: y[b, o] = act_scale[b] * acc (+ accum[b, o]), two roundings;
  // with a K split, the f32 partial sums go to part[split][b][o] instead.
  const bool vec = (M & 3) == 0;
  if (S > 1) {
#pragma unroll
    for (int c = 0; c < kBB; c++) {
      const int b = b0 + wq * (kTN / kWC) + c * 16 + r16;
      if (b >= nb) continue;
#pragma unroll
      for (int a = 0; a < kOBW; a++) {
        if (a >= nob) continue;
        const int o = o0 + (ob0 + a) * 16 + 4 * kc;
        if (o >= M) continue;
        float *dst = part + ((size_t)split * nb + b) * M + o;
        if (vec && o + 3 < M) {
          *reinterpret_cast<float4 *>(dst) = make_float4(facc[a][c][0], facc[a][c][1], facc[a][c][2], facc[a][c][3]);
        } else {
#pragma unroll
          for (int v = 0; v < 4; v++)
            if (o + v < M) dst[v] = facc[a][c][v];
        }
      }
    }
    return;
  }
#pragma unroll
  for (int c = 0; c < kBB; c++) {
    const int b = b0 + wq * (kTN / kWC) + c * 16 + r16;
    if (b >= nb) continue;
    const float sc = act_scale[b];
#pragma unroll
    for (int a = 0; a < kOBW; a++) {
      if (a >= nob) continue;
      const int o = o0 + (ob0 + a) * 16 + 4 * kc;
      if (o >= M) continue;
      float r[4];
#pragma unroll
      for (int v = 0; v < 4; v++) {
        r[v] = __fmul_rn(facc[a][c][v], sc);
        if (accum && o + v < M) r[v] = __fadd_rn(r[v], accum[(size_t)b * M + o + v]);
      }
      float *dst = y + (size_t)b * M + o;
      if (vec && o + 3 < M) {
        *reinterpret_cast<float4 *>(dst) = make_float4(r[0], r[1], r[2], r[3]);
      } else {
#pragma unroll
        for (int v = 0; v < 4; v++)
          if (o + v < M) dst[v] = r[v];
      }
    }
  }
}


// y[b, o] = act_scale[b] * sum_s part[s][b][o] (+ accum[b, o]), the splits
// added in fixed order.
// blockIdx.y selects the matrix of a pair launch: its partials start at
// part + y * S * n and its output is y0 or y1.
__global__ __launch_bounds__(256) void q2_gemm_reduce_kernel(const float *__restrict__ part, int S, size_t n, int M,
                                                            const float *__restrict__ act_scale, const float *accum,
                                                            float *y0, float *y1) {
  float *y = blockIdx.y ? y1 : y0;
  part += (size_t)blockIdx.y * S * n;
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
  return S < 1 ? 1 : (int)S;
}

hipError_t launch_q2_gemm(const void *codes, const void *scales, int M, int K, int group, const int8_t *xq,
                          const int32_t *suma, const float *act_scale, const float *accum, float *y, int nb,
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
  const int *sa = reinterpret_cast<const int *>(suma);
  if (group == 64)
    q2_gemm_kernel<1><<<grid, kThreads, 0, stream>>>(pa, xq, sa, act_scale, accum, nb, M, K, n_ot, n_bt, S, part);
  else
    q2_gemm_kernel<2><<<grid, kThreads, 0, stream>>>(pa, xq, sa, act_scale, accum, nb, M, K, n_ot, n_bt, S, part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || S == 1) return e;
  const size_t n = (size_t)nb * M;
  const dim3 rgrid((unsigned)((n + 255) / 256), njobs);
  q2_gemm_reduce_kernel<<<rgrid, 256, 0, stream>>>(part, S, n, M, act_scale, accum, pa.y[0], pa.y[1]);
  return hipGetLastError();
}

}  // namespace qg
