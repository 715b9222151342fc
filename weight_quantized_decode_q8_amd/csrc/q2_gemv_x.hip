// q2_gemv_x.hip -- the decode Q2 GEMVs with the activation side in the same
// launch: each workgroup quantises the f32 input vector itself (optionally
// after an RMSNorm), and split-K partials are added by the last workgroup of
// each row tile instead of a second kernel.
//
// What is computed is exactly what the two- or three-launch chains compute
// (qxmx qxmx_gpu.cpp page: gpu_rmsnorm_quant or the plain quantiser, then
// gemv_dpas8 and gemv_reduce; gemv_dpas8_dual for the gate|up pair; the
// cortiq-engine 0.5.43 gpu_wgpu.rs page, moe_gate_up, for the gated product
// in the epilogue):
//   v      = x, or (x * inv) * w with inv = 1/sqrt(ms + eps) (RMSNorm)
//   sc     = max|v| / 127, inv = 1 / sc (0 when sc is 0), both rounded to
//            binary32, xq = clamp(round(v * inv)): one product per value,
//            never a division by sc; suma = per-64 sums
//   y[o]   = sc * sum_u d(o,u) * (sum_{i in u} code_i * xq_i - suma_u)
// with the same per-wave group ranges, the same f32 accumulation order, the
// same wave combine and the same split order as q2_gemv_t64_kernel and
// q2_splitk_reduce_kernel, so every output equals the multi-launch chain
// bit for bit.
//
// Why (MI355X): a kernel launch in a stream or graph costs a few
// microseconds before its first bytes arrive, as much as streaming 10-20 MB,
// and the decode FFN's quantisers and split reduce each paid it for a few
// tens of KiB of work.  Quantising in every workgroup repeats that small
// work (the vector is read from L2) but overlaps it with the workgroup's
// first weight loads, which stream in during the prologue.
//
// Layout of the work: one row tile (64 rows, one per lane) of one matrix per
// workgroup, with the plain kernel's waves per tile and K split over the
// waves as in q2_gemv_t64_kernel; the gate|up pair is two matrices' tiles in
// one grid.  The activation words, which the plain kernel reads through the
// scalar cache, come from LDS here (broadcast ds_read_b128: every lane reads
// the same address).
//
// Split-K in one launch: each (tile, split) workgroup stores its partial and
// then increments the tile's counter; the workgroup that sees the count S-1
// adds the S partials in split order, setting them and the counter back to
// zero: the workspace is all zero between calls, so one workspace serves
// calls of any shape and split.  The gate|up pair with the gated product
// meets the same way: each matrix's workgroup of a tile stores its g or u,
// and the second to arrive forms t.  No workgroup waits on another, so
// nothing can hang on a missing arrival.
#include "arrival.h"
#include "gate_rule.h"
#include "q2_unit.h"
#include "qg_internal.h"
#include "quant_rule.h"

// g128 groups per load step: the gate|up pair, and the one-matrix form fed
// partial maxima (the down projection, whose waves hold 2-3 groups each).
#ifndef QG_X_PAIR_GPB
#define QG_X_PAIR_GPB 2
#endif
#ifndef QG_X_PARTS_GPB
#define QG_X_PARTS_GPB 2
#endif

namespace qg {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

// s_waitcnt immediate for lgkmcnt(0) alone (gfx9 encoding: vmcnt and
// expcnt at their maxima, i.e. not waited for).
constexpr int kLgkm0 = 0xC07F;

// A workgroup barrier that makes this wave's LDS writes visible but leaves
// its global loads in flight (__syncthreads() would also wait for those,
// i.e. for the weight loads issued before the prologue).
__device__ inline void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(kLgkm0);
  asm volatile("s_barrier" ::: "memory");
}

// Corrected dot of one unit: sum_{64 weights} code*xq - suma, the
// activation words given as four 128-bit values.
__device__ inline int unit_dot_v(const i32x4 c, const i32x4 x0, const i32x4 x1, const i32x4 x2, const i32x4 x3,
                                 int sa) {
  return q2_unit_dot(c, x0, x1, x2, x3, sa);
}

__device__ inline float half_bits_to_f32(unsigned short h) {
  return (float)__builtin_bit_cast(_Float16, h);
}

__device__ inline float scale_add(float acc, float sc, const float *accum, int o) {
  const float y = __fmul_rn(acc, sc);
  return accum ? __fadd_rn(y, accum[o]) : y;
}

struct XArgs {
  const i32x4 *codes[2];
  const unsigned short *scales[2];
  const float4 *x;       // the f32 input vector [K]
  const float4 *norm_w;  // RMSNorm weights [K] (PRO_NORM)
  float eps;
  float *y[2];           // outputs; EPI_GLU: t in y[0]
  const float *accum;    // one matrix: residual or null
  float *part;           // S > 1: partials [S][Mp]; EPI_GLU: g and u [2][Mp]
  int *cnt;              // S > 1 or EPI_GLU: arrival counters [tiles]
  const float *xmax;     // PRO_PARTS: nxmax partial maxima of |x|
  float *tmax;           // EPI_GLU: max|t| of each row tile, or null
  unsigned long long *stamps;  // measurement only: 4 wall-clock stamps per workgroup, or null
  int M, K, S, tiles, nxmax;
};

// Measurement stamps (the timeline probe): the wall clock at the
// workgroup's start, after its prologue, when its tile result is ready and
// at its exit, by thread 0.  Null in every product call.
__device__ inline void stamp(const XArgs &a, int k) {
  if (a.stamps && threadIdx.x == 0)
    a.stamps[((size_t)blockIdx.y * gridDim.x + blockIdx.x) * 4 + k] = wall_clock64();
}

// PRO_PARTS: the caller gives max|x| as partial maxima (at most
// kMaxXParts, e.g. the per-tile max|t| the gate|up launch wrote), so a
// workgroup loads only its own split's part of the vector.
enum { PRO_X = 0, PRO_NORM = 1, PRO_PARTS = 2 };
constexpr int kPartsPerLane = kQ2XMaxParts / 64;
enum { EPI_Y = 0, EPI_GLU_SILU = 1, EPI_GLU_SIGMOID = 2 };

// Largest of every thread's m over an NT-thread workgroup (exact).
template <int NT>
__device__ inline float block_max_nt(float m, float *red) {
  for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = m;
  lds_barrier();
  float r = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; w++) r = fmaxf(r, red[w]);
  return r;
}

// grid = (row tiles x matrices, splits), one row tile of one matrix per
// workgroup of W waves (the plain kernel's waves per tile).  RQ quads of the
// vector are held per thread (K <= 4 * RQ * 64 * W).  UPG units per scale
// group, GPB groups per load step.
template <int UPG, int GPB, int W, int RQ, int PRO, int EPI>
__global__ __launch_bounds__(64 * W) void q2_gemv_x_kernel(XArgs a) {
  constexpr int NT = 64 * W;
  constexpr int VPT = 1024 / NT;  // RMSNorm: threads of the 1024-thread order per thread
  __shared__ i32x4 xl[RQ * NT / 4];  // xq of this split's units, 16 per entry
  __shared__ int sl[RQ * NT / 16];    // their 64-wide sums
  __shared__ float red[W - 1][64];
  __shared__ float rmax[W];
  __shared__ double rss[16];

  stamp(a, 0);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int mat = (int)blockIdx.x >= a.tiles ? 1 : 0;
  const int tile = (int)blockIdx.x - mat * a.tiles;
  const int split = blockIdx.y, S = a.S;
  const int M = a.M, K = a.K, Mp = a.tiles * 64;
  const int nunits = K / 64, ngroups = nunits / UPG;

  // Groups of this split (the plain kernel's partition), then of this wave:
  // contiguous ranges.
  const int gps = (ngroups + S - 1) / S;
  const int gs0 = min(ngroups, split * gps);
  const int gs1 = min(ngroups, gs0 + gps);
  const int per = (gs1 - gs0 + W - 1) / W;
  const int g0 = min(gs1, gs0 + wave * per);
  const int g1 = min(gs1, g0 + per);
  const int u0 = gs0 * UPG;  // first unit held in LDS

  const i32x4 *cp = (mat ? a.codes[1] : a.codes[0]) + (size_t)tile * nunits * 64 + lane;
  const unsigned short *sp = (mat ? a.scales[1] : a.scales[0]) + (size_t)tile * ngroups * 64 + lane;

  // 1. The whole vector (PRO_PARTS: this split's quads and the partial
  //    maxima) first, then this wave's first load step of weights.
  //    Every load is issued unconditionally, indices clamped into range (a
  //    clamped quad repeats the vector's last one; a clamped weight load
  //    repeats one of the wave's own), so the compiler counts them exactly:
  //    the loads return in order, and the prologue waits for the vector
  //    alone while the weights stream in.  (Issued after the vector, the
  //    first quantiser pass measured 2 us faster per launch than with the
  //    weights first, on HBM-cold weights.)
  const int n4 = K / 4;
  const int q0 = u0 * 16, q1 = gs1 * UPG * 16;  // quads of this split
  const int qbase = PRO == PRO_PARTS ? q0 : 0;  // quad held by thread tid at r = 0
  float4 v[RQ];
  float4 w[PRO == PRO_NORM ? RQ : 1];
#pragma unroll
  for (int r = 0; r < RQ; r++) {
    const int i = min(qbase + tid + r * NT, n4 - 1);
    v[r] = a.x[i];
    if (PRO == PRO_NORM) w[r] = a.norm_w[i];
  }
  float pm[PRO == PRO_PARTS ? kPartsPerLane : 1];
  if (PRO == PRO_PARTS) {
#pragma unroll
    for (int k = 0; k < kPartsPerLane; k++) pm[k] = a.xmax[min(lane + 64 * k, a.nxmax - 1)];
  }
  i32x4 c[GPB * UPG];
  unsigned short dh[GPB];
  auto prefetch = [&]() {
    const int gl = max(g1 - 1, 0);
#pragma unroll
    for (int j = 0; j < GPB; j++)
#pragma unroll
      for (int vv = 0; vv < UPG; vv++)
        c[j * UPG + vv] = __builtin_nontemporal_load(cp + (size_t)(min(g0 + j, gl) * UPG + vv) * 64);
#pragma unroll
    for (int j = 0; j < GPB; j++) dh[j] = __builtin_nontemporal_load(sp + (size_t)min(g0 + j, gl) * 64);
  };
  // With the RMSNorm the weights go out after the binary64 sum of squares,
  // so that its temporaries and the weights are never live together (fewer
  // registers, three workgroups per CU); loads issued after the weights
  // would wait behind them, so the norm weights come with the vector.
  if (PRO != PRO_NORM) prefetch();
  float m = 0.0f;

  // 2. Prologue: the quantised vector of this split's units into LDS.
  if (PRO == PRO_NORM) {
    // RMSNorm exactly as rmsnorm_quant_kernel: its 1024 threads' binary64
    // sums (thread t: quads t, t + 1024, ...), each wave's shuffle tree and
    // the 16 wave sums added in order; here thread tid stands for threads
    // tid + NT * j, j < VPT (quad tid + NT r belongs to thread
    // tid + NT (r % VPT)).
    double ss[VPT];
#pragma unroll
    for (int j = 0; j < VPT; j++) ss[j] = 0.0;
#pragma unroll
    for (int r = 0; r < RQ; r++)
      if (tid + r * NT < n4)
        ss[r % VPT] += ((double)v[r].x * (double)v[r].x + (double)v[r].y * (double)v[r].y) +
                       ((double)v[r].z * (double)v[r].z + (double)v[r].w * (double)v[r].w);
#pragma unroll
    for (int j = 0; j < VPT; j++) {
      for (int off = 32; off > 0; off >>= 1) ss[j] += __shfl_xor(ss[j], off);
      if (lane == 0) rss[wave + W * j] = ss[j];
    }
    lds_barrier();
    double tot = 0.0;
#pragma unroll
    for (int k = 0; k < 16; k++) tot += rss[k];
    const float ms = (float)(tot / (double)(4 * n4));
    const float inv = __fdiv_rn(1.0f, sqrt_rn(__fadd_rn(ms, a.eps)));
    prefetch();
#pragma unroll
    for (int r = 0; r < RQ; r++) v[r] = mul4(scale4(v[r], inv), w[r]);
  }
  float amax;
  if (PRO == PRO_PARTS) {
    // every wave takes the max of the parts itself: no barrier
#pragma unroll
    for (int k = 0; k < kPartsPerLane; k++) m = fmaxf(m, pm[k]);
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
    amax = m;
  } else {
#pragma unroll
    for (int r = 0; r < RQ; r++) m = fmaxf(m, abs_max4(v[r]));
    amax = block_max_nt<NT>(m, rmax);
  }
  const float sc = __fdiv_rn(amax, 127.0f);
  const float qinv = sc > 0.0f ? __fdiv_rn(1.0f, sc) : 0.0f;
#pragma unroll
  for (int r = 0; r < RQ; r++) {
    const int i = qbase + tid + r * NT;
    if (i >= q0 && i < q1) quant_quad(i - q0, v[r], qinv, reinterpret_cast<int *>(xl), sl);
  }
  lds_barrier();
  stamp(a, 1);

  // 3. The GEMV over this wave's range, activations from LDS.  Two register
  //    buffers of GPB groups: the next step's loads are issued before the
  //    current step is computed, so a wave always has a step of weights in
  //    flight.  Groups are added in the same order as in the plain kernel.
  //    A step past the wave's range loads clamped indices (a repeat of its
  //    last group) and computes only its groups in range.
  float acc = 0.0f;
  i32x4 c2[GPB * UPG];
  unsigned short dh2[GPB];
  auto load_into = [&](i32x4 (&cc)[GPB * UPG], unsigned short (&dd)[GPB], int gs) {
    const int gl = max(g1 - 1, 0);
#pragma unroll
    for (int j = 0; j < GPB; j++)
#pragma unroll
      for (int vv = 0; vv < UPG; vv++)
        cc[j * UPG + vv] = __builtin_nontemporal_load(cp + (size_t)(min(gs + j, gl) * UPG + vv) * 64);
#pragma unroll
    for (int j = 0; j < GPB; j++) dd[j] = __builtin_nontemporal_load(sp + (size_t)min(gs + j, gl) * 64);
  };
  auto compute = [&](const i32x4 (&cc)[GPB * UPG], const unsigned short (&dd)[GPB], int gs) {
#pragma unroll
    for (int j = 0; j < GPB; j++) {
      if (gs + j < g1) {
        int p = 0;
#pragma unroll
        for (int vv = 0; vv < UPG; vv++) {
          const int ul = (gs + j) * UPG + vv - u0;
          p += unit_dot_v(cc[j * UPG + vv], xl[ul * 4], xl[ul * 4 + 1], xl[ul * 4 + 2], xl[ul * 4 + 3], sl[ul]);
        }
        acc = fmaf(half_bits_to_f32(dd[j]), (float)p, acc);
      }
    }
  };
  const int nsteps = (g1 - g0 + GPB - 1) / GPB;
  for (int st = 0, gs = g0; st < nsteps; st += 2, gs += 2 * GPB) {
    if (st + 1 < nsteps) {
      load_into(c2, dh2, gs + GPB);
      compute(c, dh, gs);
    } else {
      compute(c, dh, gs);
      break;
    }
    if (st + 2 < nsteps) {
      load_into(c, dh, gs + 2 * GPB);
      compute(c2, dh2, gs + GPB);
    } else {
      compute(c2, dh2, gs + GPB);
      break;
    }
  }

  // 4. Combine the waves in order (the plain kernel's combine).
  if (wave > 0) red[wave - 1][lane] = acc;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int k = 0; k < W - 1; k++) acc += red[k][lane];
  const int o = tile * 64 + lane;
  stamp(a, 2);

  if (EPI == EPI_Y) {
    if (S == 1) {
      if (o < M) a.y[mat][o] = scale_add(acc, sc, a.accum, o);
      stamp(a, 3);
      return;
    }
    // Split partial; the last arrival of this tile adds all of them in
    // split order, leaving the workspace all zero again.
    put(a.part + (size_t)split * Mp + o, acc);
    if (!arrive_last(a.cnt + tile, S)) {
      stamp(a, 3);
      return;
    }
    float s = 0.0f;
    for (int k = 0; k < S; k++) s += take(a.part + (size_t)k * Mp + o);
    if (o < M) a.y[0][o] = scale_add(s, sc, a.accum, o);
    arrive_reset(a.cnt + tile);
    stamp(a, 3);
  } else {
    // g or u of this tile, rounded as the GEMV rounds it; the second of the
    // tile's two workgroups forms t = glu(g, u) and clears the workspace.
    const float r = __fmul_rn(acc, sc);
    put(a.part + (size_t)mat * Mp + o, r);
    if (!arrive_last(a.cnt + tile, 2)) {
      stamp(a, 3);
      return;
    }
    const float other = take(a.part + (size_t)(1 - mat) * Mp + o);
    (void)take(a.part + (size_t)mat * Mp + o);
    float tm = 0.0f;
    if (o < M) {
      const float tv = glu1<EPI == EPI_GLU_SILU ? 0 : 1>(mat ? other : r, mat ? r : other);
      a.y[0][o] = tv;
      tm = fabsf(tv);
    }
    arrive_reset(a.cnt + tile);
    if (a.tmax) {
      for (int off = 32; off > 0; off >>= 1) tm = fmaxf(tm, __shfl_xor(tm, off));
      if (lane == 0) a.tmax[tile] = tm;
    }
    stamp(a, 3);
  }
}

}  // namespace

int q2x_auto_split(int64_t M, int64_t K, int group) {
  // The split costs no launch here, only a handshake per row tile, so K is
  // split whenever the row tiles cannot fill the CUs: the largest split that
  // still runs every (tile, split) workgroup in one round (one 16-wave
  // workgroup per CU), keeping at least 8 scale groups and 64 KiB of weights
  // per split.  Measured on the 5120 x 17408 g128 down projection inside the
  // decode step: S = 3 (240 workgroups, 99 KB each) 216.7-217.2 us, S = 2
  // 217.4-218.2, S = 4 (320, two rounds) 220.6-221.2, S = 1 219.9-220.6; on
  // the 4096 x 4096 g64 matrix, one per launch, HBM-cold: S = 1 (74 KB per
  // workgroup) 5.98 us, S = 2 6.85, S = 4 7.61, S = 8 11.7.
  const int64_t tiles = (M + 63) / 64;
  const int64_t ngroups = K / group;
  if (tiles >= 128) return 1;
  const int64_t tile_bytes = 64 * (K / 4 + 2 * ngroups);  // codes and scales of a row tile
  int S = 1;
  while (S < kMaxSplit && tiles * (S + 1) <= 256 && ngroups / (S + 1) >= 8 && tile_bytes / (S + 1) >= 65536) S++;
  return S;
}

hipError_t launch_q2_gemv_x(const Q2XCall &c, hipStream_t stream) {
  const int tiles = (c.M + 63) / 64;
  const bool pair = c.codes[1] != nullptr;
  XArgs a{};
  for (int n = 0; n < (pair ? 2 : 1); n++) {
    a.codes[n] = reinterpret_cast<const i32x4 *>(c.codes[n]);
    a.scales[n] = reinterpret_cast<const unsigned short *>(c.scales[n]);
    a.y[n] = c.y[n];
  }
  a.x = reinterpret_cast<const float4 *>(c.x);
  a.norm_w = reinterpret_cast<const float4 *>(c.norm_w);
  a.eps = c.eps;
  a.accum = c.accum;
  a.M = c.M;
  a.K = c.K;
  a.S = pair ? 1 : c.split;
  a.tiles = tiles;
  a.xmax = c.xmax;
  a.nxmax = c.nxmax;
  a.tmax = c.tmax;
  a.stamps = c.stamps;
  if (a.S > 1 || c.glu >= 0) {
    a.cnt = reinterpret_cast<int *>(c.ws);
    a.part = reinterpret_cast<float *>(static_cast<char *>(c.ws) + q2x_cnt_bytes(c.M));
  }
  const bool norm = c.norm_w != nullptr;
  const bool parts = c.xmax != nullptr;
  // Waves per tile as the plain kernels: 8 when one matrix's row tiles fill
  // the CUs, else 16; quads of the vector held per thread: 4 or 8 (the whole
  // vector), or 2, 4 or 8 (one split's quads, with the partial maxima).
  const int waves = tiles >= 256 ? 8 : 16;
  const int ugroup = c.group / 64;
  const int ngroups = c.K / c.group;
  const int split_quads = (ngroups + a.S - 1) / a.S * ugroup * 16;
  const int hold = parts ? split_quads : c.K / 4;
  const int per_thread = (hold + 64 * waves - 1) / (64 * waves);
  const int rq = parts && per_thread <= 2 ? 2 : per_thread <= 4 ? 4 : 8;
  const dim3 grid(tiles * (pair ? 2 : 1), a.S);
#define QXK(UPG, GPB, W, RQ, PRO, EPI) q2_gemv_x_kernel<UPG, GPB, W, RQ, PRO, EPI><<<grid, 64 * W, 0, stream>>>(a)
#define QXE(UPG, GPB, W, RQ, PRO)                                      \
  do {                                                                 \
    if (c.glu < 0) QXK(UPG, GPB, W, RQ, PRO, EPI_Y);                   \
    else if (c.glu == 0) QXK(UPG, GPB, W, RQ, PRO, EPI_GLU_SILU);      \
    else QXK(UPG, GPB, W, RQ, PRO, EPI_GLU_SIGMOID);                   \
  } while (0)
#define QXP(UPG, GPB, W, RQ)                                           \
  do {                                                                 \
    if (norm) QXE(UPG, GPB, W, RQ, PRO_NORM); else QXE(UPG, GPB, W, RQ, PRO_X); \
  } while (0)
#define QXQ(UPG, GPB, W, RQ) QXK(UPG, (UPG == 2 ? QG_X_PARTS_GPB : 2 * QG_X_PARTS_GPB), W, RQ, PRO_PARTS, EPI_Y)
#define QXR(UPG, GPB, W)                                               \
  do {                                                                 \
    if (parts) {                                                       \
      if (rq == 2) QXQ(UPG, GPB, W, 2);                                \
      else if (rq == 4) QXQ(UPG, GPB, W, 4);                           \
      else QXQ(UPG, GPB, W, 8);                                        \
    } else if (rq == 4) QXP(UPG, GPB, W, 4); else QXP(UPG, GPB, W, 8); \
  } while (0)
  if (c.group == 64) {
    if (waves == 8) QXR(1, 4, 8); else QXR(1, 4, 16);
  } else {
    if (waves == 8) QXR(2, QG_X_PAIR_GPB, 8); else QXR(2, QG_X_PAIR_GPB, 16);
  }
#undef QXK
#undef QXE
#undef QXP
#undef QXQ
#undef QXR
  return hipGetLastError();
}

}  // namespace qg
