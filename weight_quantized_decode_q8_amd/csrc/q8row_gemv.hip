// q8row_gemv.hip -- batch-1 q8_row matvec on the T64 tiled weight image.
//
// What is computed (cortiq-engine 0.5.43 gpu_wgpu.rs page, module doc and
// q8_matvec shader; cortiq-engine 0.3.7 gpu_metal.rs page, q8_matvec):
//     y[o] = rs[o] * sum_i q[o,i] * xs[i]
// with int8 q, f32 row scales rs and f32 activations xs that the caller has
// already prescaled.  Products and sums are f32; q converts exactly.
//
// gfx950 design (differs from the pages' one-workgroup-per-row kernels):
//  - one lane owns one row; a 64-row tile is one wavefront's rows, so no
//    cross-lane reduction is ever needed;
//  - T64 puts the 16-byte chunk c of all 64 rows of a tile in 1 KiB of
//    contiguous memory: every 128-bit load of a wavefront is fully coalesced;
//  - the 16 activations of chunk c are the same for all lanes, so they are
//    fetched with scalar loads into SGPRs and used directly as the f32 FMA
//    operand (no LDS, no VGPRs for xs);
//  - int8 -> f32 is one SDWA convert per byte, then one FMA: two VALU ops
//    per weight byte, far below the CU's issue rate at HBM speed;
//  - the workgroup's waves split the K chunks of one tile into contiguous
//    ranges and combine their row sums through LDS (no second launch).
// Rounding: each lane keeps 16 accumulators (one per byte position), so an
// accumulator chain has K/16/8 terms, then a 16-way tree and an 8-way sum;
// at K = 5120 the worst-case chain is about 50 roundings.
//
// Balanced form: a launch of T tiles on 256 CUs runs T / 256 full rounds and
// then a partial one, in which R = T mod 256 tiles keep R CUs busy while the
// rest idle (measured on the 248320-row lm_head: its last 40 tiles cost
// 8.6 us of 196 against 1.8 us at the full-round rate).  The balanced launch
// runs the T - R tiles of the full rounds as above and splits each of the R
// others along K into S pieces, R * S >= 256, one per workgroup at the end of
// the grid (measured: 190.6-191.8 us against 192.2-193.2 for the plain
// launch; the pieces at the start of the grid, or split 16 ways, were slower
// than the plain launch); the pieces' row sums meet in a workspace and the
// last piece of a tile to arrive adds them in piece order (arrival.h).  Only the summation
// order of those R tiles differs from the plain launch.
#include <algorithm>

#include "arrival.h"
#include "qg_internal.h"

namespace qg {
namespace {

constexpr int kWaves = 8;   // 512 threads: 8 waves split the K chunks of one tile
constexpr int kUnroll = 8;  // 128-bit loads in flight per lane

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
// Wave-uniform activation reads through the constant address space become
// scalar (SMEM) loads; xs is never written while the kernel runs.
typedef const __attribute__((address_space(4))) f32x4 uniform_f32x4;

struct Chunk {
  int w0, w1, w2, w3;
};

__device__ inline float byte_f32(int w, int b) {
  return (float)(int)(int8_t)(w >> (8 * b));
}

__device__ inline void fma_chunk(float (&acc)[16], const Chunk &c, const uniform_f32x4 *x) {
  const f32x4 x0 = x[0], x1 = x[1], x2 = x[2], x3 = x[3];
  acc[0] = fmaf(byte_f32(c.w0, 0), x0.x, acc[0]);
  acc[1] = fmaf(byte_f32(c.w0, 1), x0.y, acc[1]);
  acc[2] = fmaf(byte_f32(c.w0, 2), x0.z, acc[2]);
  acc[3] = fmaf(byte_f32(c.w0, 3), x0.w, acc[3]);
  acc[4] = fmaf(byte_f32(c.w1, 0), x1.x, acc[4]);
  acc[5] = fmaf(byte_f32(c.w1, 1), x1.y, acc[5]);
  acc[6] = fmaf(byte_f32(c.w1, 2), x1.z, acc[6]);
  acc[7] = fmaf(byte_f32(c.w1, 3), x1.w, acc[7]);
  acc[8] = fmaf(byte_f32(c.w2, 0), x2.x, acc[8]);
  acc[9] = fmaf(byte_f32(c.w2, 1), x2.y, acc[9]);
  acc[10] = fmaf(byte_f32(c.w2, 2), x2.z, acc[10]);
  acc[11] = fmaf(byte_f32(c.w2, 3), x2.w, acc[11]);
  acc[12] = fmaf(byte_f32(c.w3, 0), x3.x, acc[12]);
  acc[13] = fmaf(byte_f32(c.w3, 1), x3.y, acc[13]);
  acc[14] = fmaf(byte_f32(c.w3, 2), x3.z, acc[14]);
  acc[15] = fmaf(byte_f32(c.w3, 3), x3.w, acc[15]);
}

// Weights are streamed once per call: non-temporal loads keep them from
// evicting the activations and row scales from the caches.
__device__ inline Chunk load_chunk(const i32x4 *p) {
  i32x4 v = __builtin_nontemporal_load(p);
  return Chunk{v.x, v.y, v.z, v.w};
}

// The split tail of the balanced launch: the tiles from tiles_full on are
// cut into S pieces along K; part holds [tile - tiles_full][S][64] f32 row
// sums, cnt one arrival counter per split tile.
struct SplitTail {
  int tiles_full, S;
  float *part;
  int *cnt;
};

// grid.x = number of 64-row tiles (kSplit: the full tiles, then S pieces of
// each tile from tiles_full on); block = kWaves wavefronts.
template <bool kSplit>
__global__ __launch_bounds__(64 * kWaves) void q8row_gemv_t64_kernel(
    const i32x4 *__restrict__ qp, const float *__restrict__ rs, const float *__restrict__ xs,
    float *__restrict__ y, int M, int K, int nchunk, SplitTail st) {
  __shared__ float red[kWaves - 1][64];
  const int lane = threadIdx.x & 63;
  // The wave index is uniform across the wavefront; saying so lets every
  // address derived from it (and from the chunk counter) live in SGPRs.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  int tile = blockIdx.x;
  // This workgroup's chunks: all of the tile's, or (split tail) piece `piece`.
  int w0 = 0, w1 = nchunk, piece = 0;
  const bool split = kSplit && tile >= st.tiles_full;
  if (split) {
    const int j = tile - st.tiles_full;
    tile = st.tiles_full + j / st.S;
    piece = j % st.S;
    const int cps = (nchunk + st.S - 1) / st.S;
    w0 = min(nchunk, piece * cps);
    w1 = min(nchunk, w0 + cps);
  }

  // Contiguous chunk range of this wave.
  const int per = (w1 - w0 + kWaves - 1) / kWaves;
  const int c0 = min(w1, w0 + wave * per);
  const int c1 = min(w1, c0 + per);
  const int cfull = min(c1, K / kQ8Chunk);  // chunks lying wholly inside K

  const i32x4 *wp = qp + (size_t)tile * nchunk * 64 + lane;
  const uniform_f32x4 *xv = (const uniform_f32x4 *)xs;

  float acc[16];
#pragma unroll
  for (int j = 0; j < 16; j++) acc[j] = 0.0f;

  int c = c0;
  for (; c + kUnroll <= cfull; c += kUnroll) {
    Chunk ch[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; u++) ch[u] = load_chunk(wp + (size_t)(c + u) * 64);
#pragma unroll
    for (int u = 0; u < kUnroll; u++) fma_chunk(acc, ch[u], xv + (size_t)(c + u) * 4);
  }
  for (; c < cfull; c++) fma_chunk(acc, load_chunk(wp + (size_t)c * 64), xv + (size_t)c * 4);
  if (c < c1) {
    // The chunk that straddles K (K % 16 != 0): weights past K are zero
    // padding, activations past K must not be read.
    const Chunk ch = load_chunk(wp + (size_t)c * 64);
    const int w[4] = {ch.w0, ch.w1, ch.w2, ch.w3};
    const int rem = K - c * kQ8Chunk;
    for (int j = 0; j < rem; j++) acc[j] = fmaf(byte_f32(w[j >> 2], j & 3), xs[c * kQ8Chunk + j], acc[j]);
  }

  float s = (((acc[0] + acc[1]) + (acc[2] + acc[3])) + ((acc[4] + acc[5]) + (acc[6] + acc[7]))) +
            (((acc[8] + acc[9]) + (acc[10] + acc[11])) + ((acc[12] + acc[13]) + (acc[14] + acc[15])));

  if (wave > 0) red[wave - 1][lane] = s;
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 0; w < kWaves - 1; w++) s += red[w][lane];
  const int o = tile * 64 + lane;
  if (split) {
    const int t = tile - st.tiles_full;
    float *pp = st.part + (size_t)t * st.S * 64 + lane;
    put(pp + piece * 64, s);
    if (!arrive_last(st.cnt + t, st.S)) return;
    s = 0.0f;
    for (int k = 0; k < st.S; k++) s += take(pp + k * 64);
    arrive_reset(st.cnt + t);
  }
  if (o < M) y[o] = s * rs[o];
}

}  // namespace

hipError_t launch_q8row_gemv(const void *qpacked, const float *rs, const float *xs, float *y,
                             int M, int K, hipStream_t stream) {
  const int tiles = (M + 63) / 64;
  const int nchunk = (K + kQ8Chunk - 1) / kQ8Chunk;
  q8row_gemv_t64_kernel<false><<<tiles, 64 * kWaves, 0, stream>>>(
      reinterpret_cast<const i32x4 *>(qpacked), rs, xs, y, M, K, nchunk, SplitTail{tiles, 1, nullptr, nullptr});
  return hipGetLastError();
}

Q8TailSplit q8row_tail_split(int64_t M, int64_t K) {
  const int64_t tiles = (M + 63) / 64;
  const int64_t nchunk = (K + kQ8Chunk - 1) / kQ8Chunk;
  Q8TailSplit t{(int)tiles, 0, 1};
  const int64_t rest = tiles % kQ8Cus;
  // Below one full round the whole launch is the tail: nothing to balance
  // against (every tile already has a CU of its own).
  if (tiles < kQ8Cus || rest == 0) return t;
  int S = (int)((kQ8Cus + rest - 1) / rest);
  S = (int)std::min<int64_t>({(int64_t)S, (int64_t)kQ8MaxTailSplit, nchunk});
  if (S < 2) return t;
  t.tiles_full = (int)(tiles - rest);
  t.tiles_split = (int)rest;
  t.S = S;
  return t;
}

hipError_t launch_q8row_gemv_balanced(const void *qpacked, const float *rs, const float *xs, float *y, int M,
                                      int K, void *ws, hipStream_t stream) {
  const Q8TailSplit t = q8row_tail_split(M, K);
  if (t.tiles_split == 0) return launch_q8row_gemv(qpacked, rs, xs, y, M, K, stream);
  const int nchunk = (K + kQ8Chunk - 1) / kQ8Chunk;
  SplitTail st{t.tiles_full, t.S, nullptr, nullptr};
  st.cnt = static_cast<int *>(ws);
  st.part = reinterpret_cast<float *>(static_cast<char *>(ws) + q8_tail_cnt_bytes(t.tiles_split));
  q8row_gemv_t64_kernel<true><<<t.tiles_full + t.tiles_split * t.S, 64 * kWaves, 0, stream>>>(
      reinterpret_cast<const i32x4 *>(qpacked), rs, xs, y, M, K, nchunk, st);
  return hipGetLastError();
}

}  // namespace qg
