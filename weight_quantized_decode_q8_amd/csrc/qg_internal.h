// qg_internal.h -- private declarations shared by the library's translation
// units: launchers (one per kernel family) and the error-message helper.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qgemv.h"

namespace qg {

// Tiles of the T64 device formats: 64 rows, one row per lane of a wavefront.
constexpr int kTileRows = 64;
// q8_row chunk: 16 bytes of one row (one 128-bit load per lane).
constexpr int kQ8Chunk = 16;
// Q2 unit: 64 weights = 16 code bytes of one row.
constexpr int kQ2Unit = 64;
constexpr int kMaxSplit = 16;

inline int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

// Records a formatted message for qg_last_error() and returns `s`.
qg_status fail(qg_status s, const char *fmt, ...);

// Launchers.  Arguments are validated by the C-ABI layer before any call.
hipError_t launch_act_quant(const float *x, int rows, int K, int8_t *xq, float *act_scale,
                            int32_t *suma, hipStream_t stream);

// Fused producers: RMSNorm (x, w, eps) or a gated product (kind 0 silu(g)*u,
// kind 1 u*sigmoid(g); t optional) followed by the quantiser.
// rows >= 1 token rows of K values each ([rows][K] row-major; w shared).
hipError_t launch_rmsnorm_quant(const float *x, const float *w, int rows, int K, float eps, int8_t *xq,
                                float *act_scale, int32_t *suma, hipStream_t stream);
hipError_t launch_glu_quant(const float *g, const float *u, int rows, int K, int kind, float *t, int8_t *xq,
                            float *act_scale, int32_t *suma, hipStream_t stream);

// Column prescale act = silu(g) * u * col over rows x n values (col null: no
// column field); vec: n % 4 == 0 and every pointer 16-byte aligned.
hipError_t launch_silu_mul_pre(const float *g, const float *u, const float *col, float *act, int64_t rows, int n,
                               bool vec, hipStream_t stream);

hipError_t launch_q8row_gemv(const void *qpacked, const float *rs, const float *xs,
                             float *y, int M, int K, hipStream_t stream);
// The balanced q8_row GEMV: the tiles past the last full round over the
// kQ8Cus CUs are split along K into S pieces (tiles_split * S >= kQ8Cus,
// S <= kQ8MaxTailSplit); ws holds one arrival counter per split tile
// (q8_tail_cnt_bytes) then [tiles_split][S][64] f32, all zero between calls.
constexpr int kQ8Cus = 256;
constexpr int kQ8MaxTailSplit = 16;
struct Q8TailSplit {
  int tiles_full, tiles_split, S;
};
Q8TailSplit q8row_tail_split(int64_t M, int64_t K);
inline size_t q8_tail_cnt_bytes(int64_t tiles_split) { return (size_t)round_up(tiles_split, 64) * sizeof(int); }
hipError_t launch_q8row_gemv_balanced(const void *qpacked, const float *rs, const float *xs, float *y, int M,
                                      int K, void *ws, hipStream_t stream);

// One Q2 GEMV launch over one matrix, or two of one shape sharing the
// activation (codes[1] non-null).  y[m] receive the results; with split > 1
// the partials hold [njobs][split][round_up(M, 64)] floats.  accum (one
// matrix only) is added to the result; dots (one matrix only, test export)
// receives [M][K/64] int32.
struct Q2Call {
  const void *codes[2];
  const void *scales[2];
  float *y[2];
  int M, K, group;
  const int8_t *xq;
  const int32_t *suma;
  const float *act_scale;
  const float *accum;
  int32_t *dots;
  float *partials;
  int split;
};
hipError_t launch_q2_gemv(const Q2Call &call, hipStream_t stream);

// Q2 GEMVs that quantise their f32 input in the same launch (optionally
// after an RMSNorm, for the gate|up pair), with split-K partials reduced by
// the last workgroup of each row tile.  codes[1] non-null: the gate|up pair
// (no split), written to y[0], y[1], or with glu >= 0 (0 silu, 1 sigmoid)
// t = glu(g, u) to y[0], g and u meeting in ws.  One matrix: split S,
// accum optional.  ws: the arrival counters (q2x_cnt_bytes) then [S][Mp]
// (or [2][Mp]) f32, all zero between calls.
inline size_t q2x_cnt_bytes(int64_t M) { return (size_t)round_up((M + 63) / 64, 64) * sizeof(int); }
// Largest K: every workgroup holds the whole vector in registers, 8 quads
// per thread of its 8 (M >= 16384) or 16 waves; with the RMSNorm (the norm
// weights held too) at most 16384.
constexpr int kQ2XMaxK = 32768;
constexpr int kQ2XNormMaxK = 16384;
// Largest number of partial maxima of |x| a caller may give (8 per lane).
constexpr int kQ2XMaxParts = QG_Q2X_MAX_PARTS;
inline int64_t q2x_max_k(int64_t M) { return (M + 63) / 64 >= 256 ? 16384 : 32768; }
struct Q2XCall {
  const void *codes[2];
  const void *scales[2];
  float *y[2];
  int M, K, group;
  const float *x, *norm_w;
  float eps;
  const float *accum;
  void *ws;
  int split;
  int glu;
  const float *xmax;  // one matrix: partial maxima of |x| (nxmax of them), or null
  int nxmax;
  float *tmax;        // glu: max|t| per row tile, or null
  unsigned long long *stamps;  // measurement only (the timeline probe), else null
};
hipError_t launch_q2_gemv_x(const Q2XCall &call, hipStream_t stream);
int q2x_auto_split(int64_t M, int64_t K, int group);

// Several independent Q2 GEMVs of one group size in one launch (no split).
constexpr int kMaxQ2Jobs = QG_Q2_BATCH_MAX;
struct Q2BatchCall {
  const void *codes, *scales;
  const int8_t *xq;
  const int32_t *suma;
  const float *act_scale, *accum;
  float *y;
  int M, K;
};
hipError_t launch_q2_batch(const Q2BatchCall *jobs, int njobs, int group, hipStream_t stream);

int q2_auto_split(int64_t M, int64_t K, int group);

// The static device scratch of the entry point that allocates nothing
// (static_scratch.hip): kStaticScratchBytes per device, 256-byte aligned.
// static_scratch() returns its device address on the current device (looked
// up once per device; no allocation).
constexpr size_t kStaticScratchBytes = QG_STATIC_SCRATCH_BYTES;
hipError_t static_scratch(void **ptr);

// Gate|up Q2 GEMV (call.codes[0], [1]; no split) with t = glu(g, u) (kind 0
// silu, 1 sigmoid) in its epilogue, each tile's max|t| in suma_out[tile],
// then the quantiser's second step over t into xq_out, act_scale_out and
// suma_out.  M % 64 == 0.
hipError_t launch_q2_gate_up_glu(const Q2Call &call, int kind, float *t, int8_t *xq_out, float *act_scale_out,
                                 int32_t *suma_out, hipStream_t stream);
// The quantiser's second step: rows of t [rows][K] whose max|t| is spread
// over nparts partial maxima (float bits) at the start of each row's suma.
hipError_t launch_quant_from_parts(const float *t, int rows, int K, int nparts, int8_t *xq, float *act_scale,
                                   int32_t *suma, hipStream_t stream);

// Batched Q2 product over nb token rows (int8 MFMA), y [nb][M] token-major.
// part: [S][nb][M] f32 partials when q2_gemm_split(...) = S > 1, else unused.
int q2_gemm_split(int64_t M, int64_t K, int group, int64_t nb);
// codes1 non-null: a pair launch, the second matrix (same M, K, group) into
// y1 with its partials after the first's ([2][S][nb][M]); accum then null.
hipError_t launch_q2_gemm(const void *codes, const void *scales, int M, int K, int group, const int8_t *xq,
                          const float *act_scale, const float *accum, float *y, int nb,
                          float *part, hipStream_t stream, const void *codes1 = nullptr,
                          const void *scales1 = nullptr, float *y1 = nullptr);

// Batched q8_row GEMM: largest K (a multiple of 4) whose int32 limb sums
// cannot overflow, |sum_i q_i * limb_i| <= 128 * 128 * K < 2^31.
constexpr int kGemmMaxK = 131068;

// Batched q8_row GEMM: workspace layout (limbs, exponents, flags) and launch.
size_t gemm_ws_layout(int64_t nb, int64_t K, size_t *off_exp, size_t *off_need, size_t *off_zero);
// The activation rows of the batched q8_row product: xs itself, or (g non-
// null) act = silu(g) * u * col formed in the prep kernel (col null: none).
struct GemmAct {
  const float *xs;
  const float *g, *u, *col;
};
hipError_t launch_q8row_gemm(const void *w, const float *rs, const GemmAct &act, float *y, int nb,
                             int M, int K, int limbs, void *ws, hipStream_t stream);

}  // namespace qg
