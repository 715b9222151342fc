/*
 * qgemv.h -- C-ABI of the weight-only-quantized decode library for MI355X
 * (gfx950).  Plain C: pointers, sizes and status codes; no C++ or framework
 * types.  Library: weight_quantized_decode_q8_amd/libqgemv.so.
 *
 * Conventions shared by every entry point
 *  - "device" pointers are HIP device memory on the current device; "host"
 *    pointers are ordinary CPU memory.  The caller owns every buffer.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Device entry
 *    points only enqueue work on it: they never synchronise, never allocate
 *    and never copy between host and device.
 *  - Every argument is validated before anything is launched.  A bad
 *    argument returns QG_EINVAL and enqueues nothing; qg_last_error() then
 *    names the argument.  A failed kernel launch returns QG_ELAUNCH.  There
 *    is no fallback path of any kind.
 *  - Sizes are int64_t element counts unless the name says bytes.
 *  - Entry points are re-entrant and keep no global state besides the
 *    thread-local error message and the static device scratch of
 *    qgemv_q2_noalloc.
 *
 * Sources of the operations (page and function; the pages are third-party
 * source files of LLM inference engines):
 *  [Q8]  cortiq-engine 0.5.43 gpu_wgpu.rs page: module doc, shaders
 *        q8_matvec and q8_matmat; cortiq-engine 0.3.7 gpu_metal.rs page:
 *        kernels q8_matvec / q8_matmat, host q8_matvec / q8_matvec_range /
 *        q8_matmat.
 *  [Q2]  qxmx qxmx_gpu.cpp page: dequant_embd (code and value rule),
 *        repack_q2_g64 / repack_q2_g128 (host repack, g128 = two g64 halves
 *        sharing d), upload_q2 (block footprints, padded rows).
 *  [AQ]  qxmx qxmx_gpu.cpp page: gpu_rmsnorm_quant (per-vector int8
 *        activation quantisation with per-64 group sums).
 *  [GV]  qxmx qxmx_gpu.cpp page: gemv_dpas8 (int8-activation Q2 GEMV,
 *        split-K partials, the suma correction) and gemv_reduce.
 *  [QG]  qxmx qxmx_gpu.cpp page: ffn_forward_b (the batched FFN: the
 *        token rows quantised by the batched producers, gemm_gpu_v4 /
 *        gemm_gpu_v4_dual writing token-major outputs, the residual folded
 *        into the down projection).
 *  [PQ]  qxmx qxmx_gpu.cpp page: gpu_rmsnorm_quant, gpu_swiglu_quant,
 *        gpu_silu_mul_quant, gpu_sigmoid_mul_quant (the activation-side
 *        producers that form and quantise the next GEMV's input in one
 *        kernel).
 *  [LB]  cortiq-engine 0.5.43 gpu_wgpu.rs page: matvec_pair (two jobs laid
 *        end to end in one row space of one dispatch); cortiq-engine 0.3.7
 *        gpu_metal.rs page: matvec_batch (several independent matvecs in one
 *        command buffer).
 *  [GD]  qxmx qxmx_gpu.cpp page: gemv_dpas8_dual (the FFN gate and up
 *        matrices against one shared quantized activation, bit-exact to two
 *        separate GEMVs) and tmatvec_accum (the residual add folded into the
 *        GEMV epilogue, bit-exact to the GEMV followed by the add).
 *  [SP]  cortiq-engine 0.5.43 gpu_wgpu.rs page: silu_mul_pre (the MoE
 *        block's element-wise pass forming the down projection's input
 *        silu(g) * u, times the q8_2f column field when the tensor has one);
 *        cortiq-engine 0.3.7 gpu_metal.rs page: silu_mul_pre (has_col) and
 *        q8_mul_mm_silu (the batched down product with silu(g) * u formed in
 *        its activation load).
 *  [GU]  cortiq-engine 0.5.43 gpu_wgpu.rs page: moe_gate_up (one workgroup
 *        computes both the gate and the up row dot of a row and writes
 *        act = silu(g) * u).
 */
#ifndef QGEMV_H
#define QGEMV_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum qg_status {
    QG_OK = 0,
    QG_EINVAL = 1,   /* bad argument; nothing was enqueued */
    QG_ELAUNCH = 2,  /* a kernel launch failed */
} qg_status;

/* Human-readable name of a status. */
const char *qg_status_string(qg_status s);

/* Message describing the last non-OK status returned on this thread. */
const char *qg_last_error(void);

/* Version of this ABI (bumped on any incompatible change). */
int qg_abi_version(void);

/* ======================================================================
 * q8_row weights  [Q8]
 *
 * Source format (the pages' q8_row): int8 q[M][K] row-major, K % 4 == 0,
 * plus one f32 row scale rs[M] kept separately.
 *
 * Device format "T64" (this library): rows in tiles of 64, K in chunks of
 * 16 bytes; byte (o, i) lives at
 *     ((o/64) * (Kp/16) + i/16) * 1024 + (o%64) * 16 + i%16
 * with Mp = M rounded up to 64 and Kp = K rounded up to 16; padding bytes
 * are zero.  A wavefront load of one chunk of a tile is 1 KiB contiguous.
 * ==================================================================== */

/* Bytes of the T64 image of an M x K q8_row matrix (0 if M<1, K<4 or K%4). */
size_t qg_q8row_packed_bytes(int64_t M, int64_t K);

/* Host: repack row-major q[M][K] (host) into the T64 image dst (host,
 * dst_bytes >= qg_q8row_packed_bytes).  The caller uploads dst.
 * QG_EINVAL: null pointer, M < 1, K < 4, K % 4 != 0, dst too small.      */
qg_status qg_repack_q8row(const int8_t *q, int64_t M, int64_t K,
                          void *dst, size_t dst_bytes);

/* Host: inverse of qg_repack_q8row (for tests and export).              */
qg_status qg_unpack_q8row(const void *packed, size_t packed_bytes,
                          int64_t M, int64_t K, int8_t *q);

/* Device: y[o] = rs[o] * sum_i q[o,i] * xs[i]   [Q8, q8_matvec]
 *   qpacked: device, T64 image of q (qg_q8row_packed_bytes(M, K) bytes)
 *   rs:      device, f32[M];  xs: device, f32[K] (already prescaled by the
 *            caller, as on the pages);  y: device, f32[M], written.
 * Accumulation in f32 (no activation quantisation).  A row range of a
 * larger matrix is a call on a pointer offset by whole 64-row tiles.
 * QG_EINVAL: null pointer, M < 1, K < 4, K % 4 != 0.                     */
qg_status qgemv_q8row(const void *qpacked, const float *rs, const float *xs,
                      float *y, int64_t M, int64_t K, void *stream);

/* Bytes of workspace qgemv_q8row_balanced needs for this shape (0 when M
 * gives whole rounds of row tiles over the 256 CUs, or less than one).    */
size_t qgemv_q8row_balanced_ws_bytes(int64_t M, int64_t K);

/* Device: the same GEMV as qgemv_q8row, with its last partial round of row
 * tiles spread over the whole GPU   [Q8]
 *   A launch of T = ceil(M/64) tiles runs T / 256 full rounds on the 256
 *   CUs and then R = T mod 256 tiles on R CUs while the others idle (on
 *   the 248320-row lm_head, 40 tiles costing 8.6 us).  Here each of those
 *   R tiles is split along K into S pieces (R * S >= 256, S <= 16), one
 *   workgroup each at the end of the grid, and the last piece of a tile to
 *   finish adds the pieces' row sums in piece order.
 *   ws:        device, >= qgemv_q8row_balanced_ws_bytes(M, K) bytes,
 *              16-byte aligned (may be NULL when that is 0), all zero before
 *              the first call that uses it (allocate it zero-filled); every
 *              call leaves it all zero again.  Calls sharing one ws must not
 *              overlap in time.
 *   Other arguments as qgemv_q8row.  The outputs of the full rounds' tiles
 *   equal qgemv_q8row's bit for bit; those of the R split tiles differ only
 *   in the f32 summation order (the same bound holds).
 * QG_EINVAL: as qgemv_q8row, or a short, misaligned or overlapping
 * workspace.                                                              */
qg_status qgemv_q8row_balanced(const void *qpacked, const float *rs,
                               const float *xs, float *y, int64_t M,
                               int64_t K, void *ws, size_t ws_bytes,
                               void *stream);

/* ======================================================================
 * Q2 weights  [Q2]
 *
 * Source format (GGUF-style, as the pages read it): per row, K/group blocks
 * of (2 + group/4) bytes -- an IEEE binary16 scale d (little-endian), then
 * group/4 code bytes; code k of a block is (qs[k/4] >> 2*(k%4)) & 3 and the
 * weight is d * (code - 1).  group is 64 (18-byte blocks) or 128 (34-byte
 * blocks); a 128 block is two 64-wide units sharing d.
 *
 * Device format "T64" (this library), two planes:
 *  codes:  [Mp/64 tiles][K/64 units][64 rows][16 bytes]; inside the 16
 *          bytes of (row, unit), 32-bit word j covers weights 16j..16j+15
 *          and weight 16j + 4a + b sits at bits 8b + 2a of that word, so
 *          (word >> 2a) & 0x03030303 yields the codes of weights
 *          16j+4a .. 16j+4a+3 as four bytes.
 *  scales: [Mp/64 tiles][K/group][64 rows] binary16, one per group (not
 *          duplicated for 128-wide groups).
 * Padding rows (M..Mp) have zero codes and zero scales.
 * ==================================================================== */

typedef struct qg_q2_weight {
    const void *codes;    /* device, qg_q2_codes_bytes(M, K) bytes        */
    const void *scales;   /* device, qg_q2_scales_bytes(M, K, group) bytes */
    int64_t M;            /* rows (outputs)                               */
    int64_t K;            /* columns (inputs), K % group == 0             */
    int32_t group;        /* 64 or 128                                    */
    int32_t reserved;     /* must be 0                                    */
} qg_q2_weight;

/* Size of the GGUF-style block blob: M * (K/group) * (2 + group/4). */
size_t qg_q2_blocks_bytes(int64_t M, int64_t K, int group);
/* Sizes of the two device planes (0 on bad shape). */
size_t qg_q2_codes_bytes(int64_t M, int64_t K);
size_t qg_q2_scales_bytes(int64_t M, int64_t K, int group);

/* Host: repack a GGUF-style block blob (host, src_bytes must equal
 * qg_q2_blocks_bytes) into the two T64 planes (host).  The scales are
 * copied bit for bit.  QG_EINVAL: null pointer, M < 1, group not 64/128,
 * K % group != 0, wrong src_bytes, destination too small.                */
qg_status qg_repack_q2(const void *blocks, size_t src_bytes,
                       int64_t M, int64_t K, int group,
                       void *codes, size_t codes_bytes,
                       void *scales, size_t scales_bytes);

/* Host: inverse of qg_repack_q2 (for tests and export). */
qg_status qg_unpack_q2(const void *codes, size_t codes_bytes,
                       const void *scales, size_t scales_bytes,
                       int64_t M, int64_t K, int group,
                       void *blocks, size_t blocks_bytes);

/* Device: per-vector int8 activation quantisation   [AQ]
 *   x:         device, f32[K], finite.
 *   xq:        device, int8[K], written: clamp(round(x * inv), -128, 127),
 *              round half away from zero, inv = 1/act_scale (0 if
 *              act_scale is 0), all in IEEE binary32.
 *   act_scale: device, f32[1], written: max|x| / 127.
 *   suma:      device, int32[K/64], written: sum of xq over each 64-wide
 *              group (the correction term of the Q2 GEMV).
 * QG_EINVAL: null pointer, K < 64, K % 64 != 0, K > 1 << 24.             */
qg_status qquant_act_i8(const float *x, int64_t K, int8_t *xq,
                        float *act_scale, int32_t *suma, void *stream);

/* Device: qquant_act_i8 on each row of a [nb][K] batch (the prefill form,
 * one act_scale per token row)   [AQ, gpu_rmsnorm_quant with n_tok]
 *   x:         device, f32[nb][K] row-major, 16-byte aligned, finite.
 *   xq:        device, int8[nb][K]; act_scale: f32[nb]; suma: int32[nb][K/64].
 *   Row b of each output is exactly what qquant_act_i8 writes for row b.
 * QG_EINVAL: as qquant_act_i8, or nb < 1.                                 */
qg_status qquant_act_i8_rows(const float *x, int64_t nb, int64_t K,
                             int8_t *xq, float *act_scale, int32_t *suma,
                             void *stream);

/* Device: RMSNorm, then the quantiser of qquant_act_i8, in one launch
 *   [PQ, gpu_rmsnorm_quant]
 *   x, w:      device, f32[K] each (the vector and the norm weights),
 *              16-byte aligned, finite.
 *   eps:       the norm's epsilon, finite and >= 0 (with eps = 0 an all-zero
 *              x has no defined result).
 *   Quantised vector v_i = (x_i * inv) * w_i with inv = 1 / sqrt(ms + eps),
 *   ms = binary32(sum_i x_i^2 / K) (the squares summed in binary64), every
 *   other step one correctly rounded binary32 operation; xq, act_scale and
 *   suma are then exactly what qquant_act_i8 writes for v.
 * QG_EINVAL: null pointer, K < 64, K % 64 != 0, K > 1 << 24, misaligned
 * input, eps negative or not finite.                                       */
qg_status qquant_rmsnorm_i8(const float *x, const float *w, int64_t K,
                            float eps, int8_t *xq, float *act_scale,
                            int32_t *suma, void *stream);

/* Device: qquant_rmsnorm_i8 on each row of a [nb][K] batch (the prefill
 * form, gpu_rmsnorm_quant with n_tok): x f32[nb][K]; w f32[K], shared by
 * all rows; xq int8[nb][K], act_scale f32[nb], suma int32[nb][K/64].  Row b
 * of each output is exactly what qquant_rmsnorm_i8 writes for row b.
 * QG_EINVAL: as qquant_rmsnorm_i8, or nb < 1.                              */
qg_status qquant_rmsnorm_i8_rows(const float *x, const float *w, int64_t nb,
                                 int64_t K, float eps, int8_t *xq,
                                 float *act_scale, int32_t *suma,
                                 void *stream);

/* Gate functions of qquant_glu_i8. */
enum { QG_GLU_SILU = 0, QG_GLU_SIGMOID = 1 };

/* Device: gated product, then the quantiser of qquant_act_i8 (two
 * launches: the product over the whole GPU, then the quantiser)
 *   [PQ, gpu_swiglu_quant / gpu_silu_mul_quant (SILU),
 *    gpu_sigmoid_mul_quant (SIGMOID)]
 *   g, u:      device, f32[K] each (gate and value), 16-byte aligned.
 *   kind:      QG_GLU_SILU:    t_i = (g_i / (1 + exp(-g_i))) * u_i
 *              QG_GLU_SIGMOID: t_i = u_i * (1 / (1 + exp(-g_i)))
 *              every step one binary32 operation; exp is the correctly
 *              rounded binary32 exponential.
 *   t:         device, f32[K] receiving the product, 16-byte aligned; may
 *              be g or u itself (in place), otherwise must not overlap them.
 *   xq, act_scale, suma: exactly what qquant_act_i8 writes for t (suma
 *              also serves as scratch between the two launches).
 *   The outputs must not overlap g, u or t.
 * QG_EINVAL: as qquant_rmsnorm_i8, or a bad kind, null t, or t partly
 * overlapping g or u.                                                      */
qg_status qquant_glu_i8(const float *g, const float *u, int64_t K, int kind,
                        float *t, int8_t *xq, float *act_scale,
                        int32_t *suma, void *stream);

/* Device: qquant_glu_i8 on each row of a [nb][K] batch (the prefill form,
 * gpu_swiglu_quant / gpu_silu_mul_quant / gpu_sigmoid_mul_quant with
 * n_tok): g, u, t f32[nb][K]; xq int8[nb][K], act_scale f32[nb], suma
 * int32[nb][K/64].  Row b of each output is exactly what qquant_glu_i8
 * writes for row b.  QG_EINVAL: as qquant_glu_i8, or nb < 1.              */
qg_status qquant_glu_i8_rows(const float *g, const float *u, int64_t nb,
                             int64_t K, int kind, float *t, int8_t *xq,
                             float *act_scale, int32_t *suma, void *stream);

/* Bytes of split-K workspace qgemv_q2 needs for this shape and split
 * (split_k 0 = the library's choice).                                    */
size_t qgemv_q2_ws_bytes(int64_t M, int64_t K, int group, int split_k);

/* Split factor qgemv_q2 uses for split_k = 0 (auto) on this shape.       */
int qgemv_q2_auto_split(int64_t M, int64_t K, int group);

/* Device: y[o] = act_scale * sum_u d(o,u) * sum_{i in unit u} (code-1)*xq_i
 *   [GV, gemv_dpas8 + gemv_reduce]
 *   w:         host struct describing the device planes.
 *   xq, suma, act_scale: device, as written by qquant_act_i8 (K entries,
 *              K/64 entries, 1 entry).
 *   y:         device, f32[M], written.
 *   ws:        device workspace of >= qgemv_q2_ws_bytes(M, K, group,
 *              split_k) bytes (may be NULL when that is 0); holds the f32
 *              split-K partials [split][Mp]; contents on entry are ignored.
 *   split_k:   0 = auto, else 1..16 contiguous ranges of 64-wide units.
 * The int32 unit dots are exact; y is accumulated in f32 from d * dot.
 * QG_EINVAL: null pointer, bad weight struct, split_k out of range,
 * workspace too small or overlapping y (or a residual).                   */
qg_status qgemv_q2(const qg_q2_weight *w, const int8_t *xq,
                   const int32_t *suma, const float *act_scale, float *y,
                   void *ws, size_t ws_bytes, int split_k, void *stream);

/* Device: qgemv_q2 with no workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc).  The split-K partials go to a
 * static device array of QG_STATIC_SCRATCH_BYTES that the library holds on
 * each GPU it runs on until the process ends (looked up on the first call on
 * a device; nothing is allocated, on that call or any other).
 *   Arguments as qgemv_q2; the current device must be the stream's.
 *   y equals qgemv_q2 with the same split_k bit for bit.
 * Every call on one GPU shares that GPU's scratch, and it keeps the last
 * call's partials: calls that overlap in time on one GPU (other streams,
 * other threads) race and give wrong results; calls in order on one stream
 * are safe.  Nothing in it must start at zero.
 * QG_EINVAL: as qgemv_q2, or the split's partials (split * round_up(M, 64)
 * floats, qgemv_q2_ws_bytes) exceed QG_STATIC_SCRATCH_BYTES.
 * QG_ELAUNCH: the scratch's device address cannot be found, or a launch
 * fails.                                                                  */
#define QG_STATIC_SCRATCH_BYTES (1u << 20)
qg_status qgemv_q2_noalloc(const qg_q2_weight *w, const int8_t *xq,
                           const int32_t *suma, const float *act_scale,
                           float *y, int split_k, void *stream);

/* Test entry: qgemv_q2 that also writes the exact int32 unit dots
 *   dots[o][u] = sum_{i in unit u} (code - 1) * xq_i   (device,
 *   int32[M][K/64]) from the same kernel, to prove them bit-exact.        */
qg_status qgemv_q2_dots(const qg_q2_weight *w, const int8_t *xq,
                        const int32_t *suma, const float *act_scale,
                        float *y, int32_t *dots, void *ws, size_t ws_bytes,
                        int split_k, void *stream);

/* Device: qgemv_q2 with a residual added in the epilogue   [GD]
 *   y[o] = fl(fl(act_scale * acc[o]) + accum[o])
 * two binary32 roundings in that order (never one fused multiply-add), so
 * y equals qgemv_q2 with the same split_k followed by a separate f32 add of
 * accum, bit for bit.
 *   accum:     device, f32[M]; may be y itself (in-place residual update),
 *              otherwise must not overlap y.
 * Other arguments, workspace and errors as qgemv_q2; QG_EINVAL also for a
 * null or partly overlapping accum.                                       */
qg_status qgemv_q2_accum(const qg_q2_weight *w, const int8_t *xq,
                         const int32_t *suma, const float *act_scale,
                         const float *accum, float *y, void *ws,
                         size_t ws_bytes, int split_k, void *stream);

/* Bytes of workspace qgemv_q2_dual needs: twice qgemv_q2_ws_bytes.       */
size_t qgemv_q2_dual_ws_bytes(int64_t M, int64_t K, int group, int split_k);

/* Device: two Q2 GEMVs of one shape against one quantized activation, in
 * one launch (plus one reduce launch when split)   [GD]
 *   w0, w1:    host structs of two weights with equal M, K and group (the
 *              FFN gate and up projections).
 *   y0, y1:    device, f32[M] each, written; must not overlap.
 *   ws:        >= qgemv_q2_dual_ws_bytes(M, K, group, split_k) bytes.
 * y0 and y1 equal qgemv_q2 on w0 and on w1 with the same split_k (auto
 * picks the split qgemv_q2 picks for one matrix), bit for bit.
 * QG_EINVAL: as qgemv_q2, or the weights differ in shape, or the outputs
 * overlap.                                                                */
qg_status qgemv_q2_dual(const qg_q2_weight *w0, const qg_q2_weight *w1,
                        const int8_t *xq, const int32_t *suma,
                        const float *act_scale, float *y0, float *y1,
                        void *ws, size_t ws_bytes, int split_k, void *stream);

/* Gate|up GEMV with the gated product and its quantiser  [GD, GU, PQ]
 *
 *   g = qgemv_q2(w_gate, xq),  u = qgemv_q2(w_up, xq)          (one launch)
 *   t = silu(g) * u (kind QG_GLU_SILU) or u * sigmoid(g) (QG_GLU_SIGMOID)
 *   xq_out, act_scale_out, suma_out = the int8 quantiser of t
 *
 * The FFN's gate and up projections and the next projection's input in two
 * launches instead of three: each workgroup computes the gate and the up dot
 * of the same 64 rows (as the page's moe_gate_up does per row) and forms t
 * in its epilogue; a second launch quantises t.  t, xq_out, act_scale_out
 * and suma_out are bit-identical to qgemv_q2_dual with split_k = 1 followed
 * by qquant_glu_i8 on its two outputs (g and u are not written).
 * Arguments: w_gate, w_up: same M, K and group, M % 64 == 0; xq, suma,
 * act_scale: the quantised input as for qgemv_q2; t: device f32[M] (16-byte
 * aligned), written; xq_out int8[M], act_scale_out f32[1], suma_out
 * int32[M/64]: device, written.  No workspace (suma_out holds the per-tile
 * maxima between the two launches).
 * QG_EINVAL: as qgemv_q2_dual, or a bad kind, M % 64 != 0, misalignment,
 * or outputs overlapping each other or the inputs.                        */
qg_status qgemv_q2_gate_up_glu(const qg_q2_weight *w_gate,
                               const qg_q2_weight *w_up, const int8_t *xq,
                               const int32_t *suma, const float *act_scale,
                               int kind, float *t, int8_t *xq_out,
                               float *act_scale_out, int32_t *suma_out,
                               void *stream);

/* One GEMV of a qgemv_q2_batch launch. */
typedef struct {
    qg_q2_weight w;          /* the matrix (host struct of device planes)  */
    const int8_t *xq;        /* device, int8[w.K]: its quantised input     */
    const int32_t *suma;     /* device, int32[w.K/64]                      */
    const float *act_scale;  /* device, f32[1]                             */
    const float *accum;      /* device, f32[w.M] residual, or NULL; may be
                                y itself                                   */
    float *y;                /* device, f32[w.M], written                  */
} qg_q2_job;

/* Most GEMVs one qgemv_q2_batch call takes. */
#define QG_Q2_BATCH_MAX 16

/* Device: up to QG_Q2_BATCH_MAX independent Q2 GEMVs in one launch (each
 * launch has a fixed cost of a few microseconds, as much as streaming tens
 * of MB, so small GEMVs of one decode step -- several projections, or the
 * experts of a layer -- are better issued together)   [LB, GV, GD]
 *   jobs:      host array of njobs descriptors; each job may have its own
 *              shape and activation (all with the same group size) and an
 *              optional residual, added as in qgemv_q2_accum.
 * No K split and no workspace.  Each y equals qgemv_q2 (or qgemv_q2_accum)
 * of that job with split_k = 1 bit for bit when the job's row tiles
 * (ceil(M/64)) and the launch's total row tiles are on the same side of
 * 256 (the rule that picks 8 or 16 waves per tile); otherwise only the f32
 * summation order differs, within the same bound.
 * QG_EINVAL: null table, njobs outside 1..QG_Q2_BATCH_MAX, a bad weight
 * struct, mixed group sizes, a null or misaligned pointer, a residual
 * partly overlapping its y, or an output overlapping another job's output
 * or residual.                                                             */
qg_status qgemv_q2_batch(const qg_q2_job *jobs, int njobs, void *stream);

/* ---- The decode GEMVs with the activation quantiser in the same launch --
 *
 * Each workgroup of these launches quantises the f32 input vector itself by
 * the rule of qquant_act_i8 (after the RMSNorm of qquant_rmsnorm_i8 when
 * norm_w is given) and keeps the int8 vector in LDS, so the quantiser is not
 * a launch of its own; a K split is added up by the last workgroup of each
 * row tile, so it needs no reduce launch either.  Every output equals the
 * multi-launch chain it replaces bit for bit.  What a launch saves is its
 * fixed cost of a few microseconds, which at decode sizes is as much as
 * streaming 10-20 MB of weights.
 *   [AQ, PQ gpu_rmsnorm_quant; GV gemv_dpas8 + gemv_reduce; GD
 *    gemv_dpas8_dual, tmatvec_accum; GU moe_gate_up]
 * The vector is read by every workgroup while outputs are written, so it
 * must not overlap any output.  Each workgroup holds the whole vector: K
 * is at most 32768, or 16384 when M >= 16384 (256 row tiles or more, the
 * shapes run with 8 waves per tile) or with the RMSNorm.                  */

/* Split factor qgemv_q2_x uses for split_k = 0 (auto) on this shape: 1
 * when the row tiles fill the GPU (M >= 8192), else the largest split whose
 * workgroups still all run at once on the 256 CUs (the split costs no
 * launch here) while each keeps at least 8 scale groups and 64 KiB of
 * weights (5120 x 17408 g128: 3; 4096 x 4096 g64: 1).                     */
int qgemv_q2_x_auto_split(int64_t M, int64_t K, int group);

/* Bytes of workspace qgemv_q2_x needs for this shape and split (split_k 0 =
 * qgemv_q2_x_auto_split): 0 without a split, else the arrival counters
 * then the f32 partials.                                                  */
size_t qgemv_q2_x_ws_bytes(int64_t M, int64_t K, int group, int split_k);

/* Device: y = qgemv_q2(w, quantised x) (+ accum), one launch
 *   x:         device, f32[K], 16-byte aligned, finite; must not overlap y,
 *              accum or ws.
 *   xmax, nxmax: NULL and 0, or device f32[nxmax] (1 <= nxmax <=
 *              QG_Q2X_MAX_PARTS, 4-byte aligned) whose largest entry is
 *              max_i |x_i|, for instance the tmax that
 *              qgemv_q2_gate_up_glu_x wrote along with x = t.  Then each
 *              workgroup reads only its own split's part of x instead of
 *              the whole vector to find the scale.  act_scale is always
 *              max/127 of the max used, so given a wrong max the result
 *              is that of the quantiser with that scale (codes clamped to
 *              [-128, 127]), never an out-of-bounds access.
 *   accum:     device, f32[M] residual added as in qgemv_q2_accum, or NULL;
 *              may be y itself.
 *   y:         device, f32[M], written.
 *   ws:        device, >= qgemv_q2_x_ws_bytes(M, K, group, split_k) bytes,
 *              16-byte aligned (may be NULL when that is 0).  It must be
 *              all zero before the first call that uses it (allocate it
 *              zero-filled, or clear it once); every call leaves it all
 *              zero again, so one workspace serves calls of any shape and
 *              split.  Calls sharing one ws must not overlap in time.
 *   split_k:   0 = auto (qgemv_q2_x_auto_split), else 1..16.
 * y equals qquant_act_i8(x) followed by qgemv_q2 (or qgemv_q2_accum) with
 * the same split (given explicitly to both), bit for bit.
 * QG_EINVAL: as qgemv_q2_accum, or null or misaligned x, K above the
 * limit above, x overlapping y, or a workspace overlapping x.             */
#define QG_Q2X_MAX_PARTS 512
qg_status qgemv_q2_x(const qg_q2_weight *w, const float *x,
                     const float *xmax, int64_t nxmax,
                     const float *accum, float *y, void *ws, size_t ws_bytes,
                     int split_k, void *stream);

/* Device: the gate|up pair against one vector quantised in the launch
 *   x:         device, f32[K], 16-byte aligned.
 *   norm_w:    device, f32[K] RMSNorm weights (16-byte aligned), or NULL:
 *              with it the quantised vector is the RMSNorm of
 *              qquant_rmsnorm_i8 (x, norm_w, eps), K <= 16384.
 *   y0, y1:    device, f32[M] each, written; must not overlap each other,
 *              x or norm_w.
 * y0, y1 equal qquant_act_i8 (or qquant_rmsnorm_i8) followed by
 * qgemv_q2_dual with split_k = 1, bit for bit.  No workspace, no split.
 * QG_EINVAL: as qgemv_q2_dual, or as qgemv_q2_x for x, or eps negative
 * or not finite when norm_w is given.                                     */
qg_status qgemv_q2_dual_x(const qg_q2_weight *w0, const qg_q2_weight *w1,
                          const float *x, const float *norm_w, float eps,
                          float *y0, float *y1, void *stream);

/* Bytes of workspace qgemv_q2_gate_up_glu_x needs for M rows: the
 * arrival counters, then g and u of each row tile.                        */
size_t qgemv_q2_gate_up_glu_x_ws_bytes(int64_t M);

/* Device: the gate|up pair with the gated product in its epilogue, against
 * a vector quantised (optionally RMSNorm-ed) in the same launch
 *   t = silu(g) * u (kind QG_GLU_SILU) or u * sigmoid(g) (QG_GLU_SIGMOID)
 *   with g, u the qgemv_q2_dual_x outputs, which meet in ws: the second of
 *   the two workgroups of a row tile (gate, up) to finish forms t.
 *   t:         device, f32[M], written; must not overlap x or norm_w.
 *   tmax:      device, f32[ceil(M/64)] (4-byte aligned), or NULL: receives
 *              max |t| over each 64-row tile, so that max_o |t_o| is the
 *              largest entry (pass it to qgemv_q2_x as xmax); must not
 *              overlap t, x, norm_w or ws.
 *   ws:        device, >= qgemv_q2_gate_up_glu_x_ws_bytes(M) bytes, 16-byte
 *              aligned, all zero before the first call (allocate it
 *              zero-filled); every call leaves it all zero again.  Calls
 *              sharing one ws must not overlap in time.
 * t equals qgemv_q2_dual_x followed by the gated product of
 * qquant_glu_i8, bit for bit; feed it to qgemv_q2_x (the down projection,
 * with the residual as accum) to finish the FFN block in two launches.
 * Any M >= 1.  QG_EINVAL: as qgemv_q2_dual_x, or a bad kind, or a short,
 * misaligned or overlapping workspace.                                    */
qg_status qgemv_q2_gate_up_glu_x(const qg_q2_weight *w_gate,
                                 const qg_q2_weight *w_up, const float *x,
                                 const float *norm_w, float eps, int kind,
                                 float *t, float *tmax, void *ws,
                                 size_t ws_bytes, void *stream);

/* Device: the batched (prefill) Q2 product over nb token rows, on int8
 * MFMA   [QG, ffn_forward_b with gemm_gpu_v4]
 *   y[b, o] = act_scale[b] * sum_g d(o, g) * sum_{i in g} (code - 1) * xq[b, i]
 *             (+ accum[b, o])
 *   w:         host struct of the device planes (scales 8-byte aligned).
 *   xq, act_scale: device, as written by qquant_act_i8_rows: int8[nb][K]
 *              (16-byte aligned), f32[nb].
 *   suma:      the row quantiser's group sums (int32[nb][K/64]) in the
 *              GEMV's calling convention; not read (the product multiplies
 *              code - 1 directly), may be NULL.
 *   accum:     device, f32[nb][M] residual, or NULL; may be y itself,
 *              otherwise must not overlap it.
 *   y:         device, f32[nb][M] (token-major), 16-byte aligned, written.
 *   ws:        device workspace of >= qgemm_q2_batched_ws_bytes(M, K,
 *              group, nb) bytes, 16-byte aligned (may be NULL when that is
 *              0): f32 partial sums [S][nb][M] of a K split, used when the
 *              row and token tiles alone cannot fill the GPU; contents on
 *              entry are ignored.
 * The per-group int32 dots are exact; each output accumulates d * dot over
 * the groups in f32 (split partials added in fixed order), then act_scale[b]
 * and the residual are applied with one binary32 rounding each.
 * QG_EINVAL: null pointer, bad weight struct, nb < 1, misaligned pointer,
 * accum partly overlapping y, workspace too small or overlapping y/accum. */
qg_status qgemm_q2_batched(const qg_q2_weight *w, const int8_t *xq,
                           const int32_t *suma, const float *act_scale,
                           const float *accum, float *y, int64_t nb,
                           void *ws, size_t ws_bytes, void *stream);

/* Bytes of workspace qgemm_q2_batched needs for this shape (0: none). */
size_t qgemm_q2_batched_ws_bytes(int64_t M, int64_t K, int group, int64_t nb);

/* Gate|up pair of the batched Q2 product  [QG, gemm_gpu_v4_dual]
 *
 *   y0[b, o] = act_scale[b] * sum_g d0(o, g) * sum_{i in g} (code0(o, i) - 1) * xq[b, i]
 *   y1[b, o] = the same with the second matrix
 *
 * One launch over two matrices of the same M, K and group against the same
 * token rows (the FFN's gate and up projections).  Each output is computed
 * exactly as qgemm_q2_batched computes it (same tiles, same K split), so
 * y0 and y1 are bit-identical to two qgemm_q2_batched calls without a
 * residual.
 * Arguments as qgemm_q2_batched, with w0, w1 the two matrices and y0, y1:
 * device f32[nb][M] each (16-byte aligned, not overlapping); ws holds
 * qgemm_q2_batched_dual_ws_bytes(M, K, group, nb) bytes (0: none needed).
 * QG_EINVAL: as qgemm_q2_batched, or the matrices differ in M, K or group,
 * or the outputs overlap (each other or the workspace).                   */
qg_status qgemm_q2_batched_dual(const qg_q2_weight *w0, const qg_q2_weight *w1,
                                const int8_t *xq, const int32_t *suma,
                                const float *act_scale, float *y0, float *y1,
                                int64_t nb, void *ws, size_t ws_bytes,
                                void *stream);

/* Bytes of workspace qgemm_q2_batched_dual needs (twice the one-matrix need). */
size_t qgemm_q2_batched_dual_ws_bytes(int64_t M, int64_t K, int group, int64_t nb);

/* ======================================================================
 * Batched prefill q8_row GEMM  [Q8, q8_matmat / q8_mul_mm]
 *
 *   y[b, o] = rs[o] * sum_i q[o, i] * xs[b, i]
 *
 * The weights are exact int8 in the T64 image (the same image qgemv_q8row
 * reads).  The f32 activations are split exactly into int8 limbs of a
 * per-row fixed-point value, xs[b, i] ~= 2^e_b * (h*65536 + m*256 + l)
 * (24 bits, rounded to nearest; 2^e_b the smallest power of two bringing
 * max_i |xs[b, i]| to at most 126*65536), and each limb is an exact int8
 * MFMA product with int32 accumulation.  xs_limbs selects the form:
 *   3  all three limbs (24-bit activations);
 *   2  the two upper limbs only (16-bit activations, 2/3 of the work);
 *   0  auto: per 128 rows of xs, 2 limbs when every row satisfies
 *      2^(e_b+8) <= 0.9e-5 * sum_i |xs[b,i]| / sqrt(K) (the 16-bit error
 *      then stays well inside 2e-5 * sum_i |w_i xs_i| for q8_row weights),
 *      else 3 limbs.
 * Accuracy contract.  Row b's fixed point rounds each xs[b, i] by at most
 * u_b = 2^(e_b - 1) (3 limbs) or 257 * 2^(e_b - 1) (2 limbs: the dropped
 * low limb is at most 128 * 2^e_b in magnitude); everything after
 * that is exact (int32 limb sums) up to six binary32 roundings of the
 * output.  So, with A[o, b] = sum_i |q[o, i]| and S[o, b] = sum_i
 * |q[o, i] * xs[b, i]|, output (b, o) is certain to meet
 * |y - y_exact| <= 2e-5 * rs[o] * S[o, b] whenever
 *     u_b * A[o, b] <= 1.9e-5 * S[o, b]                        (C)
 * for the limb count used.  With 3 limbs (C) holds for dense weight rows
 * against activation rows without extreme outliers (uniform int8 rows and
 * N(0,1) xs: u_b * A is 1/35 to 1/70 of 1.9e-5 * S).  With 2 limbs (C) does
 * not hold in general: auto's 2-limb choice rests on the rounding errors
 * of different elements partly cancelling, which holds (at six standard
 * deviations) for weight rows whose mass is spread, E|q| / sqrt(E q^2) >=
 * 0.8, as in dense int8 matrices.  Outside (C) -- e.g. a weight row with
 * one or a few non-zeros on activations far below the row maximum
 * (|xs| below about 0.5 % of max|xs_b| with 3 limbs) -- no fixed-point
 * form of this product meets the bound; such rows need the per-element
 * floating arithmetic of the q8_row GEMV (qgemv_q8row, per row b).
 * A row of xs holding an infinity or NaN gives NaN for all its outputs.
 * Arguments:
 *   qpacked: device, T64 image of q [M][K] (16-byte aligned);
 *   rs: device f32[M];  xs: device f32[nb][K] row-major (16-byte aligned);
 *   y: device f32[nb][M] row-major, written;
 *   ws: device workspace, 256-byte aligned, >= qgemm_q8row_batched_ws_bytes
 *       (nb, K) bytes; holds the limbs and per-row exponents; contents on
 *       entry are ignored.
 * K is at most 131068: each limb's exact int32 sum over K, at most
 * 128 * 128 * K in magnitude, then stays below 2^31.
 * QG_EINVAL: null pointer, nb < 1, M < 1, K < 4, K % 4 != 0, K > 131068, xs_limbs
 * not 0/2/3, misalignment, workspace too small or overlapping y or xs.   */
size_t qgemm_q8row_batched_ws_bytes(int64_t nb, int64_t K);

qg_status qgemm_q8row_batched(const void *qpacked, const float *rs,
                              const float *xs, float *y, int64_t nb,
                              int64_t M, int64_t K, int xs_limbs, void *ws,
                              size_t ws_bytes, void *stream);

/* ======================================================================
 * Column prescale of the q8_row down projection's input  [SP]
 *
 *   act[r][i] = silu(g[r][i]) * u[r][i] * col[i]
 *
 * in IEEE binary32, one correctly rounded operation per step: e = exp(-g)
 * (the binary64 exponential rounded once), s = g / (1 + e), then s * u,
 * then times col[i].  col == NULL means the tensor has no column field
 * (the product is left unscaled).  The result is the prescaled xs that
 * qgemv_q8row / qgemm_q8row_batched expect.
 * Arguments:
 *   g, u: device f32[rows][n] row-major;  col: device f32[n] or NULL, shared
 *   by every row;  act: device f32[rows][n], written; it may be g or u
 *   itself, otherwise it must not overlap g, u or col.
 *   rows >= 1, n >= 1 (any n; n % 4 == 0 with 16-byte aligned pointers takes
 *   128-bit accesses).
 * QG_EINVAL: null g/u/act, bad shape, pointers not 4-byte aligned, act
 * partly overlapping g or u, or overlapping col.                          */
qg_status qact_silu_mul_pre(const float *g, const float *u, const float *col,
                            float *act, int64_t rows, int64_t n, void *stream);

/* Batched q8_row product of the prescaled down-projection input  [Q8, SP]
 *
 *   y[b, o] = rs[o] * sum_i q[o, i] * act[b, i],
 *   act[b, i] = silu(g[b, i]) * u[b, i] * col[i]
 *
 * act is formed inside the product's activation prep (never written to
 * memory) by exactly the rule of qact_silu_mul_pre, so y is bit-identical to
 * qact_silu_mul_pre followed by qgemm_q8row_batched with the same xs_limbs.
 * Arguments as qgemm_q8row_batched, with g, u: device f32[nb][K] row-major
 * and col: device f32[K] or NULL, all 16-byte aligned; the workspace is
 * qgemm_q8row_batched_ws_bytes(nb, K) bytes.
 * QG_EINVAL: as qgemm_q8row_batched, or null g/u, or g/u/col misaligned.  */
qg_status qgemm_q8row_batched_silu(const void *qpacked, const float *rs,
                                   const float *g, const float *u,
                                   const float *col, float *y, int64_t nb,
                                   int64_t M, int64_t K, int xs_limbs,
                                   void *ws, size_t ws_bytes, void *stream);

#ifdef __cplusplus
}
#endif
#endif /* QGEMV_H */
