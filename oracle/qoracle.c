/*
 * qoracle.c -- plain CPU oracle for the weight-only-quantized decode products.
 *
 * TEST INFRASTRUCTURE.  Only the tests, the smoke check and the bench's CPU
 * baseline leg load this file's library.  It shares no source, header, table
 * or helper with the HIP library; the two meet only in the seeded inputs.
 *
 * Every function is the plain definition of what the pages compute, written
 * out in double precision (fp64) except the activation quantiser, whose
 * integer outputs are decided in IEEE binary32 exactly as the page fixes it.
 * No blocking, no reordering beyond a single left-to-right loop.
 *
 * Sources (cited by page and function, no line numbers):
 *  [Q8]  cortiq-engine 0.5.43 gpu_wgpu.rs page, module doc and the q8_matvec /
 *        q8_matmat shaders; cortiq-engine 0.3.7 gpu_metal.rs page, q8_matvec /
 *        q8_matmat kernels: y[o] = rs[o] * sum_i q[o,i] * xs[i], xs already
 *        prescaled, batched y[b,o] with xs [nb][K] and y [nb][M] row-major.
 *  [Q2]  qxmx qxmx_gpu.cpp page, dequant_embd: code k of a block is
 *        (qs[k/4] >> 2*(k%4)) & 3, weight = d * (code - 1); blocks are 18 B
 *        per 64 weights or 34 B per 128 (upload_q2), d a binary16 scale.
 *  [AQ]  qxmx qxmx_gpu.cpp page, gpu_rmsnorm_quant: act_scale = amax/127,
 *        inv = 1/act_scale (0 when act_scale is 0), v = round(x*inv) with
 *        round-half-away-from-zero, clamped to [-128, 127]; suma = sum of the
 *        int8 values of each 64-wide group.
 *  [GV]  qxmx qxmx_gpu.cpp page, gemv_dpas8 and gemv_reduce: per 64-wide
 *        group the integer dot of codes with the int8 activations, corrected
 *        by suma to sum (code-1)*xq, scaled by d, summed over groups and
 *        multiplied by act_scale.
 *  [GA]  qxmx qxmx_gpu.cpp page, tmatvec_accum and the accum argument of
 *        gemv_dpas8: the projection plus a residual vector.
 *  [QG]  qxmx qxmx_gpu.cpp page, ffn_forward_b with gemm_gpu_v4 /
 *        gemm_gpu_v4_dual: the batched (prefill) Q2 product over tokens b,
 *        each token's activation quantised with its own act_scale[b] and
 *        group sums, the output token-major y[b][o], an optional residual.
 *  [PQ]  qxmx qxmx_gpu.cpp page, gpu_rmsnorm_quant, gpu_swiglu_quant,
 *        gpu_silu_mul_quant, gpu_sigmoid_mul_quant: the quantiser [AQ]
 *        applied to a vector formed in binary32 first: x * inv * w with
 *        inv = 1 / sqrt(mean(x^2) + eps) (the sum of squares in binary64),
 *        or silu(g) * u = (g / (1 + exp(-g))) * u, or u * sigmoid(g) =
 *        u * (1 / (1 + exp(-g))).
 *
 * Readings where the pages are silent (each listed in the design notes):
 *  - binary16 is decoded per IEEE 754 (subnormal = m * 2^-24); the page's
 *    host helper f16_to_f32 uses 2^-14 for subnormals, its device code uses
 *    native half.
 *  - a block is the 2-byte little-endian d followed by the code bytes.
 *  - the quantiser acts on the given f32 vector (no fused norm).
 *  - the Q2 reference result is built from sc*xq, the quantised activations.
 *  - the binary32 exponential of the activation producers is the correctly
 *    rounded one, exp evaluated in binary64 and rounded once (the page calls
 *    its runtime's single-precision exp; the pages do not fix its accuracy).
 *  - the norm's epsilon is an argument (its value is not on the pages); the
 *    binary64 sum of squares runs left to right, sqrt and the divisions are
 *    IEEE (correctly rounded) binary32 operations.
 *
 * Build: gcc -O2 -ffp-contract=off -fPIC -shared qoracle.c -lm
 *  [SP]  cortiq-engine 0.5.43 gpu_wgpu.rs page, silu_mul_pre shader of the
 *        MoE block, and cortiq-engine 0.3.7 gpu_metal.rs page, silu_mul_pre
 *        kernel (has_col): the down projection's prescaled input
 *        act = silu(g) * u * col in binary32, with col the q8_2f column
 *        field (left out when a tensor has none); the Metal page's
 *        q8_mul_mm_silu forms silu(g) * u inside the batched product.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

/* ---- binary16 -> double, IEEE 754 definition ---------------------------- */
double qo_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);                /* 0.m * 2^-14 */
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);    /* 1.m * 2^(e-15) */
    return sign ? -v : v;
}

/* ---- q8_row: y[o] = rs[o] * sum_i q[o,i] * xs[i]  [Q8] ------------------- */
/* rows == NULL: all M rows, y[o]; else y[j] for o = rows[j], j < nrows.
 * mass[.] = sum_i |rs[o] q[o,i] xs[i]|, the per-output error yardstick.   */
void qo_q8row_gemv(const int8_t *q, const float *rs, const float *xs,
                   int64_t M, int64_t K, const int64_t *rows, int64_t nrows,
                   double *y, double *mass)
{
    int64_t n = rows ? nrows : M;
    for (int64_t j = 0; j < n; j++) {
        int64_t o = rows ? rows[j] : j;
        const int8_t *qr = q + o * K;
        double acc = 0.0, am = 0.0;
        for (int64_t i = 0; i < K; i++) {
            double t = (double)qr[i] * (double)xs[i];
            acc += t;
            am += fabs(t);
        }
        y[j] = (double)rs[o] * acc;
        if (mass) mass[j] = fabs((double)rs[o]) * am;
    }
}

/* ---- batched q8_row: y[b,o] = rs[o] * sum_i q[o,i] * xs[b,i]  [Q8] ------- */
/* bs/os == NULL: the full [nb][M] output; else the n listed (b, o) entries. */
void qo_q8row_gemm(const int8_t *q, const float *rs, const float *xs,
                   int64_t nb, int64_t M, int64_t K,
                   const int64_t *bs, const int64_t *os, int64_t n,
                   double *y, double *mass)
{
    int64_t total = bs ? n : nb * M;
    for (int64_t j = 0; j < total; j++) {
        int64_t b = bs ? bs[j] : j / M;
        int64_t o = bs ? os[j] : j % M;
        const int8_t *qr = q + o * K;
        const float *xr = xs + b * K;
        double acc = 0.0, am = 0.0;
        for (int64_t i = 0; i < K; i++) {
            double t = (double)qr[i] * (double)xr[i];
            acc += t;
            am += fabs(t);
        }
        y[j] = (double)rs[o] * acc;
        if (mass) mass[j] = fabs((double)rs[o]) * am;
    }
}

/* ---- Q2 blocks [Q2] ------------------------------------------------------ */
static int64_t blk_bytes(int group) { return 2 + group / 4; }

static const uint8_t *q2_blk(const uint8_t *blob, int64_t K, int group,
                             int64_t o, int64_t g)
{
    return blob + (o * (K / group) + g) * blk_bytes(group);
}

static double q2_d(const uint8_t *blk)
{
    return qo_f16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));
}

static int q2_code(const uint8_t *blk, int k)
{
    return (blk[2 + k / 4] >> (2 * (k % 4))) & 3;
}

/* Dense dequantisation w[o][i] = d * (code - 1) of the whole matrix. */
void qo_q2_dequant(const uint8_t *blob, int64_t M, int64_t K, int group,
                   double *w)
{
    for (int64_t o = 0; o < M; o++)
        for (int64_t i = 0; i < K; i++) {
            const uint8_t *blk = q2_blk(blob, K, group, o, i / group);
            w[o * K + i] = q2_d(blk) * (double)(q2_code(blk, (int)(i % group)) - 1);
        }
}

/* ---- activation int8 quantisation, in IEEE binary32  [AQ] --------------- */
/* suma may be NULL; else K/64 entries (K % 64 == 0 is the caller's job). */
void qo_act_quant_i8(const float *x, int64_t K, int8_t *xq, float *act_scale,
                     int32_t *suma)
{
    float amax = 0.0f;
    for (int64_t i = 0; i < K; i++) {
        float a = fabsf(x[i]);
        if (a > amax) amax = a;
    }
    float sc = amax / 127.0f;
    float inv = sc > 0.0f ? 1.0f / sc : 0.0f;
    for (int64_t i = 0; i < K; i++) {
        float v = roundf(x[i] * inv);
        if (v > 127.0f) v = 127.0f;
        if (v < -128.0f) v = -128.0f;
        xq[i] = (int8_t)v;
    }
    if (suma)
        for (int64_t g = 0; g < K / 64; g++) {
            int32_t s = 0;
            for (int k = 0; k < 64; k++) s += xq[g * 64 + k];
            suma[g] = s;
        }
    *act_scale = sc;
}

/* ---- Q2 x int8 group dots  [GV] ----------------------------------------- */
/* dots[o][u] = sum over the 64 weights of 64-wide unit u of (code-1)*xq.
 * A 128-wide block is two 64-wide units sharing d.                        */
void qo_q2_dots(const uint8_t *blob, int64_t M, int64_t K, int group,
                const int8_t *xq, int32_t *dots)
{
    int64_t nu = K / 64;
    for (int64_t o = 0; o < M; o++)
        for (int64_t u = 0; u < nu; u++) {
            int32_t s = 0;
            for (int64_t i = u * 64; i < u * 64 + 64; i++) {
                const uint8_t *blk = q2_blk(blob, K, group, o, i / group);
                s += (q2_code(blk, (int)(i % group)) - 1) * (int32_t)xq[i];
            }
            dots[o * nu + u] = s;
        }
}

/* y[o] = sc * sum_u d(u) * dots[o][u], fp64  [GV]
 * rows == NULL: all rows; mass[.] = sum_i |d (code-1)| * |sc xq_i|.       */
void qo_q2_gemv(const uint8_t *blob, int64_t M, int64_t K, int group,
                const int8_t *xq, float sc, const int64_t *rows, int64_t nrows,
                double *y, double *mass)
{
    int64_t n = rows ? nrows : M;
    int64_t nu = K / 64;
    for (int64_t j = 0; j < n; j++) {
        int64_t o = rows ? rows[j] : j;
        double acc = 0.0, am = 0.0;
        for (int64_t u = 0; u < nu; u++) {
            const uint8_t *blk = q2_blk(blob, K, group, o, (u * 64) / group);
            double d = q2_d(blk);
            int64_t dot = 0, adot = 0;
            for (int64_t i = u * 64; i < u * 64 + 64; i++) {
                int c = q2_code(blk, (int)(i % group)) - 1;
                dot += (int64_t)c * xq[i];
                adot += (int64_t)(c < 0 ? -c : c) * (xq[i] < 0 ? -xq[i] : xq[i]);
            }
            acc += d * (double)dot;
            am += fabs(d) * (double)adot;
        }
        y[j] = (double)sc * acc;
        if (mass) mass[j] = fabs((double)sc) * am;
    }
}

/* ---- Q2 GEMV plus residual  [GA] ---------------------------------------- */
/* y[j] = (qo_q2_gemv result for row rows[j]) + accum[rows[j]], fp64.
 * mass as qo_q2_gemv (the residual adds no product terms).              */
void qo_q2_gemv_accum(const uint8_t *blob, int64_t M, int64_t K, int group,
                      const int8_t *xq, float sc, const float *accum,
                      const int64_t *rows, int64_t nrows, double *y,
                      double *mass)
{
    int64_t n = rows ? nrows : M;
    qo_q2_gemv(blob, M, K, group, xq, sc, rows, nrows, y, mass);
    for (int64_t j = 0; j < n; j++) {
        int64_t o = rows ? rows[j] : j;
        y[j] += (double)accum[o];
    }
}

/* ---- fused activation producers  [PQ] ----------------------------------- */
/* RMSNorm then [AQ]: v_i = (x_i * inv) * w_i in binary32, then quantised.
 * v (K floats, required) receives the normalised vector.                 */
void qo_rmsnorm_quant_i8(const float *x, const float *w, int64_t K, float eps,
                         float *v, int8_t *xq, float *act_scale, int32_t *suma)
{
    double ss = 0.0;
    for (int64_t i = 0; i < K; i++) ss += (double)x[i] * (double)x[i];
    float ms = (float)(ss / (double)K);
    float inv = 1.0f / sqrtf(ms + eps);
    for (int64_t i = 0; i < K; i++) {
        float xi = x[i] * inv;
        v[i] = xi * w[i];
    }
    qo_act_quant_i8(v, K, xq, act_scale, suma);
}

/* binary32 exp, correctly rounded: binary64 exp rounded once.            */
static float exp_f32(float a) { return (float)exp((double)a); }

/* Gated product then [AQ]: kind 0 = silu(g) * u = (g / (1 + e)) * u,
 * kind 1 = u * sigmoid(g) = u * (1 / (1 + e)), with e = exp(-g), every
 * step in binary32.  t (K floats, required) receives the product.         */
void qo_glu_quant_i8(const float *g, const float *u, int64_t K, int kind,
                     float *t, int8_t *xq, float *act_scale, int32_t *suma)
{
    for (int64_t i = 0; i < K; i++) {
        float e = exp_f32(-g[i]);
        float den = 1.0f + e;
        if (kind == 0) {
            float silu = g[i] / den;
            t[i] = silu * u[i];
        } else {
            float sig = 1.0f / den;
            t[i] = u[i] * sig;
        }
    }
    qo_act_quant_i8(t, K, xq, act_scale, suma);
}

/* [SP] act[r][i] = silu(g[r][i]) * u[r][i] * col[i] over rows x n values
 * (row-major; col shared by the rows, NULL = no column field): e = exp(-g),
 * s = g / (1 + e), then s * u, then times col[i], every step in binary32. */
void qo_silu_mul_pre(const float *g, const float *u, const float *col,
                     int64_t rows, int64_t n, float *act)
{
    for (int64_t r = 0; r < rows; r++) {
        for (int64_t i = 0; i < n; i++) {
            int64_t k = r * n + i;
            float e = exp_f32(-g[k]);
            float den = 1.0f + e;
            float s = g[k] / den;
            float v = s * u[k];
            if (col)
                v = v * col[i];
            act[k] = v;
        }
    }
}

/* ---- batched Q2: y[b,o] = sc[b] * sum_u d(o,u) * dots[b][o][u]  [QG] ---- */
/* xq [nb][K] (row b quantised with scale sc[b]); accum [nb][M] or NULL.
 * bs/os == NULL: the full [nb][M] output; else the n listed (b, o) entries.
 * mass[.] = sum_i |d (code-1)| * |sc[b] xq[b,i]|.                          */
void qo_q2_gemm(const uint8_t *blob, int64_t M, int64_t K, int group,
                const int8_t *xq, const float *sc, int64_t nb,
                const float *accum, const int64_t *bs, const int64_t *os,
                int64_t n, double *y, double *mass)
{
    int64_t total = bs ? n : nb * M;
    for (int64_t j = 0; j < total; j++) {
        int64_t b = bs ? bs[j] : j / M;
        int64_t o = bs ? os[j] : j % M;
        double yj, mj;
        qo_q2_gemv(blob, M, K, group, xq + b * K, sc[b], &o, 1, &yj, &mj);
        if (accum) yj += (double)accum[b * M + o];
        y[j] = yj;
        if (mass) mass[j] = mj;
    }
}
