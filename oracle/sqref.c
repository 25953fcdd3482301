/*
 * sqref.c -- CPU oracle for the SmoothQuant W8A8 linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, plain, obviously-correct
 * statement of what the GPU library computes.  Only tests/, the smoke check
 * in __graft_entry__.py and the cpu_baseline leg of bench.py may load it.
 * It shares no code, header, table or helper with the HIP library, and the
 * HIP library never loads it.
 *
 * Pages cited (by title and section):
 *   [P1] abeam.tech explainer of Xiao et al., "SmoothQuant: Accurate and
 *        Efficient Post-Training Quantization for Large Language Models"
 *        (arXiv 2211.10438).  Sections used: 用語解説 (Calibration, INT8 GEMM),
 *        数学的に何をしているのか (the identity Y = (X diag(s)^-1)(diag(s) W)
 *        and the offline fold), なぜ活性値が量子化しづらいのか (range set by
 *        the max absolute value), smoothing factor はどう決めるのか (equation
 *        for s_j and alpha), 学習方法 (calibrate -> s -> quantize),
 *        推論方法 (O1: per-token activations, dynamic; O2: per-tensor,
 *        dynamic; O3: per-tensor, static), 課題 (static scales come from
 *        calibration data).
 *   [P4] blogs.itmedia.co.jp, 「LLMのダイエット術、『量子化（Quantization）』」,
 *        section 3 「レイヤーごとのマッピング」 (range -> scale -> round to the
 *        nearest representable value; scale back at inference; worked
 *        example 53 -> 5.3 -> 5 -> 50).
 *
 * Precision: the quantisation decision is taken in fp32 (fp32 scales, IEEE
 * division, round half away from zero, clamp to +-127), the precision the
 * quantised codes are defined in.  The smoothing factor is evaluated in
 * double and rounded once to fp32.  The dequantised output is returned in
 * double so that the caller compares the 16-bit GPU output against the
 * (nearly) exact value.  Build with -O2 -ffp-contract=off -fno-fast-math.
 *
 * Layouts (all host memory, row-major, caller-owned):
 *   X, X_cal, X_hat : [rows x K]     W, W_hat : [K x N]  (row j = input channel j)
 *   Wq              : [N x K]        (output channel n's K codes contiguous)
 *   acc, y          : [M x N]
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

/* Largest K for which |sum_k q_x q_w| <= K * 127 * 127 fits in int32. */
#define SQREF_MAX_K 133144

/* ---------------------------------------------------------------------- */
/* Calibration statistic [P1 用語解説 "Calibration"; 学習方法; the max(|X_j|)
 * of the s_j equation]: a_j = max over all calibration tokens t of |x[t,j]|.
 * With accumulate != 0 the running maximum continues from the values already
 * in a (several calibration batches). */
void sqref_calibrate_absmax(const float* x, int64_t T, int64_t K, float* a, int accumulate)
{
    for (int64_t j = 0; j < K; ++j) {
        float m = accumulate ? a[j] : 0.0f;
        for (int64_t t = 0; t < T; ++t) {
            float v = fabsf(x[t * K + j]);
            if (v > m) m = v;
        }
        a[j] = m;
    }
}

/* max(|W_j|) of the s_j equation [P1 smoothing factor はどう決めるのか].
 * W_j is row j of W[K x N]: the weights that multiply input channel j, the
 * row that diag(s) W scales by s_j [P1 数学的に何をしているのか]. */
void sqref_weight_row_absmax(const float* w, int64_t K, int64_t N, float* b)
{
    for (int64_t j = 0; j < K; ++j) {
        float m = 0.0f;
        for (int64_t n = 0; n < N; ++n) {
            float v = fabsf(w[j * N + n]);
            if (v > m) m = v;
        }
        b[j] = m;
    }
}

/* Smoothing factor [P1 smoothing factor はどう決めるのか, the s_j equation]:
 *   s_j = max(|X_j|)^alpha / max(|W_j|)^(1 - alpha)
 * evaluated in double and rounded once to fp32.  The page does not say what
 * happens for an all-zero channel; such a channel contributes nothing to Y,
 * so any positive s keeps the identity and s_j = 1 is used. */
void sqref_smoothing_factors(const float* a, const float* b, int64_t K, double alpha, float* s)
{
    for (int64_t j = 0; j < K; ++j) {
        if (a[j] == 0.0f || b[j] == 0.0f) {
            s[j] = 1.0f;
            continue;
        }
        double num = pow((double)a[j], alpha);
        double den = pow((double)b[j], 1.0 - alpha);
        s[j] = (float)(num / den);
    }
}

/* Offline fold into the weight [P1 数学的に何をしているのか]: diag(s) W, i.e.
 * row j of W multiplied by s_j (one fp32 multiply per element). */
void sqref_fold_weight(const float* w, const float* s, int64_t K, int64_t N, float* w_hat)
{
    for (int64_t j = 0; j < K; ++j)
        for (int64_t n = 0; n < N; ++n)
            w_hat[j * N + n] = s[j] * w[j * N + n];
}

/* Offline fold of diag(s)^-1 into the preceding LayerNorm [P1
 * 数学的に何をしているのか]: LN(x)/s = (gamma/s) * normalised + beta/s, so
 * gamma_j and beta_j are each divided by s_j (fp32 division).  Either pointer
 * may be NULL. */
void sqref_fold_norm(const float* s, int64_t K, float* gamma, float* beta)
{
    for (int64_t j = 0; j < K; ++j) {
        if (gamma) gamma[j] = gamma[j] / s[j];
        if (beta) beta[j] = beta[j] / s[j];
    }
}

/* Offline fold of diag(s)^-1 into a preceding linear layer [P1
 * 数学的に何をしているのか: the scales may be absorbed by the preceding linear
 * layer as well as by a LayerNorm].  That layer's output channel j feeds
 * input channel j of this one, so column j of its weight W_prev [Kp x K]
 * and its bias_j are divided by s_j (fp32 division); its output is then
 * X diag(s)^-1 directly.  An elementwise activation f between the two layers
 * commutes with the division only if f(z / s) = f(z) / s for s > 0 (ReLU and
 * the identity do).  bias may be NULL; it is updated in place. */
void sqref_fold_prev_linear(const float* s, const float* w_prev, int64_t Kp, int64_t K,
                            float* w_out, float* bias)
{
    for (int64_t i = 0; i < Kp; ++i)
        for (int64_t j = 0; j < K; ++j)
            w_out[i * K + j] = w_prev[i * K + j] / s[j];
    if (bias)
        for (int64_t j = 0; j < K; ++j) bias[j] = bias[j] / s[j];
}

/* X diag(s)^-1 applied at run time instead of folded [P1
 * 数学的に何をしているのか]: x_hat[m,j] = x[m,j] / s_j (fp32 division). */
void sqref_smooth_activation(const float* x, const float* s, int64_t M, int64_t K, float* x_hat)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t j = 0; j < K; ++j)
            x_hat[m * K + j] = x[m * K + j] / s[j];
}

/* ---------------------------------------------------------------------- */
/* Symmetric 8-bit quantiser.  The range is set by the largest absolute value
 * [P1 なぜ活性値が量子化しづらいのか]; the range is mapped onto the codes
 * -127..127 (scale step = absmax / 127), each value is divided by the step and
 * rounded to the nearest code [P4 section 3, steps 1-3].  The page gives no
 * tie rule: halves round away from zero (C roundf).  Codes are clamped to
 * [-127, 127]. */
float sqref_step(float absmax)
{
    return absmax / 127.0f;
}

int8_t sqref_quantize_value(float v, float step)
{
    if (step == 0.0f) return 0;
    float r = roundf(v / step);
    if (r > 127.0f) r = 127.0f;
    if (r < -127.0f) r = -127.0f;
    return (int8_t)r;
}

/* Quantise n values v[i*stride] with one shared step taken from their absmax;
 * codes go to q[i*qstride]; the step is returned (0 for an all-zero vector,
 * whose codes are all 0). */
float sqref_quantize_vector(const float* v, int64_t n, int64_t stride, int8_t* q, int64_t qstride)
{
    float m = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(v[i * stride]);
        if (a > m) m = a;
    }
    float step = sqref_step(m);
    for (int64_t i = 0; i < n; ++i)
        q[i * qstride] = sqref_quantize_value(v[i * stride], step);
    return step;
}

/* Per-token dynamic activation quantisation [P1 推論方法, O1: activations
 * per token, dynamic]: each row m of X_hat[M x K] gets its own step sx[m]. */
void sqref_quant_act_pertoken(const float* x_hat, int64_t M, int64_t K, int8_t* xq, float* sx)
{
    for (int64_t m = 0; m < M; ++m)
        sx[m] = sqref_quantize_vector(x_hat + m * K, K, 1, xq + m * K, 1);
}

/* Per-output-channel weight quantisation: each column n of W_hat[K x N] gets
 * its own step sw[n]; its K codes are stored contiguously as row n of
 * Wq[N x K].  (The page's O1 uses one step for the whole tensor, the special
 * case of a constant step vector.) */
void sqref_quant_weight_perchannel(const float* w_hat, int64_t K, int64_t N, int8_t* wq, float* sw)
{
    for (int64_t n = 0; n < N; ++n)
        sw[n] = sqref_quantize_vector(w_hat + n, K, N, wq + n * K, 1);
}

/* ---------------------------------------------------------------------- */
/* Per-tensor activation quantisation [P1 推論方法: O2 quantises activations
 * per tensor, dynamically; O3 per tensor, statically].  One step for the
 * whole X_hat[M x K]:
 *   step_in == NULL (O2): step = max over all |x_hat| / 127, as for a token
 *                          but over the whole tensor;
 *   step_in != NULL (O3): step = *step_in, fixed offline from calibration
 *                          data, so values beyond the calibrated range reach
 *                          the clamp at +-127.
 * The codes follow the same quantiser; sx[m] = step for every row, the form
 * the scale-back takes. */
void sqref_quant_act_pertensor(const float* x_hat, int64_t M, int64_t K, const float* step_in,
                               int8_t* xq, float* sx)
{
    float step;
    if (step_in) {
        step = *step_in;
    } else {
        float m = 0.0f;
        for (int64_t i = 0; i < M * K; ++i) {
            float a = fabsf(x_hat[i]);
            if (a > m) m = a;
        }
        step = sqref_step(m);
    }
    for (int64_t i = 0; i < M * K; ++i) xq[i] = sqref_quantize_value(x_hat[i], step);
    for (int64_t m = 0; m < M; ++m) sx[m] = step;
}

/* The static per-tensor step of O3 [P1 推論方法; 課題 (activation scales are
 * estimated from calibration data)]: the largest |x_hat| the calibration set
 * produces, over 127.  x_hat = x / s_j per channel and the fp32 division is
 * monotone, so the largest calibration |x_hat| in channel j is a_j / s_j:
 *   step = max_j (a_j / s_j) / 127. */
float sqref_static_act_step(const float* a, const float* s, int64_t K)
{
    float m = 0.0f;
    for (int64_t j = 0; j < K; ++j) {
        float v = a[j] / s[j];
        if (v > m) m = v;
    }
    return sqref_step(m);
}

/* Per-tensor weight quantisation [P1 推論方法: O1-O3 quantise the weights
 * per tensor]: one step = max over all |W_hat| / 127; codes stored as
 * Wq[N x K] like the per-channel case, sw[n] = step for every channel. */
void sqref_quant_weight_pertensor(const float* w_hat, int64_t K, int64_t N, int8_t* wq, float* sw)
{
    float m = 0.0f;
    for (int64_t i = 0; i < K * N; ++i) {
        float a = fabsf(w_hat[i]);
        if (a > m) m = a;
    }
    float step = sqref_step(m);
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) wq[n * K + k] = sqref_quantize_value(w_hat[k * N + n], step);
        sw[n] = step;
    }
}

/* ---------------------------------------------------------------------- */
/* INT8 GEMM [P1 用語解説 "INT8 GEMM"; 推論方法]: acc[m,n] = sum_k xq[m,k] wq[n,k],
 * summed exactly in 64-bit and stored as int32 (exact for K <= SQREF_MAX_K).
 * Returns 0, or -1 if K is out of range. */
int sqref_gemm_i32(const int8_t* xq, const int8_t* wq, int64_t M, int64_t N, int64_t K, int32_t* acc)
{
    if (K > SQREF_MAX_K) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            int64_t sum = 0;
            for (int64_t k = 0; k < K; ++k)
                sum += (int64_t)xq[m * K + k] * (int64_t)wq[n * K + k];
            acc[m * N + n] = (int32_t)sum;
        }
    return 0;
}

/* The same sums for a chosen set of rows and columns only:
 * acc[i * ncol + c] = sum_k xq[rows[i], k] * wq[cols[c], k]. */
int sqref_gemm_i32_sampled(const int8_t* xq, const int8_t* wq, int64_t K,
                           const int64_t* rows, int64_t nrow, const int64_t* cols, int64_t ncol,
                           int32_t* acc)
{
    if (K > SQREF_MAX_K) return -1;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t i = 0; i < nrow; ++i)
        for (int64_t c = 0; c < ncol; ++c) {
            int64_t sum = 0;
            for (int64_t k = 0; k < K; ++k)
                sum += (int64_t)xq[rows[i] * K + k] * (int64_t)wq[cols[c] * K + k];
            acc[i * ncol + c] = (int32_t)sum;
        }
    return 0;
}

/* Scale back [P4 section 3: multiply the scale factor back at inference]:
 * y[m,n] = acc[m,n] * sx[m] * sw[n], in double (token step times channel
 * step). */
void sqref_dequant(const int32_t* acc, const float* sx, const float* sw, int64_t M, int64_t N, double* y)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n)
            y[m * N + n] = (double)acc[m * N + n] * (double)sx[m] * (double)sw[n];
}

/* Scale back followed by the rest of a linear layer: y = acc*sx*sw + bias[n]
 * (bias over output channels, may be NULL), then max(y, 0) when relu is set,
 * in double.  The ReLU is the activation a smoothed layer may be folded
 * through (see sqref_fold_prev_linear). */
void sqref_dequant_bias_act(const int32_t* acc, const float* sx, const float* sw,
                            const float* bias, int relu, int64_t M, int64_t N, double* y)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double v = (double)acc[m * N + n] * (double)sx[m] * (double)sw[n];
            if (bias) v += (double)bias[n];
            if (relu && !(v > 0.0)) v = 0.0;
            y[m * N + n] = v;
        }
}

/* The same scale back with bias and ReLU, evaluated in fp32 in a fixed order
 * so that a quantised code taken from its output (the next layer's input)
 * is decided in the precision the layer computes in: f = fp32(acc) * sx[m]
 * (one fp32 rounding), v = f * sw[n] + bias[n] with a single rounding
 * (C99 fmaf), then ReLU as v > 0 ? v : +0.  The pages fix no precision for
 * this step; this is fp32 with one rounding per operation. */
void sqref_dequant_bias_act_f32(const int32_t* acc, const float* sx, const float* sw,
                                const float* bias, int relu, int64_t M, int64_t N, float* y)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            float f = (float)acc[m * N + n];
            f = f * sx[m];
            float v = fmaf(f, sw[n], bias ? bias[n] : 0.0f);
            if (relu && !(v > 0.0f)) v = 0.0f;
            y[m * N + n] = v;
        }
}

/* Whole run-time linear layer for timing: per-token quantisation of X_hat,
 * INT8 GEMM and scale back, one token row at a time (rows are independent).
 * xq_row / acc_row are caller scratch of K and N entries per thread slot;
 * this entry point allocates them itself. */
int sqref_linear_w8a8(const float* x_hat, const int8_t* wq, const float* sw,
                      int64_t M, int64_t N, int64_t K, double* y)
{
    if (K > SQREF_MAX_K) return -1;
    int rc = 0;
#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t m = 0; m < M; ++m) {
        int8_t* xq = (int8_t*)malloc((size_t)K);
        if (!xq) { rc = -2; continue; }
        float sx = sqref_quantize_vector(x_hat + m * K, K, 1, xq, 1);
        for (int64_t n = 0; n < N; ++n) {
            int64_t sum = 0;
            for (int64_t k = 0; k < K; ++k)
                sum += (int64_t)xq[k] * (int64_t)wq[n * K + k];
            y[m * N + n] = (double)(int32_t)sum * (double)sx * (double)sw[n];
        }
        free(xq);
    }
    return rc;
}
