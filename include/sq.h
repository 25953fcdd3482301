/*
 * sq.h -- C ABI of the SmoothQuant W8A8 linear-layer library for AMD MI355X
 * (gfx950).
 *
 * The method (pages cited by title and section):
 *   [P1] abeam.tech explainer of Xiao et al., "SmoothQuant: Accurate and
 *        Efficient Post-Training Quantization for Large Language Models"
 *        (arXiv 2211.10438).
 *   [P4] blogs.itmedia.co.jp, 「LLMのダイエット術、『量子化（Quantization）』」.
 *
 *   offline : calibrate per-input-channel activation absmax; smoothing
 *             factor s_j; fold diag(s) into W and diag(s)^-1 into the
 *             preceding LayerNorm; quantise W to INT8 per output channel.
 *   runtime : quantise each token of X_hat to INT8 by its own absmax; INT8 x
 *             INT8 -> INT32 GEMM; scale back by token step x channel step.
 *
 * Conventions for every entry point:
 *   - Tensor pointers are DEVICE pointers owned by the caller, contiguous and
 *     row-major, each 16-byte aligned.  Sizes are element counts.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *     Each call validates its arguments on the host, enqueues its kernels on
 *     `stream` and returns without synchronising; results are ready when the
 *     stream reaches that point.
 *   - On a validation error nothing is launched and nothing is written; the
 *     status says which rule failed.  A launch failure returns SQ_ERR_HIP.
 *     Faults inside a kernel surface at the caller's next synchronisation,
 *     as with any HIP call.
 *   - Inputs must be finite (NaN/Inf are outside the contract).
 *   - Every input and output buffer must be distinct (no aliasing) unless a
 *     description says otherwise.
 *   - The library keeps no state between calls and allocates no device
 *     memory; calls on different streams are independent.
 *
 * Quantiser used everywhere [P1 なぜ活性値が量子化しづらいのか: the range is
 * set by the largest absolute value; P4 section 3: range -> scale -> round
 * to nearest; scale back at inference]:
 *   step = absmax / 127.0f (fp32 IEEE division);
 *   code = clamp(round_half_away_from_zero(v / step), -127, 127), v / step an
 *          fp32 IEEE division; an all-zero vector has step 0 and codes 0.
 */
#ifndef SQ_H
#define SQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    SQ_OK = 0,
    SQ_ERR_NULL = 1,        /* a required pointer is NULL */
    SQ_ERR_SHAPE = 2,       /* a size is < 1 or > SQ_MAX_DIM */
    SQ_ERR_DTYPE = 3,       /* dtype code not accepted by this entry point */
    SQ_ERR_K_OVERFLOW = 4,  /* K > SQ_MAX_K: int32 accumulators could overflow */
    SQ_ERR_ALIGN = 5,       /* a tensor pointer is not 16-byte aligned */
    SQ_ERR_ALPHA = 6,       /* alpha outside [0, 1] or not finite */
    SQ_ERR_HIP = 7,         /* the HIP runtime reported a launch error */
    SQ_ERR_ALIAS = 8,       /* two buffers overlap where the entry point forbids it */
    SQ_ERR_ACT = 9,         /* activation code not one of sq_act */
    SQ_ERR_EPS = 10,        /* LayerNorm epsilon negative or not finite */
    SQ_ERR_WORKSPACE = 11   /* workspace NULL, misaligned or smaller than required */
} sq_status;

typedef enum { SQ_F32 = 0, SQ_F16 = 1, SQ_BF16 = 2 } sq_dtype;

/* Elementwise activation applied after the bias (sq_w8a8_gemm_dequant_ex). */
typedef enum { SQ_ACT_NONE = 0, SQ_ACT_RELU = 1 } sq_act;

/* |sum_k xq*wq| <= K * 127 * 127 < 2^31 holds for K <= 133144. */
#define SQ_MAX_K 133144
/* Largest accepted M, N, K, T (rows and columns are indexed with int). */
#define SQ_MAX_DIM 4194304

/* ---------------------------------------------------------------- offline */

/* Calibration statistic [P1 用語解説 "Calibration"; 学習方法; the max(|X_j|)
 * of the s_j equation in smoothing factor はどう決めるのか]:
 *   a[j] = max(accumulate ? a[j] : 0, max_t |x[t, j]|)
 * x: [T x K] of dtype xdt (F32, F16, BF16).  a: fp32 [K], read (accumulate
 * != 0) and written.  Call once per calibration batch with accumulate = 1
 * after the first to keep a running maximum over batches. */
sq_status sq_calibrate_absmax(const void* x, sq_dtype xdt, int64_t T, int64_t K,
                              float* a, int accumulate, void* stream);

/* Smoothing factor and offline fold [P1 smoothing factor はどう決めるのか:
 * s_j = max(|X_j|)^alpha / max(|W_j|)^(1-alpha); 数学的に何をしているのか:
 * Y = (X diag(s)^-1)(diag(s) W), diag(s) folded into W and diag(s)^-1 into
 * the preceding LayerNorm]:
 *   b_j     = max_n |w[j, n]|               (row j multiplies input channel j)
 *   s_out[j] = (float)(pow(a_j, alpha) / pow(b_j, 1 - alpha)) in double;
 *             1.0f when a_j == 0 or b_j == 0 (the channel adds nothing to Y)
 *   w_out[j, n] = s_j * w[j, n]             (one fp32 multiply)
 *   gamma[j] /= s_j, beta[j] /= s_j         (fp32 division; in place)
 * a: fp32 [K].  w: [K x N] of dtype wdt (F32, F16, BF16).  alpha in [0, 1]
 * (a double, used as given: both pow calls take exactly this value).
 * s_out: fp32 [K].  w_out: fp32 [K x N].  gamma, beta: fp32 [K] or NULL.
 * s is evaluated with the device's double pow; it may differ from another
 * libm's result by one fp32 ulp when the two double results straddle an fp32
 * rounding boundary. */
sq_status sq_smooth_fold(const float* a, const void* w, sq_dtype wdt, int64_t K, int64_t N,
                         double alpha, float* s_out, float* w_out, float* gamma, float* beta,
                         void* stream);

/* Offline fold of this layer's smoothing into a preceding linear layer [P1
 * 数学的に何をしているのか: diag(s)^-1 may be absorbed by the preceding linear
 * layer instead of a LayerNorm].  That layer's output channel j feeds input
 * channel j here, so
 *   w_out[i, j] = fp32(w_prev[i, j]) / s[j]      (fp32 division)
 *   bias[j]     = bias[j] / s[j]                 (in place; bias may be NULL)
 * and its output is X diag(s)^-1 directly.  An activation between the two
 * layers must commute with the division (f(z / s) = f(z) / s for s > 0:
 * ReLU does, GELU does not).  s: fp32 [K] (sq_smooth_fold's s_out of the
 * next layer).  w_prev: [Kp x K] of dtype wdt (its input channels in rows,
 * the convention of sq_smooth_fold).  w_out: fp32 [Kp x K]. */
sq_status sq_fold_prev_linear(const float* s, const void* w_prev, sq_dtype wdt, int64_t Kp,
                              int64_t K, float* w_out, float* bias, void* stream);

/* Per-output-channel weight quantisation (each column n of w gets its own
 * step; P1 推論方法 names per-tensor weights for O1, the special case of a
 * constant step vector):
 *   w_scale[n] = max_j |w[j, n]| / 127;   wq[n, j] = code(w[j, n], w_scale[n])
 * w: [K x N] of dtype wdt (F32, F16, BF16), normally the folded W_hat.
 * wq: int8 [N x K] (output channel n's K codes contiguous -- the transpose of
 * w's layout).  w_scale: fp32 [N]. */
sq_status sq_quant_weight_perchannel(const void* w, sq_dtype wdt, int64_t K, int64_t N,
                                     int8_t* wq, float* w_scale, void* stream);

/* Per-tensor weight quantisation [P1 推論方法, O1-O3: weights per tensor]:
 * one step for the whole matrix,
 *   step = max_{j,n} |w[j, n]| / 127;   wq[n, j] = code(w[j, n], step)
 * and every w_scale[n] = step, so the GEMM entry points take it unchanged.
 * Shapes, layouts and dtypes as sq_quant_weight_perchannel. */
sq_status sq_quant_weight_pertensor(const void* w, sq_dtype wdt, int64_t K, int64_t N,
                                    int8_t* wq, float* w_scale, void* stream);

/* ---------------------------------------------------------------- runtime */

/* Per-token dynamic activation quantisation [P1 推論方法, O1: activations per
 * token, dynamic]:
 *   v[m, k]    = smooth ? fp32(x[m, k]) / smooth[k] : fp32(x[m, k])
 *   x_scale[m] = max_k |v[m, k]| / 127;   xq[m, k] = code(v[m, k], x_scale[m])
 * x: [M x K] of dtype xdt (F32, F16, BF16), normally X_hat as the folded
 * LayerNorm emits it.  smooth: fp32 [K] or NULL (NULL: x is already
 * smoothed).  xq: int8 [M x K].  x_scale: fp32 [M]. */
sq_status sq_quant_act_pertoken(const void* x, sq_dtype xdt, int64_t M, int64_t K,
                                const float* smooth, int8_t* xq, float* x_scale, void* stream);

/* LayerNorm carrying the folded smoothing factors, fused with per-token
 * quantisation [P1 数学的に何をしているのか: diag(s)^-1 is absorbed by the
 * LayerNorm in front of the layer, which then emits X_hat; P1 推論方法, O1:
 * X_hat quantised per token].  The LayerNorm is the standard one of each row
 * (Ba, Kiros and Hinton, "Layer Normalization", 2016):
 *   mu   = fp32(S / K),  S = sum_k x[m, k]                   (double sums)
 *   var  = sum_k (x[m, k] - S / K)^2 / K                     (double)
 *   rstd = fp32(1 / sqrt(var + eps))                         (double)
 *   h[k] = dt( (((x[m, k] - mu) * rstd) * gamma[k]) + beta[k] )
 *          (fp32, one rounding per operation, no fused multiply-add, then
 *          round to nearest even to the activation dtype xdt)
 *   then xq[m, :], x_scale[m] exactly as sq_quant_act_pertoken of h.
 * gamma, beta: fp32 [K], the LayerNorm's scale and shift already divided by
 * the smoothing factors (sq_smooth_fold's in-place update).  eps >= 0.
 * x_hat: [M x K] of dtype xdt receiving h, or NULL (not written).  The double
 * sums are taken in the kernel's own order; a result can differ from a
 * correctly rounded sum only where the exact statistic lies within that
 * order's error bound (K * 2^-53 relative) of an fp32 rounding boundary.
 * One workgroup per row, the row held in registers: K up to 65536 (fp16,
 * bf16) or 32768 (fp32) when K is a multiple of 8 (4 for fp32), else up to
 * 16384; larger K: SQ_ERR_SHAPE.  Outputs must not overlap the inputs or one
 * another: SQ_ERR_ALIAS. */
sq_status sq_layernorm_quant_pertoken(const void* x, sq_dtype xdt, int64_t M, int64_t K,
                                      const float* gamma, const float* beta, double eps,
                                      int8_t* xq, float* x_scale, void* x_hat, void* stream);

/* Per-tensor activation quantisation [P1 推論方法, O2: activations per
 * tensor, dynamic; O3: per tensor, static, the step fixed offline from
 * calibration]:
 *   v[m, k] = smooth ? fp32(x[m, k]) / smooth[k] : fp32(x[m, k])
 *   step    = step_in ? *step_in                      (O3, static)
 *                     : max_{m,k} |v[m, k]| / 127      (O2, dynamic)
 *   xq[m, k] = code(v[m, k], step)  (clamped to +-127: under a static step
 *              values beyond 127 * step saturate);   x_scale[m] = step
 * Every x_scale entry holds the same step, so sq_w8a8_gemm_dequant and the
 * packed GEMM consume the result unchanged.  step_in: device pointer to one
 * fp32 (the output of sq_static_act_step) or NULL; it must not overlap
 * x_scale.  In the dynamic case x_scale first holds partial maxima (one per
 * workgroup of the first launch) until the second launch replaces every
 * entry with the step.  Other arguments as sq_quant_act_pertoken.  Dynamic:
 * three launches (partial maxima, step, codes); static: one. */
sq_status sq_quant_act_pertensor(const void* x, sq_dtype xdt, int64_t M, int64_t K,
                                 const float* smooth, const float* step_in, int8_t* xq,
                                 float* x_scale, void* stream);

/* The O3 static activation step from calibration statistics [P1 推論方法, O3;
 * smoothing factor はどう決めるのか]: the calibration maxima a_j of X's
 * channels become a_j / s_j after smoothing, so
 *   *step_out = max_j (a[j] / s[j]) / 127      (fp32 divisions)
 * a, s: fp32 [K] (sq_calibrate_absmax's and sq_smooth_fold's outputs).
 * step_out: device pointer to one fp32.  One workgroup. */
sq_status sq_static_act_step(const float* a, const float* s, int64_t K, float* step_out,
                             void* stream);

/* INT8 GEMM with fused scale back [P1 用語解説 "INT8 GEMM", 推論方法;
 * P4 section 3: multiply the scale factor back]:
 *   acc[m, n] = sum_k xq[m, k] * wq[n, k]              (exact int32)
 *   y[m, n]   = ydt( (fp32(acc) * x_scale[m]) * w_scale[n] )
 * two fp32 multiplies in that order, then round-to-nearest-even to ydt.
 * xq: int8 [M x K].  x_scale: fp32 [M].  wq: int8 [N x K].  w_scale: fp32 [N].
 * y: [M x N] of dtype ydt (F16, BF16, F32).  K <= SQ_MAX_K. */
sq_status sq_w8a8_gemm_dequant(const int8_t* xq, const float* x_scale, const int8_t* wq,
                               const float* w_scale, int64_t M, int64_t N, int64_t K,
                               void* y, sq_dtype ydt, void* stream);

/* The scale back extended by the rest of a linear layer [P1
 * 数学的に何をしているのか: a smoothed layer whose factors are folded into the
 * layer before it; SmoothQuant's target models put a bias and an activation
 * between such layers]:
 *   y[m, n] = ydt( act( fma(fp32(acc) * x_scale[m], w_scale[n], bias[n]) ) )
 * i.e. RN(RN(acc * sx) * sw + bias) in one fp32 FMA, then act: SQ_ACT_NONE,
 * or SQ_ACT_RELU (v > 0 ? v : +0), then round to nearest even to ydt.
 * bias: fp32 [N], 16-byte aligned, or NULL (treated as zeros).  act other
 * than sq_act's values: SQ_ERR_ACT.  Everything else as sq_w8a8_gemm_dequant
 * (same kernels and tiling, the epilogue extended). */
sq_status sq_w8a8_gemm_dequant_ex(const int8_t* xq, const float* x_scale, const int8_t* wq,
                                  const float* w_scale, const float* bias, int act, int64_t M,
                                  int64_t N, int64_t K, void* y, sq_dtype ydt, void* stream);

/* Batched INT8 products for attention [P1 推論方法: besides the linear layers,
 * the attention BMMs run in INT8 (Q K^T and P V)].  `batch` independent
 * products (batch x heads) lying back to back, each exactly as
 * sq_w8a8_gemm_dequant:
 *   acc[b, m, n] = sum_k xq[b, m, k] * wq[b, n, k]
 *   y[b, m, n]   = ydt( (fp32(acc) * x_scale[b, m]) * w_scale[b, n] )
 * xq: int8 [batch x M x K]; x_scale: fp32 [batch x M]; wq: int8
 * [batch x N x K]; w_scale: fp32 [batch x N]; y: [batch x M x N].  For
 * Q K^T: xq = per-token codes of Q (sq_quant_act_pertoken over batch*M rows),
 * wq = per-row codes of K (the same call over its batch*N rows: each key is
 * an output channel of the product).  For P V: xq = per-row codes of P, wq =
 * V's codes per head-dim channel, transposed (sq_quant_weight_perchannel_batched).
 * 1 <= batch <= 65535; other limits and errors as sq_w8a8_gemm_dequant.  One
 * launch (the batch entry is the grid's second dimension). */
sq_status sq_w8a8_bmm_dequant(const int8_t* xq, const float* x_scale, const int8_t* wq,
                              const float* w_scale, int64_t batch, int64_t M, int64_t N,
                              int64_t K, void* y, sq_dtype ydt, void* stream);

/* Per-output-channel quantisation of `batch` matrices w [batch x K x N]
 * lying back to back: for each entry b and column n,
 *   w_scale[b, n] = max_k |w[b, k, n]| / 127,  wq[b, n, k] = code(w[b, k, n])
 * exactly as sq_quant_weight_perchannel per entry (wq: int8 [batch x N x K],
 * w_scale: fp32 [batch x N]).  For attention: V [keys x head_dim] per head
 * becomes the weight operand of P V.  Four launches in all (zero, column
 * maxima, codes, steps).  1 <= batch <= 65535. */
sq_status sq_quant_weight_perchannel_batched(const void* w, sq_dtype wdt, int64_t batch,
                                             int64_t K, int64_t N, int8_t* wq, float* w_scale,
                                             void* stream);

/* ------------------------------------------------------------- auxiliary */

/* The INT8 GEMM's raw accumulators, for exact checking of the GEMM kernels:
 *   acc[m, n] = sum_k xq[m, k] * wq[n, k]   (int32 [M x N]).
 * Uses the same kernels and tiling that sq_w8a8_gemm_dequant selects for
 * (M, N, K). */
sq_status sq_w8a8_gemm_i32(const int8_t* xq, const int8_t* wq, int64_t M, int64_t N, int64_t K,
                           int32_t* acc, void* stream);

/* sq_w8a8_bmm_dequant's raw accumulators (int32 [batch x M x N]), same
 * kernels, for exact checking. */
sq_status sq_w8a8_bmm_i32(const int8_t* xq, const int8_t* wq, int64_t batch, int64_t M, int64_t N,
                          int64_t K, int32_t* acc, void* stream);


/* X diag(s)^-1 at run time, for inputs whose LayerNorm was not folded [P1
 * 数学的に何をしているのか]:  x_hat[m, k] = dt(fp32(x[m, k]) / s[k]), rounded to
 * nearest even when dt is 16-bit.  x, x_hat: [M x K] of dtype dt.  s: fp32 [K]. */
sq_status sq_smooth_activation(const void* x, sq_dtype dt, int64_t M, int64_t K,
                               const float* s, void* x_hat, void* stream);

/* ------------------------------------------------- fragment-packed weights */

/* The quantised weight in a layout the GEMM kernels read as whole contiguous
 * kilobytes (an offline re-layout of wq, no arithmetic; the row-major wq of
 * sq_quant_weight_perchannel stays the canonical form).  Row block b (output
 * channels 16b .. 16b+15) and 64-byte k-group c form one 1024-byte block at
 * byte (b * (K / 64) + c) * 1024; its 16-byte piece l holds channel
 * 16b + l % 16, inputs 64c + 16 (l / 16) .. +15.  Channels past N are zero.
 * Size in bytes: sq_packed_weight_bytes(N, K) = ceil(N / 16) * (K / 64) * 1024.
 * Requires K % 128 == 0 (SQ_ERR_SHAPE otherwise). */
int64_t sq_packed_weight_bytes(int64_t N, int64_t K);
sq_status sq_pack_weight(const int8_t* wq, int64_t N, int64_t K, int8_t* wq_packed,
                         void* stream);

/* sq_w8a8_gemm_dequant / sq_w8a8_gemm_i32 with the weights in the packed
 * layout; identical results.  K % 128 == 0. */
sq_status sq_w8a8_gemm_dequant_packed(const int8_t* xq, const float* x_scale,
                                      const int8_t* wq_packed, const float* w_scale, int64_t M,
                                      int64_t N, int64_t K, void* y, sq_dtype ydt, void* stream);
sq_status sq_w8a8_gemm_i32_packed(const int8_t* xq, const int8_t* wq_packed, int64_t M, int64_t N,
                                  int64_t K, int32_t* acc, void* stream);

/* Split-K forms of sq_w8a8_gemm_dequant and sq_w8a8_gemm_dequant_packed
 * (identical results), for few tokens against a narrow, deep layer, where the
 * output tiles alone leave most compute units idle (e.g. 128 tokens through a
 * 16384 x 4096 layer; the split is taken for K >= 8192 with K % 256 == 0
 * when the 128 x 64 output tiles number at most half the compute units,
 * from 65 tokens on).  K is
 * split into 2, 4 or 8 ranges; each range's int32
 * partial products go to the workspace, and the scale back runs once the
 * ranges of an output tile are summed (integer sums, so the result does not
 * depend on their order).  When the shape does not call for a split
 * (sq_gemm_workspace_bytes returns 0) the call is the plain GEMM and the
 * workspace is not touched.
 *
 * workspace: device memory owned by the caller, 16-byte aligned, at least
 * sq_gemm_workspace_bytes(M, N, K) bytes (queried with the same device
 * current), all zero before its first use; every call leaves its counters at
 * zero again, so one zero fill serves any number of calls of any shapes.
 * Calls that run at the same time must not share a workspace.  Errors:
 * SQ_ERR_WORKSPACE for a NULL, misaligned or too small workspace (when one
 * is needed), SQ_ERR_ALIAS when it overlaps an operand or y; else as the
 * plain entry points (the packed form needs K % 128 == 0). */
int64_t sq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K);
sq_status sq_w8a8_gemm_dequant_ws(const int8_t* xq, const float* x_scale, const int8_t* wq,
                                  const float* w_scale, int64_t M, int64_t N, int64_t K, void* y,
                                  sq_dtype ydt, void* workspace, int64_t workspace_bytes,
                                  void* stream);
sq_status sq_w8a8_gemm_dequant_packed_ws(const int8_t* xq, const float* x_scale,
                                         const int8_t* wq_packed, const float* w_scale, int64_t M,
                                         int64_t N, int64_t K, void* y, sq_dtype ydt,
                                         void* workspace, int64_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory -- code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc: the split-K
 * form of sq_w8a8_gemm_dequant_packed (results identical to it and to
 * sq_w8a8_gemm_dequant_packed_ws) with the int32 partial sums and tile
 * counters in a scratch array inside the library instead of a caller
 * workspace.  Nothing is allocated: the array is a static device array of
 * sq_noalloc_scratch_bytes() bytes (8 MiB + 16 KiB), one copy per GPU the
 * library runs on, held until the process ends.  It fits every split the
 * library takes on a 256-CU MI355X; a shape whose split would need more
 * returns SQ_ERR_WORKSPACE (sq_gemm_workspace_bytes(M, N, K) gives the need).
 * Shapes the library does not split run the plain packed GEMM and do not
 * touch the scratch.  Each call clears the tile counters it uses (a small
 * kernel on `stream`) before the split product.  All calls on one GPU share
 * its array: calls that can run at the same time on one GPU (on different
 * streams) race and must not overlap.  Other errors as
 * sq_w8a8_gemm_dequant_packed (K % 128 == 0). */
sq_status sq_w8a8_gemm_dequant_packed_noalloc(const int8_t* xq, const float* x_scale,
                                              const int8_t* wq_packed, const float* w_scale,
                                              int64_t M, int64_t N, int64_t K, void* y,
                                              sq_dtype ydt, void* stream);
int64_t sq_noalloc_scratch_bytes(void);

/* sq_w8a8_gemm_dequant_ex with the weights in the packed layout; identical
 * results.  K % 128 == 0. */
sq_status sq_w8a8_gemm_dequant_packed_ex(const int8_t* xq, const float* x_scale,
                                         const int8_t* wq_packed, const float* w_scale,
                                         const float* bias, int act, int64_t M, int64_t N,
                                         int64_t K, void* y, sq_dtype ydt, void* stream);

/* The whole run-time layer on packed weights: per-token quantisation of x
 * (exactly sq_quant_act_pertoken with smooth = NULL, writing xq and x_scale)
 * followed by sq_w8a8_gemm_dequant_packed, in one call.  For M <= 2 and
 * M * K <= 16384 the two steps run as one kernel (every workgroup quantises
 * the one or two tokens itself while its first weight loads are in flight,
 * then streams its share of the weight blocks); other shapes take two
 * launches.  x: [M x K] of dtype xdt; xq: int8 [M x K];
 * x_scale: fp32 [M]; wq_packed as above; w_scale: fp32 [N]; y: [M x N] of
 * ydt.  K % 128 == 0.  xq and x_scale are written in both cases. */
sq_status sq_w8a8_linear_packed(const void* x, sq_dtype xdt, int64_t M, int64_t K,
                                const int8_t* wq_packed, const float* w_scale, int64_t N,
                                int8_t* xq, float* x_scale, void* y, sq_dtype ydt, void* stream);

/* The same one-call layer with O3's static per-tensor step [P1 推論方法, O3]:
 * quantisation is exactly sq_quant_act_pertensor with smooth = NULL and
 * step_in given (no run-time maximum: every token uses *step_in, values
 * beyond 127 steps saturate), followed by sq_w8a8_gemm_dequant_packed.  One
 * kernel for M <= 2 and M * K <= 16384, else two launches.  step_in: device
 * pointer to one fp32 (sq_static_act_step's output), not inside x_scale
 * (SQ_ERR_ALIAS).  Other arguments and outputs as sq_w8a8_linear_packed;
 * every x_scale entry is *step_in. */
sq_status sq_w8a8_linear_packed_static(const void* x, sq_dtype xdt, int64_t M, int64_t K,
                                       const int8_t* wq_packed, const float* w_scale, int64_t N,
                                       const float* step_in, int8_t* xq, float* x_scale, void* y,
                                       sq_dtype ydt, void* stream);

/* sq_w8a8_linear_packed with a caller workspace that holds a second copy of
 * the activation codes in the fragment-packed layout (the weights' layout of
 * one 16-row block: 64-byte k-group c of token row m, inputs 64c + 16g ..
 * +15, at byte c * 1024 + (16 g + m) * 16), written by the quantiser beside
 * xq; the GEMM then reads each activation fragment as one contiguous
 * kilobyte rather than 16 row pieces K bytes apart.  Used at 13-16 tokens on
 * layers of at least 512 16-channel blocks (N > 8176) or of K >= 16384, where
 * the two-launch layer runs [P1 推論方法: per-token quantisation, then the
 * INT8 GEMM];
 * results identical to sq_w8a8_linear_packed (xq, x_scale and y).  Other
 * shapes run exactly as sq_w8a8_linear_packed and do not touch the
 * workspace.
 *
 * workspace: device memory owned by the caller, 16-byte aligned, at least
 * sq_linear_workspace_bytes(xdt, M, N, K) bytes (16 * K where the copy is
 * used, else 0; -1 for invalid arguments); no initial contents needed.
 * Calls that run at the same time must not share a workspace.  Errors:
 * SQ_ERR_WORKSPACE for a NULL, misaligned or too small workspace where one
 * is needed, SQ_ERR_ALIAS when it, xq, x_scale or y overlap one another or
 * an input; else as sq_w8a8_linear_packed. */
int64_t sq_linear_workspace_bytes(sq_dtype xdt, int64_t M, int64_t N, int64_t K);
sq_status sq_w8a8_linear_packed_ws(const void* x, sq_dtype xdt, int64_t M, int64_t K,
                                   const int8_t* wq_packed, const float* w_scale, int64_t N,
                                   int8_t* xq, float* x_scale, void* y, sq_dtype ydt,
                                   void* workspace, int64_t workspace_bytes, void* stream);

/* Library version string (static storage). */
const char* sq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SQ_H */
