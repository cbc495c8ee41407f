/*
 * ptq.h -- C ABI of the MI355X (gfx950) W8A8 post-training-quantized linear layer.
 *
 * The library runs the data-parallel hot path of a post-training-quantized
 * linear layer on one GPU:
 *
 *   sq_absmax_calib      column absmax calibration of activations / weights
 *   sq_smooth_factors    SmoothQuant smoothing factors s_j
 *   ssz_weight_qparams   MinMax + SSZ per-output-channel weight quantization
 *   ssz_weight_qparams_asym   the same with a per-channel offset (int8)
 *   quant_per_token_i8   per-token int8 activation quantization (with X/s)
 *   w8a8_gemm_dequant    int8 x int8 -> int32 GEMM, fused dequantization
 *   w8a8_gemm_fused      the same with bias, activation and fp32/bf16/int8 output
 *   sq_act_scale_ema     static per-tensor activation scale, moving-average range
 *   weight_scale_per_tensor   per-tensor (per-layer) weight scale
 *   quant_static_i8      int8 codes of a whole tensor with one static scale
 *
 * Conventions shared by every entry point:
 *   - Pointers are DEVICE pointers (hipMalloc'd or equivalent), owned by the
 *     caller; the library allocates no memory and keeps no state.  All
 *     matrices are dense row-major with the reduction dimension K contiguous
 *     (weights are [N = out, K = in]).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Each call checks
 *     its arguments on the host, then enqueues its kernels on `stream` and
 *     returns; it never synchronises.  Faults inside a kernel surface at the
 *     caller's next synchronisation.
 *   - The return value is a ptq_status.  On anything but PTQ_OK nothing was
 *     enqueued (except PTQ_ERR_HIP, which reports a failed launch), and
 *     ptq_last_error() returns a message for the calling thread.
 *   - Inputs must be finite; NaN or Inf inputs give unspecified results.
 *   - Rounding: fl32 denotes IEEE binary32 round-to-nearest-even.  A division
 *     R/S by a scale (or by a smoothing factor) is the IEEE quotient
 *     fl32(R / S); round() is round-half-to-even; symmetric codes saturate to
 *     [-qmax, qmax] (qmax = 127 for int8, 7 for int4), so the zero point is 0.
 *   - Folded values (x / s_j, w * s_j) must be finite as well.
 *
 * Sources, cited by page title and section:
 *   [PTQ]  tutorial chapter "4. 训练后量化（PTQ）" -- the four-step PTQ flow
 *          ("PTQ 的基本流程") and per-layer vs per-channel granularity
 *          ("逐层量化 vs 逐通道量化").
 *   [SSZ]  msModelSlim "SSZ：权重量化算法说明" -- flow ("算法流程"),
 *          initialisation ("初始化阶段"), iteration ("迭代优化阶段"),
 *          convergence ("收敛判断"), limits ("使用限制"), constants
 *          ("算法参数"), FAQ.
 *   [SQ]   "SmoothQuant大模型量化技术深度解析", section
 *          "一、SmoothQuant技术原理" (smoothing-factor formula).
 *   [INT8] CSDN article on CUDA INT8 quantized inference, sections 2.1
 *          (Q = round(R/S) + Z; range calibration; parameter computation;
 *          saturation), 2.2 (granularity), 3.1 (16-byte vector loads),
 *          3.2 (INT8 matrix multiply with integer accumulation), 4.2
 *          (quantize -> op -> dequantize fusion), 5.1 (overflow diagnosis).
 */
#ifndef PTQ_H
#define PTQ_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PTQ_ABI_VERSION 1

#if defined(__GNUC__) || defined(__clang__)
#define PTQ_API __attribute__((visibility("default")))
#else
#define PTQ_API
#endif

/* [SSZ] "算法参数": iteration limit, convergence threshold, minimum scale. */
#define PTQ_SSZ_MAX_ITER 20
#define PTQ_SSZ_THRESHOLD 1e-10
#define PTQ_SSZ_MIN_SCALE 1e-5f

/* Largest K (a multiple of 16) for which no int8 x int8 dot product can
 * overflow int32, whatever the codes -- (-128) * (-128) = 2^14 per term:
 * 2^14 K <= 2^31 - 1.  ([INT8] 5.1 overflow.) */
#define PTQ_GEMM_MAX_K 131056

/* Every K must be a multiple of this (16-byte vector rows, [INT8] 3.1). */
#define PTQ_K_MULTIPLE 16

typedef enum { PTQ_ACT_NONE = 0, PTQ_ACT_RELU = 1, PTQ_ACT_GELU = 2 } ptq_act;
typedef enum { PTQ_FOLD_DIV = 1, PTQ_FOLD_MUL = 2 } ptq_fold;
typedef enum { PTQ_OUT_F32 = 0, PTQ_OUT_BF16 = 1, PTQ_OUT_I8 = 2 } ptq_out;

typedef enum {
  PTQ_OK = 0,
  PTQ_ERR_NULL = 1,        /* a required pointer is NULL                      */
  PTQ_ERR_SHAPE = 2,       /* a size is <= 0, K not a multiple of 16, K too big */
  PTQ_ERR_DTYPE = 3,       /* unknown element type                            */
  PTQ_ERR_UNSUPPORTED = 4, /* bits not in {8, 4}, or symmetric == 0           */
  PTQ_ERR_ARG = 5,         /* alpha, max_iter, threshold or min_scale invalid */
  PTQ_ERR_ALIGN = 6,       /* a base pointer is not 16-byte aligned           */
  PTQ_ERR_HIP = 7          /* a kernel launch failed                          */
} ptq_status;

typedef enum {
  PTQ_F32 = 0, /* IEEE binary32 */
  PTQ_BF16 = 1 /* bfloat16 (upper half of a binary32), widened exactly */
} ptq_dtype;

/* ABI version of the loaded library (PTQ_ABI_VERSION). */
PTQ_API int ptq_abi_version(void);

/* Message for the last non-OK status returned on the calling thread. */
PTQ_API const char* ptq_last_error(void);

/* Static name of a status code. */
PTQ_API const char* ptq_status_string(int status);

/*
 * Column absmax calibration.  [SQ] max(|X_j|) per activation channel j over
 * the calibration data, and max(|W_j|) per input channel j of a weight (the
 * channel shared with X); [INT8] 2.1 range calibration from calibration
 * statistics.
 *
 *   x        [rows, cols] matrix of `dtype` (PTQ_F32 or PTQ_BF16), 16-B aligned
 *   rows     >= 1;  cols >= 1 and a multiple of 16
 *   amax     [cols] fp32, 16-B aligned.  accumulate == 0: amax[j] =
 *            max_i |x[i,j]|.  accumulate != 0: amax[j] = max(amax[j],
 *            max_i |x[i,j]|), a running maximum over calibration batches.
 * The result is exact (no rounding) and independent of launch order.
 */
PTQ_API ptq_status sq_absmax_calib(const void* x, int dtype, int64_t rows, int64_t cols, float* amax,
                           int accumulate, void* stream);

/*
 * SmoothQuant smoothing factors.  [SQ] s_j = max|X_j|^alpha / max|W_j|^(1-alpha),
 * alpha in [0,1].  Evaluated in fp64 and rounded once to fp32; a channel
 * whose activation or weight maximum is 0 gets s_j = 1.
 *
 *   act_amax, w_amax  [K] fp32 (from sq_absmax_calib), non-negative
 *   K                 >= 1
 *   alpha             in [0, 1] (NaN rejected)
 *   s                 [K] fp32 output
 */
PTQ_API ptq_status sq_smooth_factors(const float* act_amax, const float* w_amax, int64_t K, float alpha, float* s,
                             void* stream);

/*
 * Per-output-channel symmetric weight quantization: MinMax initial scale
 * refined by the SSZ least-squares scale search.  [SSZ] flow, init,
 * iteration, convergence, limits (int8 and int4, per-channel, symmetric, 2-D
 * weight), constants; [INT8] 2.1 quantization and saturation; [SQ] the
 * weight side of the smoothing fold.
 *
 * For each row n (output channel), with w_hat[k] = fl32(w[n,k] * s[k])
 * (w_hat = w when s is NULL):
 *   S = max(fl32(max_k |w_hat[k]| / qmax), min_scale);  q = quant(S);  best = mse(S)
 *   repeat up to max_iter times (the row stops on its own):
 *     if sum q^2 == 0: stop
 *     S' = max(fl32(A / sum(q^2)), min_scale);  cur = mse(S')
 *     converged = best == 0 || (best - cur)/best < threshold || |best - cur| < threshold
 *     if cur < best: S = S', q = quant(S'), best = cur
 *     if converged: stop
 * quant(S)[k] = clamp(rne(fl32(w_hat[k] / S)), -qmax, qmax);
 * A = sum_k w_hat[k] q[k], and mse(S) = E / K with E = sum_k (w_hat[k] - S q[k])^2,
 * where A and E are the exact sums rounded once to fp64 (the division by K in
 * fp64); every comparison and quotient above is fp64.
 *
 *   w          [N, K] of `dtype`, 16-B aligned;  N >= 1;  K multiple of 16, <= 131072
 *   s          [K] fp32 smoothing factors, or NULL for no smoothing
 *   bits       8 or 4;  symmetric must be 1 (asymmetric int8: ssz_weight_qparams_asym;
 *              symmetric = 0 here returns PTQ_ERR_UNSUPPORTED)
 *   max_iter   0..20 (PTQ_SSZ_MAX_ITER; 0 = MinMax only)
 *   threshold  >= 0 (PTQ_SSZ_THRESHOLD);  min_scale > 0 (PTQ_SSZ_MIN_SCALE)
 *   scale      [N] fp32 output: S per output channel
 *   wq         output codes, or NULL: bits 8 -> [N, K] int8;  bits 4 ->
 *              [N, K/2] bytes, byte i of a row = element 2i in the low nibble,
 *              element 2i+1 in the high nibble, two's complement.  16-B aligned.
 *   iters      [N] int32 output (least-squares steps entered), or NULL
 *   mse        [N] fp64 output (final mean squared error), or NULL
 */
PTQ_API ptq_status ssz_weight_qparams(const void* w, int dtype, int64_t N, int64_t K, const float* s, int bits,
                              int symmetric, int max_iter, double threshold, float min_scale, float* scale,
                              void* wq, int32_t* iters, double* mse, void* stream);

/*
 * Per-output-channel ASYMMETRIC int8 weight quantization: MinMax initial
 * scale and offset refined by the SSZ least-squares search over both.
 * [SSZ] asymmetric mode (scale and offset optimised together; int8 only, as
 * the method's limits exclude int4 asymmetric), flow, convergence and
 * constants as for ssz_weight_qparams; [INT8] 2.1 Q = round(R/S) + Z with
 * saturation.
 *
 * For each row n, with w_hat as above:
 *   quant(S, Z)[k] = clamp(rne(fl32(w_hat[k] / S)) + Z, -128, 127)
 *   mse(S, Z)      = mean_k (w_hat[k] - S (q[k] - Z))^2 (the exact sum rounded
 *                    once to fp64, divided by K in fp64)
 *   init: lo = min_k w_hat[k], hi = max_k w_hat[k];
 *         S = max(fl32(fl32(hi - lo) / 255), min_scale);
 *         Z = clamp(-128 - rne(fl32(lo / S)), -128, 127)
 *   step: for the offset-relative codes r = q - Z of the current (S, Z), the
 *         least-squares line w_hat ~ a r + b (2x2 normal equations;
 *         det = K sum r^2 - (sum r)^2, det == 0 stops the row; sum w_hat r and
 *         sum w_hat the exact sums rounded once to fp64;
 *         a = (K sum w_hat r - sum w_hat sum r) / det, b = (sum w_hat - a sum r) / K);
 *         S' = max(fl32(a), min_scale), Z' = clamp(Z - rne(b / a), -128, 127)
 *         (fp64 quotient);  kept only if mse(S', Z') < best;  convergence,
 *         iteration limit and per-row stop exactly as in ssz_weight_qparams.
 * Dequantized weight: S (q - Z).
 *
 *   w, s, N, K, max_iter, threshold, min_scale   as for ssz_weight_qparams
 *   scale       [N] fp32 output
 *   zero_point  [N] int32 output, in [-128, 127]
 *   wq          [N, K] int8 output codes in [-128, 127], 16-B aligned, or NULL
 *   iters, mse  [N] int32 / fp64 outputs, or NULL
 */
PTQ_API ptq_status ssz_weight_qparams_asym(const void* w, int dtype, int64_t N, int64_t K, const float* s,
                                           int max_iter, double threshold, float min_scale, float* scale,
                                           int32_t* zero_point, int8_t* wq, int32_t* iters, double* mse,
                                           void* stream);

/*
 * Per-token dynamic int8 activation quantization with the smoothing fold.
 * [SQ] the activation side of the fold (X diag(s)^-1) and the reason the
 * activation scale varies per token rather than per channel; [INT8] 2.1.
 *
 * For each token row t, with x_hat[j] = fl32(x[t,j] / s[j]) (x_hat = x
 * when s is NULL):
 *   a = max_j |x_hat[j]|;  tok_scale[t] = a > 0 ? fl32(a / 127) : 1
 *   xq[t,j] = clamp(rne(fl32(x_hat[j] / tok_scale[t])), -127, 127)
 *
 *   x          [T, K] of `dtype`, 16-B aligned;  T >= 1;  K multiple of 16, <= 131072
 *   s          [K] fp32 smoothing factors, or NULL
 *   xq         [T, K] int8 output, 16-B aligned
 *   tok_scale  [T] fp32 output
 */
PTQ_API ptq_status quant_per_token_i8(const void* x, int dtype, int64_t T, int64_t K, const float* s, int8_t* xq,
                              float* tok_scale, void* stream);

/*
 * Integer GEMM with fused dequantization.  [INT8] 3.2 (int8 operands, both
 * K-contiguous, integer accumulation), 4.2 (dequantization fused into the
 * producing kernel), 5.1 (int32 overflow); dequantization inverts
 * Q = round(R/S) with zero points 0.
 *
 *   acc[t,n] = sum_k xq[t,k] * wq[n,k]             (exact int32)
 *   y[t,n]   = fl32(fl32(acc[t,n]) * fl32(tok_scale[t] * ch_scale[n]))
 *
 *   xq         [M, K] int8, 16-B aligned;  wq [N, K] int8, 16-B aligned
 *   tok_scale  [M] fp32;  ch_scale [N] fp32
 *   M, N       >= 1;  K multiple of 16 and <= PTQ_GEMM_MAX_K
 *   y          [M, N] fp32 output, 16-B aligned
 *   acc        [M, N] int32 output of the raw sums, or NULL (diagnosis, [INT8] 5.1)
 */
PTQ_API ptq_status w8a8_gemm_dequant(const int8_t* xq, const int8_t* wq, const float* tok_scale, const float* ch_scale,
                             int64_t M, int64_t N, int64_t K, float* y, int32_t* acc, void* stream);

/*
 * The GEMM of w8a8_gemm_dequant with a fused epilogue: bias, activation and
 * the output format the next layer consumes.  [INT8] 4.2 (quantize -> op ->
 * dequantize -> activation fused into one kernel), [INT8] 2.1 (the int8
 * output's quantization and saturation), [SQ] (the next layer's fold).
 *
 * In fp32, each operation rounded, for every output element (t, n):
 *   v = fl32(acc) * fl32(tok_scale[t] * ch_scale[n])      (as w8a8_gemm_dequant)
 *   v = v + bias[n]                                       (bias may be NULL)
 *   act PTQ_ACT_RELU: v = v > 0 ? v : +0
 *       PTQ_ACT_GELU: v = 0.5 v (1 + erf(v / sqrt 2))     (erf from the erfc fit of
 *                     Numerical Recipes 2nd ed. section 6.2, relative error < 1.2e-7:
 *                     within about an ulp of the correctly rounded erf)
 *   out_type PTQ_OUT_F32:  out[t,n] = v                     float  [M, N]
 *            PTQ_OUT_BF16: out[t,n] = bf16 RNE of v         uint16 [M, N]
 *            PTQ_OUT_I8:   x = next_s ? fl32(v / next_s[n]) : v;
 *                          out[t,n] = clamp(rne(fl32(x / out_scale[0])), -127, 127)   int8 [M, N]
 *              -- the next layer's static per-tensor activation quantization
 *              (see sq_act_scale_ema) with its smoothing fold; its token
 *              scales are then out_scale[0] for every row.
 *
 *   bias       [N] fp32 or NULL
 *   act        PTQ_ACT_NONE / RELU / GELU (else PTQ_ERR_UNSUPPORTED)
 *   out_type   PTQ_OUT_F32 / BF16 / I8 (else PTQ_ERR_DTYPE)
 *   next_s     [N] fp32 or NULL; int8 output only (else PTQ_ERR_ARG)
 *   out_scale  [1] fp32 device scalar > 0, required for the int8 output only
 *   out        16-B aligned;  acc as in w8a8_gemm_dequant (may be NULL)
 */
PTQ_API ptq_status w8a8_gemm_fused(const int8_t* xq, const int8_t* wq, const float* tok_scale, const float* ch_scale,
                                   const float* bias, int act, int out_type, const float* next_s,
                                   const float* out_scale, int64_t M, int64_t N, int64_t K, void* out, int32_t* acc,
                                   void* stream);

/*
 * Static per-tensor activation scale from a moving average of the
 * activation range.  [INT8] 2.1 (tracking the range with a moving average is
 * more robust than the raw min/max), [QAT] 六 (activation quantizer type
 * moving_average_abs_max), [SQ] (the quantized tensor is the smoothed one).
 *
 * Per calibration batch: col_amax = sq_absmax_calib of the batch (not
 * accumulated), then this call:
 *   a     = max_j fl32(col_amax[j] / s[j])      (max |x_hat| of the batch; s may be NULL)
 *   state = first ? a : fl32(fl32(momentum * state) + fl32(fl32(1 - momentum) * a))
 *   scale = state > 0 ? fl32(state / 127) : 1
 * The pages give no momentum: it is the caller's parameter, in [0, 1).
 *
 *   col_amax   [K] fp32 (device)      state  [1] fp32 in/out (device)
 *   scale      [1] fp32 output        row_scale [rows] fp32 output filled with scale, or NULL
 */
PTQ_API ptq_status sq_act_scale_ema(const float* col_amax, const float* s, int64_t K, float momentum, int first,
                                    float* state, float* scale, float* row_scale, int64_t rows, void* stream);

/*
 * Per-tensor (per-layer) weight scale: one scale for the whole weight
 * ([PTQ] 逐层量化 vs 逐通道量化; the MinMax rule of the per-channel path on
 * the whole tensor -- the SSZ search is per-channel only, [SSZ] 使用限制):
 *   a = max_j fl32(col_amax[j] * s[j]);  scale = max(fl32(a / 127), min_scale)
 * with col_amax = sq_absmax_calib of the weight; ch_scale [N] (or NULL)
 * receives the same value for every output channel (what the GEMM reads).
 */
PTQ_API ptq_status weight_scale_per_tensor(const float* col_amax, const float* s, int64_t K, float min_scale,
                                           float* scale, float* ch_scale, int64_t N, void* stream);

/*
 * Int8 codes of a whole [rows, cols] tensor with one static scale (scale[0],
 * device): the static per-tensor activation quantization (fold =
 * PTQ_FOLD_DIV: x_hat = fl32(x / s_j)) or the per-tensor weight
 * quantization (fold = PTQ_FOLD_MUL: w_hat = fl32(w * s_j)); s may be NULL
 * (no fold, fold ignored).  [INT8] 2.1.
 *   q[r, j] = clamp(rne(fl32(x_hat[r, j] / scale[0])), -127, 127)
 *   row_scale [rows] fp32 output filled with scale[0] (the GEMM's token scales), or NULL
 * Shapes, dtypes and alignment as quant_per_token_i8.
 */
PTQ_API ptq_status quant_static_i8(const void* x, int dtype, int64_t rows, int64_t cols, const float* s, int fold,
                                   const float* scale, int8_t* q, float* row_scale, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PTQ_H */
