/*
 * ptq_oracle.c -- the CPU oracle of the W8A8 post-training-quantized linear layer.
 *
 * TEST INFRASTRUCTURE ONLY.  This is a plain, slow, scalar implementation
 * that the GPU path is checked against.  Only the tests, the smoke check and
 * the bench's CPU-baseline leg may load it; the product path never does.  It
 * shares no code, header, table or helper with the HIP library.
 *
 * Sources (the pages):
 *   [PTQ]  tutorial chapter "4. 训练后量化（PTQ）": the four-step flow
 *          ("PTQ 的基本流程") and per-layer vs per-channel granularity
 *          ("逐层量化 vs 逐通道量化").
 *   [SSZ]  msModelSlim document "SSZ：权重量化算法说明": algorithm flow
 *          ("算法流程"), initialisation ("初始化阶段"), iteration
 *          ("迭代优化阶段"), convergence ("收敛判断"), limits ("使用限制"),
 *          constants ("算法参数").
 *   [SQ]   article "SmoothQuant大模型量化技术深度解析", section
 *          "一、SmoothQuant技术原理": the smoothing factor s_j and the
 *          equivalent rescaling of activations and weights.
 *   [INT8] CSDN article on CUDA INT8 inference: section 2.1 (linear
 *          quantization Q = round(R/S) + Z, range calibration, parameter
 *          computation, saturation), 2.2 (granularity), 3.2 (INT8 GEMM with
 *          integer accumulation), 4.2 (quantize -> op -> dequantize fusion).
 *
 * Arithmetic conventions (the pages fix no precision; these readings are the
 * oracle's definition and the GPU path must reproduce them):
 *   - fl32(.) is IEEE binary32 round-to-nearest-even.  This file is compiled
 *     with -O2 -fno-fast-math -ffp-contract=off so no product is fused into a
 *     following add and float expressions stay in float.
 *   - R / S is the IEEE binary32 quotient fl32(R / S), the plain reading of
 *     [INT8] 2.1's Q = round(R/S) + Z; the activation fold X / s_j is the
 *     quotient fl32(X / s_j) likewise.
 *   - round() is round-half-to-even (nearbyintf under the default rounding
 *     mode), then saturation to [-qmax, qmax], qmax = 127 (int8) or 7 (int4);
 *     symmetric, so the zero point Z is 0.
 *   - the SSZ sums -- the quantization error sum (w_hat - S q)^2 and the
 *     least-squares sums sum w_hat q, sum w_hat -- are the exact real sums
 *     rounded once to fp64 (accumulated in binary128, whose 113-bit
 *     significand holds every product exactly; the fp64 result can differ from
 *     the correctly rounded exact sum only when that sum lies within about
 *     K * 2^-113 of it, relatively, of an fp64 rounding boundary).  The value
 *     is therefore independent of any summation order.
 *
 * Every function takes host pointers to row-major, K-contiguous arrays and
 * returns 0 on success, a negative value on a bad argument or a non-finite
 * input.
 */
#include <math.h>
#include <omp.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define O_OK 0
#define O_EARG -1
#define O_ENONFINITE -2
#define O_EOVERFLOW -3

/* Number of threads the OpenMP loops below use (reported by the CPU baseline). */
int o_num_threads(void) { return omp_get_max_threads(); }

static int all_finite(const float* a, int64_t n) {
  for (int64_t i = 0; i < n; ++i)
    if (!isfinite(a[i])) return 0;
  return 1;
}

/* ---------------------------------------------------------------------------
 * Range calibration: column-wise absolute maximum.
 * [SQ] max(|X_j|) over the calibration activations of channel j, and
 * max(|W_j|) over input channel j of the weight (the channel shared with X,
 * which is the only choice that keeps the rescaling equivalent).  [INT8] 2.1:
 * the dynamic range comes from statistics over a calibration set.  Several
 * calibration batches fold in as a running maximum (accumulate != 0).
 * ------------------------------------------------------------------------- */
int o_absmax_cols(const float* x, int64_t rows, int64_t cols, float* amax, int accumulate) {
  if (!x || !amax || rows < 0 || cols <= 0) return O_EARG;
  if (!all_finite(x, rows * cols)) return O_ENONFINITE;
  if (!accumulate)
    for (int64_t j = 0; j < cols; ++j) amax[j] = 0.0f;
  for (int64_t i = 0; i < rows; ++i)
    for (int64_t j = 0; j < cols; ++j) {
      float a = fabsf(x[i * cols + j]);
      if (a > amax[j]) amax[j] = a;
    }
  return O_OK;
}

/* ---------------------------------------------------------------------------
 * Smoothing factor.  [SQ] s_j = max|X_j|^alpha / max|W_j|^(1-alpha),
 * alpha in [0,1].  Evaluated in fp64 and rounded once to fp32.  A channel
 * whose activation or weight maximum is 0 gets s_j = 1 (no smoothing; the
 * pages do not cover it).
 * ------------------------------------------------------------------------- */
int o_smooth_factors(const float* ax, const float* aw, int64_t K, float alpha, float* s) {
  if (!ax || !aw || !s || K <= 0) return O_EARG;
  if (!(alpha >= 0.0f && alpha <= 1.0f)) return O_EARG;
  double a = (double)alpha;
  for (int64_t j = 0; j < K; ++j) {
    if (ax[j] == 0.0f || aw[j] == 0.0f) {
      s[j] = 1.0f;
      continue;
    }
    double v = pow((double)ax[j], a) / pow((double)aw[j], 1.0 - a);
    s[j] = (float)v;
  }
  return O_OK;
}

/* ---------------------------------------------------------------------------
 * Folding the smoothing into the operands.  [SQ] the activations of channel j
 * are divided by s_j and the weights of input channel j multiplied by s_j, so
 * (X diag(s)^-1)(diag(s) W^T) = X W^T.
 *   w_hat[n,j] = fl32(W[n,j] * s_j)
 *   x_hat[t,j] = fl32(X[t,j] / s_j)
 * With s == NULL both are the identity.
 * ------------------------------------------------------------------------- */
int o_fold_weight(const float* w, const float* s, int64_t N, int64_t K, float* wh) {
  if (!w || !wh || N < 0 || K <= 0) return O_EARG;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t j = 0; j < K; ++j) wh[n * K + j] = s ? w[n * K + j] * s[j] : w[n * K + j];
  return O_OK;
}

int o_fold_act(const float* x, const float* s, int64_t T, int64_t K, float* xh) {
  if (!x || !xh || T < 0 || K <= 0) return O_EARG;
  for (int64_t t = 0; t < T; ++t)
    for (int64_t j = 0; j < K; ++j) {
      if (s) {
        xh[t * K + j] = x[t * K + j] / s[j];
      } else {
        xh[t * K + j] = x[t * K + j];
      }
    }
  return O_OK;
}

/* Whether every folded value (x * s_j with mul, x / s_j without; x itself when s is NULL) is finite: the path
 * requires it (a folded value that overflows has no code), and the quantizers below refuse such input with
 * O_ENONFINITE instead of coding it. */
static int fold_finite(const float* x, const float* s, int64_t rows, int64_t cols, int mul) {
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t j = 0; j < cols; ++j) {
      const float v = x[r * cols + j];
      const float f = !s ? v : (mul ? v * s[j] : v / s[j]);
      if (!isfinite(f)) return 0;
    }
  return 1;
}

/* ---------------------------------------------------------------------------
 * Linear quantization, symmetric.  [INT8] 2.1: Q = round(R/S) + Z followed by
 * saturation to the representable range; Z = 0 for symmetric quantization
 * ([SSZ] iteration stage: symmetric keeps the offset at 0).
 *   code = clamp(rne(fl32(R / S)), -qmax, qmax)
 * ------------------------------------------------------------------------- */
static int code_of(float r, float S, int qmax) {
  float t = r / S;
  float q = nearbyintf(t);
  if (q > (float)qmax) q = (float)qmax;
  if (q < (float)-qmax) q = (float)-qmax;
  return (int)q;
}

int o_quant_row(const float* r, int64_t K, float S, int qmax, int8_t* q) {
  if (!r || !q || K <= 0 || !(S > 0.0f) || qmax <= 0 || qmax > 127) return O_EARG;
  if (!all_finite(r, K)) return O_ENONFINITE;
  for (int64_t k = 0; k < K; ++k) q[k] = (int8_t)code_of(r[k], S, qmax);
  return O_OK;
}

/* Exact sums, rounded once to fp64 (binary128 accumulation; see the header).
 *   sq_err_exact: sum_k (w_hat_k - S (q_k - z))^2
 *   dot_exact:    sum_k w_hat_k (q_k - z)
 *   sum_exact:    sum_k w_hat_k */
static double sq_err_exact(const float* wh, const int8_t* q, int64_t K, float S, int z) {
  __float128 acc = 0;
  for (int64_t k = 0; k < K; ++k) {
    __float128 d = (__float128)wh[k] - (__float128)S * (__float128)((int)q[k] - z);
    acc += d * d;
  }
  return (double)acc;
}

static double dot_exact(const float* wh, const int8_t* q, int64_t K, int z) {
  __float128 acc = 0;
  for (int64_t k = 0; k < K; ++k) acc += (__float128)wh[k] * (__float128)((int)q[k] - z);
  return (double)acc;
}

static double sum_exact(const float* wh, int64_t K) {
  __float128 acc = 0;
  for (int64_t k = 0; k < K; ++k) acc += (__float128)wh[k];
  return (double)acc;
}

/* Quantization error of one channel: the mean of (w_hat - S*q)^2 over its K
 * elements -- the exact sum rounded to fp64, then divided by K in fp64.
 * ([SSZ] compares "quantization error"; the mean is this oracle's reading.) */
double o_mse_row(const float* wh, const int8_t* q, int64_t K, float S) {
  return sq_err_exact(wh, q, K, S, 0) / (double)K;
}

/* Least-squares scale for fixed codes: argmin_S sum (w_hat - S q)^2 =
 * sum(w_hat q) / sum(q^2), the numerator the exact sum rounded to fp64.
 * Returns the fp64 quotient, or 0 when sum(q^2)=0.
 * ([SSZ] each iteration fits the scale by least squares.) */
double o_lsq_scale(const float* wh, const int8_t* q, int64_t K) {
  int64_t B = 0;
  for (int64_t k = 0; k < K; ++k) B += (int64_t)q[k] * (int64_t)q[k];
  return B == 0 ? 0.0 : dot_exact(wh, q, K, 0) / (double)B;
}

/* ---------------------------------------------------------------------------
 * SSZ, symmetric per-channel, one row (= one output channel).
 *
 * [SSZ] flow: MinMax initial parameters; least-squares update; keep the new
 * parameters only if the quantization error improves; repeat until converged
 * or the iteration limit; symmetric keeps offset 0 and optimises the scale
 * only.  Constants: at most 20 iterations, convergence threshold 1e-10,
 * minimum scale 1e-5 (passed in).  Convergence: relative change
 * (best - cur)/best < thr or absolute change |best - cur| < thr.
 *
 * Readings taken where the document is silent:
 *   - MinMax init: S0 = max(fl32(max_k |w_hat_k| / qmax), fl32(min_scale)).
 *   - each least-squares step refits S for the codes of the current S:
 *     S' = max(fl32(A/B), fl32(min_scale)), A = sum w_hat q (the exact sum
 *     rounded to fp64), B = sum q^2 (exact); B == 0 leaves nothing to fit
 *     and ends the row.
 *   - errors are o_mse_row's (exact sums, rounded once).
 *   - a candidate is kept only if strictly better (cur < best).
 *   - either convergence test ends the row; d = best - cur is signed, so a
 *     rejected candidate (d <= 0) also ends it (the next step would rebuild
 *     the same candidate).  best == 0 counts as converged.
 *   - each row stops on its own ("all channels converged" then ends the
 *     whole search).
 *   - iters = number of least-squares steps entered (0 when max_iter = 0).
 * hist (may be NULL) receives best after the init (index 0) and after each
 * step entered (index i); entries after the last step are left untouched.
 * ------------------------------------------------------------------------- */
static void ssz_one_row(const float* wh, int64_t K, int qmax, int max_iter, double thr, float min_scale,
                        float* S_out, int8_t* q, int32_t* iters_out, double* mse_out, double* hist,
                        int8_t* qc) {
  float m = 0.0f;
  for (int64_t k = 0; k < K; ++k) {
    float a = fabsf(wh[k]);
    if (a > m) m = a;
  }
  float S = m / (float)qmax;
  if (S < min_scale) S = min_scale;
  o_quant_row(wh, K, S, qmax, q);
  double best = o_mse_row(wh, q, K, S);
  if (hist) hist[0] = best;

  double A = dot_exact(wh, q, K, 0);
  int64_t B = 0;
  for (int64_t k = 0; k < K; ++k) B += (int64_t)q[k] * (int64_t)q[k];

  int it = 0;
  for (int i = 1; i <= max_iter; ++i) {
    it = i;
    if (B == 0) break;
    float Sc = (float)(A / (double)B);
    if (Sc < min_scale) Sc = min_scale;
    o_quant_row(wh, K, Sc, qmax, qc);
    double cur = o_mse_row(wh, qc, K, Sc);
    double d = best - cur;
    int conv = (best == 0.0) || (d / best < thr) || (fabs(d) < thr);
    if (cur < best) {
      S = Sc;
      best = cur;
      memcpy(q, qc, (size_t)K);
      A = dot_exact(wh, q, K, 0);
      B = 0;
      for (int64_t k = 0; k < K; ++k) B += (int64_t)q[k] * (int64_t)q[k];
    }
    if (hist) hist[i] = best;
    if (conv) break;
  }
  *S_out = S;
  if (iters_out) *iters_out = it;
  if (mse_out) *mse_out = best;
}

/*
 * Weight quantization parameters for a [N,K] weight: fold s (may be NULL),
 * then MinMax + SSZ per row.  bits 8 -> qmax 127, bits 4 -> qmax 7 ([SSZ]
 * limits: int8 and int4, per-channel, symmetric; the weight is 2-D).
 * Outputs: S[N], q[N,K] codes (one code per byte), iters[N], mse[N] (any of
 * iters/mse/hist may be NULL); hist is [N, max_iter+1].
 */
int o_ssz(const float* w, const float* s, int64_t N, int64_t K, int bits, int max_iter, double thr,
          float min_scale, float* S, int8_t* q, int32_t* iters, double* mse, double* hist) {
  if (!w || !S || !q || N < 0 || K <= 0) return O_EARG;
  if (bits != 8 && bits != 4) return O_EARG;
  if (max_iter < 0 || !(thr >= 0.0) || !(min_scale > 0.0f)) return O_EARG;
  if (!all_finite(w, N * K)) return O_ENONFINITE;
  if (!fold_finite(w, s, N, K, 1)) return O_ENONFINITE;
  const int qmax = bits == 8 ? 127 : 7;
  int bad = 0;
#pragma omp parallel
  {
    float* wh = (float*)malloc(sizeof(float) * (size_t)K);
    int8_t* qc = (int8_t*)malloc((size_t)K);
    if (!wh || !qc) {
#pragma omp atomic write
      bad = 1;
    } else {
#pragma omp for schedule(dynamic, 16)
      for (int64_t n = 0; n < N; ++n) {
        o_fold_weight(w + n * K, s, 1, K, wh);
        ssz_one_row(wh, K, qmax, max_iter, thr, min_scale, S + n, q + n * K, iters ? iters + n : NULL,
                    mse ? mse + n : NULL, hist ? hist + n * (int64_t)(max_iter + 1) : NULL, qc);
      }
    }
    free(wh);
    free(qc);
  }
  return bad ? O_EARG : O_OK;
}

/* ---------------------------------------------------------------------------
 * Diagnostic: the symmetric SSZ search under the other readings of the
 * silent points, to measure how much each reading matters (never used for
 * parity; o_ssz above is the reading the kernels follow).
 *   conv_and    -- a row converges only when BOTH the relative and the
 *                  absolute change are under the threshold ([SSZ] lists the
 *                  two tests without saying how they combine).
 *   err_sum     -- the error is the channel's SUM of squared differences
 *                  instead of its mean (the relative test is unchanged, the
 *                  absolute one sees K times larger changes).
 *   global_loop -- rows do not stop on their own: every row keeps taking
 *                  steps until all rows have converged at least once, or the
 *                  iteration limit ("exit when all channels have converged").
 * Each candidate is still kept only if strictly better.  Outputs S[N],
 * iters[N] (steps whose candidate the row evaluated) and mse[N] (the mean
 * squared error of the final scale, whatever the reading; may be NULL).
 * ------------------------------------------------------------------------- */
int o_ssz_variant(const float* w, const float* s, int64_t N, int64_t K, int bits, int max_iter, double thr,
                  float min_scale, int conv_and, int err_sum, int global_loop, float* S, int32_t* iters,
                  double* mse) {
  if (!w || !S || !iters || N < 0 || K <= 0) return O_EARG;
  if (bits != 8 && bits != 4) return O_EARG;
  if (max_iter < 0 || !(thr >= 0.0) || !(min_scale > 0.0f)) return O_EARG;
  if (!all_finite(w, N * K)) return O_ENONFINITE;
  if (!fold_finite(w, s, N, K, 1)) return O_ENONFINITE;
  const int qmax = bits == 8 ? 127 : 7;
  const double scale = err_sum ? (double)K : 1.0;  /* mean -> sum */
  float* wh = (float*)malloc(sizeof(float) * (size_t)(N * K));
  int8_t* q = (int8_t*)malloc((size_t)K);
  double* best = (double*)malloc(sizeof(double) * (size_t)N);
  double* A = (double*)malloc(sizeof(double) * (size_t)N);
  int64_t* B = (int64_t*)malloc(sizeof(int64_t) * (size_t)N);
  char* done = (char*)malloc((size_t)N);
  if (!wh || !q || !best || !A || !B || !done) {
    free(wh); free(q); free(best); free(A); free(B); free(done);
    return O_EARG;
  }
  o_fold_weight(w, s, N, K, wh);
  for (int64_t n = 0; n < N; ++n) {
    const float* r = wh + n * K;
    float m = 0.0f;
    for (int64_t k = 0; k < K; ++k) m = fabsf(r[k]) > m ? fabsf(r[k]) : m;
    float S0 = m / (float)qmax;
    S[n] = S0 < min_scale ? min_scale : S0;
    o_quant_row(r, K, S[n], qmax, q);
    best[n] = o_mse_row(r, q, K, S[n]) * scale;
    A[n] = dot_exact(r, q, K, 0);
    B[n] = 0;
    for (int64_t k = 0; k < K; ++k) B[n] += (int64_t)q[k] * (int64_t)q[k];
    iters[n] = 0;
    done[n] = 0;
  }
  for (int i = 1; i <= max_iter; ++i) {
    int64_t active = 0;
    for (int64_t n = 0; n < N; ++n) {
      if (!global_loop && done[n]) continue;
      const float* r = wh + n * K;
      if (B[n] == 0) {  /* nothing to fit: the row is converged and never changes */
        if (!done[n]) iters[n] = i;
        done[n] = 1;
        continue;
      }
      float Sc = (float)(A[n] / (double)B[n]);
      if (Sc < min_scale) Sc = min_scale;
      o_quant_row(r, K, Sc, qmax, q);
      const double cur = o_mse_row(r, q, K, Sc) * scale;
      const double d = best[n] - cur;
      const int rel = best[n] == 0.0 || d / best[n] < thr, ab = fabs(d) < thr;
      const int conv = best[n] == 0.0 || (conv_and ? (rel && ab) : (rel || ab));
      iters[n] = i;
      if (cur < best[n]) {
        S[n] = Sc;
        best[n] = cur;
        A[n] = dot_exact(r, q, K, 0);
        B[n] = 0;
        for (int64_t k = 0; k < K; ++k) B[n] += (int64_t)q[k] * (int64_t)q[k];
      }
      if (conv) done[n] = 1;
    }
    for (int64_t n = 0; n < N; ++n) active += !done[n];
    if (active == 0) break;
  }
  if (mse)
    for (int64_t n = 0; n < N; ++n) mse[n] = best[n] / scale;
  free(wh); free(q); free(best); free(A); free(B); free(done);
  return O_OK;
}

/* ---------------------------------------------------------------------------
 * Asymmetric linear quantization, int8.  [INT8] 2.1: Q = round(R/S) + Z with
 * saturation; the SSZ document's asymmetric mode lets the offset move
 * ([SSZ] iteration stage; "symmetric: false" in the option table) and
 * supports it for int8 only ([SSZ] limits: no int4 asymmetric).
 *   code = clamp(rne(fl32(R / S)) + Z, -128, 127),  Z an integer,
 *   dequantized value S * (code - Z).
 * Readings: the full two's-complement range [-128, 127] (256 levels); Z is
 * an integer in that range.
 * ------------------------------------------------------------------------- */
#define O_QMIN_ASYM (-128)
#define O_QMAX_ASYM 127

static int code_asym(float r, float S, int z) {
  float t = nearbyintf(r / S);
  /* saturate (in floating point) before converting and adding Z, so that a quotient beyond the int range
   * still lands on its own end of the code range */
  if (t > 1000.0f) t = 1000.0f;
  if (t < -1000.0f) t = -1000.0f;
  int q = (int)t + z;
  if (q > O_QMAX_ASYM) q = O_QMAX_ASYM;
  if (q < O_QMIN_ASYM) q = O_QMIN_ASYM;
  return q;
}

int o_quant_row_asym(const float* r, int64_t K, float S, int Z, int8_t* q) {
  if (!r || !q || K <= 0 || !(S > 0.0f) || Z < O_QMIN_ASYM || Z > O_QMAX_ASYM) return O_EARG;
  if (!all_finite(r, K)) return O_ENONFINITE;
  for (int64_t k = 0; k < K; ++k) q[k] = (int8_t)code_asym(r[k], S, Z);
  return O_OK;
}

/* mean of (w_hat - S*(q - Z))^2: the exact sum rounded to fp64, divided by K in fp64 */
double o_mse_row_asym(const float* wh, const int8_t* q, int64_t K, float S, int Z) {
  return sq_err_exact(wh, q, K, S, Z) / (double)K;
}

/* Least squares over scale and offset for fixed codes.  The dequantized weight
 * is S (q - Z), so the fit is taken in the offset-relative codes r = q - Z:
 * the line w ~ a*r + b that minimises sum (w_hat - a r - b)^2, from its 2x2
 * normal equations
 *   [sum r^2  sum r] [a]   [sum w r]
 *   [sum r    K    ] [b] = [sum w  ]
 * solved as a = (K sum wr - sum w sum r) / det, b = (sum w - a sum r) / K,
 * det = K sum r^2 - (sum r)^2 (exact integers; sum w r and sum w are the
 * exact sums rounded to fp64; each fp64 operation in the order written).
 * a is the scale of the fitted line and b its intercept, so the refit
 * parameters are S' = a and Z' = Z - b/a (rounded; see ssz_asym_one_row).
 * ([SSZ] asymmetric mode fits scale and offset together by least squares.)
 * Returns 1 and a, b when det > 0; 0 when all codes are equal (nothing to fit). */
int o_lsq_affine(const float* wh, const int8_t* q, int64_t K, int Z, double* a, double* b) {
  int64_t sr = 0, srr = 0;
  for (int64_t k = 0; k < K; ++k) {
    int64_t r = (int64_t)q[k] - Z;
    sr += r;
    srr += r * r;
  }
  int64_t det = K * srr - sr * sr;
  if (det <= 0) return 0;
  double sw = sum_exact(wh, K), swr = dot_exact(wh, q, K, Z);
  double aa = ((double)K * swr - sw * (double)sr) / (double)det;
  *a = aa;
  *b = (sw - aa * (double)sr) / (double)K;
  return 1;
}

/* ---------------------------------------------------------------------------
 * SSZ, asymmetric per-channel int8, one row.  Same flow, constants, greedy
 * rule and convergence tests as the symmetric search above; the parameters
 * are the pair (S, Z) ([SSZ] asymmetric: scale and offset optimised
 * together).
 *
 * Readings taken where the document is silent:
 *   - MinMax init from the channel's min lo and max hi:
 *       S0 = max(fl32(fl32(hi - lo) / 255), fl32(min_scale)),
 *       Z0 = clamp(-128 - rne(fl32(lo / S0)), -128, 127),
 *     which maps lo to -128 and hi to (about) 127.
 *   - each least-squares step fits the line w ~ a r + b to the offset-relative
 *     codes r = q - Z of the current (S, Z) (o_lsq_affine) and converts it to
 *     parameters:
 *       S' = max(fl32(a), fl32(min_scale)),
 *       Z' = clamp(Z - rne(b / a), -128, 127)   (fp64 quotient, ties to even),
 *     since a r + b = a (q - (Z - b/a)).  All codes equal (det = 0) leaves
 *     nothing to fit and ends the row.
 *   - the candidate's error is computed with its own codes; kept only if
 *     strictly better; iters, convergence and hist as in the symmetric case.
 * ------------------------------------------------------------------------- */
static void ssz_asym_one_row(const float* wh, int64_t K, int max_iter, double thr, float min_scale, float* S_out,
                             int32_t* Z_out, int8_t* q, int32_t* iters_out, double* mse_out, double* hist,
                             int8_t* qc) {
  float lo = wh[0], hi = wh[0];
  for (int64_t k = 1; k < K; ++k) {
    if (wh[k] < lo) lo = wh[k];
    if (wh[k] > hi) hi = wh[k];
  }
  float range = hi - lo;
  float S = range / 255.0f;
  if (S < min_scale) S = min_scale;
  double zd = (double)O_QMIN_ASYM - (double)nearbyintf(lo / S); /* saturated before the int conversion */
  if (zd < O_QMIN_ASYM) zd = O_QMIN_ASYM;
  if (zd > O_QMAX_ASYM) zd = O_QMAX_ASYM;
  int Z = (int)zd;
  o_quant_row_asym(wh, K, S, Z, q);
  double best = o_mse_row_asym(wh, q, K, S, Z);
  if (hist) hist[0] = best;

  int it = 0;
  for (int i = 1; i <= max_iter; ++i) {
    it = i;
    double a, b;
    if (!o_lsq_affine(wh, q, K, Z, &a, &b)) break;
    float Sc = (float)a;
    if (Sc < min_scale) Sc = min_scale;
    double zr = (double)Z - nearbyint(b / a);
    int Zc = zr < (double)O_QMIN_ASYM ? O_QMIN_ASYM : (zr > (double)O_QMAX_ASYM ? O_QMAX_ASYM : (int)zr);
    o_quant_row_asym(wh, K, Sc, Zc, qc);
    double cur = o_mse_row_asym(wh, qc, K, Sc, Zc);
    double d = best - cur;
    int conv = (best == 0.0) || (d / best < thr) || (fabs(d) < thr);
    if (cur < best) {
      S = Sc;
      Z = Zc;
      best = cur;
      memcpy(q, qc, (size_t)K);
    }
    if (hist) hist[i] = best;
    if (conv) break;
  }
  *S_out = S;
  *Z_out = Z;
  if (iters_out) *iters_out = it;
  if (mse_out) *mse_out = best;
}

/* Asymmetric int8 weight quantization parameters for a [N,K] weight: fold s
 * (may be NULL), then MinMax + asymmetric SSZ per row.  Outputs S[N], Z[N],
 * q[N,K] codes in [-128,127], iters[N], mse[N], hist[N, max_iter+1] (the
 * last three may be NULL). */
int o_ssz_asym(const float* w, const float* s, int64_t N, int64_t K, int max_iter, double thr, float min_scale,
               float* S, int32_t* Z, int8_t* q, int32_t* iters, double* mse, double* hist) {
  if (!w || !S || !Z || !q || N < 0 || K <= 0) return O_EARG;
  if (max_iter < 0 || !(thr >= 0.0) || !(min_scale > 0.0f)) return O_EARG;
  if (!all_finite(w, N * K)) return O_ENONFINITE;
  if (!fold_finite(w, s, N, K, 1)) return O_ENONFINITE;
  int bad = 0;
#pragma omp parallel
  {
    float* wh = (float*)malloc(sizeof(float) * (size_t)K);
    int8_t* qc = (int8_t*)malloc((size_t)K);
    if (!wh || !qc) {
#pragma omp atomic write
      bad = 1;
    } else {
#pragma omp for schedule(dynamic, 16)
      for (int64_t n = 0; n < N; ++n) {
        o_fold_weight(w + n * K, s, 1, K, wh);
        ssz_asym_one_row(wh, K, max_iter, thr, min_scale, S + n, Z + n, q + n * K, iters ? iters + n : NULL,
                         mse ? mse + n : NULL, hist ? hist + n * (int64_t)(max_iter + 1) : NULL, qc);
      }
    }
    free(wh);
    free(qc);
  }
  return bad ? O_EARG : O_OK;
}

/* Per-tensor (per-layer) MinMax for comparison with per-channel ([PTQ]
 * granularity section): one S for the whole tensor,
 * S = max(fl32(max|W| / qmax), fl32(min_scale)); codes for every row. */
int o_minmax_per_tensor(const float* w, int64_t N, int64_t K, int bits, float min_scale, float* S_out,
                        int8_t* q) {
  if (!w || !S_out || !q || N <= 0 || K <= 0 || (bits != 8 && bits != 4)) return O_EARG;
  if (!all_finite(w, N * K)) return O_ENONFINITE;
  const int qmax = bits == 8 ? 127 : 7;
  float m = 0.0f;
  for (int64_t i = 0; i < N * K; ++i) {
    float a = fabsf(w[i]);
    if (a > m) m = a;
  }
  float S = m / (float)qmax;
  if (S < min_scale) S = min_scale;
  for (int64_t n = 0; n < N; ++n) o_quant_row(w + n * K, K, S, qmax, q + n * K);
  *S_out = S;
  return O_OK;
}

/* int4 storage: byte i of a row holds element 2i in the low nibble and
 * element 2i+1 in the high nibble, each a 4-bit two's-complement code.
 * (The SSZ document supports int4 codes but gives no storage format; this is
 * the library's.) */
int o_pack_int4(const int8_t* q, int64_t N, int64_t K, uint8_t* packed) {
  if (!q || !packed || N < 0 || K <= 0 || (K & 1)) return O_EARG;
  for (int64_t n = 0; n < N; ++n)
    for (int64_t i = 0; i < K / 2; ++i) {
      uint8_t lo = (uint8_t)q[n * K + 2 * i] & 0xF, hi = (uint8_t)q[n * K + 2 * i + 1] & 0xF;
      packed[n * (K / 2) + i] = (uint8_t)(lo | (hi << 4));
    }
  return O_OK;
}

/* ---------------------------------------------------------------------------
 * Per-token dynamic activation quantization, int8, symmetric.  One scale per
 * token row computed from that row at run time; the smoothing fold X/s is
 * applied first.
 *   a_t = max_j |x_hat[t,j]|,  delta_t = a_t > 0 ? fl32(a_t / 127) : 1,
 *   Xq[t,j] = clamp(rne(fl32(x_hat[t,j] / delta_t)), -127, 127).
 * ([SQ] per-channel activation scales do not fit integer GEMM kernels, which
 * is why the activation scale varies per token and the channel variation is
 * moved into the weights; [INT8] 2.1 for the formula; section 6 closes on
 * dynamic quantization.)
 * ------------------------------------------------------------------------- */
int o_quant_per_token(const float* x, const float* s, int64_t T, int64_t K, int8_t* xq, float* delta) {
  if (!x || !xq || !delta || T < 0 || K <= 0) return O_EARG;
  if (!all_finite(x, T * K)) return O_ENONFINITE;
  if (!fold_finite(x, s, T, K, 0)) return O_ENONFINITE;
  int bad = 0;
#pragma omp parallel
  {
    float* xh = (float*)malloc(sizeof(float) * (size_t)K);
    if (!xh) {
#pragma omp atomic write
      bad = 1;
    } else {
#pragma omp for schedule(static)
      for (int64_t t = 0; t < T; ++t) {
        o_fold_act(x + t * K, s, 1, K, xh);
        float a = 0.0f;
        for (int64_t j = 0; j < K; ++j) {
          float v = fabsf(xh[j]);
          if (v > a) a = v;
        }
        float d = a > 0.0f ? a / 127.0f : 1.0f;
        for (int64_t j = 0; j < K; ++j) xq[t * K + j] = (int8_t)code_of(xh[j], d, 127);
        delta[t] = d;
      }
    }
    free(xh);
  }
  return bad ? O_EARG : O_OK;
}

/* ---------------------------------------------------------------------------
 * Integer GEMM.  [INT8] 3.2: int8 x int8 products accumulated in integers;
 * both operands are K-contiguous (the snippet loads both tiles with leading
 * dimension K).  acc[t,n] = sum_k Xq[t,k] * Wq[n,k], in int64; returns
 * O_EOVERFLOW if any sum leaves the int32 range ([INT8] 5.1 overflow).
 * ------------------------------------------------------------------------- */
int o_gemm_i8(const int8_t* xq, const int8_t* wq, int64_t M, int64_t N, int64_t K, int64_t* acc) {
  if (!xq || !wq || !acc || M < 0 || N < 0 || K <= 0) return O_EARG;
  int ovf = 0;
#pragma omp parallel for schedule(static)
  for (int64_t t = 0; t < M; ++t)
    for (int64_t n = 0; n < N; ++n) {
      int64_t a = 0;
      for (int64_t k = 0; k < K; ++k) a += (int64_t)xq[t * K + k] * (int64_t)wq[n * K + k];
      acc[t * N + n] = a;
      if (a > INT32_MAX || a < INT32_MIN) {
#pragma omp atomic write
        ovf = 1;
      }
    }
  return ovf ? O_EOVERFLOW : O_OK;
}

/* Dequantization, the inverse of Q = round(R/S) with Z = 0 for both operands:
 * y[t,n] = acc[t,n] * delta_t * S_n, fp64 (the reference output; the GPU
 * writes fp32). */
int o_dequant(const int64_t* acc, const float* delta, const float* S, int64_t M, int64_t N, double* y) {
  if (!acc || !delta || !S || !y || M < 0 || N < 0) return O_EARG;
  for (int64_t t = 0; t < M; ++t)
    for (int64_t n = 0; n < N; ++n) y[t * N + n] = (double)acc[t * N + n] * (double)delta[t] * (double)S[n];
  return O_OK;
}

/* ===========================================================================
 * Epilogue fusion ([INT8] 4.2: quantize -> op -> dequantize -> activation in
 * one kernel) and the output formats the next layer consumes.
 *
 * Readings (the pages give the fused chain, not its arithmetic):
 *   - the epilogue works in fp32, in this order, each operation rounded:
 *       v = fl32(fl32(acc) * fl32(tok_scale[t] * ch_scale[n]))   (the dequant)
 *       v = fl32(v + bias[n])                                     (optional bias)
 *       relu: v > 0 ? v : +0;   gelu: fl32(0.5 v (1 + erf(v / sqrt 2))) (fp32 erff)
 *   - output f32: v;  bf16: v rounded to nearest-even bf16;  int8: the next
 *     layer's static per-tensor quantization of v, with its smoothing fold
 *     x_hat = fl32(v / next_s[n]) when next_s is given, then
 *     clamp(rne(fl32(x_hat / out_scale)), -127, 127).
 *   - the q_sigmoid snippet of [INT8] 3.3 is an integer sigmoid for a
 *     convolutional network; the linear layers here use ReLU (OPT) or GELU
 *     (GPT) instead.
 * ========================================================================= */
#define O_ACT_NONE 0
#define O_ACT_RELU 1
#define O_ACT_GELU 2
#define O_OUT_F32 0
#define O_OUT_BF16 1
#define O_OUT_I8 2

/* float -> bf16 bits, round to nearest, ties to even (finite inputs) */
uint16_t o_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  uint32_t lsb = (u >> 16) & 1u;
  u += 0x7FFFu + lsb;
  return (uint16_t)(u >> 16);
}

static float o_gelu32(float v) {
  const float c = 0.70710678118654752440f; /* fl32(1/sqrt(2)) */
  float e = erff(v * c);
  float h = 0.5f * v;
  return h * (1.0f + e);
}

int o_epilogue(const int64_t* acc, int64_t M, int64_t N, const float* tok_scale, const float* ch_scale,
               const float* bias, int act, int out_type, const float* next_s, float out_scale, void* out) {
  if (!acc || !tok_scale || !ch_scale || !out || M < 0 || N < 0) return O_EARG;
  if (act < O_ACT_NONE || act > O_ACT_GELU || out_type < O_OUT_F32 || out_type > O_OUT_I8) return O_EARG;
  if (out_type == O_OUT_I8 && !(out_scale > 0.0f)) return O_EARG;
  for (int64_t t = 0; t < M; ++t) {
    for (int64_t n = 0; n < N; ++n) {
      int64_t a = acc[t * N + n];
      if (a > INT32_MAX || a < INT32_MIN) return O_EOVERFLOW;
      float sc = tok_scale[t] * ch_scale[n];
      float v = (float)a * sc;
      if (bias) v = v + bias[n];
      if (act == O_ACT_RELU) v = v > 0.0f ? v : 0.0f;
      else if (act == O_ACT_GELU) v = o_gelu32(v);
      if (out_type == O_OUT_F32) {
        ((float*)out)[t * N + n] = v;
      } else if (out_type == O_OUT_BF16) {
        ((uint16_t*)out)[t * N + n] = o_bf16_rne(v);
      } else {
        float xh = next_s ? v / next_s[n] : v;
        if (isnan(xh)) return O_ENONFINITE; /* 0 * inf or inf - inf upstream: no code */
        ((int8_t*)out)[t * N + n] = (int8_t)code_of(xh, out_scale, 127);
      }
    }
  }
  return O_OK;
}

/* ===========================================================================
 * Static (calibrated) per-tensor scales: the moving-average absmax of the
 * activations ([INT8] 2.1 tip: a moving average of the range is more robust
 * than the raw min/max; [QAT] 六: activation_quantize_type
 * moving_average_abs_max) and the per-tensor (per-layer) weight scale ([PTQ]
 * 逐层量化: one scale for the whole tensor).
 *
 * Readings:
 *   - the tracked range is per tensor: a = max over the batch of |x_hat|,
 *     x_hat the smoothed activation fl32(x / s_j) (s may be NULL);
 *   - moving average: the first batch sets the state, later batches update
 *     state = fl32(fl32(m * state) + fl32(fl32(1 - m) * a)) with momentum m in
 *     [0, 1) -- the pages give no momentum; it is a labelled parameter
 *     (0.9 in the tests and the bench);
 *   - static activation scale = state > 0 ? fl32(state / 127) : 1;
 *   - per-tensor weight scale = max(fl32(max|w_hat| / 127), fl32(min_scale)),
 *     w_hat = fl32(w * s_j) (the MinMax rule of the per-channel path on the
 *     whole tensor; the SSZ search itself is per-channel only, [SSZ] 使用限制).
 * Both can be computed from column maxima: for a positive constant c and RNE,
 * max_t |fl32(x_tj / c)| = fl32(max_t |x_tj| / c) and likewise for x_tj * c
 * (rounding is monotone).
 * ========================================================================= */
#define O_FOLD_NONE 0
#define O_FOLD_DIV 1 /* activation side: x / s_j */
#define O_FOLD_MUL 2 /* weight side: w * s_j */

static float fold_one(float x, const float* s, int64_t j, int fold) {
  if (!s || fold == O_FOLD_NONE) return x;
  return fold == O_FOLD_DIV ? x / s[j] : x * s[j];
}

/* max over the whole [rows, cols] tensor of |fold(x)| (element by element, no shortcut) */
int o_absmax_tensor(const float* x, int64_t rows, int64_t cols, const float* s, int fold, float* amax) {
  if (!x || !amax || rows < 0 || cols <= 0 || fold < O_FOLD_NONE || fold > O_FOLD_MUL) return O_EARG;
  if (!all_finite(x, rows * cols)) return O_ENONFINITE;
  float m = 0.0f;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t j = 0; j < cols; ++j) {
      float v = fabsf(fold_one(x[r * cols + j], s, j, fold));
      if (v > m) m = v;
    }
  *amax = m;
  return O_OK;
}

int o_ema_update(float* state, float a, float momentum, int first) {
  if (!state || !(momentum >= 0.0f && momentum < 1.0f) || !(a >= 0.0f)) return O_EARG;
  if (first) {
    *state = a;
  } else {
    float t1 = momentum * *state;
    float w = 1.0f - momentum;
    float t2 = w * a;
    *state = t1 + t2;
  }
  return O_OK;
}

float o_act_static_scale(float state) { return state > 0.0f ? state / 127.0f : 1.0f; }

float o_weight_scale_per_tensor(float amax, float min_scale) {
  float S = amax / 127.0f;
  return S < min_scale ? min_scale : S;
}

/* codes of a whole tensor with one static scale S: clamp(rne(fl32(fold(x) / S)), -127, 127) */
int o_quant_static(const float* x, int64_t rows, int64_t cols, const float* s, int fold, float S, int8_t* q) {
  if (!x || !q || rows < 0 || cols <= 0 || !(S > 0.0f) || fold < O_FOLD_NONE || fold > O_FOLD_MUL) return O_EARG;
  if (!all_finite(x, rows * cols)) return O_ENONFINITE;
  if (fold != O_FOLD_NONE && !fold_finite(x, s, rows, cols, fold == O_FOLD_MUL)) return O_ENONFINITE;
  for (int64_t r = 0; r < rows; ++r)
    for (int64_t j = 0; j < cols; ++j) q[r * cols + j] = (int8_t)code_of(fold_one(x[r * cols + j], s, j, fold), S, 127);
  return O_OK;
}
