// capi.hip -- the exported C ABI of libptq: argument checks, then kernel launches.
//
// Every entry point validates on the host before touching the GPU, so each
// error class can be raised without a device: required pointers, shapes
// (sizes >= 1, K a multiple of 16 for the 16-byte vector rows, K bounds),
// element type, supported settings ([SSZ] limits: int8/int4, per-channel,
// symmetric), argument ranges ([SQ] alpha in [0,1]; [SSZ] constants) and
// 16-byte alignment.  A failed launch is reported as PTQ_ERR_HIP.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include "ptq_launch.hpp"
#include "../../include/ptq.h"

namespace {

thread_local char g_err[512] = "";

ptq_status fail(ptq_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

ptq_status from_hip(hipError_t e, const char* fn) {
  if (e == hipSuccess) return PTQ_OK;
  return fail(PTQ_ERR_HIP, "%s: kernel launch failed: %s", fn, hipGetErrorString(e));
}

bool known_dtype(int dt) { return dt == PTQ_F32 || dt == PTQ_BF16; }

}  // namespace

extern "C" {

int ptq_abi_version(void) { return PTQ_ABI_VERSION; }

const char* ptq_last_error(void) { return g_err; }

const char* ptq_status_string(int st) {
  switch (st) {
    case PTQ_OK: return "PTQ_OK";
    case PTQ_ERR_NULL: return "PTQ_ERR_NULL";
    case PTQ_ERR_SHAPE: return "PTQ_ERR_SHAPE";
    case PTQ_ERR_DTYPE: return "PTQ_ERR_DTYPE";
    case PTQ_ERR_UNSUPPORTED: return "PTQ_ERR_UNSUPPORTED";
    case PTQ_ERR_ARG: return "PTQ_ERR_ARG";
    case PTQ_ERR_ALIGN: return "PTQ_ERR_ALIGN";
    case PTQ_ERR_HIP: return "PTQ_ERR_HIP";
    default: return "PTQ_ERR_UNKNOWN";
  }
}

ptq_status sq_absmax_calib(const void* x, int dtype, int64_t rows, int64_t cols, float* amax, int accumulate,
                           void* stream) {
  const char* fn = "sq_absmax_calib";
  if (!x || !amax) return fail(PTQ_ERR_NULL, "%s: x and amax are required", fn);
  if (!known_dtype(dtype)) return fail(PTQ_ERR_DTYPE, "%s: unknown dtype %d", fn, dtype);
  if (rows <= 0 || cols <= 0) return fail(PTQ_ERR_SHAPE, "%s: rows=%lld cols=%lld must be >= 1", fn, (long long)rows,
                                          (long long)cols);
  if (cols % PTQ_K_MULTIPLE) return fail(PTQ_ERR_SHAPE, "%s: cols=%lld is not a multiple of 16", fn, (long long)cols);
  if (rows > INT64_MAX / cols) return fail(PTQ_ERR_SHAPE, "%s: rows*cols overflows", fn);
  if ((cols / PTQ_K_MULTIPLE + 15) / 16 > 0x7fffffff)
    return fail(PTQ_ERR_SHAPE, "%s: cols=%lld too large", fn, (long long)cols);
  if (!aligned16(x) || !aligned16(amax)) return fail(PTQ_ERR_ALIGN, "%s: x and amax must be 16-byte aligned", fn);
  return from_hip(ptq::launch_absmax_cols(x, dtype, rows, cols, amax, accumulate, (hipStream_t)stream), fn);
}

ptq_status sq_smooth_factors(const float* act_amax, const float* w_amax, int64_t K, float alpha, float* s,
                             void* stream) {
  const char* fn = "sq_smooth_factors";
  if (!act_amax || !w_amax || !s) return fail(PTQ_ERR_NULL, "%s: act_amax, w_amax and s are required", fn);
  if (K <= 0 || K > ((int64_t)1 << 40)) return fail(PTQ_ERR_SHAPE, "%s: K=%lld out of range", fn, (long long)K);
  if (!(alpha >= 0.0f && alpha <= 1.0f)) return fail(PTQ_ERR_ARG, "%s: alpha=%g must lie in [0, 1]", fn, (double)alpha);
  return from_hip(ptq::launch_smooth_factors(act_amax, w_amax, K, alpha, s, (hipStream_t)stream), fn);
}

ptq_status ssz_weight_qparams(const void* w, int dtype, int64_t N, int64_t K, const float* s, int bits, int symmetric,
                              int max_iter, double threshold, float min_scale, float* scale, void* wq, int32_t* iters,
                              double* mse, void* stream) {
  const char* fn = "ssz_weight_qparams";
  if (!w || !scale) return fail(PTQ_ERR_NULL, "%s: w and scale are required", fn);
  if (!known_dtype(dtype)) return fail(PTQ_ERR_DTYPE, "%s: unknown dtype %d", fn, dtype);
  if (N <= 0 || K <= 0) return fail(PTQ_ERR_SHAPE, "%s: N=%lld K=%lld must be >= 1", fn, (long long)N, (long long)K);
  if (K % PTQ_K_MULTIPLE) return fail(PTQ_ERR_SHAPE, "%s: K=%lld is not a multiple of 16", fn, (long long)K);
  if (K > ptq::kMaxRowK) return fail(PTQ_ERR_SHAPE, "%s: K=%lld exceeds %lld", fn, (long long)K,
                                     (long long)ptq::kMaxRowK);
  if (N > 0x7fffffff) return fail(PTQ_ERR_SHAPE, "%s: N=%lld too large", fn, (long long)N);
  if (bits != 8 && bits != 4) return fail(PTQ_ERR_UNSUPPORTED, "%s: bits=%d (only 8 and 4 are supported)", fn, bits);
  if (symmetric != 1)
    return fail(PTQ_ERR_UNSUPPORTED,
                "%s: symmetric=0 is served by ssz_weight_qparams_asym (int8 only; the SSZ method has no int4 "
                "asymmetric mode)", fn);
  if (max_iter < 0 || max_iter > PTQ_SSZ_MAX_ITER)
    return fail(PTQ_ERR_ARG, "%s: max_iter=%d must lie in [0, %d]", fn, max_iter, PTQ_SSZ_MAX_ITER);
  if (!(threshold >= 0.0) || isinf(threshold)) return fail(PTQ_ERR_ARG, "%s: threshold=%g invalid", fn, threshold);
  if (!(min_scale > 0.0f) || isinf(min_scale))
    return fail(PTQ_ERR_ARG, "%s: min_scale=%g must be positive", fn, (double)min_scale);
  if (!aligned16(w) || (s && !aligned16(s)) || (wq && !aligned16(wq)))
    return fail(PTQ_ERR_ALIGN, "%s: w, s and wq must be 16-byte aligned", fn);
  return from_hip(ptq::launch_ssz(w, dtype, N, K, s, bits, max_iter, threshold, min_scale, scale, wq, iters, mse,
                                  (hipStream_t)stream),
                  fn);
}

ptq_status ssz_weight_qparams_asym(const void* w, int dtype, int64_t N, int64_t K, const float* s, int max_iter,
                                   double threshold, float min_scale, float* scale, int32_t* zero_point, int8_t* wq,
                                   int32_t* iters, double* mse, void* stream) {
  const char* fn = "ssz_weight_qparams_asym";
  if (!w || !scale || !zero_point) return fail(PTQ_ERR_NULL, "%s: w, scale and zero_point are required", fn);
  if (!known_dtype(dtype)) return fail(PTQ_ERR_DTYPE, "%s: unknown dtype %d", fn, dtype);
  if (N <= 0 || K <= 0) return fail(PTQ_ERR_SHAPE, "%s: N=%lld K=%lld must be >= 1", fn, (long long)N, (long long)K);
  if (K % PTQ_K_MULTIPLE) return fail(PTQ_ERR_SHAPE, "%s: K=%lld is not a multiple of 16", fn, (long long)K);
  if (K > ptq::kMaxRowK) return fail(PTQ_ERR_SHAPE, "%s: K=%lld exceeds %lld", fn, (long long)K,
                                     (long long)ptq::kMaxRowK);
  if (N > 0x7fffffff) return fail(PTQ_ERR_SHAPE, "%s: N=%lld too large", fn, (long long)N);
  if (max_iter < 0 || max_iter > PTQ_SSZ_MAX_ITER)
    return fail(PTQ_ERR_ARG, "%s: max_iter=%d must lie in [0, %d]", fn, max_iter, PTQ_SSZ_MAX_ITER);
  if (!(threshold >= 0.0) || isinf(threshold)) return fail(PTQ_ERR_ARG, "%s: threshold=%g invalid", fn, threshold);
  if (!(min_scale > 0.0f) || isinf(min_scale))
    return fail(PTQ_ERR_ARG, "%s: min_scale=%g must be positive", fn, (double)min_scale);
  if (!aligned16(w) || (s && !aligned16(s)) || (wq && !aligned16(wq)))
    return fail(PTQ_ERR_ALIGN, "%s: w, s and wq must be 16-byte aligned", fn);
  return from_hip(ptq::launch_ssz_asym(w, dtype, N, K, s, max_iter, threshold, min_scale, scale, zero_point, wq,
                                       iters, mse, (hipStream_t)stream),
                  fn);
}

ptq_status quant_per_token_i8(const void* x, int dtype, int64_t T, int64_t K, const float* s, int8_t* xq,
                              float* tok_scale, void* stream) {
  const char* fn = "quant_per_token_i8";
  if (!x || !xq || !tok_scale) return fail(PTQ_ERR_NULL, "%s: x, xq and tok_scale are required", fn);
  if (!known_dtype(dtype)) return fail(PTQ_ERR_DTYPE, "%s: unknown dtype %d", fn, dtype);
  if (T <= 0 || K <= 0) return fail(PTQ_ERR_SHAPE, "%s: T=%lld K=%lld must be >= 1", fn, (long long)T, (long long)K);
  if (K % PTQ_K_MULTIPLE) return fail(PTQ_ERR_SHAPE, "%s: K=%lld is not a multiple of 16", fn, (long long)K);
  if (K > ptq::kMaxRowK) return fail(PTQ_ERR_SHAPE, "%s: K=%lld exceeds %lld", fn, (long long)K,
                                     (long long)ptq::kMaxRowK);
  if (T > INT64_MAX / K) return fail(PTQ_ERR_SHAPE, "%s: T*K overflows", fn);
  if (!aligned16(x) || !aligned16(xq) || (s && !aligned16(s)))
    return fail(PTQ_ERR_ALIGN, "%s: x, xq and s must be 16-byte aligned", fn);
  return from_hip(ptq::launch_quant_per_token(x, dtype, T, K, s, xq, tok_scale, (hipStream_t)stream), fn);
}

ptq_status w8a8_gemm_dequant(const int8_t* xq, const int8_t* wq, const float* tok_scale, const float* ch_scale,
                             int64_t M, int64_t N, int64_t K, float* y, int32_t* acc, void* stream) {
  const char* fn = "w8a8_gemm_dequant";
  if (!xq || !wq || !tok_scale || !ch_scale || !y)
    return fail(PTQ_ERR_NULL, "%s: xq, wq, tok_scale, ch_scale and y are required", fn);
  if (M <= 0 || N <= 0 || K <= 0)
    return fail(PTQ_ERR_SHAPE, "%s: M=%lld N=%lld K=%lld must be >= 1", fn, (long long)M, (long long)N, (long long)K);
  if (K % PTQ_K_MULTIPLE) return fail(PTQ_ERR_SHAPE, "%s: K=%lld is not a multiple of 16", fn, (long long)K);
  if (K > PTQ_GEMM_MAX_K)
    return fail(PTQ_ERR_SHAPE, "%s: K=%lld exceeds %d, int32 sums could overflow", fn, (long long)K, PTQ_GEMM_MAX_K);
  if (M > 0x7fffffff || N > 0x7fffffff) return fail(PTQ_ERR_SHAPE, "%s: M or N too large", fn);
  if (!aligned16(xq) || !aligned16(wq) || !aligned16(y) || (acc && !aligned16(acc)))
    return fail(PTQ_ERR_ALIGN, "%s: xq, wq, y and acc must be 16-byte aligned", fn);
  return from_hip(ptq::launch_gemm_dequant(xq, wq, tok_scale, ch_scale, M, N, K, y, acc, (hipStream_t)stream), fn);
}

ptq_status w8a8_gemm_fused(const int8_t* xq, const int8_t* wq, const float* tok_scale, const float* ch_scale,
                           const float* bias, int act, int out_type, const float* next_s, const float* out_scale,
                           int64_t M, int64_t N, int64_t K, void* out, int32_t* acc, void* stream) {
  const char* fn = "w8a8_gemm_fused";
  if (!xq || !wq || !tok_scale || !ch_scale || !out)
    return fail(PTQ_ERR_NULL, "%s: xq, wq, tok_scale, ch_scale and out are required", fn);
  if (act != PTQ_ACT_NONE && act != PTQ_ACT_RELU && act != PTQ_ACT_GELU)
    return fail(PTQ_ERR_UNSUPPORTED, "%s: act=%d (none, relu and gelu are supported)", fn, act);
  if (out_type != PTQ_OUT_F32 && out_type != PTQ_OUT_BF16 && out_type != PTQ_OUT_I8)
    return fail(PTQ_ERR_DTYPE, "%s: out_type=%d unknown", fn, out_type);
  if (out_type == PTQ_OUT_I8 && !out_scale)
    return fail(PTQ_ERR_NULL, "%s: the int8 output needs out_scale", fn);
  if (out_type != PTQ_OUT_I8 && (next_s || out_scale))
    return fail(PTQ_ERR_ARG, "%s: next_s and out_scale apply to the int8 output only", fn);
  if (M <= 0 || N <= 0 || K <= 0)
    return fail(PTQ_ERR_SHAPE, "%s: M=%lld N=%lld K=%lld must be >= 1", fn, (long long)M, (long long)N, (long long)K);
  if (K % PTQ_K_MULTIPLE) return fail(PTQ_ERR_SHAPE, "%s: K=%lld is not a multiple of 16", fn, (long long)K);
  if (K > PTQ_GEMM_MAX_K)
    return fail(PTQ_ERR_SHAPE, "%s: K=%lld exceeds %d, int32 sums could overflow", fn, (long long)K, PTQ_GEMM_MAX_K);
  if (M > 0x7fffffff || N > 0x7fffffff) return fail(PTQ_ERR_SHAPE, "%s: M or N too large", fn);
  if (!aligned16(xq) || !aligned16(wq) || !aligned16(out) || (acc && !aligned16(acc)))
    return fail(PTQ_ERR_ALIGN, "%s: xq, wq, out and acc must be 16-byte aligned", fn);
  return from_hip(ptq::launch_gemm_fused(xq, wq, tok_scale, ch_scale, bias, act, out_type, next_s, out_scale, M, N, K,
                                         out, acc, (hipStream_t)stream),
                  fn);
}

ptq_status sq_act_scale_ema(const float* col_amax, const float* s, int64_t K, float momentum, int first, float* state,
                            float* scale, float* row_scale, int64_t rows, void* stream) {
  const char* fn = "sq_act_scale_ema";
  if (!col_amax || !state || !scale) return fail(PTQ_ERR_NULL, "%s: col_amax, state and scale are required", fn);
  if (K <= 0) return fail(PTQ_ERR_SHAPE, "%s: K=%lld must be >= 1", fn, (long long)K);
  if (row_scale && rows <= 0) return fail(PTQ_ERR_SHAPE, "%s: rows=%lld must be >= 1", fn, (long long)rows);
  if (!(momentum >= 0.0f && momentum < 1.0f))
    return fail(PTQ_ERR_ARG, "%s: momentum=%g must lie in [0, 1)", fn, (double)momentum);
  return from_hip(ptq::launch_tensor_scale(col_amax, s, K, 0, momentum, first != 0, 0.0f, state, scale, row_scale,
                                           rows, (hipStream_t)stream),
                  fn);
}

ptq_status weight_scale_per_tensor(const float* col_amax, const float* s, int64_t K, float min_scale, float* scale,
                                   float* ch_scale, int64_t N, void* stream) {
  const char* fn = "weight_scale_per_tensor";
  if (!col_amax || !scale) return fail(PTQ_ERR_NULL, "%s: col_amax and scale are required", fn);
  if (K <= 0) return fail(PTQ_ERR_SHAPE, "%s: K=%lld must be >= 1", fn, (long long)K);
  if (ch_scale && N <= 0) return fail(PTQ_ERR_SHAPE, "%s: N=%lld must be >= 1", fn, (long long)N);
  if (!(min_scale > 0.0f) || isinf(min_scale))
    return fail(PTQ_ERR_ARG, "%s: min_scale=%g must be positive", fn, (double)min_scale);
  return from_hip(ptq::launch_tensor_scale(col_amax, s, K, 1, 0.0f, 0, min_scale, nullptr, scale, ch_scale, N,
                                           (hipStream_t)stream),
                  fn);
}

ptq_status quant_static_i8(const void* x, int dtype, int64_t rows, int64_t cols, const float* s, int fold,
                           const float* scale, int8_t* q, float* row_scale, void* stream) {
  const char* fn = "quant_static_i8";
  if (!x || !scale || !q) return fail(PTQ_ERR_NULL, "%s: x, scale and q are required", fn);
  if (!known_dtype(dtype)) return fail(PTQ_ERR_DTYPE, "%s: unknown dtype %d", fn, dtype);
  if (rows <= 0 || cols <= 0)
    return fail(PTQ_ERR_SHAPE, "%s: rows=%lld cols=%lld must be >= 1", fn, (long long)rows, (long long)cols);
  if (cols % PTQ_K_MULTIPLE) return fail(PTQ_ERR_SHAPE, "%s: cols=%lld is not a multiple of 16", fn, (long long)cols);
  if (cols > ptq::kMaxRowK) return fail(PTQ_ERR_SHAPE, "%s: cols=%lld exceeds %lld", fn, (long long)cols,
                                        (long long)ptq::kMaxRowK);
  if (rows > INT64_MAX / cols) return fail(PTQ_ERR_SHAPE, "%s: rows*cols overflows", fn);
  if (s && fold != PTQ_FOLD_DIV && fold != PTQ_FOLD_MUL)
    return fail(PTQ_ERR_ARG, "%s: fold=%d (PTQ_FOLD_DIV or PTQ_FOLD_MUL with s)", fn, fold);
  if (!aligned16(x) || !aligned16(q) || (s && !aligned16(s)))
    return fail(PTQ_ERR_ALIGN, "%s: x, q and s must be 16-byte aligned", fn);
  return from_hip(ptq::launch_quant_static(x, dtype, rows, cols, s, fold == PTQ_FOLD_MUL, scale, q, row_scale,
                                           (hipStream_t)stream),
                  fn);
}

}  // extern "C"
