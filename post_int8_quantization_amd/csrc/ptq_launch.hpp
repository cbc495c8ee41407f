// ptq_launch.hpp -- internal launchers behind the C ABI (C++ linkage, not exported).
// Each launcher assumes its arguments were validated by capi.hip and enqueues
// its kernels on `stream`; it returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ptq {

hipError_t launch_absmax_cols(const void* x, int dtype, int64_t rows, int64_t cols, float* amax, int accumulate,
                              hipStream_t stream);

hipError_t launch_smooth_factors(const float* ax, const float* aw, int64_t K, float alpha, float* s,
                                 hipStream_t stream);

hipError_t launch_quant_per_token(const void* x, int dtype, int64_t T, int64_t K, const float* s, int8_t* xq,
                                  float* tok_scale, hipStream_t stream);

hipError_t launch_quant_per_token_rpb(const void* x, int dtype, int64_t T, int64_t K, const float* s, int8_t* xq,
                                      float* tok_scale, int64_t rows_per_block, hipStream_t stream);

// static per-tensor quantization: one scale (scale[0], device) for every row; fold_mul: x * s_j instead of
// x * fl32(1/s_j); row_scale (may be null) receives scale[0] per row
hipError_t launch_quant_static(const void* x, int dtype, int64_t rows, int64_t cols, const float* s, int fold_mul,
                               const float* scale, int8_t* q, float* row_scale, hipStream_t stream);

// single-block scale kernels over column maxima: activation (moving average, mode 0) or weight
// (per-tensor MinMax, mode 1); see calib.hip
hipError_t launch_tensor_scale(const float* col_amax, const float* s, int64_t K, int mode, float momentum, int first,
                               float min_scale, float* state, float* scale, float* bcast, int64_t n_bcast,
                               hipStream_t stream);

hipError_t launch_ssz(const void* w, int dtype, int64_t N, int64_t K, const float* s, int bits, int max_iter,
                      double threshold, float min_scale, float* scale, void* wq, int32_t* iters, double* mse,
                      hipStream_t stream);

hipError_t launch_ssz_asym(const void* w, int dtype, int64_t N, int64_t K, const float* s, int max_iter,
                           double threshold, float min_scale, float* scale, int32_t* zero_point, int8_t* wq,
                           int32_t* iters, double* mse, hipStream_t stream);

hipError_t launch_gemm_dequant(const int8_t* xq, const int8_t* wq, const float* tok_scale, const float* ch_scale,
                               int64_t M, int64_t N, int64_t K, float* y, int32_t* acc, hipStream_t stream);

// act: 0 none, 1 relu, 2 gelu;  out_type: 0 fp32, 1 bf16, 2 int8
hipError_t launch_gemm_fused(const int8_t* xq, const int8_t* wq, const float* tok_scale, const float* ch_scale,
                             const float* bias, int act, int out_type, const float* next_s, const float* out_scale,
                             int64_t M, int64_t N, int64_t K, void* out, int32_t* acc, hipStream_t stream);

// Largest K the row-resident kernels (per-token quantization, SSZ) accept.
constexpr int64_t kMaxRowK = 131072;

}  // namespace ptq
