// Stand-ins for the kernel launchers behind the C ABI (post_int8_quantization_amd/csrc/ptq_launch.hpp), so that
// the ABI's host code (capi.hip) can run under AddressSanitizer and UndefinedBehaviorSanitizer with no GPU: each
// records which launcher was reached and with which leading pointer, and returns the status the driver chose.
#include "../../post_int8_quantization_amd/csrc/ptq_launch.hpp"

extern "C" {
const char* g_stub_last = "";
const void* g_stub_ptr = nullptr;
int g_stub_status = 0;  // hipError_t value the next launcher returns
}

namespace {
hipError_t hit(const char* name, const void* p) {
  g_stub_last = name;
  g_stub_ptr = p;
  return (hipError_t)g_stub_status;
}
}  // namespace

namespace ptq {

hipError_t launch_absmax_cols(const void* x, int, int64_t, int64_t, float*, int, hipStream_t) {
  return hit("absmax_cols", x);
}
hipError_t launch_smooth_factors(const float* ax, const float*, int64_t, float, float*, hipStream_t) {
  return hit("smooth_factors", ax);
}
hipError_t launch_quant_per_token(const void* x, int, int64_t, int64_t, const float*, int8_t*, float*, hipStream_t) {
  return hit("quant_per_token", x);
}
hipError_t launch_quant_per_token_rpb(const void* x, int, int64_t, int64_t, const float*, int8_t*, float*, int64_t,
                                      hipStream_t) {
  return hit("quant_per_token_rpb", x);
}
hipError_t launch_quant_static(const void* x, int, int64_t, int64_t, const float*, int, const float*, int8_t*, float*,
                               hipStream_t) {
  return hit("quant_static", x);
}
hipError_t launch_tensor_scale(const float* col_amax, const float*, int64_t, int, float, int, float, float*, float*,
                               float*, int64_t, hipStream_t) {
  return hit("tensor_scale", col_amax);
}
hipError_t launch_ssz(const void* w, int, int64_t, int64_t, const float*, int, int, double, float, float*, void*,
                      int32_t*, double*, hipStream_t) {
  return hit("ssz", w);
}
hipError_t launch_ssz_asym(const void* w, int, int64_t, int64_t, const float*, int, double, float, float*, int32_t*,
                           int8_t*, int32_t*, double*, hipStream_t) {
  return hit("ssz_asym", w);
}
hipError_t launch_gemm_dequant(const int8_t* xq, const int8_t*, const float*, const float*, int64_t, int64_t, int64_t,
                               float*, int32_t*, hipStream_t) {
  return hit("gemm_dequant", xq);
}
hipError_t launch_gemm_fused(const int8_t* xq, const int8_t*, const float*, const float*, const float*, int, int,
                             const float*, const float*, int64_t, int64_t, int64_t, void*, int32_t*, hipStream_t) {
  return hit("gemm_fused", xq);
}

}  // namespace ptq
