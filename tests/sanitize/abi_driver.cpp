// Drives the host code of the C ABI (capi.hip) under AddressSanitizer and UndefinedBehaviorSanitizer, with the
// kernel launchers replaced by stand-ins (launch_stubs.cpp): every invalid argument class of every entry point
// must return its status with a message, every valid call must reach its launcher with the caller's pointer, and
// a failed launch must come back as PTQ_ERR_HIP.  Nothing touches a GPU.  Exit 0 when every check holds.
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <cmath>
#include <limits>

#include "../../include/ptq.h"

extern "C" {
extern const char* g_stub_last;
extern const void* g_stub_ptr;
extern int g_stub_status;
}

static int g_fail = 0, g_checks = 0;

static void expect(int got, int want, const char* what) {
  ++g_checks;
  const char* msg = ptq_last_error();
  if (got != want) {
    fprintf(stderr, "FAIL %s: status %d (%s), expected %d; last error: %s\n", what, got, ptq_status_string(got), want,
            msg);
    ++g_fail;
  } else if (want != PTQ_OK && (!msg || !*msg)) {
    fprintf(stderr, "FAIL %s: no error message\n", what);
    ++g_fail;
  }
}

static void expect_launch(int got, const char* stub, const void* p, const char* what) {
  expect(got, PTQ_OK, what);
  ++g_checks;
  if (strcmp(g_stub_last, stub) != 0 || g_stub_ptr != p) {
    fprintf(stderr, "FAIL %s: reached %s with %p, expected %s with %p\n", what, g_stub_last, g_stub_ptr, stub, p);
    ++g_fail;
  }
  g_stub_last = "";
  g_stub_ptr = nullptr;
}

int main() {
  // host buffers standing in for device memory: the ABI checks only their presence and alignment
  const size_t bytes = 1 << 16;
  unsigned char* buf = static_cast<unsigned char*>(aligned_alloc(64, bytes));
  memset(buf, 0, bytes);
  void* A = buf;                 // 16-byte aligned
  void* B = buf + 4096;          // 16-byte aligned
  void* C = buf + 8192;          // 16-byte aligned
  void* D = buf + 12288;         // 16-byte aligned
  void* MIS = buf + 16384 + 4;   // misaligned
  float* f = reinterpret_cast<float*>(buf + 20480);
  const double inf = std::numeric_limits<double>::infinity();
  const float nanf = std::numeric_limits<float>::quiet_NaN();

  // status strings and version
  for (int st = 0; st <= 8; ++st) expect(ptq_status_string(st) != nullptr ? PTQ_OK : -1, PTQ_OK, "status string");
  expect(ptq_abi_version() == PTQ_ABI_VERSION ? PTQ_OK : -1, PTQ_OK, "abi version");

  // sq_absmax_calib
  expect(sq_absmax_calib(nullptr, PTQ_F32, 4, 16, f, 0, nullptr), PTQ_ERR_NULL, "calib null x");
  expect(sq_absmax_calib(A, 7, 4, 16, f, 0, nullptr), PTQ_ERR_DTYPE, "calib dtype");
  expect(sq_absmax_calib(A, PTQ_F32, 0, 16, f, 0, nullptr), PTQ_ERR_SHAPE, "calib rows");
  expect(sq_absmax_calib(A, PTQ_F32, 4, 15, f, 0, nullptr), PTQ_ERR_SHAPE, "calib cols multiple");
  expect(sq_absmax_calib(A, PTQ_F32, INT64_MAX / 8, 16, f, 0, nullptr), PTQ_ERR_SHAPE, "calib overflow");
  expect(sq_absmax_calib(MIS, PTQ_F32, 4, 16, f, 0, nullptr), PTQ_ERR_ALIGN, "calib align");
  expect_launch(sq_absmax_calib(A, PTQ_BF16, 4, 16, f, 1, nullptr), "absmax_cols", A, "calib ok");

  // sq_smooth_factors
  expect(sq_smooth_factors(nullptr, f, 16, 0.5f, f, nullptr), PTQ_ERR_NULL, "smooth null");
  expect(sq_smooth_factors(f, f, 0, 0.5f, f, nullptr), PTQ_ERR_SHAPE, "smooth K");
  expect(sq_smooth_factors(f, f, 16, 1.5f, f, nullptr), PTQ_ERR_ARG, "smooth alpha > 1");
  expect(sq_smooth_factors(f, f, 16, nanf, f, nullptr), PTQ_ERR_ARG, "smooth alpha nan");
  expect_launch(sq_smooth_factors(f, f, 16, 0.5f, f, nullptr), "smooth_factors", f, "smooth ok");

  // ssz_weight_qparams
  expect(ssz_weight_qparams(nullptr, PTQ_F32, 4, 16, nullptr, 8, 1, 20, 1e-10, 1e-5f, f, B, nullptr, nullptr, nullptr),
         PTQ_ERR_NULL, "ssz null");
  expect(ssz_weight_qparams(A, 9, 4, 16, nullptr, 8, 1, 20, 1e-10, 1e-5f, f, B, nullptr, nullptr, nullptr),
         PTQ_ERR_DTYPE, "ssz dtype");
  expect(ssz_weight_qparams(A, PTQ_F32, 4, 24, nullptr, 8, 1, 20, 1e-10, 1e-5f, f, B, nullptr, nullptr, nullptr),
         PTQ_ERR_SHAPE, "ssz K multiple");
  expect(ssz_weight_qparams(A, PTQ_F32, 4, 131088, nullptr, 8, 1, 20, 1e-10, 1e-5f, f, B, nullptr, nullptr, nullptr),
         PTQ_ERR_SHAPE, "ssz K max");
  expect(ssz_weight_qparams(A, PTQ_F32, 4, 16, nullptr, 2, 1, 20, 1e-10, 1e-5f, f, B, nullptr, nullptr, nullptr),
         PTQ_ERR_UNSUPPORTED, "ssz bits");
  expect(ssz_weight_qparams(A, PTQ_F32, 4, 16, nullptr, 8, 0, 20, 1e-10, 1e-5f, f, B, nullptr, nullptr, nullptr),
         PTQ_ERR_UNSUPPORTED, "ssz asym via sym");
  expect(ssz_weight_qparams(A, PTQ_F32, 4, 16, nullptr, 8, 1, 21, 1e-10, 1e-5f, f, B, nullptr, nullptr, nullptr),
         PTQ_ERR_ARG, "ssz max_iter");
  expect(ssz_weight_qparams(A, PTQ_F32, 4, 16, nullptr, 8, 1, 20, inf, 1e-5f, f, B, nullptr, nullptr, nullptr),
         PTQ_ERR_ARG, "ssz threshold inf");
  expect(ssz_weight_qparams(A, PTQ_F32, 4, 16, nullptr, 8, 1, 20, 1e-10, 0.0f, f, B, nullptr, nullptr, nullptr),
         PTQ_ERR_ARG, "ssz min_scale");
  expect(ssz_weight_qparams(A, PTQ_F32, 4, 16, static_cast<const float*>(MIS), 8, 1, 20, 1e-10, 1e-5f, f, B, nullptr,
                            nullptr, nullptr),
         PTQ_ERR_ALIGN, "ssz align s");
  expect_launch(ssz_weight_qparams(A, PTQ_BF16, 4, 16, nullptr, 4, 1, 0, 0.0, 1e-5f, f, B, nullptr, nullptr, nullptr),
                "ssz", A, "ssz ok");

  // ssz_weight_qparams_asym
  int32_t* zp = reinterpret_cast<int32_t*>(D);
  expect(ssz_weight_qparams_asym(A, PTQ_F32, 4, 16, nullptr, 20, 1e-10, 1e-5f, f, nullptr, static_cast<int8_t*>(B),
                                 nullptr, nullptr, nullptr),
         PTQ_ERR_NULL, "asym null zp");
  expect(ssz_weight_qparams_asym(A, PTQ_F32, -1, 16, nullptr, 20, 1e-10, 1e-5f, f, zp, static_cast<int8_t*>(B),
                                 nullptr, nullptr, nullptr),
         PTQ_ERR_SHAPE, "asym N");
  expect(ssz_weight_qparams_asym(A, PTQ_F32, 4, 16, nullptr, -1, 1e-10, 1e-5f, f, zp, static_cast<int8_t*>(B),
                                 nullptr, nullptr, nullptr),
         PTQ_ERR_ARG, "asym max_iter");
  expect(ssz_weight_qparams_asym(A, PTQ_F32, 4, 16, nullptr, 20, 1e-10, 1e-5f, f, zp, static_cast<int8_t*>(MIS),
                                 nullptr, nullptr, nullptr),
         PTQ_ERR_ALIGN, "asym align");
  expect_launch(ssz_weight_qparams_asym(A, PTQ_F32, 4, 16, f, 20, 1e-10, 1e-5f, f, zp, static_cast<int8_t*>(B),
                                        nullptr, nullptr, nullptr),
                "ssz_asym", A, "asym ok");

  // quant_per_token_i8
  expect(quant_per_token_i8(A, PTQ_F32, 4, 16, nullptr, nullptr, f, nullptr), PTQ_ERR_NULL, "quant null");
  expect(quant_per_token_i8(A, PTQ_F32, 4, 0, nullptr, static_cast<int8_t*>(B), f, nullptr), PTQ_ERR_SHAPE, "quant K");
  expect(quant_per_token_i8(A, PTQ_F32, INT64_MAX / 16 + 1, 16, nullptr, static_cast<int8_t*>(B), f, nullptr),
         PTQ_ERR_SHAPE, "quant overflow");
  expect(quant_per_token_i8(A, PTQ_F32, 4, 16, nullptr, static_cast<int8_t*>(MIS), f, nullptr), PTQ_ERR_ALIGN,
         "quant align");
  expect_launch(quant_per_token_i8(A, PTQ_F32, 4, 16, f, static_cast<int8_t*>(B), f, nullptr), "quant_per_token", A,
                "quant ok");

  // w8a8_gemm_dequant
  const int8_t* xq = static_cast<const int8_t*>(A);
  const int8_t* wq = static_cast<const int8_t*>(B);
  float* y = static_cast<float*>(C);
  expect(w8a8_gemm_dequant(xq, wq, f, f, 4, 4, 16, nullptr, nullptr, nullptr), PTQ_ERR_NULL, "gemm null y");
  expect(w8a8_gemm_dequant(xq, wq, f, f, 4, 4, PTQ_GEMM_MAX_K + 16, y, nullptr, nullptr), PTQ_ERR_SHAPE, "gemm K max");
  expect(w8a8_gemm_dequant(xq, wq, f, f, (int64_t)1 << 31, 4, 16, y, nullptr, nullptr), PTQ_ERR_SHAPE, "gemm M");
  expect(w8a8_gemm_dequant(xq, wq, f, f, 4, 4, 16, y, static_cast<int32_t*>(MIS), nullptr), PTQ_ERR_ALIGN,
         "gemm align acc");
  expect_launch(w8a8_gemm_dequant(xq, wq, f, f, 4, 4, PTQ_GEMM_MAX_K, y, nullptr, nullptr), "gemm_dequant", xq,
                "gemm ok");

  // w8a8_gemm_fused
  expect(w8a8_gemm_fused(xq, wq, f, f, nullptr, 3, PTQ_OUT_F32, nullptr, nullptr, 4, 4, 16, C, nullptr, nullptr),
         PTQ_ERR_UNSUPPORTED, "fused act");
  expect(w8a8_gemm_fused(xq, wq, f, f, nullptr, 0, 3, nullptr, nullptr, 4, 4, 16, C, nullptr, nullptr), PTQ_ERR_DTYPE,
         "fused out");
  expect(w8a8_gemm_fused(xq, wq, f, f, nullptr, 0, PTQ_OUT_I8, f, nullptr, 4, 4, 16, C, nullptr, nullptr), PTQ_ERR_NULL,
         "fused i8 no scale");
  expect(w8a8_gemm_fused(xq, wq, f, f, nullptr, 0, PTQ_OUT_BF16, f, nullptr, 4, 4, 16, C, nullptr, nullptr),
         PTQ_ERR_ARG, "fused next_s on bf16");
  expect_launch(w8a8_gemm_fused(xq, wq, f, f, f, PTQ_ACT_GELU, PTQ_OUT_I8, f, f, 4, 4, 16, C, nullptr, nullptr),
                "gemm_fused", xq, "fused ok");

  // sq_act_scale_ema, weight_scale_per_tensor
  expect(sq_act_scale_ema(f, nullptr, 16, 1.0f, 1, f, f, nullptr, 0, nullptr), PTQ_ERR_ARG, "ema momentum");
  expect(sq_act_scale_ema(f, nullptr, 16, 0.9f, 1, f, f, f, 0, nullptr), PTQ_ERR_SHAPE, "ema rows");
  expect_launch(sq_act_scale_ema(f, nullptr, 16, 0.9f, 0, f, f, f, 8, nullptr), "tensor_scale", f, "ema ok");
  expect(weight_scale_per_tensor(f, nullptr, 16, -1.0f, f, nullptr, 0, nullptr), PTQ_ERR_ARG, "wscale min_scale");
  expect(weight_scale_per_tensor(f, nullptr, 16, 1e-5f, f, f, 0, nullptr), PTQ_ERR_SHAPE, "wscale N");
  expect_launch(weight_scale_per_tensor(f, f, 16, 1e-5f, f, f, 4, nullptr), "tensor_scale", f, "wscale ok");

  // quant_static_i8
  int8_t* q = static_cast<int8_t*>(B);
  expect(quant_static_i8(A, PTQ_F32, 4, 16, f, 0, f, q, nullptr, nullptr), PTQ_ERR_ARG, "static fold");
  expect(quant_static_i8(A, PTQ_F32, 4, 131088, nullptr, 0, f, q, nullptr, nullptr), PTQ_ERR_SHAPE, "static cols max");
  expect(quant_static_i8(MIS, PTQ_F32, 4, 16, nullptr, 0, f, q, nullptr, nullptr), PTQ_ERR_ALIGN, "static align");
  expect_launch(quant_static_i8(A, PTQ_BF16, 4, 16, f, PTQ_FOLD_MUL, f, q, f, nullptr), "quant_static", A,
                "static ok");

  // a failed launch comes back as PTQ_ERR_HIP with the runtime's message
  g_stub_status = 1;  // hipErrorInvalidValue
  expect(sq_smooth_factors(f, f, 16, 0.5f, f, nullptr), PTQ_ERR_HIP, "launch failure");
  g_stub_status = 0;

  free(buf);
  printf("abi sanitizer driver: %d checks, %d failed\n", g_checks, g_fail);
  return g_fail ? 1 : 0;
}
