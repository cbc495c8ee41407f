// A client of the C ABI with no Python and no torch: device memory from hipMalloc, one stream of its own, and the
// five calls of the path (calibration, smoothing factors, MinMax + SSZ, per-token quantization, GEMM + dequant)
// on fp32 inputs read from files; every output is written back to files for the test to compare.
//
//   ptq_path DIR T K N ALPHA     reads DIR/x.f32 [T,K] and DIR/w.f32 [N,K]; writes DIR/{ax,aw,s,S,d,y}.f32,
//                                DIR/{wq,xq}.i8, DIR/{it,acc}.i32
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <string>
#include <vector>

#include "ptq.h"

#define HIP_OK(call)                                                                       \
  do {                                                                                     \
    hipError_t e_ = (call);                                                                \
    if (e_ != hipSuccess) {                                                                \
      std::fprintf(stderr, "%s failed: %s\n", #call, hipGetErrorString(e_));               \
      std::exit(2);                                                                        \
    }                                                                                      \
  } while (0)

#define PTQ_OK_(call)                                                                      \
  do {                                                                                     \
    ptq_status s_ = (call);                                                                \
    if (s_ != PTQ_OK) {                                                                    \
      std::fprintf(stderr, "%s: %s (%s)\n", #call, ptq_status_string(s_), ptq_last_error()); \
      std::exit(3);                                                                        \
    }                                                                                      \
  } while (0)

template <typename T>
static std::vector<T> read_file(const std::string& path, size_t n) {
  std::vector<T> v(n);
  FILE* f = std::fopen(path.c_str(), "rb");
  if (!f || std::fread(v.data(), sizeof(T), n, f) != n) {
    std::fprintf(stderr, "cannot read %zu values from %s\n", n, path.c_str());
    std::exit(4);
  }
  std::fclose(f);
  return v;
}

template <typename T>
static void write_file(const std::string& path, const T* d_src, size_t n) {
  std::vector<T> v(n);
  HIP_OK(hipMemcpy(v.data(), d_src, n * sizeof(T), hipMemcpyDeviceToHost));
  FILE* f = std::fopen(path.c_str(), "wb");
  if (!f || std::fwrite(v.data(), sizeof(T), n, f) != n) {
    std::fprintf(stderr, "cannot write %s\n", path.c_str());
    std::exit(4);
  }
  std::fclose(f);
}

template <typename T>
static T* device(size_t n) {
  void* p = nullptr;
  HIP_OK(hipMalloc(&p, n * sizeof(T) + 16));
  return static_cast<T*>(p);
}

int main(int argc, char** argv) {
  if (argc != 6) {
    std::fprintf(stderr, "usage: %s DIR T K N ALPHA\n", argv[0]);
    return 1;
  }
  const std::string dir = argv[1];
  const int64_t T = std::atoll(argv[2]), K = std::atoll(argv[3]), N = std::atoll(argv[4]);
  const float alpha = std::strtof(argv[5], nullptr);
  if (ptq_abi_version() != PTQ_ABI_VERSION) {
    std::fprintf(stderr, "ABI version %d, header %d\n", ptq_abi_version(), PTQ_ABI_VERSION);
    return 5;
  }
  const std::vector<float> x = read_file<float>(dir + "/x.f32", size_t(T * K));
  const std::vector<float> w = read_file<float>(dir + "/w.f32", size_t(N * K));

  hipStream_t st;
  HIP_OK(hipStreamCreate(&st));
  float* d_x = device<float>(T * K);
  float* d_w = device<float>(N * K);
  float *d_ax = device<float>(K), *d_aw = device<float>(K), *d_s = device<float>(K);
  float *d_S = device<float>(N), *d_d = device<float>(T), *d_y = device<float>(T * N);
  int8_t *d_wq = device<int8_t>(N * K), *d_xq = device<int8_t>(T * K);
  int32_t *d_it = device<int32_t>(N), *d_acc = device<int32_t>(T * N);
  HIP_OK(hipMemcpyAsync(d_x, x.data(), x.size() * sizeof(float), hipMemcpyHostToDevice, st));
  HIP_OK(hipMemcpyAsync(d_w, w.data(), w.size() * sizeof(float), hipMemcpyHostToDevice, st));

  PTQ_OK_(sq_absmax_calib(d_x, PTQ_F32, T, K, d_ax, 0, st));
  PTQ_OK_(sq_absmax_calib(d_w, PTQ_F32, N, K, d_aw, 0, st));
  PTQ_OK_(sq_smooth_factors(d_ax, d_aw, K, alpha, d_s, st));
  PTQ_OK_(ssz_weight_qparams(d_w, PTQ_F32, N, K, d_s, 8, 1, PTQ_SSZ_MAX_ITER, PTQ_SSZ_THRESHOLD, PTQ_SSZ_MIN_SCALE,
                             d_S, d_wq, d_it, nullptr, st));
  PTQ_OK_(quant_per_token_i8(d_x, PTQ_F32, T, K, d_s, d_xq, d_d, st));
  PTQ_OK_(w8a8_gemm_dequant(d_xq, d_wq, d_d, d_S, T, N, K, d_y, d_acc, st));
  HIP_OK(hipStreamSynchronize(st));

  write_file(dir + "/ax.f32", d_ax, K);
  write_file(dir + "/aw.f32", d_aw, K);
  write_file(dir + "/s.f32", d_s, K);
  write_file(dir + "/S.f32", d_S, N);
  write_file(dir + "/wq.i8", d_wq, N * K);
  write_file(dir + "/it.i32", d_it, N);
  write_file(dir + "/xq.i8", d_xq, T * K);
  write_file(dir + "/d.f32", d_d, T);
  write_file(dir + "/y.f32", d_y, T * N);
  write_file(dir + "/acc.i32", d_acc, T * N);
  for (void* p : {(void*)d_x, (void*)d_w, (void*)d_ax, (void*)d_aw, (void*)d_s, (void*)d_S, (void*)d_d, (void*)d_y,
                  (void*)d_wq, (void*)d_xq, (void*)d_it, (void*)d_acc})
    HIP_OK(hipFree(p));
  HIP_OK(hipStreamDestroy(st));
  std::printf("ptq_path: T=%lld K=%lld N=%lld done\n", (long long)T, (long long)K, (long long)N);
  return 0;
}
