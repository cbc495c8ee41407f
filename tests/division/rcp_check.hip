// Checks the kernels' reciprocal rcp_rn (post_int8_quantization_amd/csrc/ptq_dev.hpp) against the IEEE quotient
// 1.0f / s (this file is compiled with correctly rounded fp32 division) for every fp32 s in [2^-100, 2^101):
// every mantissa of each of the 201 binades, one thread per value.  Prints the count checked, the mismatches of
// rcp_rn, and (for contrast) the mismatches of the hardware approximation alone; exit status 0 when it ran.
#include <cstdio>
#include <cstdint>

#include "../../post_int8_quantization_amd/csrc/ptq_dev.hpp"

namespace {

constexpr int kLoExp = -100, kBinades = 201;

__global__ void k_check(unsigned long long* __restrict__ bad, unsigned long long* __restrict__ raw_bad,
                        unsigned int* __restrict__ first) {
  const uint64_t id = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= ((uint64_t)kBinades << 23)) return;
  const int e = kLoExp + (int)(id >> 23);
  const uint32_t bits = ((uint32_t)(e + 127) << 23) | (uint32_t)(id & 0x7FFFFFu);
  const float s = __uint_as_float(bits);
  const float ref = 1.0f / s;
  if (__float_as_uint(ptq::rcp_rn(s)) != __float_as_uint(ref)) {
    const unsigned long long n = atomicAdd(bad, 1ull);
    if (n < 4) first[n] = bits;
  }
  if (__float_as_uint(__builtin_amdgcn_rcpf(s)) != __float_as_uint(ref)) {
    // one atomic per wave for the contrast count (a tenth of the values differ)
    const uint64_t m = __ballot(1);
    if ((threadIdx.x & 63) == __builtin_ctzll(m)) atomicAdd(raw_bad, (unsigned long long)__builtin_popcountll(m));
  }
}

}  // namespace

#define CK(x)                                                                         \
  do {                                                                                \
    hipError_t e_ = (x);                                                              \
    if (e_ != hipSuccess) {                                                           \
      fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));                  \
      return 2;                                                                       \
    }                                                                                 \
  } while (0)

int main() {
  unsigned long long* d = nullptr;  // [0] mismatches, [1] raw mismatches, then 4 first offenders (as uint32)
  CK(hipMalloc(&d, 32));
  CK(hipMemset(d, 0, 32));
  const uint64_t total = (uint64_t)kBinades << 23;
  k_check<<<(unsigned)((total + 255) / 256), 256>>>(d, d + 1, reinterpret_cast<unsigned int*>(d + 2));
  CK(hipGetLastError());
  CK(hipDeviceSynchronize());
  unsigned long long h[4];
  CK(hipMemcpy(h, d, 32, hipMemcpyDeviceToHost));
  const unsigned int* f = reinterpret_cast<const unsigned int*>(h + 2);
  printf("checked %llu mismatches %llu approximation_mismatches %llu\n", (unsigned long long)total, h[0], h[1]);
  for (unsigned long long i = 0; i < h[0] && i < 4; ++i) printf("offender 0x%08x\n", f[i]);
  CK(hipFree(d));
  return 0;
}
