// Checks the kernels' division helpers (post_int8_quantization_amd/csrc/ptq_dev.hpp) against the IEEE quotient
// (this file is compiled with correctly rounded fp32 division), one thread per value:
//  * rcp_rn(s) against 1.0f / s for every fp32 s in [2^-100, 2^101): every mantissa of each of the 201 binades;
//  * rcp64(s) on the same values: its relative error |1 - s rcp64(s)| (one fused multiply-add, exact to within a
//    rounding of that small residual) at most 2^-51, and the largest one seen;
//  * quot64((double)x, rcp64(s)) against x / s, bit for bit wherever x / s is a normal fp32 number (else its
//    rounding to an integer): for 4096 divisors s (special values, then seeded random mantissas and exponents in
//    [-100, 100]), every mantissa of the twelve binades of x that put x / s in [2^-4, 2^9); and for the first 8
//    divisors every non-negative finite fp32 x (every exponent field 0..254).
// Prints the counts checked and the mismatches, and, for contrast, the mismatches of the hardware reciprocal alone
// and of the fp32 product x * rcp_rn(s); exit status 0 when it ran.
#include <cstdio>
#include <cstdint>
#include <vector>

#include "../../post_int8_quantization_amd/csrc/ptq_dev.hpp"

namespace {

constexpr int kLoExp = -100, kBinades = 201;

__global__ void k_check(unsigned long long* __restrict__ bad, unsigned long long* __restrict__ raw_bad,
                        unsigned int* __restrict__ first, unsigned long long* __restrict__ r64_bad,
                        unsigned long long* __restrict__ r64_max) {
  const uint64_t id = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= ((uint64_t)kBinades << 23)) return;  // the grid is a whole number of waves of this range
  const int e = kLoExp + (int)(id >> 23);
  const uint32_t bits = ((uint32_t)(e + 127) << 23) | (uint32_t)(id & 0x7FFFFFu);
  const float s = __uint_as_float(bits);
  const float ref = 1.0f / s;
  {
    const double res = fabs(__builtin_fma(-(double)s, ptq::rcp64(s), 1.0));
    if (!(res <= 0x1p-51)) atomicAdd(r64_bad, 1ull);
    double m = res;
    for (int o = 32; o > 0; o >>= 1) m = fmax(m, __shfl_xor(m, o));
    if ((threadIdx.x & 63) == 0) atomicMax(r64_max, (unsigned long long)__double_as_longlong(m));
  }
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

// quot64 sweep.  Block (x, y): divisor divs[y]; thread t of block x covers the mantissas t + 256 (x kMpt + j),
// j < kMpt, of every x binade in [lo, hi] -- exponent fields (rel ? field(s) : 0) + lo .. + hi, each in 0..254.
constexpr int kMpt = 16;
constexpr unsigned kGridX = (1u << 23) / (256u * kMpt);  // 2048 blocks cover the 2^23 mantissas

struct QuotCounts {
  unsigned long long bad;       // normal quotients that differ, or codes that differ
  unsigned long long sub_diff;  // subnormal quotients within one step (allowed), codes equal
  unsigned long long f32_bad;   // contrast: fl32(x * rcp_rn(s)) differs from x / s (normal quotients)
  unsigned int first[8];        // first offenders: (s bits, x bits) pairs
};

__global__ void k_quot(const float* __restrict__ divs, int rel, int lo, int hi, QuotCounts* __restrict__ out) {
  __shared__ unsigned long long blk_f32_bad;  // the block's contrast count, one global atomic per block
  if (threadIdx.x == 0) blk_f32_bad = 0;
  __syncthreads();
  const float s = divs[blockIdx.y];
  const double r64 = ptq::rcp64(s);
  const float rs = ptq::rcp_rn(s);
  const int fs = (int)((__float_as_uint(s) >> 23) & 0xFFu);
  unsigned int f32_bad = 0;
  for (int k = lo; k <= hi; ++k) {
    const int fx = (rel ? fs : 0) + k;
    if (fx < 0 || fx > 254) continue;
    for (int j = 0; j < kMpt; ++j) {
      const uint32_t mant = threadIdx.x + 256u * (blockIdx.x * kMpt + j);
      const uint32_t xb = ((uint32_t)fx << 23) | mant;
      const float x = __uint_as_float(xb);
      const float ref = x / s;
      const float got = ptq::quot64((double)x, r64);
      const bool normal = !(fabsf(ref) < 0x1p-126f);
      if (__float_as_uint(got) != __float_as_uint(ref)) {
        const uint32_t gb = __float_as_uint(got), rb = __float_as_uint(ref);
        const uint32_t step = gb > rb ? gb - rb : rb - gb;  // same sign: the distance in subnormal steps
        if (normal || step > 1 || __builtin_rintf(got) != __builtin_rintf(ref)) {
          const unsigned long long n = atomicAdd(&out->bad, 1ull);
          if (n < 4) {
            out->first[2 * n] = __float_as_uint(s);
            out->first[2 * n + 1] = xb;
          }
        } else {
          atomicAdd(&out->sub_diff, 1ull);
        }
      }
      if (normal && __float_as_uint(x * rs) != __float_as_uint(ref)) ++f32_bad;
    }
  }
  if (f32_bad) atomicAdd(&blk_f32_bad, (unsigned long long)f32_bad);
  __syncthreads();
  if (threadIdx.x == 0 && blk_f32_bad) atomicAdd(&out->f32_bad, blk_f32_bad);
}

uint64_t splitmix(uint64_t& z) {
  uint64_t r = (z += 0x9E3779B97F4A7C15ull);
  r = (r ^ (r >> 30)) * 0xBF58476D1CE4E5B9ull;
  r = (r ^ (r >> 27)) * 0x94D049BB133111EBull;
  return r ^ (r >> 31);
}

float f32_of(int e, uint32_t mant) {
  const uint32_t b = ((uint32_t)(e + 127) << 23) | (mant & 0x7FFFFFu);
  float f;
  __builtin_memcpy(&f, &b, 4);
  return f;
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
  // [0] mismatches, [1] raw mismatches, [2..3] 4 first offenders (as uint32), [4] rcp64 over the bound,
  // [5] rcp64's largest residual (fp64 bits)
  unsigned long long* d = nullptr;
  CK(hipMalloc(&d, 48));
  CK(hipMemset(d, 0, 48));
  const uint64_t total = (uint64_t)kBinades << 23;
  k_check<<<(unsigned)((total + 255) / 256), 256>>>(d, d + 1, reinterpret_cast<unsigned int*>(d + 2), d + 4, d + 5);
  CK(hipGetLastError());
  CK(hipDeviceSynchronize());
  unsigned long long h[6];
  CK(hipMemcpy(h, d, 48, hipMemcpyDeviceToHost));
  const unsigned int* f = reinterpret_cast<const unsigned int*>(h + 2);
  printf("checked %llu mismatches %llu approximation_mismatches %llu\n", (unsigned long long)total, h[0], h[1]);
  for (unsigned long long i = 0; i < h[0] && i < 4; ++i) printf("offender 0x%08x\n", f[i]);
  double r64_max;
  __builtin_memcpy(&r64_max, &h[5], 8);
  printf("rcp64 checked %llu over_bound %llu max_residual %.6e\n", (unsigned long long)total, h[4], r64_max);
  CK(hipFree(d));

  // divisors: special values first, then seeded random ones
  constexpr int kDivs = 4096, kFull = 8;
  std::vector<float> divs = {1.0f, f32_of(0, 1), f32_of(0, 0x7FFFFF), f32_of(-100, 0), f32_of(100, 0x7FFFFF),
                             3.0f, 0.1f, 1.0f / 127.0f};
  uint64_t z = 20240917;
  while ((int)divs.size() < kDivs) {
    const uint64_t r = splitmix(z);
    divs.push_back(f32_of(-100 + (int)((r >> 32) % 201u), (uint32_t)r));
  }
  float* dd = nullptr;
  QuotCounts* dq = nullptr;
  CK(hipMalloc(&dd, sizeof(float) * kDivs));
  CK(hipMalloc(&dq, sizeof(QuotCounts)));
  CK(hipMemcpy(dd, divs.data(), sizeof(float) * kDivs, hipMemcpyHostToDevice));
  CK(hipMemset(dq, 0, sizeof(QuotCounts)));
  // x / s in [2^-4, 2^9): x exponent fields field(s) - 3 .. field(s) + 8 (all in 0..254 for s in [2^-100, 2^101))
  k_quot<<<dim3(kGridX, kDivs), 256>>>(dd, 1, -3, 8, dq);
  CK(hipGetLastError());
  // every non-negative finite x for the special divisors
  k_quot<<<dim3(kGridX, kFull), 256>>>(dd, 0, 0, 254, dq);
  CK(hipGetLastError());
  CK(hipDeviceSynchronize());
  QuotCounts q;
  CK(hipMemcpy(&q, dq, sizeof(QuotCounts), hipMemcpyDeviceToHost));
  const unsigned long long qtotal = ((unsigned long long)kDivs * 12 + (unsigned long long)kFull * 255) << 23;
  printf("quot64 checked %llu mismatches %llu subnormal_within_one_step %llu f32_product_mismatches %llu\n", qtotal,
         q.bad, q.sub_diff, q.f32_bad);
  for (unsigned long long i = 0; i < q.bad && i < 4; ++i)
    printf("quot64 offender s 0x%08x x 0x%08x\n", q.first[2 * i], q.first[2 * i + 1]);
  CK(hipFree(dq));
  CK(hipFree(dd));
  return 0;
}
