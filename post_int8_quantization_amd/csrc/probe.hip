// probe.hip -- matrix-core clock probe, VALU probe and HBM stream probe (measurement aids for the rooflines, not
// steps of the method).
//
// Every block (one per CU: 512 threads, two waves per SIMD, 64 KB of LDS) issues int8 MFMAs back to back into
// 32 independent accumulators, on operands drawn from a hash of (seed, thread, register), so consecutive
// instructions see unrelated bytes as the GEMM's do.  Wave 0 of each block reads the shader-clock counter
// (s_memtime) and the constant 100 MHz counter (s_memrealtime) around the loop; their ratio is the shader
// clock the chip held while doing it.  Kinds:
//   0  v_mfma_i32_16x16x64_i8, pseudo-random operands
//   1  v_mfma_i32_32x32x32_i8, pseudo-random operands (the same multiply-adds per iteration)
//   2  as 0, plus the GEMM kernel's operand traffic: 24 ds_read_b128 of pseudo-random LDS per 64 MFMAs
//   3  as 0, all operands zero
// The published dense int8 peak assumes the 2.4 GHz top clock; under a power limit the clock that random
// operands allow is lower, and kinds 0 and 2 measure what the GEMM's own instruction mix can reach.
//
// The VALU probe measures the ALU bound of the SSZ search the same way, one wave per block (64 threads) so the
// caller sets the waves per SIMD by the block count, wave 0 timing its loop as above.  Kinds:
//   0  the SSZ pass loop alone: 64 fp32 row values per lane held in fp64, per pass the fp64 reciprocal of the
//      scale, then per element the fp64 product rounded to fp32, round, clamp to [-127, 127], widening of the code,
//      the fp64 multiply-add of sum w q and the fp32 one of sum q^2 -- the search's own instructions, without its
//      reductions, decisions or memory traffic
//   1  as 0, plus the per-pass 64-lane butterflies of both sums (fp64 and integer)
//   2  fp32 multiply-adds only (8 independent chains per lane)
//   3  fp64 multiply-adds only (8 independent chains per lane)
//
// The HBM stream probe measures the memory bound the same way: the rate at which plain streaming reads (or a
// copy) of a buffer far larger than the 256 MB last-level cache move bytes, with each wave reading 1 KB of
// consecutive bytes per load instruction and 16 such loads in flight per lane -- the access pattern of the
// path's HBM-bound kernels without their arithmetic.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

#include "../../include/ptq_probe.h"
#include "ptq_dev.hpp"

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int hash3(uint32_t seed, uint32_t a, uint32_t b) {
  uint32_t h = seed * 0x9E3779B9u ^ (a * 0x85EBCA6Bu + b * 0xC2B2AE35u + 0x27D4EB2Fu);
  h ^= h >> 15;
  h *= 0x2C1B3C6Du;
  h ^= h >> 12;
  h *= 0x297A2D39u;
  h ^= h >> 15;
  return (int)h;
}

constexpr int kLdsChunks = 4096;  // 64 KB of 16-byte chunks

template <int KIND>
__global__ __launch_bounds__(512) void k_probe_mfma(int iters, uint32_t seed, unsigned long long* __restrict__ out) {
  __shared__ uint4 sm[kLdsChunks];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int i = tid; i < kLdsChunks; i += 512)
    sm[i] = make_uint4((uint32_t)hash3(seed, i, 0), (uint32_t)hash3(seed, i, 1), (uint32_t)hash3(seed, i, 2),
                       (uint32_t)hash3(seed, i, 3));
  __syncthreads();
  const uint32_t t = blockIdx.x * 512u + tid;
  int sink = 0;
  unsigned long long c0 = 0, r0 = 0;
  if constexpr (KIND == 1) {
    v16i acc[4][2];
    v4i a[4], b[2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) a[i][e] = hash3(seed, t, 16 + i * 4 + e);
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) b[j][e] = hash3(seed, t, 64 + j * 4 + e);
    c0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 2; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[i], b[j], acc[i][j], 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) sink ^= acc[i][j][r];
  } else {
    v4i acc[8][4];
    v4i a[8], b[4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = v4i{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) a[i][e] = KIND == 3 ? 0 : hash3(seed, t, 16 + i * 4 + e);
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) b[j][e] = KIND == 3 ? 0 : hash3(seed, t, 64 + j * 4 + e);
    c0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], b[j], acc[i][j], 0, 0, 0);
          if constexpr (KIND == 2) {
            // the GEMM's per-wave fragment reads: an A fragment after each group, a B fragment after the first four
            const uint4 v = sm[((wave * 8 + i) * 64 + lane + ks * 16 + it) & (kLdsChunks - 1)];
            a[i] = v4i{(int)v.x, (int)v.y, (int)v.z, (int)v.w};
            if (i < 4) {
              const uint4 w = sm[((wave * 4 + i) * 64 + lane + kLdsChunks / 2 + ks * 16 + it) & (kLdsChunks - 1)];
              b[i] = v4i{(int)w.x, (int)w.y, (int)w.z, (int)w.w};
            }
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) sink ^= acc[i][j][0] ^ acc[i][j][1] ^ acc[i][j][2] ^ acc[i][j][3];
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if (tid == 0) {
    out[3 * blockIdx.x] = c1 - c0;
    out[3 * blockIdx.x + 1] = r1 - r0;
  }
  // keeps the accumulators live; the value itself is meaningless
  if (lane == 0 && wave == 0) out[3 * blockIdx.x + 2] = (unsigned long long)(uint32_t)sink;
}

template <int KIND>
__global__ __launch_bounds__(64) __attribute__((amdgpu_waves_per_eu(2))) void k_probe_valu(
    int iters, uint32_t seed, unsigned long long* __restrict__ out) {
  const int lane = threadIdx.x;
  const uint32_t t = blockIdx.x * 64u + lane;
  unsigned long long c0 = 0, r0 = 0;
  double sink = 0.0;
  if constexpr (KIND <= 1) {
    // row values in [-1/8, 1/8), as fp32 then widened; scales near max / 127, alternating between two values
    double wh[64];
#pragma unroll
    for (int i = 0; i < 64; ++i) wh[i] = (double)((float)(hash3(seed, t, i) >> 8) * 0x1p-26f);
    const float s0 = 0.125f / 127.0f, s1 = s0 * 1.0009765625f;
    double P = 0.0;
    float R2 = 0.0f;
    c0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
      const double r64 = ptq::rcp64((it & 1) ? s1 : s0);
      double a = 0.0;
      float b = 0.0f;
#pragma unroll
      for (int i = 0; i < 64; ++i) {
        const float q = fminf(fmaxf(__builtin_rintf(ptq::quot64(wh[i], r64)), -127.0f), 127.0f);
        a = __builtin_fma(wh[i], (double)q, a);
        b = __builtin_fmaf(q, q, b);
      }
      if constexpr (KIND == 1) {
        a = ptq::wave_sum(a);
        b = (float)ptq::wave_sum((int)b);
      }
      P += a;
      R2 += b;
    }
    sink = P + (double)R2;
  } else if constexpr (KIND == 2) {
    float f[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = (float)(hash3(seed, t, i) & 0xFFFF) * 0x1p-16f;
    const float m = 0.99998f, c = (float)(hash3(seed, t, 99) & 0xFF) * 0x1p-20f;
    c0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int u = 0; u < 16; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = __builtin_fmaf(f[i], m, c);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) sink += (double)f[i];
  } else {
    double d[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) d[i] = (double)(hash3(seed, t, i) & 0xFFFF) * 0x1p-16;
    const double m = 0.99998, c = (double)(hash3(seed, t, 99) & 0xFF) * 0x1p-20;
    c0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
    for (int it = 0; it < iters; ++it) {
#pragma unroll
      for (int u = 0; u < 16; ++u)
#pragma unroll
        for (int i = 0; i < 8; ++i) d[i] = __builtin_fma(d[i], m, c);
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) sink += d[i];
  }
  const unsigned long long c1 = __builtin_amdgcn_s_memtime();
  const unsigned long long r1 = __builtin_amdgcn_s_memrealtime();
  if (lane == 0) {
    out[3 * blockIdx.x] = c1 - c0;
    out[3 * blockIdx.x + 1] = r1 - r0;
    out[3 * blockIdx.x + 2] = (unsigned long long)__double_as_longlong(sink);  // keeps the loop live; meaningless
  }
}

constexpr int kStreamThreads = 256;
constexpr int kStreamUnroll = 16;  // 16-byte loads in flight per lane

// kind 0: read every 16-byte vector of src once (a per-block xor of the words keeps the loads live: out[block]);
// kind 1: copy src to dst.  Blocks take rounds of 64 KB of consecutive bytes in turn; block 0 takes the tail.
template <int KIND>
__global__ __launch_bounds__(kStreamThreads) void k_probe_stream(const u32x4* __restrict__ src, uint64_t n16,
                                                                 u32x4* __restrict__ dst, uint32_t* __restrict__ out) {
  constexpr uint64_t R = (uint64_t)kStreamThreads * kStreamUnroll;  // vectors per round
  __shared__ uint32_t red[kStreamThreads / 64];
  const int tid = threadIdx.x;
  const uint64_t rounds = n16 / R;
  uint32_t x = 0;
  for (uint64_t r = blockIdx.x; r < rounds; r += gridDim.x) {
    const uint64_t base = r * R + (uint64_t)tid;
    u32x4 v[kStreamUnroll];
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) v[u] = __builtin_nontemporal_load(src + base + (uint64_t)u * kStreamThreads);
#pragma unroll
    for (int u = 0; u < kStreamUnroll; ++u) {
      if constexpr (KIND == 1) __builtin_nontemporal_store(v[u], dst + base + (uint64_t)u * kStreamThreads);
      else x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
  }
  if (blockIdx.x == 0) {
    for (uint64_t i = rounds * R + (uint64_t)tid; i < n16; i += kStreamThreads) {
      const u32x4 v = src[i];
      if constexpr (KIND == 1) dst[i] = v;
      else x ^= v.x ^ v.y ^ v.z ^ v.w;
    }
  }
  if constexpr (KIND == 0) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) x ^= (uint32_t)__shfl_xor((int)x, o);
    if ((tid & 63) == 0) red[tid >> 6] = x;
    __syncthreads();
    if (tid == 0) {
      uint32_t t = 0;
#pragma unroll
      for (int w = 0; w < kStreamThreads / 64; ++w) t ^= red[w];
      out[blockIdx.x] = t;
    }
  }
}

thread_local char g_probe_err[256] = "";

}  // namespace

extern "C" {

const char* ptq_probe_last_error(void) { return g_probe_err; }

int ptq_probe_mfma(int kind, int blocks, int iters, uint32_t seed, uint64_t* out, void* stream) {
  if (!out) {
    snprintf(g_probe_err, sizeof g_probe_err, "ptq_probe_mfma: out is required");
    return PTQ_PROBE_ERR_ARG;
  }
  if (kind < 0 || kind > 3 || blocks < 1 || blocks > 65536 || iters < 1 || iters > 1000000) {
    snprintf(g_probe_err, sizeof g_probe_err, "ptq_probe_mfma: kind=%d blocks=%d iters=%d out of range", kind, blocks,
             iters);
    return PTQ_PROBE_ERR_ARG;
  }
  if (reinterpret_cast<uintptr_t>(out) & 7u) {
    snprintf(g_probe_err, sizeof g_probe_err, "ptq_probe_mfma: out must be 8-byte aligned");
    return PTQ_PROBE_ERR_ARG;
  }
  hipStream_t s = (hipStream_t)stream;
  unsigned long long* o = reinterpret_cast<unsigned long long*>(out);
  switch (kind) {
    case 0: k_probe_mfma<0><<<blocks, 512, 0, s>>>(iters, seed, o); break;
    case 1: k_probe_mfma<1><<<blocks, 512, 0, s>>>(iters, seed, o); break;
    case 2: k_probe_mfma<2><<<blocks, 512, 0, s>>>(iters, seed, o); break;
    default: k_probe_mfma<3><<<blocks, 512, 0, s>>>(iters, seed, o); break;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    snprintf(g_probe_err, sizeof g_probe_err, "ptq_probe_mfma: launch failed: %s", hipGetErrorString(e));
    return PTQ_PROBE_ERR_HIP;
  }
  return 0;
}

int ptq_probe_valu(int kind, int blocks, int iters, uint32_t seed, uint64_t* out, void* stream) {
  if (!out) {
    snprintf(g_probe_err, sizeof g_probe_err, "ptq_probe_valu: out is required");
    return PTQ_PROBE_ERR_ARG;
  }
  if (kind < 0 || kind > 3 || blocks < 1 || blocks > 65536 || iters < 1 || iters > 1000000) {
    snprintf(g_probe_err, sizeof g_probe_err, "ptq_probe_valu: kind=%d blocks=%d iters=%d out of range", kind, blocks,
             iters);
    return PTQ_PROBE_ERR_ARG;
  }
  if (reinterpret_cast<uintptr_t>(out) & 7u) {
    snprintf(g_probe_err, sizeof g_probe_err, "ptq_probe_valu: out must be 8-byte aligned");
    return PTQ_PROBE_ERR_ARG;
  }
  hipStream_t s = (hipStream_t)stream;
  unsigned long long* o = reinterpret_cast<unsigned long long*>(out);
  switch (kind) {
    case 0: k_probe_valu<0><<<blocks, 64, 0, s>>>(iters, seed, o); break;
    case 1: k_probe_valu<1><<<blocks, 64, 0, s>>>(iters, seed, o); break;
    case 2: k_probe_valu<2><<<blocks, 64, 0, s>>>(iters, seed, o); break;
    default: k_probe_valu<3><<<blocks, 64, 0, s>>>(iters, seed, o); break;
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    snprintf(g_probe_err, sizeof g_probe_err, "ptq_probe_valu: launch failed: %s", hipGetErrorString(e));
    return PTQ_PROBE_ERR_HIP;
  }
  return 0;
}

int ptq_probe_stream(int kind, const void* src, uint64_t bytes, void* dst, int blocks, uint32_t* out, void* stream) {
  if (kind < 0 || kind > 1 || blocks < 1 || blocks > 65536 || bytes == 0 || (bytes & 15u) != 0) {
    snprintf(g_probe_err, sizeof g_probe_err, "ptq_probe_stream: kind=%d blocks=%d bytes=%llu out of range", kind,
             blocks, (unsigned long long)bytes);
    return PTQ_PROBE_ERR_ARG;
  }
  if (!src || (kind == 1 && !dst) || (kind == 0 && !out)) {
    snprintf(g_probe_err, sizeof g_probe_err, "ptq_probe_stream: src, and dst (copy) or out (read), are required");
    return PTQ_PROBE_ERR_ARG;
  }
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst)) & 15u ||
      reinterpret_cast<uintptr_t>(out) & 3u) {
    snprintf(g_probe_err, sizeof g_probe_err, "ptq_probe_stream: src and dst must be 16-byte aligned, out 4-byte");
    return PTQ_PROBE_ERR_ARG;
  }
  hipStream_t s = (hipStream_t)stream;
  const u32x4* sp = reinterpret_cast<const u32x4*>(src);
  u32x4* dp = reinterpret_cast<u32x4*>(dst);
  if (kind == 0) k_probe_stream<0><<<blocks, kStreamThreads, 0, s>>>(sp, bytes / 16, dp, out);
  else k_probe_stream<1><<<blocks, kStreamThreads, 0, s>>>(sp, bytes / 16, dp, out);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    snprintf(g_probe_err, sizeof g_probe_err, "ptq_probe_stream: launch failed: %s", hipGetErrorString(e));
    return PTQ_PROBE_ERR_HIP;
  }
  return 0;
}

}  // extern "C"
