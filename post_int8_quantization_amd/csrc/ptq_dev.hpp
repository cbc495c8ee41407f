// ptq_dev.hpp -- device helpers shared by the gfx950 kernels of libptq.
//
// Wavefronts are 64 lanes.  Cross-lane reductions use xor butterflies: every
// lane ends with the same bits (fp addition is commutative, so partner lanes
// add the same two partials), which keeps per-row decisions uniform.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ptq.h"

namespace ptq {

constexpr int kWave = 64;

typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte load of data read exactly once (streaming; nontemporal hint)
__device__ __forceinline__ uint4 load_once(const void* p) {
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(v.x, v.y, v.z, v.w);
}

// bf16 pair in one dword -> two fp32 (exact widening)
__device__ __forceinline__ float bf16_lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t u) { return __uint_as_float(u & 0xFFFF0000u); }

// Load 8 consecutive elements (16 bytes of bf16 or 32 bytes of fp32) as fp32.
template <int DT>
__device__ __forceinline__ void load8(const void* base, int64_t elem, float (&v)[8]) {
  if constexpr (DT == PTQ_BF16) {
    const uint4 d = load_once(reinterpret_cast<const uint16_t*>(base) + elem);
    v[0] = bf16_lo(d.x); v[1] = bf16_hi(d.x);
    v[2] = bf16_lo(d.y); v[3] = bf16_hi(d.y);
    v[4] = bf16_lo(d.z); v[5] = bf16_hi(d.z);
    v[6] = bf16_lo(d.w); v[7] = bf16_hi(d.w);
  } else {
    const float* p = reinterpret_cast<const float*>(base) + elem;
    const uint4 a = load_once(p), b = load_once(p + 4);
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y); v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y); v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}

// Symmetric code of one value: clamp(rne(x * inv), -qmax, qmax), as fp32.
__device__ __forceinline__ float code_f(float x, float inv, float qmax) {
  const float t = x * inv;
  return fminf(fmaxf(__builtin_rintf(t), -qmax), qmax);
}

// Four codes in [-128,127] packed into one dword, element 0 in the low byte.
__device__ __forceinline__ uint32_t pack4_i8(float a, float b, float c, float d) {
  const uint32_t ia = (uint32_t)(int)a & 0xFFu, ib = (uint32_t)(int)b & 0xFFu;
  const uint32_t ic = (uint32_t)(int)c & 0xFFu, id = (uint32_t)(int)d & 0xFFu;
  return ia | (ib << 8) | (ic << 16) | (id << 24);
}

// Eight int4 codes packed into one dword: element 2i in the low nibble of byte i.
__device__ __forceinline__ uint32_t pack8_i4(const float* q) {
  uint32_t r = 0;
#pragma unroll
  for (int e = 0; e < 8; ++e) r |= ((uint32_t)(int)q[e] & 0xFu) << (4 * e);
  return r;
}

}  // namespace ptq
