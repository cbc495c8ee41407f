// ptq_dev.hpp -- device helpers shared by the gfx950 kernels of libptq.
//
// Wavefronts are 64 lanes.  Cross-lane reductions are butterflies in which
// every lane ends with the same bits (fp addition and max are commutative, so
// the two lanes of a pair combine the same two partials), which keeps per-row
// decisions uniform.
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

// Buffer accesses with hardware range checking (gfx9 raw buffer, stride 0):
// a load at a byte offset past num_records returns zeros and a store there is
// dropped, so tails and absent rows need no branches -- every lane issues the
// same loads and stores, which also lets the compiler count them exactly when
// it places its waits.  Descriptor word 3 is the gfx9 default.
typedef unsigned u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}

// 16-byte load of read-once data (nontemporal)
__device__ __forceinline__ uint4 buf_load16_once(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 2);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  const u32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void buf_store8(__amdgpu_buffer_rsrc_t r, uint32_t off, uint2 v) {
  const u32x2_t d = {v.x, v.y};
  __builtin_amdgcn_raw_buffer_store_b64(d, r, (int)off, 0, 0);
}

__device__ __forceinline__ void buf_store4(__amdgpu_buffer_rsrc_t r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)off, 0, 0);
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

// Lane exchanges for the butterflies.  Steps 1, 2, 4 and 8 stay inside a row of
// 16 lanes and use DPP moves (quad permutes, then the half-row and row
// mirrors, which pair each group of 4 or 8 lanes with the other half of the
// group after the earlier steps have made the group uniform); steps 16 and 32
// use the gfx950 row swaps (v_permlane16_swap / v_permlane32_swap), which
// hand every lane the same lane of the paired row or half.  All are VALU
// moves: no LDS round trip.
// (every lane of these patterns reads a valid source lane, so no lane keeps the destination's old value:
// the move form without an `old` operand spares the compiler a zeroing move per DPP move)
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

constexpr int kDppXor1 = 0xB1;         // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;         // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;  // lane i <-> 7-i within 8
constexpr int kDppMirror = 0x140;      // lane i <-> 15-i within 16

// Applies OP(v, partner) for each butterfly step; partner values are the same
// lanes' values of the other half of every group, so both lanes of a pair
// combine the same two operands.
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_u32(uint32_t v, Op op) {
  v = op(v, dpp_u32<kDppXor1>(v));
  v = op(v, dpp_u32<kDppXor2>(v));
  v = op(v, dpp_u32<kDppHalfMirror>(v));
  v = op(v, dpp_u32<kDppMirror>(v));
  {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = op(r[0], r[1]);
  }
  {
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    v = op(r[0], r[1]);
  }
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
  return __uint_as_float(
      wave_reduce_u32(__float_as_uint(v), [](uint32_t a, uint32_t b) { return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b))); }));
}

__device__ __forceinline__ int wave_sum(int v) {
  return (int)wave_reduce_u32((uint32_t)v, [](uint32_t a, uint32_t b) { return (uint32_t)((int)a + (int)b); });
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = dpp_u32<CTRL>((uint32_t)b), hi = dpp_u32<CTRL>((uint32_t)(b >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ double join_f64(uint32_t lo, uint32_t hi) {
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

__device__ __forceinline__ double wave_sum(double v) {
  v += dpp_f64<kDppXor1>(v);
  v += dpp_f64<kDppXor2>(v);
  v += dpp_f64<kDppHalfMirror>(v);
  v += dpp_f64<kDppMirror>(v);
  {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)b, (uint32_t)b, false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(b >> 32), (uint32_t)(b >> 32), false, false);
    v = join_f64(lo[0], hi[0]) + join_f64(lo[1], hi[1]);
  }
  {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const auto lo = __builtin_amdgcn_permlane32_swap((uint32_t)b, (uint32_t)b, false, false);
    const auto hi = __builtin_amdgcn_permlane32_swap((uint32_t)(b >> 32), (uint32_t)(b >> 32), false, false);
    v = join_f64(lo[0], hi[0]) + join_f64(lo[1], hi[1]);
  }
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
