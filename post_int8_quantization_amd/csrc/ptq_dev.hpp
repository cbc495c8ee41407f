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

// The IEEE binary32 quotient fl32(x / s) from r = fl32(1 / s) (itself an IEEE quotient) by one residual
// correction (Markstein; Muller et al., Handbook of Floating-Point Arithmetic, division chapter):
//   q0 = fl32(x r),  e = x - q0 s  (exact, by the fused multiply-add),  q = fl32(q0 + e r).
// q equals fl32(x / s) whenever |x| >= 2^-102 and 2^-126 <= |s| < 2^126 (so that r is a normal number) and the
// quotient does not overflow: the residual then stays a normal number.  A host sweep over every fp32 mantissa
// of x against thousands of divisor mantissas confirms it bit for bit.  Below |x| = 2^-102 the result is still
// within a few units of the smallest subnormal of the quotient; every caller either proves that such x cannot
// change its outputs or takes the IEEE division (`/`, correctly rounded in this build) instead.
__device__ __forceinline__ float div_rn(float x, float s, float r) {
  const float q0 = x * r;
  const float e = __builtin_fmaf(-q0, s, x);
  return __builtin_fmaf(e, r, q0);
}

// The domain of div_rn for a divisor: r normal and x / s far from overflow for the callers' operands.
__device__ __forceinline__ bool div_rn_divisor_ok(float s) { return s >= 0x1p-100f && s <= 0x1p100f; }

// 1 / s in fp64 for a normal fp32 s, within 2^-51 relative: the hardware's approximate fp64 reciprocal and two
// Newton-Raphson steps with the fused multiply-add, r <- r + r (1 - s r), each of which squares the relative error
// (up to the step's own rounding).  Five instructions against the IEEE division's eleven.  The bound |1 - s r| <=
// 2^-51 holds for every fp32 s in [2^-100, 2^101): checked one by one on the GPU (tests/division/rcp_check.hip,
// tests/test_gpu_rcp.py).
__device__ __forceinline__ double rcp64(float s) {
  const double d = (double)s;
  double r = __builtin_amdgcn_rcp(d);
  r = __builtin_fma(r, __builtin_fma(-d, r, 1.0), r);
  r = __builtin_fma(r, __builtin_fma(-d, r, 1.0), r);
  return r;
}

// fl32(x / s) for an fp32 value x held in fp64 and r64 within 2^-51 relative of 1 / s (rcp64(s), or fl64(1 / s)),
// s a normal fp32 number: the fp64 product x r64 rounded to fp32, two instructions.  The product rounds with a
// relative error of at most 2^-53 (it is a normal fp64 number for every fp32 x), so x r64 lies within 2^-50.6
// relative of the exact quotient.
// The rounding to fp32 can pick another value than the IEEE quotient only if a rounding boundary of fp32 -- a
// midpoint m of two adjacent fp32 numbers, whose significand is odd and 25 bits long -- lies between the two.  An
// exact quotient is never such a midpoint (m s has an odd significand of at least 25 bits, which no fp32 x has),
// and it lies at least 2^-49 relative from every one: x - m s is a non-zero multiple of the smaller of the two
// operands' last-bit weights, and m s has at most 49 significant bits.  So the result is the IEEE quotient
// whenever that is a normal fp32 number; a smaller quotient comes out within one subnormal step of it.  Checked
// bit for bit on the GPU over every mantissa of twelve binades of x around each of thousands of divisors
// (tests/division/rcp_check.hip, tests/test_gpu_rcp.py).
__device__ __forceinline__ float quot64(double x, double r64) { return (float)(x * r64); }

// fl32(1 / s), the IEEE reciprocal, as one Newton-Raphson step with the fused multiply-add from the hardware's
// approximate reciprocal: r = r0 + r0 (1 - s r0), r0 = v_rcp_f32(s).  It equals the IEEE quotient 1.0f / s for
// every fp32 s in [2^-100, 2^101) -- every mantissa of every binade, checked on the GPU by
// tests/division/rcp_check.hip (tests/test_gpu_rcp.py) -- in three instructions instead of the division
// sequence's ten.  Callers use it only for divisors inside div_rn's domain (the approximation alone differs from
// the IEEE reciprocal on about a tenth of those values; outside the domain the callers divide).
__device__ __forceinline__ float rcp_rn(float s) {
  const float r0 = __builtin_amdgcn_rcpf(s);
  return __builtin_fmaf(__builtin_fmaf(-s, r0, 1.0f), r0, r0);
}

// A value known to be the same in every lane, moved to scalar registers (frees vector registers in
// register-bound kernels; the value is unchanged).
__device__ __forceinline__ float uni(float v) {
  return __uint_as_float((uint32_t)__builtin_amdgcn_readfirstlane((int)__float_as_uint(v)));
}
__device__ __forceinline__ double uni(double v) {
  const uint64_t b = (uint64_t)__double_as_longlong(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(b >> 32));
  return __longlong_as_double((long long)(((uint64_t)hi << 32) | lo));
}

// Symmetric code of one value: clamp(rne(fl32(x / s)), -qmax, qmax), as fp32; r = fl32(1 / s).
__device__ __forceinline__ float code_f(float x, float s, float r, float qmax) {
  return fminf(fmaxf(__builtin_rintf(div_rn(x, s, r)), -qmax), qmax);
}

// The same code through the IEEE division.
__device__ __forceinline__ float code_f_ieee(float x, float s, float qmax) {
  return fminf(fmaxf(__builtin_rintf(x / s), -qmax), qmax);
}

// ---------------------------------------------------------------------------
// Double-double sums (Dekker, Knuth): a value hi + lo with |lo| <= ulp(hi) / 2, for sums that must come out as
// the exact real sum rounded once to fp64.  Used only on rare fallback paths.
struct DD {
  double hi, lo;
};

// s + e = a + b exactly (Knuth's TwoSum)
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
  s = a + b;
  const double bb = s - a;
  e = (a - (s - bb)) + (b - bb);
}

// x + y; the same bits whichever operand comes first (the rounding error of hi + hi is unique and the two lo
// parts are added to each other first), so butterfly partners stay identical
__device__ __forceinline__ DD dd_add(DD x, DD y) {
  double s, e;
  two_sum(x.hi, y.hi, s, e);
  e += x.lo + y.lo;
  DD r;
  r.hi = s + e;
  r.lo = e - (r.hi - s);
  return r;
}

__device__ __forceinline__ DD dd_add_d(DD x, double y) { return dd_add(x, DD{y, 0.0}); }

// the exact square of an fp64 value as a double-double (the product error by the fused multiply-add)
__device__ __forceinline__ DD two_sqr(double d) {
  DD r;
  r.hi = d * d;
  r.lo = __builtin_fma(d, d, -r.hi);
  return r;
}

__device__ __forceinline__ DD dd_dpp_xor(DD v, int step) {
  switch (step) {
    case 0: return DD{dpp_f64<kDppXor1>(v.hi), dpp_f64<kDppXor1>(v.lo)};
    case 1: return DD{dpp_f64<kDppXor2>(v.hi), dpp_f64<kDppXor2>(v.lo)};
    case 2: return DD{dpp_f64<kDppHalfMirror>(v.hi), dpp_f64<kDppHalfMirror>(v.lo)};
    default: return DD{dpp_f64<kDppMirror>(v.hi), dpp_f64<kDppMirror>(v.lo)};
  }
}

__device__ __forceinline__ DD dd_swap16(DD v, bool second) {
  const uint64_t bh = (uint64_t)__double_as_longlong(v.hi), bl = (uint64_t)__double_as_longlong(v.lo);
  const auto h0 = __builtin_amdgcn_permlane16_swap((uint32_t)bh, (uint32_t)bh, false, false);
  const auto h1 = __builtin_amdgcn_permlane16_swap((uint32_t)(bh >> 32), (uint32_t)(bh >> 32), false, false);
  const auto l0 = __builtin_amdgcn_permlane16_swap((uint32_t)bl, (uint32_t)bl, false, false);
  const auto l1 = __builtin_amdgcn_permlane16_swap((uint32_t)(bl >> 32), (uint32_t)(bl >> 32), false, false);
  return second ? DD{join_f64(h0[1], h1[1]), join_f64(l0[1], l1[1])} : DD{join_f64(h0[0], h1[0]), join_f64(l0[0], l1[0])};
}

__device__ __forceinline__ DD dd_swap32(DD v, bool second) {
  const uint64_t bh = (uint64_t)__double_as_longlong(v.hi), bl = (uint64_t)__double_as_longlong(v.lo);
  const auto h0 = __builtin_amdgcn_permlane32_swap((uint32_t)bh, (uint32_t)bh, false, false);
  const auto h1 = __builtin_amdgcn_permlane32_swap((uint32_t)(bh >> 32), (uint32_t)(bh >> 32), false, false);
  const auto l0 = __builtin_amdgcn_permlane32_swap((uint32_t)bl, (uint32_t)bl, false, false);
  const auto l1 = __builtin_amdgcn_permlane32_swap((uint32_t)(bl >> 32), (uint32_t)(bl >> 32), false, false);
  return second ? DD{join_f64(h0[1], h1[1]), join_f64(l0[1], l1[1])} : DD{join_f64(h0[0], h1[0]), join_f64(l0[0], l1[0])};
}

// Sum over aligned groups of G lanes (G a power of two up to 64); every lane of a group ends with the same bits.
template <int G>
__device__ __forceinline__ DD group_sum_dd(DD v) {
  if constexpr (G >= 2) v = dd_add(v, dd_dpp_xor(v, 0));
  if constexpr (G >= 4) v = dd_add(v, dd_dpp_xor(v, 1));
  if constexpr (G >= 8) v = dd_add(v, dd_dpp_xor(v, 2));
  if constexpr (G >= 16) v = dd_add(v, dd_dpp_xor(v, 3));
  if constexpr (G >= 32) v = dd_add(dd_swap16(v, false), dd_swap16(v, true));
  if constexpr (G >= 64) v = dd_add(dd_swap32(v, false), dd_swap32(v, true));
  return v;
}

// rne(t) for |t| < 2^22, as the low bits of fl32(t + 1.5 * 2^23): the addition rounds the exact sum to an
// integer (ties to even) inside the binade [2^23, 2^24), so the low mantissa bits hold rne(t) in two's
// complement -- one instruction instead of a rounding and a conversion.
__device__ __forceinline__ uint32_t rne_bits(float t) { return __float_as_uint(t + 12582912.0f); }

// The low bytes of four words packed into one dword, word 0's in the low byte (three byte permutes).
__device__ __forceinline__ uint32_t pack4_low_bytes(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const uint32_t ab = __builtin_amdgcn_perm(b, a, 0x0c0c0400u);  // [a0, b0, 0, 0]
  const uint32_t cd = __builtin_amdgcn_perm(d, c, 0x0c0c0400u);  // [c0, d0, 0, 0]
  return __builtin_amdgcn_perm(cd, ab, 0x05040100u);               // [a0, b0, c0, d0]
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
