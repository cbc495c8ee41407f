// ssz.hip -- MinMax + SSZ per-output-channel weight quantization (gfx950):
// symmetric int8/int4 (k_ssz; k_ssz_rows for rows of at most 512 elements,
// several rows per wave) and asymmetric int8 (k_ssz_asym, further down).
//
// [SSZ] flow: MinMax initial scale, then least-squares refits of the scale for
// the current codes, a refit kept only when it lowers the quantization error,
// until the relative or absolute change falls under the threshold or the
// iteration limit is reached; symmetric quantization fixes the offset at 0.
// [SQ] the weight side of the smoothing fold, w_hat = fl32(w * s_j).
//
// One block of TPR threads owns one row (output channel).  The row is read
// from HBM once and stays in registers (CPT chunks of 16 elements per
// thread, in fp32, widened to fp64 where a pass needs it) for every pass;
// all passes are ALU work.  One pass over the row for a scale S computes, per
// element, the code q = clamp(rne(w_hat * inv S)) and accumulates A =
// sum(w_hat q) in fp64 and B = sum(q^2) exactly (fp32 per lane, integer
// across lanes) -- the two sums the least-squares step needs.  The error of
// the pass follows from the same sums and the row's sum of squares W2
// (computed once): K * mse(S) = W2 - 2 S A + S^2 B, the expansion of
// sum (w_hat - S q)^2, evaluated in fp64 and clamped at 0.  The sums are
// reduced with xor butterflies (identical in every lane) and, for multi-wave
// rows, through LDS in wave order, so every decision is uniform across the
// row.
#include "ptq_dev.hpp"
#include "ptq_launch.hpp"

namespace ptq {

namespace {

struct PassSums {
  double a;  // sum w_hat q
  int b;     // sum q^2
};

template <int TPR, int CPT, bool WIDE>
__device__ __forceinline__ PassSums row_pass(const float (&wh)[CPT][16], const double (&wd)[WIDE ? CPT : 1][16],
                                             float S, float qmax, double* red_d, int* red_i, int tid) {
  const float inv = 1.0f / S;
  double a = 0.0;
  float bq = 0.0f;  // at most 16*CPT terms of <= 127^2 each: exact in fp32
#pragma unroll
  for (int m = 0; m < CPT; ++m) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float q = code_f(wh[m][k], inv, qmax);
      const double w = WIDE ? wd[WIDE ? m : 0][k] : (double)wh[m][k];
      a = __builtin_fma(w, (double)q, a);
      bq = __builtin_fmaf(q, q, bq);
    }
  }
  PassSums r;
  r.a = wave_sum(a);
  r.b = wave_sum((int)bq);
  constexpr int NW = TPR / kWave;
  if constexpr (NW > 1) {
    // red_d / red_i point at this pass's half of a two-pass slot ring: the previous readers of
    // these slots (two passes ago) finished before the barrier of the pass in between
    const int w = tid / kWave;
    if ((tid & (kWave - 1)) == 0) {
      red_d[w] = r.a;
      red_i[w] = r.b;
    }
    __syncthreads();
    r.a = red_d[0];
    r.b = red_i[0];
#pragma unroll
    for (int i = 1; i < NW; ++i) {
      r.a += red_d[i];
      r.b += red_i[i];
    }
  }
  return r;
}

// Row n of w, folded (w_hat = fl32(w * s_j)), into registers: CPT chunks of 16 elements per thread,
// chunk c8 of thread tid at elements (tid + TPR*c8)*16 ..; chunks past the row are zeros (they add
// nothing to any sum and never change a max of magnitudes).  WIDE also keeps an fp64 copy.
template <int DT, bool HAS_S, int TPR, int CPT, bool WIDE>
__device__ __forceinline__ void load_row(const void* __restrict__ w, int64_t n, int64_t K, const float* __restrict__ s,
                                         int tid, float (&wh)[CPT][16], double (&wd)[WIDE ? CPT : 1][16]) {
  const int64_t nchunk = K / 16;
#pragma unroll
  for (int c8 = 0; c8 < CPT; ++c8) {
    const int64_t c = tid + (int64_t)TPR * c8;
    if (c < nchunk) {
      float a8[8], b8[8];
      load8<DT>(w, n * K + c * 16, a8);
      load8<DT>(w, n * K + c * 16 + 8, b8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        wh[c8][e] = a8[e];
        wh[c8][e + 8] = b8[e];
      }
      if constexpr (HAS_S) {
        const float4* sp = reinterpret_cast<const float4*>(s + c * 16);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 sv = sp[q4];
          wh[c8][4 * q4 + 0] = wh[c8][4 * q4 + 0] * sv.x;
          wh[c8][4 * q4 + 1] = wh[c8][4 * q4 + 1] * sv.y;
          wh[c8][4 * q4 + 2] = wh[c8][4 * q4 + 2] * sv.z;
          wh[c8][4 * q4 + 3] = wh[c8][4 * q4 + 3] * sv.w;
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) wh[c8][e] = 0.0f;
    }
    if constexpr (WIDE) {
#pragma unroll
      for (int e = 0; e < 16; ++e) wd[c8][e] = (double)wh[c8][e];
    }
  }
}

// e / K in fp64.  For a power-of-two K the quotient is an exact scaling, so it is taken with
// ldexp (one instruction) instead of the division sequence; the result is the same double.
struct DivK {
  double kd;
  int lg;  // log2 K when K is a power of two, else -1
  __device__ __forceinline__ double operator()(double e) const {
    if (lg >= 0) return __builtin_ldexp(e, -lg);
    return e / kd;
  }
};

__device__ __forceinline__ DivK make_divk(int64_t K) {
  DivK d;
  d.kd = (double)K;
  d.lg = (K & (K - 1)) == 0 ? 63 - __builtin_clzll((unsigned long long)K) : -1;
  return d;
}

// The relative convergence test fl64(d / best) < thr, for best > 0 and thr >= 0, with the division
// taken only where its rounding can decide.  d <= 0 gives a quotient <= 0, below any thr > 0.
// d >= 2 fl64(thr * best) means d > thr * best exactly (one rounding, or an underflow below the
// smallest positive d, cannot halve the product), so the quotient exceeds thr and rounds to >= thr.
// On these weights the division then runs only for improvements within a factor of two of the
// threshold; it was 15 of the ~95 per-pass instructions of a row's wave.
__device__ __forceinline__ bool rel_below(double d, double best, double thr) {
  if (thr > 0.0 && d <= 0.0) return true;
  if (d >= 2.0 * (thr * best)) return false;
  return d / best < thr;
}

// K * mse(S) from the pass sums: W2 - 2 S A + S^2 B, never below 0
__device__ __forceinline__ double sq_err(double w2, float S, const PassSums& p) {
  const double Sd = (double)S;
  const double e = (w2 - 2.0 * Sd * p.a) + Sd * Sd * (double)p.b;
  return e > 0.0 ? e : 0.0;
}

// WIDE_MODE 1 keeps an explicit fp64 copy of the row in registers.  The default (0) leaves the
// widening to the compiler, which hoists it out of the pass loop: the same 6 VALU operations per
// element and pass in about 2/3 of the registers (2 waves per SIMD instead of 1 on 4096- and
// 16384-wide rows; measured 25-30% faster, int8 and int4).  Forcing the conversion into every pass
// (3 waves per SIMD, 7 operations) measured 5% slower than the default.
template <int DT, bool HAS_S, int BITS, int TPR, int CPT, int WIDE_MODE = 0>
__global__ __launch_bounds__(TPR) void k_ssz(const void* __restrict__ w, int64_t N, int64_t K,
                                             const float* __restrict__ s, int max_iter, double thr, float min_scale,
                                             float* __restrict__ scale, void* __restrict__ wq,
                                             int32_t* __restrict__ iters, double* __restrict__ mse) {
  constexpr int NW = TPR / kWave;
  constexpr bool WIDE = WIDE_MODE == 1;
  constexpr float QMAX = BITS == 8 ? 127.0f : 7.0f;
  __shared__ double red_d[NW];
  __shared__ float red_f[NW];
  __shared__ double ring_d[2][NW];  // pass sums, alternating halves
  __shared__ int ring_i[2][NW];
  int par = 0;
  const int tid = threadIdx.x;
  const int64_t nchunk = K / 16;
  const DivK per_elem = make_divk(K);

  for (int64_t n = blockIdx.x; n < N; n += gridDim.x) {
    float wh[CPT][16];
    double wd[WIDE ? CPT : 1][16];
    load_row<DT, HAS_S, TPR, CPT, WIDE>(w, n, K, s, tid, wh, wd);
    float m = 0.0f;
    double w2 = 0.0;
#pragma unroll
    for (int c8 = 0; c8 < CPT; ++c8) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        m = fmaxf(m, fabsf(wh[c8][e]));
        const double x = (double)wh[c8][e];
        w2 = __builtin_fma(x, x, w2);
      }
    }
    m = wave_max(m);
    w2 = wave_sum(w2);
    if constexpr (NW > 1) {
      __syncthreads();
      if ((tid & (kWave - 1)) == 0) {
        red_f[tid / kWave] = m;
        red_d[tid / kWave] = w2;
      }
      __syncthreads();
      m = red_f[0];
      w2 = red_d[0];
#pragma unroll
      for (int i = 1; i < NW; ++i) {
        m = fmaxf(m, red_f[i]);
        w2 += red_d[i];
      }
    }

    // MinMax init
    float S = m / QMAX;
    S = S < min_scale ? min_scale : S;
    PassSums cur = row_pass<TPR, CPT, WIDE>(wh, wd, S, QMAX, ring_d[par], ring_i[par], tid);
    par ^= 1;
    double best = per_elem(sq_err(w2, S, cur));
    double A = cur.a;
    int B = cur.b;

    // least-squares refits, greedy, per-row convergence
    int it = 0;
    for (int i = 1; i <= max_iter; ++i) {
      it = i;
      if (B == 0) break;
      float Sc = (float)(A / (double)B);
      Sc = Sc < min_scale ? min_scale : Sc;
      const PassSums p = row_pass<TPR, CPT, WIDE>(wh, wd, Sc, QMAX, ring_d[par], ring_i[par], tid);
      par ^= 1;
      const double c = per_elem(sq_err(w2, Sc, p));
      const double d = best - c;
      const bool conv = (best == 0.0) || (fabs(d) < thr) || rel_below(d, best, thr);
      if (c < best) {
        S = Sc;
        best = c;
        A = p.a;
        B = p.b;
      }
      if (conv) break;
    }

    // codes of the kept scale, and its error summed directly (the reported mse; the expansion
    // above loses relative accuracy when the error is tiny next to W2)
    double e_dir = 0.0;
    if (wq || mse) {
      const float inv = 1.0f / S;
      const double Sd = (double)S;
#pragma unroll
      for (int c8 = 0; c8 < CPT; ++c8) {
        const int64_t c = tid + (int64_t)TPR * c8;
        float q[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          q[e] = code_f(wh[c8][e], inv, QMAX);
          const double dd = __builtin_fma(-Sd, (double)q[e], (double)wh[c8][e]);  // S*q is exact in fp64
          e_dir = __builtin_fma(dd, dd, e_dir);
        }
        if (wq && c < nchunk) {
          if constexpr (BITS == 8) {
            uint4 o;
            o.x = pack4_i8(q[0], q[1], q[2], q[3]);
            o.y = pack4_i8(q[4], q[5], q[6], q[7]);
            o.z = pack4_i8(q[8], q[9], q[10], q[11]);
            o.w = pack4_i8(q[12], q[13], q[14], q[15]);
            *reinterpret_cast<uint4*>(reinterpret_cast<int8_t*>(wq) + n * K + c * 16) = o;
          } else {
            uint2 o;
            o.x = pack8_i4(q);
            o.y = pack8_i4(q + 8);
            *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(wq) + n * (K / 2) + c * 8) = o;
          }
        }
      }
      if (mse) {
        e_dir = wave_sum(e_dir);
        if constexpr (NW > 1) {
          __syncthreads();
          if ((tid & (kWave - 1)) == 0) red_d[tid / kWave] = e_dir;
          __syncthreads();
          e_dir = red_d[0];
#pragma unroll
          for (int i = 1; i < NW; ++i) e_dir += red_d[i];
        }
      }
    }
    if (tid == 0) {
      scale[n] = S;
      if (iters) iters[n] = it;
      if (mse) mse[n] = per_elem(e_dir);
    }
  }
}

// ---------------------------------------------------------------------------
// Short rows (K <= 512, at most 32 chunks of 16): one wave holds R = 64 / G rows, G lanes each
// (G = the chunk count rounded up to a power of two, 1 to 32), one 16-element chunk per lane -- the
// same pass length per lane as the one-wave row kernel, which at these K leaves half its lanes or
// more idle.  Each group
// of G lanes carries its own row's state, reduces inside the group only (DPP moves within the 16-lane
// row, plus the 16-lane swap for G = 32), and stops updating when its row converges, while the wave
// runs until all its rows have; a pass never takes longer than in the row kernel, and R rows share it.
// Same formulas and decisions per row as k_ssz.

// sums and maximum over aligned groups of G lanes (G a power of two up to 32); every lane of a group
// ends with the group's total, bit-identical across the group (each step adds the same two operands)
template <int G>
__device__ __forceinline__ double group_sum(double v) {
  if constexpr (G >= 2) v += dpp_f64<kDppXor1>(v);
  if constexpr (G >= 4) v += dpp_f64<kDppXor2>(v);
  if constexpr (G >= 8) v += dpp_f64<kDppHalfMirror>(v);
  if constexpr (G >= 16) v += dpp_f64<kDppMirror>(v);
  if constexpr (G == 32) {
    const uint64_t b = (uint64_t)__double_as_longlong(v);
    const auto lo = __builtin_amdgcn_permlane16_swap((uint32_t)b, (uint32_t)b, false, false);
    const auto hi = __builtin_amdgcn_permlane16_swap((uint32_t)(b >> 32), (uint32_t)(b >> 32), false, false);
    v = join_f64(lo[0], hi[0]) + join_f64(lo[1], hi[1]);
  }
  return v;
}

template <int G, typename Op>
__device__ __forceinline__ uint32_t group_reduce_u32(uint32_t v, Op op) {
  if constexpr (G >= 2) v = op(v, dpp_u32<kDppXor1>(v));
  if constexpr (G >= 4) v = op(v, dpp_u32<kDppXor2>(v));
  if constexpr (G >= 8) v = op(v, dpp_u32<kDppHalfMirror>(v));
  if constexpr (G >= 16) v = op(v, dpp_u32<kDppMirror>(v));
  if constexpr (G == 32) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    v = op(r[0], r[1]);
  }
  return v;
}

template <int G>
__device__ __forceinline__ int group_sum(int v) {
  return (int)group_reduce_u32<G>((uint32_t)v, [](uint32_t a, uint32_t b) { return (uint32_t)((int)a + (int)b); });
}

template <int G>
__device__ __forceinline__ float group_max(float v) {
  return __uint_as_float(group_reduce_u32<G>(
      __float_as_uint(v), [](uint32_t a, uint32_t b) { return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b))); }));
}

template <int DT, bool HAS_S, int BITS, int G>
__global__ __launch_bounds__(kWave) void k_ssz_rows(const void* __restrict__ w, int64_t N, int64_t K,
                                                    const float* __restrict__ s, int max_iter, double thr,
                                                    float min_scale, float* __restrict__ scale,
                                                    void* __restrict__ wq, int32_t* __restrict__ iters,
                                                    double* __restrict__ mse) {
  static_assert(G >= 1 && G <= 32 && (G & (G - 1)) == 0, "1 to 32 lanes per row, a power of two");
  constexpr int R = kWave / G;  // rows per wave
  constexpr int CPT = 1;        // chunks of 16 per lane
  constexpr float QMAX = BITS == 8 ? 127.0f : 7.0f;
  const int lane = threadIdx.x;
  const int gl = lane % G;  // lane in the row's group
  const int64_t nchunk = K / 16;
  const DivK per_elem = make_divk(K);

  // every lane runs the same number of row groups (uniform loop); rows past N compute on zeros, unwritten
  for (int64_t n0 = (int64_t)blockIdx.x * R; n0 < N; n0 += (int64_t)gridDim.x * R) {
    const int64_t n = n0 + lane / G;
    const bool live = n < N;
    float wh[CPT][16];
    double wd[1][16];
    load_row<DT, HAS_S, G, CPT, false>(w, live ? n : n0, K, s, gl, wh, wd);
    if (!live) {
#pragma unroll
      for (int c8 = 0; c8 < CPT; ++c8)
#pragma unroll
        for (int e = 0; e < 16; ++e) wh[c8][e] = 0.0f;
    }
    float m = 0.0f;
    double w2 = 0.0;
#pragma unroll
    for (int c8 = 0; c8 < CPT; ++c8) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        m = fmaxf(m, fabsf(wh[c8][e]));
        const double x = (double)wh[c8][e];
        w2 = __builtin_fma(x, x, w2);
      }
    }
    m = group_max<G>(m);
    w2 = group_sum<G>(w2);

    // one pass over the group's row for the scale S of that row: A = sum w_hat q (fp64), B = sum q^2
    auto pass = [&](float Sx, double& A, int& B) {
      const float inv = 1.0f / Sx;
      double a = 0.0;
      float bq = 0.0f;
#pragma unroll
      for (int c8 = 0; c8 < CPT; ++c8) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float q = code_f(wh[c8][e], inv, QMAX);
          a = __builtin_fma((double)wh[c8][e], (double)q, a);
          bq = __builtin_fmaf(q, q, bq);
        }
      }
      A = group_sum<G>(a);
      B = group_sum<G>((int)bq);
    };

    // MinMax init
    float S = m / QMAX;
    S = S < min_scale ? min_scale : S;
    double A;
    int B;
    pass(S, A, B);
    double best = per_elem(sq_err(w2, S, PassSums{A, B}));

    // least-squares refits, greedy, per-row convergence; a row's state stays fixed once it stops
    int it = 0;
    bool active = live;  // rows past N take no step
    for (int i = 1; i <= max_iter; ++i) {
      if (!__builtin_amdgcn_ballot_w64(active)) break;
      if (active) it = i;
      const bool fit = active && B != 0;
      if (active && B == 0) active = false;
      float Sc = fit ? (float)(A / (double)B) : S;
      Sc = Sc < min_scale ? min_scale : Sc;
      double Ap;
      int Bp;
      pass(Sc, Ap, Bp);
      const double c = per_elem(sq_err(w2, Sc, PassSums{Ap, Bp}));
      const double d = best - c;
      const bool conv = (best == 0.0) || (fabs(d) < thr) || rel_below(d, best, thr);
      if (fit && c < best) {
        S = Sc;
        best = c;
        A = Ap;
        B = Bp;
      }
      if (fit && conv) active = false;
    }

    // codes of the kept scale, and its error summed directly
    double e_dir = 0.0;
    if (wq || mse) {
      const float inv = 1.0f / S;
      const double Sd = (double)S;
#pragma unroll
      for (int c8 = 0; c8 < CPT; ++c8) {
        const int64_t c = gl + (int64_t)G * c8;
        float q[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          q[e] = code_f(wh[c8][e], inv, QMAX);
          const double dd = __builtin_fma(-Sd, (double)q[e], (double)wh[c8][e]);  // S*q is exact in fp64
          e_dir = __builtin_fma(dd, dd, e_dir);
        }
        if (wq && live && c < nchunk) {
          if constexpr (BITS == 8) {
            uint4 o;
            o.x = pack4_i8(q[0], q[1], q[2], q[3]);
            o.y = pack4_i8(q[4], q[5], q[6], q[7]);
            o.z = pack4_i8(q[8], q[9], q[10], q[11]);
            o.w = pack4_i8(q[12], q[13], q[14], q[15]);
            *reinterpret_cast<uint4*>(reinterpret_cast<int8_t*>(wq) + n * K + c * 16) = o;
          } else {
            uint2 o;
            o.x = pack8_i4(q);
            o.y = pack8_i4(q + 8);
            *reinterpret_cast<uint2*>(reinterpret_cast<uint8_t*>(wq) + n * (K / 2) + c * 8) = o;
          }
        }
      }
      if (mse) e_dir = group_sum<G>(e_dir);
    }
    if (live && gl == 0) {
      scale[n] = S;
      if (iters) iters[n] = it;
      if (mse) mse[n] = per_elem(e_dir);
    }
  }
}

// ---------------------------------------------------------------------------
// Asymmetric int8 ([SSZ] asymmetric mode: scale and offset fitted together;
// [INT8] 2.1 Q = round(R/S) + Z with saturation).  Codes
//   q = clamp(rne(fl32(w_hat * inv S)) + Z, -128, 127),  dequantized S (q - Z).
// A pass for (S, Z) accumulates A = sum w_hat q (fp64), B = sum q^2 and
// C = sum q (exact).  With the row's W1 = sum w_hat and W2 = sum w_hat^2:
//   K mse = W2 - 2 S (A - Z W1) + S^2 (B - 2 Z C + K Z^2),
// and the least-squares line w_hat ~ a q + b through the pass's codes solves
// the 2x2 normal equations: det = K B - C^2, a = (K A - W1 C) / det,
// b = (W1 - a C) / K, giving S' = max(fl32(a), min_scale) and
// Z' = clamp(rne(-b / a), -128, 127).  MinMax init from the row's min lo and
// max hi: S0 = max(fl32(fl32(hi - lo) / 255), min_scale),
// Z0 = clamp(-128 - rne(fl32(lo * inv S0)), -128, 127).
// Register slots past the row hold w_hat = 0, whose code is Z: each adds Z^2
// to B and Z to C, which the pass subtracts exactly.

struct PassSumsA {
  double a;  // sum w_hat q
  double b;  // sum q^2 (an exact integer)
  double c;  // sum q   (an exact integer)
};

__device__ __forceinline__ float code_asym_f(float x, float inv, float zf) {
  return fminf(fmaxf(__builtin_rintf(x * inv) + zf, -128.0f), 127.0f);
}

template <int TPR, int CPT, bool WIDE>
__device__ __forceinline__ PassSumsA row_pass_asym(const float (&wh)[CPT][16], const double (&wd)[WIDE ? CPT : 1][16],
                                                   float S, int Z, double pad, double* red_d, int tid) {
  const float inv = 1.0f / S;
  const float zf = (float)Z;
  double a = 0.0;
  float bq = 0.0f;  // at most 16*CPT terms of <= 128^2 each: exact in fp32
  float cq = 0.0f;
#pragma unroll
  for (int m = 0; m < CPT; ++m) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float q = code_asym_f(wh[m][k], inv, zf);
      const double w = WIDE ? wd[WIDE ? m : 0][k] : (double)wh[m][k];
      a = __builtin_fma(w, (double)q, a);
      bq = __builtin_fmaf(q, q, bq);
      cq += q;
    }
  }
  PassSumsA r;
  r.a = wave_sum(a);
  r.b = (double)wave_sum((int)bq);
  r.c = (double)wave_sum((int)cq);
  constexpr int NW = TPR / kWave;
  if constexpr (NW > 1) {
    // red_d points at this pass's half of a two-pass slot ring (see row_pass)
    const int w = tid / kWave;
    if ((tid & (kWave - 1)) == 0) {
      red_d[w] = r.a;
      red_d[NW + w] = r.b;
      red_d[2 * NW + w] = r.c;
    }
    __syncthreads();
    r.a = red_d[0];
    r.b = red_d[NW];
    r.c = red_d[2 * NW];
#pragma unroll
    for (int i = 1; i < NW; ++i) {
      r.a += red_d[i];
      r.b += red_d[NW + i];
      r.c += red_d[2 * NW + i];
    }
  }
  const double zd = (double)Z;
  r.b -= pad * zd * zd;
  r.c -= pad * zd;
  return r;
}

// K * mse(S, Z) from the pass sums, never below 0
__device__ __forceinline__ double sq_err_asym(double w2, double w1, double Kd, float S, int Z, const PassSumsA& p) {
  const double Sd = (double)S, zd = (double)Z;
  const double cross = p.a - zd * w1;
  const double quad = (p.b - 2.0 * zd * p.c) + Kd * zd * zd;  // sum (q - Z)^2, exact
  const double e = (w2 - 2.0 * Sd * cross) + Sd * Sd * quad;
  return e > 0.0 ? e : 0.0;
}

template <int DT, bool HAS_S, int TPR, int CPT, int WIDE_MODE = 0>
__global__ __launch_bounds__(TPR) void k_ssz_asym(const void* __restrict__ w, int64_t N, int64_t K,
                                                  const float* __restrict__ s, int max_iter, double thr,
                                                  float min_scale, float* __restrict__ scale,
                                                  int32_t* __restrict__ zero_point, int8_t* __restrict__ wq,
                                                  int32_t* __restrict__ iters, double* __restrict__ mse) {
  constexpr int NW = TPR / kWave;
  constexpr bool WIDE = WIDE_MODE == 1;
  __shared__ double red_d[3 * NW];
  __shared__ float red_f[2 * NW];
  __shared__ double ring_d[2][3 * NW];  // pass sums, alternating halves
  int par = 0;
  const int tid = threadIdx.x;
  const int64_t nchunk = K / 16;
  const double Kd = (double)K;
  const DivK per_elem = make_divk(K);
  const double pad = (double)((int64_t)TPR * CPT * 16 - K);  // zero slots per row

  for (int64_t n = blockIdx.x; n < N; n += gridDim.x) {
    float wh[CPT][16];
    double wd[WIDE ? CPT : 1][16];
    load_row<DT, HAS_S, TPR, CPT, WIDE>(w, n, K, s, tid, wh, wd);
    float lo = __builtin_huge_valf(), hi = -__builtin_huge_valf();
    double w1 = 0.0, w2 = 0.0;
#pragma unroll
    for (int c8 = 0; c8 < CPT; ++c8) {
      const bool in = tid + (int64_t)TPR * c8 < nchunk;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float v = wh[c8][e];
        lo = fminf(lo, in ? v : lo);
        hi = fmaxf(hi, in ? v : hi);
        const double x = (double)v;
        w1 += x;
        w2 = __builtin_fma(x, x, w2);
      }
    }
    lo = -wave_max(-lo);
    hi = wave_max(hi);
    w1 = wave_sum(w1);
    w2 = wave_sum(w2);
    if constexpr (NW > 1) {
      __syncthreads();
      if ((tid & (kWave - 1)) == 0) {
        red_f[tid / kWave] = lo;
        red_f[NW + tid / kWave] = hi;
        red_d[tid / kWave] = w1;
        red_d[NW + tid / kWave] = w2;
      }
      __syncthreads();
      lo = red_f[0];
      hi = red_f[NW];
      w1 = red_d[0];
      w2 = red_d[NW];
#pragma unroll
      for (int i = 1; i < NW; ++i) {
        lo = fminf(lo, red_f[i]);
        hi = fmaxf(hi, red_f[NW + i]);
        w1 += red_d[i];
        w2 += red_d[NW + i];
      }
    }

    // MinMax init
    const float range = hi - lo;
    float S = range / 255.0f;
    S = S < min_scale ? min_scale : S;
    int Z;
    {
      const float inv0 = 1.0f / S;
      const float z0 = -128.0f - __builtin_rintf(lo * inv0);
      Z = (int)fminf(fmaxf(z0, -128.0f), 127.0f);
    }
    PassSumsA cur = row_pass_asym<TPR, CPT, WIDE>(wh, wd, S, Z, pad, ring_d[par], tid);
    par ^= 1;
    double best = per_elem(sq_err_asym(w2, w1, Kd, S, Z, cur));

    int it = 0;
    for (int i = 1; i <= max_iter; ++i) {
      it = i;
      const double det = Kd * cur.b - cur.c * cur.c;  // exact: integers below 2^53
      if (det <= 0.0) break;
      const double a = (Kd * cur.a - w1 * cur.c) / det;
      const double b = per_elem(w1 - a * cur.c);
      float Sc = (float)a;
      Sc = Sc < min_scale ? min_scale : Sc;
      const double zr = __builtin_rint(-b / a);
      const int Zc = zr < -128.0 ? -128 : (zr > 127.0 ? 127 : (int)zr);
      const PassSumsA p = row_pass_asym<TPR, CPT, WIDE>(wh, wd, Sc, Zc, pad, ring_d[par], tid);
      par ^= 1;
      const double c = per_elem(sq_err_asym(w2, w1, Kd, Sc, Zc, p));
      const double d = best - c;
      const bool conv = (best == 0.0) || (fabs(d) < thr) || rel_below(d, best, thr);
      if (c < best) {
        S = Sc;
        Z = Zc;
        best = c;
        cur = p;
      }
      if (conv) break;
    }

    // codes of the kept (S, Z) and their error summed directly (the reported mse)
    double e_dir = 0.0;
    if (wq || mse) {
      const float inv = 1.0f / S;
      const float zf = (float)Z;
      const double Sd = (double)S;
#pragma unroll
      for (int c8 = 0; c8 < CPT; ++c8) {
        const int64_t c = tid + (int64_t)TPR * c8;
        float q[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          q[e] = code_asym_f(wh[c8][e], inv, zf);
          // slots past the row: w_hat = 0 and q = Z, so they add 0
          const double dd = __builtin_fma(-Sd, (double)(q[e] - zf), (double)wh[c8][e]);  // S*(q-Z) exact in fp64
          e_dir = __builtin_fma(dd, dd, e_dir);
        }
        if (wq && c < nchunk) {
          uint4 o;
          o.x = pack4_i8(q[0], q[1], q[2], q[3]);
          o.y = pack4_i8(q[4], q[5], q[6], q[7]);
          o.z = pack4_i8(q[8], q[9], q[10], q[11]);
          o.w = pack4_i8(q[12], q[13], q[14], q[15]);
          *reinterpret_cast<uint4*>(wq + n * K + c * 16) = o;
        }
      }
      if (mse) {
        e_dir = wave_sum(e_dir);
        if constexpr (NW > 1) {
          __syncthreads();
          if ((tid & (kWave - 1)) == 0) red_d[tid / kWave] = e_dir;
          __syncthreads();
          e_dir = red_d[0];
#pragma unroll
          for (int i = 1; i < NW; ++i) e_dir += red_d[i];
        }
      }
    }
    if (tid == 0) {
      scale[n] = S;
      zero_point[n] = Z;
      if (iters) iters[n] = it;
      if (mse) mse[n] = per_elem(e_dir);
    }
  }
}

template <int DT, bool HAS_S>
hipError_t dispatch_asym(const void* w, int64_t N, int64_t K, const float* s, int max_iter, double thr,
                         float min_scale, float* scale, int32_t* zp, int8_t* wq, int32_t* iters, double* mse,
                         hipStream_t stream) {
  const int64_t nchunk = K / 16;
  int tpr = 64;
  while (tpr < 1024 && (nchunk + tpr - 1) / tpr > 4) tpr *= 2;
  const int64_t cpt = (nchunk + tpr - 1) / tpr;
#define PTQ_SA(TPR_, CPT_)                                                                                \
  if (tpr == TPR_ && cpt <= CPT_) {                                                                       \
    k_ssz_asym<DT, HAS_S, TPR_, CPT_><<<(unsigned)N, TPR_, 0, stream>>>(w, N, K, s, max_iter, thr,        \
                                                                        min_scale, scale, zp, wq, iters,  \
                                                                        mse);                             \
    return hipGetLastError();                                                                             \
  }
  PTQ_SA(64, 1) PTQ_SA(64, 2) PTQ_SA(64, 4)
  PTQ_SA(128, 4) PTQ_SA(256, 4) PTQ_SA(512, 4) PTQ_SA(1024, 4) PTQ_SA(1024, 8)
#undef PTQ_SA
  return hipErrorInvalidValue;
}

template <int DT, bool HAS_S, int BITS>
hipError_t dispatch(const void* w, int64_t N, int64_t K, const float* s, int max_iter, double thr, float min_scale,
                    float* scale, void* wq, int32_t* iters, double* mse, hipStream_t stream) {
  const int64_t nchunk = K / 16;
  // short rows: several rows per wave, one chunk per lane
  if (nchunk <= 32) {
#define PTQ_SR(G_)                                                                                        \
  if (nchunk <= G_) {                                                                                     \
    constexpr int64_t R_ = kWave / G_;                                                                    \
    k_ssz_rows<DT, HAS_S, BITS, G_><<<(unsigned)((N + R_ - 1) / R_), kWave, 0, stream>>>(                 \
        w, N, K, s, max_iter, thr, min_scale, scale, wq, iters, mse);                                     \
    return hipGetLastError();                                                                             \
  }
    PTQ_SR(1) PTQ_SR(2) PTQ_SR(4) PTQ_SR(8) PTQ_SR(16) PTQ_SR(32)
#undef PTQ_SR
  }
  // longer rows: about 64 elements per thread; one wave per row up to K = 4096
  int tpr = 64;
  while (tpr < 1024 && (nchunk + tpr - 1) / tpr > 4) tpr *= 2;
  const int64_t cpt = (nchunk + tpr - 1) / tpr;
  const int64_t blocks = N;
#define PTQ_S(TPR_, CPT_)                                                                                 \
  if (tpr == TPR_ && cpt <= CPT_) {                                                                       \
    k_ssz<DT, HAS_S, BITS, TPR_, CPT_><<<(unsigned)blocks, TPR_, 0, stream>>>(                            \
        w, N, K, s, max_iter, thr, min_scale, scale, wq, iters, mse);                                     \
    return hipGetLastError();                                                                             \
  }
  PTQ_S(64, 1) PTQ_S(64, 2) PTQ_S(64, 4)
  PTQ_S(128, 4) PTQ_S(256, 4) PTQ_S(512, 4) PTQ_S(1024, 4) PTQ_S(1024, 8)
#undef PTQ_S
  return hipErrorInvalidValue;
}

template <int DT, bool HAS_S>
hipError_t dispatch_bits(const void* w, int64_t N, int64_t K, const float* s, int bits, int max_iter, double thr,
                         float min_scale, float* scale, void* wq, int32_t* iters, double* mse, hipStream_t stream) {
  if (bits == 8) return dispatch<DT, HAS_S, 8>(w, N, K, s, max_iter, thr, min_scale, scale, wq, iters, mse, stream);
  return dispatch<DT, HAS_S, 4>(w, N, K, s, max_iter, thr, min_scale, scale, wq, iters, mse, stream);
}

}  // namespace

hipError_t launch_ssz_asym(const void* w, int dtype, int64_t N, int64_t K, const float* s, int max_iter,
                           double threshold, float min_scale, float* scale, int32_t* zero_point, int8_t* wq,
                           int32_t* iters, double* mse, hipStream_t stream) {
  if (dtype == PTQ_BF16)
    return s ? dispatch_asym<PTQ_BF16, true>(w, N, K, s, max_iter, threshold, min_scale, scale, zero_point, wq,
                                             iters, mse, stream)
             : dispatch_asym<PTQ_BF16, false>(w, N, K, s, max_iter, threshold, min_scale, scale, zero_point, wq,
                                              iters, mse, stream);
  return s ? dispatch_asym<PTQ_F32, true>(w, N, K, s, max_iter, threshold, min_scale, scale, zero_point, wq, iters,
                                          mse, stream)
           : dispatch_asym<PTQ_F32, false>(w, N, K, s, max_iter, threshold, min_scale, scale, zero_point, wq, iters,
                                           mse, stream);
}

hipError_t launch_ssz(const void* w, int dtype, int64_t N, int64_t K, const float* s, int bits, int max_iter,
                      double threshold, float min_scale, float* scale, void* wq, int32_t* iters, double* mse,
                      hipStream_t stream) {
  if (dtype == PTQ_BF16)
    return s ? dispatch_bits<PTQ_BF16, true>(w, N, K, s, bits, max_iter, threshold, min_scale, scale, wq, iters,
                                             mse, stream)
             : dispatch_bits<PTQ_BF16, false>(w, N, K, s, bits, max_iter, threshold, min_scale, scale, wq, iters,
                                              mse, stream);
  return s ? dispatch_bits<PTQ_F32, true>(w, N, K, s, bits, max_iter, threshold, min_scale, scale, wq, iters, mse,
                                          stream)
           : dispatch_bits<PTQ_F32, false>(w, N, K, s, bits, max_iter, threshold, min_scale, scale, wq, iters, mse,
                                           stream);
}

}  // namespace ptq
