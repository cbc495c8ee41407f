// ssz.hip -- MinMax + SSZ per-output-channel weight quantization (gfx950):
// symmetric int8/int4 and asymmetric int8 (k_ssz), short symmetric rows of at
// most 512 elements, several rows per wave (k_ssz_rows), and the exact search
// (exact_row) for the rows those two cannot certify: inside the symmetric
// k_ssz instances of up to 128 threads, else in a launch of its own
// (k_ssz_exact).
//
// [SSZ] flow: MinMax initial parameters, then least-squares refits for the
// current codes, a refit kept only when it lowers the quantization error,
// until the relative or absolute change falls under the threshold or the
// iteration limit is reached; symmetric quantization fixes the offset at 0.
// [SQ] the weight side of the smoothing fold, w_hat = fl32(w * s_j).
// [INT8] 2.1 the codes: clamp(rne(fl32(w_hat / S)) + Z).
//
// One block of TPR threads owns one row (output channel).  The row is read
// from HBM once and stays in registers (CPT chunks of 16 elements per thread)
// for every pass; all passes are ALU work.  A pass for (S, Z) computes per
// element the code q, its offset-relative value r = q - Z (r = q when
// symmetric) and accumulates
//   P = sum w_hat r (fp64),  R2 = sum r^2,  R1 = sum r (exact integers),
// the sums the least-squares step needs.  The quotient w_hat / S is the IEEE
// quotient whenever 2^-100 <= S <= 2^100: for rows of up to 32768 elements
// (at most 64 per thread), held in fp64, the fp64 product with an fp64
// reciprocal (rcp64) rounded to fp32 (quot64); for longer rows, held in fp32,
// div_rn's corrected product with the IEEE reciprocal (an element under
// 2^-102 then has |w_hat / S| < 1/4 and the code 0 either way).
//
// Every decision is the one the exact values give:
//  * P is exact.  A non-zero r needs |w_hat / S| > 1/2, so every non-zero term
//    w_hat r is a multiple of 2^(E-25) (E the binary exponent of S), and it is
//    never negative (r has the sign of w_hat).  While the sum stays under
//    2^(E+28) every partial sum is an integer multiple of 2^(E-25) below
//    2^53 of them: no fp64 addition rounds, in any order.  A computed sum under
//    2^(E+27) proves that (a sum that had rounded would be at least
//    2^(E+28)(1 - 2^-40)).
//  * The error of a pass comes from the expansion
//      K mse = W2 - 2 S P + S^2 R2,  W2 = sum w_hat^2 (fp64, once per row),
//    whose rounding is bounded by (h + 8) u (W2 + 2 S P + S^2 R2), u = 2^-53,
//    h the longest chain of fp64 additions in the reduction of W2 (serial per
//    lane, then the butterfly, then the waves).  Each error is therefore
//    known as an interval holding the exact error (its exact sum rounded to
//    fp64, divided by K), and a keep or convergence decision that the
//    intervals settle is the exact decision.
//  * A refit that returns the kept parameters exactly is the same candidate:
//    its error equals the best one, so the step converges (threshold > 0)
//    without a pass.
// A row for which any of this fails -- a scale outside div_rn's range, a P
// the certificate does not cover, a decision the intervals leave open (none
// in 330,000 passes over the workloads' weights) -- is searched again with the
// IEEE division and every sum in double-double, rounded once: by the same
// block, right away, in the k_ssz instances that can (ssz_inline_exact); the
// others and k_ssz_rows write a NaN scale and nothing else for it, and
// k_ssz_exact, launched next on the same stream, searches the rows so marked.
// The exact search's roundings of the exact sums give the correctly rounded
// fp64 value unless an exact sum lies within about 2^-90 relative of an fp64
// rounding boundary.
// Sums are reduced with butterflies in which both lanes of a pair combine the
// same two operands, and across waves through LDS in wave order, so every
// lane of a row holds identical bits and every decision is uniform.
#include "ptq_dev.hpp"
#include "ptq_launch.hpp"

namespace ptq {

namespace {

constexpr double kU = 0x1p-53;  // unit roundoff of binary64

// An interval [lo, hi] holding an exact error value.
struct Ival {
  double lo, hi;
};

enum : int { kNo = 0, kYes = 1, kUnk = 2 };

__device__ __forceinline__ int tri_or(int a, int b) {
  return (a == kYes || b == kYes) ? kYes : ((a == kNo && b == kNo) ? kNo : kUnk);
}

struct Decision {
  int keep, conv;
};

// The greedy rule (keep the candidate iff cur < best) and the convergence test
//   best == 0  or  |d| < thr  or  fl64(d / best) < thr,   d = fl64(best - cur),
// for every best in b and cur in c.  Rounding is monotone, so fl64(best - cur) lies in
// [fl64(b.lo - c.hi), fl64(b.hi - c.lo)] and the quotient between the quotients of the end points.  The
// relative test matters only when best > 0 (best == 0 converges anyway).  On points the result is the plain
// rule and test.
__device__ __forceinline__ int conv_of(Ival b, double dlo, double dhi, double thr) {
  const int z = b.hi == 0.0 ? kYes : (b.lo > 0.0 ? kNo : kUnk);
  const int ab = (dlo > -thr && dhi < thr) ? kYes : ((dlo >= thr || dhi <= -thr) ? kNo : kUnk);
  int rel;
  if (thr > 0.0 && dhi <= 0.0) {
    rel = kYes;  // quotient <= 0 < thr
  } else if (dlo >= 2.0 * (thr * b.hi)) {
    rel = kNo;  // d > thr * best exactly (one rounding cannot halve the product), so the quotient rounds to >= thr
  } else {
    const double inf = __builtin_huge_val();
    const double fmax = dhi >= 0.0 ? (b.lo > 0.0 ? dhi / b.lo : inf) : dhi / b.hi;
    const double fmin = dlo >= 0.0 ? dlo / b.hi : (b.lo > 0.0 ? dlo / b.lo : -inf);
    rel = fmax < thr ? kYes : (fmin >= thr ? kNo : kUnk);
  }
  return tri_or(z, tri_or(ab, rel));
}

__device__ __forceinline__ Decision decide(Ival b, Ival c, double thr) {
  Decision r;
  r.keep = c.hi < b.lo ? kYes : (c.lo >= b.hi ? kNo : kUnk);
  r.conv = conv_of(b, b.lo - c.hi, b.hi - c.lo, thr);
  return r;
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

// The interval of the exact mean error for exact pass sums, from the expansion and its rounding bound
// hu * (W2 + 2 S P + S^2 R2), hu = (h + 8) u.
__device__ __forceinline__ Ival err_ival(double w2, float S, double P, double R2, double hu, const DivK& per_elem) {
  const double Sd = (double)S;
  const double s2 = Sd * Sd * R2;
  const double e = (w2 - 2.0 * Sd * P) + s2;
  const double bnd = hu * ((w2 + 2.0 * Sd * P) + s2);
  const double lo = e - bnd, hi = e + bnd;
  return Ival{per_elem(lo > 0.0 ? lo : 0.0), per_elem(hi > 0.0 ? hi : 0.0)};
}

// A candidate S1 whose pass sums P and R2 equal the kept scale S0's (the same codes, or codes with the same two
// sums) has the same error function e(S) = (W2 - 2 S P + S^2 R2) / K, so the difference of the two errors is
//   e(S0) - e(S1) = (S0 - S1) (R2 (S0 + S1) - 2 P) / K,
// free of the cancellation against W2 that widens the expansion's intervals -- such candidates differ from the
// kept error by as little as 1e-11 relative when S1 is S0's neighbour.  With S1 in [S0/2, 2 S0] and R2 < 2^27,
// S0 - S1, S0 + S1, R2 (S0 + S1) and 2 P are exact, so the computed difference d carries three or four roundings
// (relative error below 8u).  The oracle's own fl64(best - cur), of its two rounded errors, lies within
// 2^-51 (best + |d|) of the exact difference.  The decisions follow from d, and the candidate's error interval
// from the kept one.  Returns false (nothing decided) outside those conditions.
__device__ __forceinline__ bool same_sums_decide(float S0, float S1, double P, double R2, Ival best, double thr,
                                                 const DivK& per_elem, Decision& dc, Ival& cur) {
  if (!(R2 < 0x1p27) || !(S1 >= 0.5f * S0 && S1 <= 2.0f * S0)) return false;
  const double s0 = (double)S0, s1 = (double)S1;
  const double t = R2 * (s0 + s1) - 2.0 * P;
  const double d = per_elem((s0 - s1) * t);
  const double ad = __builtin_fabs(d);
  const double ed = 8.0 * kU * ad;                        // the exact difference is within d +- ed
  const double eo = ed + 0x1p-50 * (best.hi + ad);        // the oracle's difference is within d +- eo
  dc.keep = d - eo > 0.0 ? kYes : (d <= 0.0 ? kNo : kUnk);  // d has the exact difference's sign
  dc.conv = conv_of(best, d - eo, d + eo, thr);
  const double clo = best.lo - (d + eo), chi = best.hi - (d - eo);
  cur = Ival{clo > 0.0 ? clo : 0.0, chi > 0.0 ? chi : 0.0};
  return true;
}

// 2^(E + 27), E the binary exponent of a normal S: a computed P below it is exact (see the file header)
__device__ __forceinline__ double p_cert(float S) {
  const int e = (int)((__float_as_uint(S) >> 23) & 0xFFu) - 127;
  return __builtin_ldexp(1.0, e + 27);
}

// Offset-relative code r = q - Z of one element, q = clamp(rne(fl32(w / S)) + Z); symmetric: Z = 0 and the
// range [-qmax, qmax].  rS = fl32(1 / S), 2^-100 <= S <= 2^100.
template <bool ASYM>
__device__ __forceinline__ float rel_code(float w, float S, float rS, float zf, float qmax) {
  const float t = __builtin_rintf(div_rn(w, S, rS));
  if constexpr (ASYM) return fminf(fmaxf(t + zf, -128.0f), 127.0f) - zf;
  return fminf(fmaxf(t, -qmax), qmax);
}

// the same code through the IEEE division (any S)
template <bool ASYM>
__device__ __forceinline__ float rel_code_ieee(float w, float S, float zf, float qmax) {
  const float t = __builtin_rintf(w / S);
  if constexpr (ASYM) return fminf(fmaxf(t + zf, -128.0f), 127.0f) - zf;
  return fminf(fmaxf(t, -qmax), qmax);
}

// the same code from the fp64 row value and r64 = rcp64(S) (quot64), 2^-100 <= S <= 2^100
template <bool ASYM>
__device__ __forceinline__ float rel_code64(double w, double r64, float zf, float qmax) {
  const float t = __builtin_rintf(quot64(w, r64));
  if constexpr (ASYM) return fminf(fmaxf(t + zf, -128.0f), 127.0f) - zf;
  return fminf(fmaxf(t, -qmax), qmax);
}

template <typename T>
__device__ __forceinline__ T tmin(T a, T b) {
  if constexpr (sizeof(T) == 8) return __builtin_fmin(a, b);
  else return __builtin_fminf(a, b);
}
template <typename T>
__device__ __forceinline__ T tmax(T a, T b) {
  if constexpr (sizeof(T) == 8) return __builtin_fmax(a, b);
  else return __builtin_fmaxf(a, b);
}
template <typename T>
__device__ __forceinline__ T tabs(T a) {
  if constexpr (sizeof(T) == 8) return __builtin_fabs(a);
  else return __builtin_fabsf(a);
}

// A row's elements in registers: fp64 (the widening done once, 2 registers per element) up to 64 per thread in
// blocks of up to 512 threads, else fp32, where the doubles would not fit (1024 threads leave 128 registers).
template <bool F64>
struct RowElemOf {
  using type = double;
};
template <>
struct RowElemOf<false> {
  using type = float;
};
template <int TPR, int CPT>
using RowElem = RowElemOf<(CPT <= 4 && TPR <= 512)>;

// Row n of w, folded (w_hat = fl32(w * s_j)), into registers: CPT chunks of 16 elements per thread,
// chunk c8 of thread tid at elements (tid + TPR*c8)*16 ..; chunks past the row are zeros (they add
// nothing to any sum, have the code r = 0, and never change a max of magnitudes).
template <int DT, bool HAS_S, int TPR, int CPT, typename T>
__device__ __forceinline__ void load_row(const void* __restrict__ w, int64_t n, int64_t K, const float* __restrict__ s,
                                         int tid, T (&wh)[CPT][16]) {
  const int64_t nchunk = K / 16;
#pragma unroll
  for (int c8 = 0; c8 < CPT; ++c8) {
    const int64_t c = tid + (int64_t)TPR * c8;
    if (c < nchunk) {
      float a8[8], b8[8], f[16];
      load8<DT>(w, n * K + c * 16, a8);
      load8<DT>(w, n * K + c * 16 + 8, b8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        f[e] = a8[e];
        f[e + 8] = b8[e];
      }
      if constexpr (HAS_S) {
        const float4* sp = reinterpret_cast<const float4*>(s + c * 16);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const float4 sv = sp[q4];
          f[4 * q4 + 0] = f[4 * q4 + 0] * sv.x;
          f[4 * q4 + 1] = f[4 * q4 + 1] * sv.y;
          f[4 * q4 + 2] = f[4 * q4 + 2] * sv.z;
          f[4 * q4 + 3] = f[4 * q4 + 3] * sv.w;
        }
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) wh[c8][e] = (T)f[e];  // the fold in fp32, then widened exactly
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) wh[c8][e] = (T)0.0f;
    }
  }
}

// One pass over a thread's elements for (S, Z): P, R2, R1 of its elements.  S is in div_rn's domain (the callers
// check it); elements held in fp64 take the fp64 product's quotient, elements in fp32 div_rn's.
template <int CPT, bool ASYM, typename T>
__device__ __forceinline__ void lane_pass(const T (&wh)[CPT][16], float S, float zf, float qmax, double& p,
                                          float& r2, float& r1) {
  double a = 0.0;
  float b = 0.0f;  // at most 16*CPT terms of <= 255^2 each: exact in fp32
  float c = 0.0f;
  if constexpr (sizeof(T) == 8) {
    const double r64 = rcp64(S);
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float r = rel_code64<ASYM>(wh[m][k], r64, zf, qmax);
        a = __builtin_fma(wh[m][k], (double)r, a);
        b = __builtin_fmaf(r, r, b);
        if constexpr (ASYM) c += r;
      }
    }
  } else {
    const float rS = rcp_rn(S);
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float r = rel_code<ASYM>(wh[m][k], S, rS, zf, qmax);
        a = __builtin_fma((double)wh[m][k], (double)r, a);
        b = __builtin_fmaf(r, r, b);
        if constexpr (ASYM) c += r;
      }
    }
  }
  p = a;
  r2 = b;
  r1 = c;
}

// Writes a row's codes (int8, or int4 nibbles) for chunk c of the row.
template <int BITS>
__device__ __forceinline__ void store_codes(void* wq, int64_t n, int64_t K, int64_t c, const float (&q)[16]) {
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

// The state of a row's search, identical in every lane of the row.
struct RowState {
  float S;
  int Z;
  double P, R2, R1;  // the kept parameters' pass sums (exact)
  Ival best;
};

// One step of the search from the kept state st: the least-squares refit.  Returns false when there is nothing
// to fit (the row stops); else the candidate (Sc, Zc).
template <bool ASYM>
__device__ __forceinline__ bool refit(const RowState& st, double Kd, double w1, const DivK& per_elem,
                                      float min_scale, float& Sc, int& Zc) {
  if constexpr (ASYM) {
    const double det = Kd * st.R2 - st.R1 * st.R1;  // exact: integers below 2^53
    if (det <= 0.0) return false;
    const double a = (Kd * st.P - w1 * st.R1) / det;
    const double b = per_elem(w1 - a * st.R1);
    Sc = (float)a;
    Sc = Sc < min_scale ? min_scale : Sc;
    const double zr = (double)st.Z - __builtin_rint(b / a);
    Zc = zr < -128.0 ? -128 : (zr > 127.0 ? 127 : (int)zr);
  } else {
    if (st.R2 == 0.0) return false;
    Sc = (float)(st.P / st.R2);
    Sc = Sc < min_scale ? min_scale : Sc;
    Zc = 0;
  }
  return true;
}

// MinMax init of the parameters from the row's max magnitude (symmetric, `hi`) or min lo and max hi
template <bool ASYM>
__device__ __forceinline__ void minmax_init(float lo, float hi, float qmax, float min_scale, float& S, int& Z) {
  if constexpr (ASYM) {
    S = (hi - lo) / 255.0f;
    S = S < min_scale ? min_scale : S;
    const float z0 = -128.0f - __builtin_rintf(lo / S);
    Z = (int)fminf(fmaxf(z0, -128.0f), 127.0f);
  } else {
    S = hi / qmax;
    S = S < min_scale ? min_scale : S;
    Z = 0;
  }
}

constexpr int kExactTpr = 256;

template <int DT, bool HAS_S>
__device__ __forceinline__ float load_folded(const void* __restrict__ w, const float* __restrict__ s, int64_t n,
                                             int64_t K, int64_t k) {
  float v;
  if constexpr (DT == PTQ_BF16)
    v = __uint_as_float((uint32_t)reinterpret_cast<const uint16_t*>(w)[n * K + k] << 16);
  else
    v = reinterpret_cast<const float*>(w)[n * K + k];
  if constexpr (HAS_S) v = v * s[k];
  return v;
}

// The exact search of row n by a block of NT threads, reading the row from memory on every pass: codes by the
// IEEE division, P, the error and the asymmetric W1 summed in double-double and rounded once, R2 and R1 exact;
// then the plain greedy rule and convergence test on those values.  Writes all of the row's outputs.  Every
// thread of the block calls it (it synchronises the block); xd holds 4 NT/64 doubles and xf 2 NT/64 floats of LDS.
template <int DT, bool HAS_S, int BITS, bool ASYM, int NT>
__device__ __forceinline__ void exact_row(const void* __restrict__ w, int64_t n, int64_t K, const float* __restrict__ s,
                                          int max_iter, double thr, float min_scale, float* __restrict__ scale,
                                          int32_t* __restrict__ zero_point, void* __restrict__ wq,
                                          int32_t* __restrict__ iters, double* __restrict__ mse, double* xd, float* xf,
                                          int tid) {
  constexpr int NW = NT / kWave;
  constexpr float QMAX = BITS == 8 ? 127.0f : 7.0f;
  const double Kd = (double)K;
  const DivK per_elem = make_divk(K);

  // sums over the block (every thread gets the same bits)
  auto bsum_dd = [&](DD v) -> double {
    v = group_sum_dd<64>(v);
    __syncthreads();
    if ((tid & (kWave - 1)) == 0) {
      xd[tid / kWave] = v.hi;
      xd[NW + tid / kWave] = v.lo;
    }
    __syncthreads();
    DD t{xd[0], xd[NW]};
#pragma unroll
    for (int i = 1; i < NW; ++i) t = dd_add(t, DD{xd[i], xd[NW + i]});
    return t.hi + t.lo;
  };
  auto bsum = [&](double v) -> double {  // exact integer sums
    v = wave_sum(v);
    __syncthreads();
    if ((tid & (kWave - 1)) == 0) xd[2 * NW + tid / kWave] = v;
    __syncthreads();
    double t = xd[2 * NW];
#pragma unroll
    for (int i = 1; i < NW; ++i) t += xd[2 * NW + i];
    return t;
  };
  auto bminmax = [&](float& lo, float& hi) {
    lo = -wave_max(-lo);
    hi = wave_max(hi);
    __syncthreads();
    if ((tid & (kWave - 1)) == 0) {
      xf[tid / kWave] = lo;
      xf[NW + tid / kWave] = hi;
    }
    __syncthreads();
    lo = xf[0];
    hi = xf[NW];
#pragma unroll
    for (int i = 1; i < NW; ++i) {
      lo = fminf(lo, xf[i]);
      hi = fmaxf(hi, xf[NW + i]);
    }
  };

  float lo = __builtin_huge_valf(), hi = ASYM ? -__builtin_huge_valf() : 0.0f;
  DD w1{0.0, 0.0};
  for (int64_t k = tid; k < K; k += NT) {
    const float v = load_folded<DT, HAS_S>(w, s, n, K, k);
    if constexpr (ASYM) {
      lo = fminf(lo, v);
      hi = fmaxf(hi, v);
      w1 = dd_add_d(w1, (double)v);
    } else {
      hi = fmaxf(hi, fabsf(v));
    }
  }
  bminmax(lo, hi);
  const double W1 = ASYM ? bsum_dd(w1) : 0.0;

  // P, R2, R1 and the mean error of (S, Z), every sum exact
  auto pass = [&](float S, int Z, double& P, double& R2, double& R1) -> double {
    const float zf = (float)Z;
    const double Sd = (double)S;
    DD p{0.0, 0.0}, e{0.0, 0.0};
    double r2 = 0.0, r1 = 0.0;
    for (int64_t k = tid; k < K; k += NT) {
      const float v = load_folded<DT, HAS_S>(w, s, n, K, k);
      const float r = rel_code_ieee<ASYM>(v, S, zf, QMAX);
      p = dd_add_d(p, (double)v * (double)r);  // exact product
      double dh, dl;
      two_sum((double)v, -(Sd * (double)r), dh, dl);  // S r is exact in fp64
      DD t = two_sqr(dh);
      t.lo += dh * (2.0 * dl) + dl * dl;
      e = dd_add(e, t);
      r2 += (double)r * (double)r;
      r1 += (double)r;
    }
    P = bsum_dd(p);
    R2 = bsum(r2);
    R1 = ASYM ? bsum(r1) : 0.0;
    return per_elem(bsum_dd(e));
  };

  RowState st;
  minmax_init<ASYM>(lo, hi, QMAX, min_scale, st.S, st.Z);
  const double b0 = pass(st.S, st.Z, st.P, st.R2, st.R1);
  double best = b0;
  int it = 0;
  for (int i = 1; i <= max_iter; ++i) {
    it = i;
    float Sc;
    int Zc;
    if (!refit<ASYM>(st, Kd, W1, per_elem, min_scale, Sc, Zc)) break;
    RowState c;
    c.S = Sc;
    c.Z = Zc;
    const double cur = pass(Sc, Zc, c.P, c.R2, c.R1);
    const double d = best - cur;
    const bool conv = (best == 0.0) || (fabs(d) < thr) || (d / best < thr);
    if (cur < best) {
      st = c;
      best = cur;
    }
    if (conv) break;
  }

  // codes of the kept parameters
  if (wq) {
    const float zf = (float)st.Z;
    for (int64_t k = tid; k < K; k += NT) {
      const float v = load_folded<DT, HAS_S>(w, s, n, K, k);
      const float q = rel_code_ieee<ASYM>(v, st.S, zf, QMAX) + (ASYM ? zf : 0.0f);
      if constexpr (BITS == 8) {
        reinterpret_cast<int8_t*>(wq)[n * K + k] = (int8_t)(int)q;
      } else {
        // two codes per byte: the thread of the even element writes the pair
        const float v1 = load_folded<DT, HAS_S>(w, s, n, K, k ^ 1);
        const float q1 = rel_code_ieee<false>(v1, st.S, 0.0f, QMAX);
        if ((k & 1) == 0)
          reinterpret_cast<uint8_t*>(wq)[n * (K / 2) + k / 2] =
              (uint8_t)(((uint32_t)(int)q & 0xFu) | (((uint32_t)(int)q1 & 0xFu) << 4));
      }
    }
  }
  if (tid == 0) {
    scale[n] = st.S;
    if constexpr (ASYM) zero_point[n] = st.Z;
    if (iters) iters[n] = it;
    if (mse) mse[n] = best;
  }
}

// Whether k_ssz searches the rows it cannot certify itself (exact_row, by the same block, right away), which
// spares the launch of k_ssz_exact: the symmetric instances of up to 128 threads (rows of up to 8192 elements).
// The others mark such rows with a NaN scale (and no other output) for k_ssz_exact: the asymmetric and
// 1024-thread instances have no registers to spare, and the 256-thread one ran ~1% slower with the search inside.
constexpr bool ssz_inline_exact(bool asym, int tpr) { return !asym && tpr <= 128; }

// MinMax + SSZ, symmetric (ASYM = false; qmax 127 or 7) or asymmetric int8; one row per block of TPR threads.
// Rows it cannot certify are searched exactly (see ssz_inline_exact).  Register use is capped at two waves
// per SIMD (256 registers): left free, the asymmetric variant takes more and runs one wave per SIMD.
template <int DT, bool HAS_S, int BITS, bool ASYM, int TPR, int CPT>
__global__ __launch_bounds__(TPR) __attribute__((amdgpu_waves_per_eu(2))) void k_ssz(
                                             const void* __restrict__ w, int64_t N, int64_t K,
                                             const float* __restrict__ s, int max_iter, double thr, float min_scale,
                                             float* __restrict__ scale, int32_t* __restrict__ zero_point,
                                             void* __restrict__ wq, int32_t* __restrict__ iters,
                                             double* __restrict__ mse) {
  constexpr int NW = TPR / kWave;
  constexpr float QMAX = BITS == 8 ? 127.0f : 7.0f;
  __shared__ double ring[2][3 * NW];  // pass sums, alternating halves
  __shared__ double xd[4 * NW];  // (also the exact search's block sums)
  __shared__ float xf[2 * NW];
  int par = 0;
  const int tid = threadIdx.x;
  const int64_t nchunk = K / 16;
  const double Kd = (double)K;
  const DivK per_elem = make_divk(K);
  // rounding bound of the expansion: the longest addition chain of W2 is CPT*16 per lane, 6 butterfly steps,
  // NW - 1 wave partials; (h + 8) u, rounded up
  const double hu = (double)(CPT * 16 + 6 + NW + 8) * kU * (1.0 + 0x1p-20);

  for (int64_t n = blockIdx.x; n < N; n += gridDim.x) {
    using T = typename RowElem<TPR, CPT>::type;
    T wh[CPT][16];
    load_row<DT, HAS_S, TPR, CPT>(w, n, K, s, tid, wh);

    // row statistics: W2 = sum w_hat^2 (fp64); the max magnitude (symmetric) or min and max; W1 = sum w_hat
    T lo_t = (T)__builtin_huge_valf(), hi_t = (T)(ASYM ? -__builtin_huge_valf() : 0.0f);
    double w2 = 0.0;
    DD w1dd{0.0, 0.0};
#pragma unroll
    for (int c8 = 0; c8 < CPT; ++c8) {
      const bool in = tid + (int64_t)TPR * c8 < nchunk;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const T v = wh[c8][e];
        if constexpr (ASYM) {
          lo_t = tmin(lo_t, in ? v : lo_t);
          hi_t = tmax(hi_t, in ? v : hi_t);
          w1dd = dd_add_d(w1dd, (double)v);
        } else {
          hi_t = tmax(hi_t, tabs(v));
        }
        const double x = (double)v;
        w2 = __builtin_fma(x, x, w2);
      }
    }
    float lo = (float)lo_t, hi = (float)hi_t;  // fp32 values: exact
    if constexpr (ASYM) lo = -wave_max(-lo);
    hi = wave_max(hi);
    w2 = wave_sum(w2);
    if constexpr (ASYM) w1dd = group_sum_dd<64>(w1dd);
    if constexpr (NW > 1) {
      __syncthreads();
      if ((tid & (kWave - 1)) == 0) {
        xf[tid / kWave] = lo;
        xf[NW + tid / kWave] = hi;
        xd[tid / kWave] = w2;
      }
      __syncthreads();
      lo = xf[0];
      hi = xf[NW];
      w2 = xd[0];
#pragma unroll
      for (int i = 1; i < NW; ++i) {
        lo = fminf(lo, xf[i]);
        hi = fmaxf(hi, xf[NW + i]);
        w2 += xd[i];
      }
      if constexpr (ASYM) {
        __syncthreads();
        if ((tid & (kWave - 1)) == 0) {
          xd[tid / kWave] = w1dd.hi;
          xd[NW + tid / kWave] = w1dd.lo;
        }
        __syncthreads();
        DD t{xd[0], xd[NW]};
#pragma unroll
        for (int i = 1; i < NW; ++i) t = dd_add(t, DD{xd[i], xd[NW + i]});
        w1dd = t;
      }
    }
    const double w1 = uni(w1dd.hi + w1dd.lo);
    w2 = uni(w2);
    lo = uni(lo);
    hi = uni(hi);

    // pass sums for (S, Z) over the row; false when the scale is outside div_rn's range or P is not certified
    auto pass = [&](float Sx, int Zx, double& P, double& R2, double& R1) -> bool {
      if (!div_rn_divisor_ok(Sx)) return false;
      float r2, r1;
      lane_pass<CPT, ASYM>(wh, Sx, (float)Zx, QMAX, P, r2, r1);
      P = wave_sum(P);
      int i2 = wave_sum((int)r2), i1 = ASYM ? wave_sum((int)r1) : 0;
      R2 = (double)i2;
      R1 = (double)i1;
      if constexpr (NW > 1) {
        // a two-pass slot ring: the readers of a slot two passes ago finished before the barrier in between
        double* rs = ring[par];
        par ^= 1;
        const int wv = tid / kWave;
        if ((tid & (kWave - 1)) == 0) {
          rs[wv] = P;
          rs[NW + wv] = R2;
          if constexpr (ASYM) rs[2 * NW + wv] = R1;
        }
        __syncthreads();
        P = rs[0];
        R2 = rs[NW];
        if constexpr (ASYM) R1 = rs[2 * NW];
#pragma unroll
        for (int i = 1; i < NW; ++i) {
          P += rs[i];
          R2 += rs[NW + i];
          if constexpr (ASYM) R1 += rs[2 * NW + i];
        }
      }
      P = uni(P);
      R2 = uni(R2);
      if constexpr (ASYM) R1 = uni(R1);
      return P < p_cert(Sx);
    };

    RowState st;
    minmax_init<ASYM>(lo, hi, QMAX, min_scale, st.S, st.Z);
    bool ok = pass(st.S, st.Z, st.P, st.R2, st.R1);
    st.best = err_ival(w2, st.S, st.P, st.R2, hu, per_elem);
    st.best = Ival{uni(st.best.lo), uni(st.best.hi)};

    // least-squares refits, greedy, per-row convergence
    int it = 0, i = 1;
    RowState c;  // the last candidate
    for (;;) {
      bool open = false;  // the intervals left the last candidate's decision open
      for (; ok && i <= max_iter; ++i) {
        it = i;
        float Sc;
        int Zc;
        if (!refit<ASYM>(st, Kd, w1, per_elem, min_scale, Sc, Zc)) break;
        if (Sc == st.S && Zc == st.Z) {
          // the kept parameters again: the same codes and error, d = 0
          if (thr > 0.0 || st.best.hi == 0.0) break;
          if (st.best.lo > 0.0) it = max_iter;  // thr == 0, best > 0: the same candidate at every remaining step
          else ok = false;
          break;
        }
        c.S = Sc;
        c.Z = Zc;
        if (!pass(Sc, Zc, c.P, c.R2, c.R1)) {
          ok = false;
          break;
        }
        c.best = err_ival(w2, Sc, c.P, c.R2, hu, per_elem);
        c.best = Ival{uni(c.best.lo), uni(c.best.hi)};
        Decision dc;
        const double dlo = st.best.lo - c.best.hi;
        if (dlo > 0.0 && dlo >= thr && st.best.lo > 0.0 && dlo >= 2.0 * (thr * st.best.hi)) {
          // (wave-uniform) the common outcome, which decide() reaches through the same comparisons: a definite
          // improvement of at least thr, absolute and relative, for every error in the intervals
          dc.keep = kYes;
          dc.conv = kNo;
        } else {
          dc = decide(st.best, c.best, thr);
        }
        if (dc.keep == kUnk || dc.conv == kUnk) {
          open = true;
          break;
        }
        if (dc.keep == kYes) st = c;
        if (dc.conv == kYes) break;
      }
      if (!open) break;
      // (off the loop, so the common path stays as it is) a candidate with the kept codes' sums again: decide
      // from the exact difference of the two errors, then go on with the next step
      Decision dc;
      Ival cs;
      if (!(c.P == st.P && c.R2 == st.R2 && same_sums_decide(st.S, c.S, st.P, st.R2, st.best, thr, per_elem, dc, cs)) ||
          dc.keep == kUnk || dc.conv == kUnk) {
        ok = false;
        break;
      }
      c.best = Ival{uni(cs.lo), uni(cs.hi)};
      if (dc.keep == kYes) st = c;
      if (dc.conv == kYes) break;
      ++i;
    }

    if (!ok) {
      // a row this search cannot certify: the exact search
      if constexpr (ssz_inline_exact(ASYM, TPR))
        exact_row<DT, HAS_S, BITS, ASYM, TPR>(w, n, K, s, max_iter, thr, min_scale, scale, zero_point, wq, iters, mse,
                                              xd, xf, tid);
      else if (tid == 0)
        scale[n] = __builtin_nanf("");
      continue;
    }
    // codes of the kept parameters, and their error summed directly (the reported mse)
    double e_dir = 0.0;
    if (wq || mse) {
      // st.S passed the domain check of its pass
      const float rS = sizeof(T) == 8 ? 0.0f : rcp_rn(st.S), zf = (float)st.Z;
      const double r64 = sizeof(T) == 8 ? rcp64(st.S) : 0.0;
      const double Sd = (double)st.S;
#pragma unroll
      for (int c8 = 0; c8 < CPT; ++c8) {
        const int64_t c = tid + (int64_t)TPR * c8;
        float q[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          float r;
          if constexpr (sizeof(T) == 8) r = rel_code64<ASYM>(wh[c8][e], r64, zf, QMAX);
          else r = rel_code<ASYM>(wh[c8][e], st.S, rS, zf, QMAX);
          q[e] = ASYM ? r + zf : r;
          const double dd = __builtin_fma(-Sd, (double)r, (double)wh[c8][e]);  // S r is exact in fp64
          e_dir = __builtin_fma(dd, dd, e_dir);
        }
        if (wq && c < nchunk) store_codes<BITS>(wq, n, K, c, q);
      }
      if (mse) {
        e_dir = wave_sum(e_dir);
        if constexpr (NW > 1) {
          __syncthreads();
          if ((tid & (kWave - 1)) == 0) xd[tid / kWave] = e_dir;
          __syncthreads();
          e_dir = xd[0];
#pragma unroll
          for (int i = 1; i < NW; ++i) e_dir += xd[i];
        }
      }
    }
    if (tid == 0) {
      scale[n] = st.S;
      if constexpr (ASYM) zero_point[n] = st.Z;
      if (iters) iters[n] = it;
      if (mse) mse[n] = per_elem(e_dir);
    }
  }
}

// ---------------------------------------------------------------------------
// Short symmetric rows (K <= 512, at most 32 chunks of 16): one wave holds R = 64 / G rows, G lanes each
// (G = the chunk count rounded up to a power of two, 1 to 32), one 16-element chunk per lane -- the same pass
// length per lane as the one-wave row kernel, which at these K leaves half its lanes or more idle.  Each group
// of G lanes carries its own row's state, reduces inside the group only (DPP moves within the 16-lane row, plus
// the 16-lane swap for G = 32), and stops updating when its row converges or is deferred, while the wave runs
// until all its rows have.  Same formulas and decisions per row as k_ssz.

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
  int lg = 0;
  while ((1 << lg) < G) ++lg;
  const double hu = (double)(16 + lg + 8) * kU * (1.0 + 0x1p-20);

  // every lane runs the same number of row groups (uniform loop); rows past N compute on zeros, unwritten
  for (int64_t n0 = (int64_t)blockIdx.x * R; n0 < N; n0 += (int64_t)gridDim.x * R) {
    const int64_t n = n0 + lane / G;
    const bool live = n < N;
    float wh[CPT][16];
    load_row<DT, HAS_S, G, CPT>(w, live ? n : n0, K, s, gl, wh);
    if (!live) {
#pragma unroll
      for (int e = 0; e < 16; ++e) wh[0][e] = 0.0f;
    }
    float m = 0.0f;
    double w2 = 0.0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      m = fmaxf(m, fabsf(wh[0][e]));
      const double x = (double)wh[0][e];
      w2 = __builtin_fma(x, x, w2);
    }
    m = group_max<G>(m);
    w2 = group_sum<G>(w2);

    // the group's pass sums for its own scale Sx (a scale outside div_rn's range computes garbage, and the
    // caller defers the row); returns whether P is certified
    auto pass = [&](float Sx, double& P, double& R2) -> bool {
      const bool in = div_rn_divisor_ok(Sx);
      const float Su = in ? Sx : 1.0f;
      float r2, r1;
      lane_pass<CPT, false>(wh, Su, 0.0f, QMAX, P, r2, r1);
      P = group_sum<G>(P);
      R2 = (double)group_sum<G>((int)r2);
      return in && P < p_cert(Su);
    };

    // MinMax init
    float S, Sp;
    int Z;
    minmax_init<false>(0.0f, m, QMAX, min_scale, S, Z);
    double P, R2;
    bool ok = pass(S, P, R2);
    Ival best = err_ival(w2, S, P, R2, hu, per_elem);

    // least-squares refits, greedy, per-row convergence; a row's state stays fixed once it stops
    int it = 0;
    bool active = live && ok;  // rows past N take no step
    for (int i = 1; i <= max_iter; ++i) {
      if (!__builtin_amdgcn_ballot_w64(active)) break;
      if (active) it = i;
      if (active && R2 == 0.0) active = false;
      float Sc = active ? (float)(P / R2) : S;
      Sc = Sc < min_scale ? min_scale : Sc;
      if (active && Sc == S) {
        // the kept scale again: the same codes and error (see k_ssz)
        if (!(thr > 0.0 || best.hi == 0.0)) {
          if (best.lo > 0.0) it = max_iter;
          else ok = false;
        }
        active = false;
      }
      Sp = active ? Sc : S;
      double Pc, R2c;
      const bool pok = pass(Sp, Pc, R2c);
      if (active && !pok) {
        ok = false;
        active = false;
      }
      Ival cur = err_ival(w2, Sc, Pc, R2c, hu, per_elem);
      Decision dc = decide(best, cur, thr);
      if ((dc.keep == kUnk || dc.conv == kUnk) && Pc == P && R2c == R2) {
        Ival cs;
        if (same_sums_decide(S, Sc, P, R2, best, thr, per_elem, dc, cs)) cur = cs;
      }
      if (active && (dc.keep == kUnk || dc.conv == kUnk)) {
        ok = false;
        active = false;
      }
      if (active && dc.keep == kYes) {
        S = Sc;
        best = cur;
        P = Pc;
        R2 = R2c;
      }
      if (active && dc.conv == kYes) active = false;
    }

    // codes of the kept scale, and its error summed directly
    double e_dir = 0.0;
    if (wq || mse) {
      const float Su = div_rn_divisor_ok(S) ? S : 1.0f;
      const float rS = rcp_rn(Su);
      const double Sd = (double)Su;
      const int64_t c = gl;
      float q[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        q[e] = rel_code<false>(wh[0][e], Su, rS, 0.0f, QMAX);
        const double dd = __builtin_fma(-Sd, (double)q[e], (double)wh[0][e]);  // S*q is exact in fp64
        e_dir = __builtin_fma(dd, dd, e_dir);
      }
      if (wq && live && ok && c < nchunk) store_codes<BITS>(wq, n, K, c, q);
      if (mse) e_dir = group_sum<G>(e_dir);
    }
    if (live && gl == 0) {
      scale[n] = ok ? S : __builtin_nanf("");
      if (ok && iters) iters[n] = it;
      if (ok && mse) mse[n] = per_elem(e_dir);
    }
  }
}

// ---------------------------------------------------------------------------
// The exact search (exact_row) for the rows k_ssz_rows and the k_ssz instances without the inline search defer
// (scale[n] is NaN), one row at a time per block of 256 threads.  Rows with a finite scale are left as they are.

template <int DT, bool HAS_S, int BITS, bool ASYM>
__global__ __launch_bounds__(kExactTpr) void k_ssz_exact(const void* __restrict__ w, int64_t N, int64_t K,
                                                         const float* __restrict__ s, int max_iter, double thr,
                                                         float min_scale, float* __restrict__ scale,
                                                         int32_t* __restrict__ zero_point, void* __restrict__ wq,
                                                         int32_t* __restrict__ iters, double* __restrict__ mse) {
  constexpr int NW = kExactTpr / kWave;
  __shared__ double xd[4 * NW];
  __shared__ float xf[2 * NW];
  __shared__ int flag;                // deferred rows in the current chunk
  __shared__ int list[kExactTpr];     // and their indices in the chunk
  const int tid = threadIdx.x;

  // chunks of kExactTpr rows: every thread reads one row's scale, the deferred rows of the chunk are listed in
  // LDS (in any order), then searched one at a time by the whole block
  const int64_t nchunks = (N + kExactTpr - 1) / kExactTpr;
  for (int64_t ch = blockIdx.x; ch < nchunks; ch += gridDim.x) {
    if (tid == 0) flag = 0;
    __syncthreads();
    const int64_t mine = ch * kExactTpr + tid;
    if (mine < N && __builtin_isnan(scale[mine])) list[atomicAdd(&flag, 1)] = (int)tid;
    __syncthreads();
    const int count = flag;
    for (int li = 0; li < count; ++li)
      exact_row<DT, HAS_S, BITS, ASYM, kExactTpr>(w, ch * kExactTpr + list[li], K, s, max_iter, thr, min_scale, scale,
                                                  zero_point, wq, iters, mse, xd, xf, tid);
    __syncthreads();  // the chunk's list is read by all before the next chunk rebuilds it
  }
}

// ---------------------------------------------------------------------------

template <int DT, bool HAS_S, int BITS, bool ASYM>
hipError_t dispatch(const void* w, int64_t N, int64_t K, const float* s, int max_iter, double thr, float min_scale,
                    float* scale, int32_t* zp, void* wq, int32_t* iters, double* mse, hipStream_t stream) {
  const int64_t nchunk = K / 16;
  bool launched = false;
  // short symmetric rows: several rows per wave, one chunk per lane
  if (!ASYM && nchunk <= 32) {
#define PTQ_SR(G_)                                                                                        \
  if (!launched && nchunk <= G_) {                                                                        \
    constexpr int64_t R_ = kWave / G_;                                                                    \
    k_ssz_rows<DT, HAS_S, BITS, G_><<<(unsigned)((N + R_ - 1) / R_), kWave, 0, stream>>>(                 \
        w, N, K, s, max_iter, thr, min_scale, scale, wq, iters, mse);                                     \
    launched = true;                                                                                      \
  }
    PTQ_SR(1) PTQ_SR(2) PTQ_SR(4) PTQ_SR(8) PTQ_SR(16) PTQ_SR(32)
#undef PTQ_SR
  }
  bool exact_launch = launched;  // the short-row kernel leaves its deferred rows to k_ssz_exact
  if (!launched) {
    // longer rows: about 64 elements per thread; one wave per row up to K = 4096
    int tpr = 64;
    while (tpr < 1024 && (nchunk + tpr - 1) / tpr > 4) tpr *= 2;
    const int64_t cpt = (nchunk + tpr - 1) / tpr;
#define PTQ_S(TPR_, CPT_)                                                                                 \
  if (!launched && tpr == TPR_ && cpt <= CPT_) {                                                          \
    k_ssz<DT, HAS_S, BITS, ASYM, TPR_, CPT_><<<(unsigned)N, TPR_, 0, stream>>>(                           \
        w, N, K, s, max_iter, thr, min_scale, scale, zp, wq, iters, mse);                                 \
    launched = true;                                                                                      \
    exact_launch = !ssz_inline_exact(ASYM, TPR_);                                                         \
  }
    PTQ_S(64, 1) PTQ_S(64, 2) PTQ_S(64, 4)
    PTQ_S(128, 4) PTQ_S(256, 4) PTQ_S(512, 4) PTQ_S(1024, 4) PTQ_S(1024, 8)
#undef PTQ_S
  }
  if (!launched) return hipErrorInvalidValue;
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !exact_launch) return e;
  // the deferred rows, if any: a block per chunk of kExactTpr rows (up to 1024 blocks), which reads the chunk's
  // scales first, so a launch with nothing deferred costs one load per row
  const int64_t nchunks = (N + kExactTpr - 1) / kExactTpr;
  const int64_t blocks = nchunks < 1024 ? nchunks : 1024;
  k_ssz_exact<DT, HAS_S, BITS, ASYM><<<(unsigned)blocks, kExactTpr, 0, stream>>>(w, N, K, s, max_iter, thr,
                                                                                 min_scale, scale, zp, wq, iters,
                                                                                 mse);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_ssz_asym(const void* w, int dtype, int64_t N, int64_t K, const float* s, int max_iter,
                           double threshold, float min_scale, float* scale, int32_t* zero_point, int8_t* wq,
                           int32_t* iters, double* mse, hipStream_t stream) {
  if (dtype == PTQ_BF16)
    return s ? dispatch<PTQ_BF16, true, 8, true>(w, N, K, s, max_iter, threshold, min_scale, scale, zero_point, wq,
                                                 iters, mse, stream)
             : dispatch<PTQ_BF16, false, 8, true>(w, N, K, s, max_iter, threshold, min_scale, scale, zero_point, wq,
                                                  iters, mse, stream);
  return s ? dispatch<PTQ_F32, true, 8, true>(w, N, K, s, max_iter, threshold, min_scale, scale, zero_point, wq,
                                              iters, mse, stream)
           : dispatch<PTQ_F32, false, 8, true>(w, N, K, s, max_iter, threshold, min_scale, scale, zero_point, wq,
                                               iters, mse, stream);
}

hipError_t launch_ssz(const void* w, int dtype, int64_t N, int64_t K, const float* s, int bits, int max_iter,
                      double threshold, float min_scale, float* scale, void* wq, int32_t* iters, double* mse,
                      hipStream_t stream) {
#define PTQ_B(DT_, HS_)                                                                                       \
  return bits == 8 ? dispatch<DT_, HS_, 8, false>(w, N, K, s, max_iter, threshold, min_scale, scale, nullptr, wq, \
                                                  iters, mse, stream)                                         \
                   : dispatch<DT_, HS_, 4, false>(w, N, K, s, max_iter, threshold, min_scale, scale, nullptr, wq, \
                                                  iters, mse, stream)
  if (dtype == PTQ_BF16) {
    if (s) PTQ_B(PTQ_BF16, true);
    PTQ_B(PTQ_BF16, false);
  }
  if (s) PTQ_B(PTQ_F32, true);
  PTQ_B(PTQ_F32, false);
#undef PTQ_B
}

}  // namespace ptq
