// quant.hip -- per-token int8 activation quantization with the smoothing fold (gfx950).
//
// One block of TPR threads owns one token row at a time and walks rows with a
// grid stride, loading the next row while it quantizes the current one.  Each
// thread holds CPT groups of 16 elements of the row in registers, so a row is
// read from HBM once and written once as int8.  A group is split into pieces
// of E elements (one 16-byte load: E = 8 for bf16, 4 for fp32); piece p of
// group m of thread tid starts at column
//     m*TPR*16 + p*TPR*E + tid*E,
// so the 64 lanes of a wave read 1 KB of consecutive bytes per load
// instruction (whole cache lines) and write E*64 consecutive code bytes per
// store ([INT8] 3.1: 16-byte vectorised accesses).  The smoothing fold
// x_hat = fl32(x / s_j) ([SQ] X diag(s)^-1) is div_rn's corrected product
// with the per-column reciprocals fl32(1 / s_j), which each thread computes
// once (rcp_rn, the IEEE reciprocal) for its own columns and keeps in registers, beside
// s_j, across the rows it visits; the grid size trades that reuse against
// rows in flight.
//
// All row accesses are range-checked buffer loads and stores on a per-row
// descriptor (zero bytes for a row past T), so no lane or row takes a branch
// around a memory access and the loads of the rows in flight stay in flight.
//
// Per row: a = max|x_hat| (wave butterfly + LDS across waves),
// delta = a > 0 ? fl32(a/127) : 1, code = clamp(rne(fl32(x_hat / delta)),
// -127, 127) ([INT8] 2.1), the quotient again by div_rn.
//
// div_rn gives the IEEE quotient of every operand at least 2^-102 in
// magnitude.  With every s_j in [2^-20, 2^100] (checked once per block) an x
// under 2^-102 has |x_hat| < 2^-81, so a row whose computed maximum a lies in
// [2^-60, 2^100] has the exact a and delta, and its small elements have the
// code 0 either way: such rows take the fast path.  Any other row (a zero or
// tiny row, a huge one), and every row when some s_j is outside that range,
// is folded and quantized with the IEEE division instead.  The static mode
// takes the fast path when its scale lies in [2^-60, 2^100] (and the s_j
// check holds for the division fold).
#include "ptq_dev.hpp"
#include "ptq_launch.hpp"

namespace ptq {

namespace {

template <int DT>
struct Piece {
  static constexpr int E = DT == PTQ_BF16 ? 8 : 4;  // elements per 16-byte load
  static constexpr int P = 16 / E;                  // pieces per 16-element group
};

template <int DT, int TPR>
__device__ __forceinline__ int64_t piece_col(int m, int p, int tid) {
  return (int64_t)m * TPR * 16 + (int64_t)p * TPR * Piece<DT>::E + (int64_t)tid * Piece<DT>::E;
}

// Row t of x (zero-length past T: the loads then return zeros).
template <int DT, int TPR, int CPT>
__device__ __forceinline__ void load_raw(const void* x, int64_t t, int64_t T, int64_t K, int tid,
                                         uint4 (&raw)[CPT][Piece<DT>::P]) {
  constexpr int P = Piece<DT>::P;
  constexpr int BYTES = DT == PTQ_BF16 ? 2 : 4;
  const __amdgpu_buffer_rsrc_t rs =
      buf_rsrc(reinterpret_cast<const char*>(x) + (t < T ? t : 0) * K * BYTES, t < T ? (uint32_t)(K * BYTES) : 0u);
#pragma unroll
  for (int m = 0; m < CPT; ++m) {
#pragma unroll
    for (int p = 0; p < P; ++p) raw[m][p] = buf_load16_once(rs, (uint32_t)(piece_col<DT, TPR>(m, p, tid) * BYTES));
  }
}

template <int DT>
__device__ __forceinline__ void unpack16(const uint4 (&raw)[Piece<DT>::P], float (&v)[16]) {
  if constexpr (DT == PTQ_BF16) {
#pragma unroll
    for (int q = 0; q < 2; ++q) {
      const uint32_t w[4] = {raw[q].x, raw[q].y, raw[q].z, raw[q].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[q * 8 + 2 * i] = bf16_lo(w[i]);
        v[q * 8 + 2 * i + 1] = bf16_hi(w[i]);
      }
    }
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      v[q * 4 + 0] = __uint_as_float(raw[q].x);
      v[q * 4 + 1] = __uint_as_float(raw[q].y);
      v[q * 4 + 2] = __uint_as_float(raw[q].z);
      v[q * 4 + 3] = __uint_as_float(raw[q].w);
    }
  }
}

enum { FOLD_NONE = 0, FOLD_DIV = 1, FOLD_MUL = 2 };

// The per-column factors of a thread's columns, in registers: s_j, and for the division fold also
// r_j = fl32(1/s_j).  (Keeping s_j in LDS instead, read per element, measured slower.)
template <int DT, int FOLD, int TPR, int CPT>
struct ColFactors {
  static constexpr int kRegS = FOLD != FOLD_NONE ? CPT : 1;
  static constexpr int kRegR = FOLD == FOLD_DIV ? CPT : 1;
  float sreg[kRegS][16];
  float rreg[kRegR][16];

  __device__ __forceinline__ float s(int m, int e, int) const { return sreg[kRegS == 1 ? 0 : m][e]; }
  __device__ __forceinline__ float r(int m, int e) const { return rreg[kRegR == 1 ? 0 : m][e]; }
};

// One row: fold, absmax (wave butterfly + LDS across waves), codes, store.  STATIC: the scale is given
// (static_delta, its reciprocal static_inv) and no maximum is taken.  FOLD: none, x / s_j (div_rn with the
// reciprocals), or x * s_j.  cols_ok: every s_j of the launch is in div_rn's fold range (see the file header);
// the row takes the IEEE division when it is not, or when its maximum (or the static scale) is out of range --
// re-reading the row from memory, so that the loaded words need not stay live for that rare path.
// refill() is called as soon as the row's words are unpacked: the caller reuses their registers for the
// next row's loads, which then overlap this row's reduction and codes.
template <int DT, int FOLD, int TPR, int CPT, bool STATIC, typename Refill>
__device__ __forceinline__ void quant_row(uint4 (&raw)[CPT][Piece<DT>::P], const ColFactors<DT, FOLD, TPR, CPT>& cf,
                                          bool cols_ok, const void* __restrict__ x, int64_t t, int64_t T, int64_t K,
                                          int tid, int8_t* __restrict__ xq, float* __restrict__ tok_scale,
                                          float (*red)[TPR / kWave], int parity, float static_delta,
                                          float static_inv, Refill refill) {
  constexpr int NW = TPR / kWave;
  constexpr int E = Piece<DT>::E, P = Piece<DT>::P;
  float v[CPT][16];
  float amax = 0.0f;
#pragma unroll
  for (int m = 0; m < CPT; ++m) {
    unpack16<DT>(raw[m], v[m]);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if constexpr (FOLD == FOLD_DIV) v[m][e] = div_rn(v[m][e], cf.s(m, e, tid), cf.r(m, e));
      else if constexpr (FOLD == FOLD_MUL) v[m][e] = v[m][e] * cf.s(m, e, tid);
      if constexpr (!STATIC) amax = fmaxf(amax, fabsf(v[m][e]));
    }
  }
  refill(raw);
  float delta, inv;
  if constexpr (STATIC) {
    delta = static_delta;
    inv = static_inv;
  } else {
    amax = wave_max(amax);
    if constexpr (NW > 1) {
      if ((tid & (kWave - 1)) == 0) red[parity][tid / kWave] = amax;
      __syncthreads();
      amax = red[parity][0];
#pragma unroll
      for (int w = 1; w < NW; ++w) amax = fmaxf(amax, red[parity][w]);
    }
  }
  const bool fast = cols_ok && (STATIC ? (delta >= 0x1p-60f && delta <= 0x1p100f)
                                       : (amax >= 0x1p-60f && amax <= 0x1p100f));
  if (!fast) {
    // the IEEE division throughout (uniform over the row), on the row read again
    uint4 again[CPT][P];
    load_raw<DT, TPR, CPT>(x, t, T, K, tid, again);
    amax = 0.0f;
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
      unpack16<DT>(again[m], v[m]);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        if constexpr (FOLD == FOLD_DIV) v[m][e] = v[m][e] / cf.s(m, e, tid);
        else if constexpr (FOLD == FOLD_MUL) v[m][e] = v[m][e] * cf.s(m, e, tid);
        if constexpr (!STATIC) amax = fmaxf(amax, fabsf(v[m][e]));
      }
    }
    if constexpr (!STATIC) {
      amax = wave_max(amax);
      if constexpr (NW > 1) {
        __syncthreads();
        if ((tid & (kWave - 1)) == 0) red[parity ^ 1][tid / kWave] = amax;
        __syncthreads();
        amax = red[parity ^ 1][0];
#pragma unroll
        for (int w = 1; w < NW; ++w) amax = fmaxf(amax, red[parity ^ 1][w]);
        __syncthreads();
      }
    }
  }
  if constexpr (!STATIC) {
    delta = amax > 0.0f ? amax / 127.0f : 1.0f;
    inv = rcp_rn(delta);  // used only on the fast path: delta in [2^-67, 2^93]
  }
  const bool live = t < T;
  const __amdgpu_buffer_rsrc_t rq = buf_rsrc(xq + (live ? t : 0) * K, live ? (uint32_t)K : 0u);
#pragma unroll
  for (int m = 0; m < CPT; ++m) {
    // the quotients x_hat / delta; a per-token one needs no saturation: |x_hat| <= a, so the quotient is at
    // most 127 (1 + 2^-24) and rounds to at most 127.  The static scale saturates (before rounding: the same
    // code, since the bounds are integers).  The codes are rounded by rne_bits and packed byte-wise.
    uint32_t qb[16];
    float tq[16];
    if (fast) {
#pragma unroll
      for (int e = 0; e < 16; ++e) tq[e] = div_rn(v[m][e], delta, inv);
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) tq[e] = v[m][e] / delta;
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if constexpr (STATIC) tq[e] = fminf(fmaxf(tq[e], -127.0f), 127.0f);
      qb[e] = rne_bits(tq[e]);
    }
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const uint32_t c = (uint32_t)piece_col<DT, TPR>(m, p, tid);
      if constexpr (E == 8) {
        uint2 o;
        o.x = pack4_low_bytes(qb[p * 8 + 0], qb[p * 8 + 1], qb[p * 8 + 2], qb[p * 8 + 3]);
        o.y = pack4_low_bytes(qb[p * 8 + 4], qb[p * 8 + 5], qb[p * 8 + 6], qb[p * 8 + 7]);
        buf_store8(rq, c, o);
      } else {
        buf_store4(rq, c, pack4_low_bytes(qb[p * 4 + 0], qb[p * 4 + 1], qb[p * 4 + 2], qb[p * 4 + 3]));
      }
    }
  }
  // lane 0 writes delta: the other lanes' offsets fall past the 4-byte range (a NULL tok_scale, allowed
  // in the static mode, gets a zero-length range)
  const bool put = live && tok_scale != nullptr;
  const __amdgpu_buffer_rsrc_t rt = buf_rsrc(put ? tok_scale + t : reinterpret_cast<float*>(xq), put ? 4u : 0u);
  buf_store4(rt, tid == 0 ? 0u : 4u, __float_as_uint(delta));
}

// Grid-stride over rows with D rows in flight: slot d of the register ring is
// refilled with the row D strides ahead as soon as its row is quantized (a
// row past T loads nothing: zero-length descriptor).  A block stops at its
// first row past T, so a last round with fewer rows costs no work for the
// missing ones.
// STATIC: one given scale (scale[0]) for every row, as a per-tensor static quantization.  FOLD_MUL folds by
// s_j (the weight side, fl32(x * s_j)), FOLD_DIV by fl32(x / s_j) (the activation side).
template <int DT, int FOLD, int TPR, int CPT, int D, bool STATIC>
__global__ __launch_bounds__(TPR) void k_quant_tok(const void* __restrict__ x, int64_t T, int64_t K,
                                                   const float* __restrict__ s, int8_t* __restrict__ xq,
                                                   float* __restrict__ tok_scale, const float* __restrict__ scale) {
  using CF = ColFactors<DT, FOLD, TPR, CPT>;
  constexpr int E = Piece<DT>::E, P = Piece<DT>::P;
  __shared__ float red[2][TPR / kWave];
  const int tid = threadIdx.x;
  const int64_t G = gridDim.x;

  // the smoothing factors of this thread's columns are loaded first, so that waiting for them (loads
  // complete in issue order) leaves the first D rows in flight while the reciprocals are computed
  constexpr bool HAS_S = FOLD != FOLD_NONE;
  uint4 sv[HAS_S ? CPT : 1][4];
  if constexpr (HAS_S) {
    const __amdgpu_buffer_rsrc_t rsc = buf_rsrc(s, (uint32_t)(K * 4));
#pragma unroll
    for (int m = 0; m < CPT; ++m)
#pragma unroll
      for (int p = 0; p < P; ++p)
#pragma unroll
        for (int h = 0; h < E / 4; ++h)
          sv[m][p * (E / 4) + h] = buf_load16(rsc, (uint32_t)((piece_col<DT, TPR>(m, p, tid) + 4 * h) * 4));
  }
  uint4 ring[D][CPT][P];
#pragma unroll
  for (int d = 0; d < D; ++d) load_raw<DT, TPR, CPT>(x, blockIdx.x + d * G, T, K, tid, ring[d]);

  CF cf;
  bool cols_ok = true;
  if constexpr (HAS_S) {
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int64_t c0 = piece_col<DT, TPR>(m, p, tid);
        const bool in = c0 < K;
#pragma unroll
        for (int h = 0; h < E / 4; ++h) {
          const uint4 w = sv[m][p * (E / 4) + h];
          const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int e = p * E + 4 * h + i;
            const float sj = in ? __uint_as_float(u[i]) : 1.0f;
            cf.sreg[m][e] = sj;
            if constexpr (FOLD == FOLD_DIV) {
              cf.rreg[m][e] = rcp_rn(sj);  // used only when every s_j is in div_rn's domain
              cols_ok = cols_ok && (sj >= 0x1p-20f && sj <= 0x1p100f);
            }
          }
        }
      }
    }
    cols_ok = __syncthreads_and(cols_ok) != 0;
  }
  float static_delta = 1.0f, static_inv = 1.0f;
  if constexpr (STATIC) {
    static_delta = scale[0];
    static_inv = rcp_rn(static_delta);  // used only on the fast path (scale in [2^-60, 2^100])
  }
  int parity = 0;
  for (int64_t base = blockIdx.x; base < T; base += D * G) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int64_t t = base + d * G;
      if (t >= T) break;  // block-uniform: the round's remaining rows, and every later one, are past T
      quant_row<DT, FOLD, TPR, CPT, STATIC>(
          ring[d], cf, cols_ok, x, t, T, K, tid, xq, tok_scale, red, parity, static_delta, static_inv,
          [&](uint4 (&slot)[CPT][P]) { load_raw<DT, TPR, CPT>(x, t + D * G, T, K, tid, slot); });
      parity ^= 1;
    }
  }
}

template <int DT, int FOLD, int TPR, int CPT, bool STATIC>
void launch_one(const void* x, int64_t T, int64_t K, const float* s, int8_t* xq, float* ts, const float* scale,
                int64_t blocks, hipStream_t stream) {
  constexpr int D = CPT >= 4 ? 1 : 4 / CPT;  // rows in flight per block: about 4 groups of 16 elements per thread
  k_quant_tok<DT, FOLD, TPR, CPT, D, STATIC><<<(unsigned)blocks, TPR, 0, stream>>>(x, T, K, s, xq, ts, scale);
}

template <int DT, int FOLD, bool STATIC>
hipError_t dispatch(const void* x, int64_t T, int64_t K, const float* s, int8_t* xq, float* ts, const float* scale,
                    int64_t rows_per_block, hipStream_t stream) {
  const int64_t ngroup = K / 16;
  // the narrowest block with at most 2 groups of 16 elements per thread (up to 8 at 1024 threads)
  int tpr = 64;
  int64_t cpt = (ngroup + tpr - 1) / tpr;
  while (cpt > 2 && tpr < 1024) {
    tpr *= 2;
    cpt = (ngroup + tpr - 1) / tpr;
  }
  // rows per block: the per-column reciprocals are computed once per block and reused for its rows
  int64_t blocks = (T + rows_per_block - 1) / rows_per_block;
  if (blocks < 1) blocks = 1;
#define PTQ_Q(TPR_, CPT_)                                                           \
  if (tpr == TPR_ && cpt <= CPT_) {                                                 \
    launch_one<DT, FOLD, TPR_, CPT_, STATIC>(x, T, K, s, xq, ts, scale, blocks, stream); \
    return hipGetLastError();                                                       \
  }
  PTQ_Q(64, 1) PTQ_Q(64, 2) PTQ_Q(128, 2) PTQ_Q(256, 2) PTQ_Q(512, 2)
  PTQ_Q(1024, 2) PTQ_Q(1024, 4) PTQ_Q(1024, 8)
#undef PTQ_Q
  return hipErrorInvalidValue;
}

}  // namespace

static int64_t default_rows_per_block(int64_t T, int64_t K) {
  // enough blocks to keep rows in flight on every CU, enough rows per block to reuse the reciprocals
  int64_t r = T / (K >= 8192 ? 512 : 1024);
  return r < 1 ? 1 : (r > 16 ? 16 : r);
}

template <int DT, bool STATIC>
hipError_t dispatch_fold(const void* x, int64_t T, int64_t K, const float* s, int fold_mul, int8_t* xq, float* ts,
                         const float* scale, int64_t rpb, hipStream_t stream) {
  if (!s) return dispatch<DT, FOLD_NONE, STATIC>(x, T, K, s, xq, ts, scale, rpb, stream);
  if (fold_mul) return dispatch<DT, FOLD_MUL, STATIC>(x, T, K, s, xq, ts, scale, rpb, stream);
  return dispatch<DT, FOLD_DIV, STATIC>(x, T, K, s, xq, ts, scale, rpb, stream);
}

// rows_per_block <= 0 picks the default
hipError_t launch_quant_per_token_rpb(const void* x, int dtype, int64_t T, int64_t K, const float* s, int8_t* xq,
                                      float* tok_scale, int64_t rows_per_block, hipStream_t stream) {
  if (rows_per_block <= 0) rows_per_block = default_rows_per_block(T, K);
  if (dtype == PTQ_BF16)
    return dispatch_fold<PTQ_BF16, false>(x, T, K, s, 0, xq, tok_scale, nullptr, rows_per_block, stream);
  return dispatch_fold<PTQ_F32, false>(x, T, K, s, 0, xq, tok_scale, nullptr, rows_per_block, stream);
}

hipError_t launch_quant_static(const void* x, int dtype, int64_t rows, int64_t cols, const float* s, int fold_mul,
                               const float* scale, int8_t* q, float* row_scale, hipStream_t stream) {
  const int64_t rpb = default_rows_per_block(rows, cols);
  if (dtype == PTQ_BF16) return dispatch_fold<PTQ_BF16, true>(x, rows, cols, s, fold_mul, q, row_scale, scale, rpb, stream);
  return dispatch_fold<PTQ_F32, true>(x, rows, cols, s, fold_mul, q, row_scale, scale, rpb, stream);
}

hipError_t launch_quant_per_token(const void* x, int dtype, int64_t T, int64_t K, const float* s, int8_t* xq,
                                  float* tok_scale, hipStream_t stream) {
  return launch_quant_per_token_rpb(x, dtype, T, K, s, xq, tok_scale, 0, stream);
}

}  // namespace ptq
