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
// x_hat = fl32(x * fl32(1/s_j)) ([SQ] X diag(s)^-1) uses per-column
// reciprocals that each thread computes once (IEEE division) for its own
// columns and keeps in registers across the rows it visits; the grid size
// trades that reuse against rows in flight.
//
// All row accesses are range-checked buffer loads and stores on a per-row
// descriptor (zero bytes for a row past T), so no lane or row takes a branch
// around a memory access and the loads of the rows in flight stay in flight.
//
// Per row: a = max|x_hat| (wave butterfly + LDS across waves),
// delta = a > 0 ? fl32(a/127) : 1, inv = fl32(1/delta),
// code = clamp(rne(fl32(x_hat * inv)), -127, 127)   ([INT8] 2.1).
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

// One row: fold, absmax (wave butterfly + LDS across waves), codes, store.  STATIC: the scale is
// given (static_delta, its reciprocal static_inv) and no maximum is taken.
template <int DT, bool HAS_S, int TPR, int CPT, bool STATIC>
__device__ __forceinline__ void quant_row(const uint4 (&raw)[CPT][Piece<DT>::P], const float (&r)[CPT][16], int64_t t,
                                          int64_t T, int64_t K, int tid, int8_t* __restrict__ xq,
                                          float* __restrict__ tok_scale, float (*red)[TPR / kWave], int parity,
                                          float static_delta, float static_inv) {
  constexpr int NW = TPR / kWave;
  constexpr int E = Piece<DT>::E, P = Piece<DT>::P;
  float v[CPT][16];
  float amax = 0.0f;
#pragma unroll
  for (int m = 0; m < CPT; ++m) {
    unpack16<DT>(raw[m], v[m]);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if constexpr (HAS_S) v[m][e] = v[m][e] * r[m][e];
      if constexpr (!STATIC) amax = fmaxf(amax, fabsf(v[m][e]));
    }
  }
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
    delta = amax > 0.0f ? amax / 127.0f : 1.0f;
    inv = 1.0f / delta;
  }
  const bool live = t < T;
  const __amdgpu_buffer_rsrc_t rq = buf_rsrc(xq + (live ? t : 0) * K, live ? (uint32_t)K : 0u);
#pragma unroll
  for (int m = 0; m < CPT; ++m) {
    float q[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) q[e] = code_f(v[m][e], inv, 127.0f);
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const uint32_t c = (uint32_t)piece_col<DT, TPR>(m, p, tid);
      if constexpr (E == 8) {
        uint2 o;
        o.x = pack4_i8(q[p * 8 + 0], q[p * 8 + 1], q[p * 8 + 2], q[p * 8 + 3]);
        o.y = pack4_i8(q[p * 8 + 4], q[p * 8 + 5], q[p * 8 + 6], q[p * 8 + 7]);
        buf_store8(rq, c, o);
      } else {
        buf_store4(rq, c, pack4_i8(q[p * 4 + 0], q[p * 4 + 1], q[p * 4 + 2], q[p * 4 + 3]));
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
// refilled with the row D strides ahead as soon as its row is quantized.  A
// block walks whole rounds of D rows; the rows of a round past T are no-ops
// (zero-length descriptors).
// STATIC: one given scale (scale[0]) for every row, as a per-tensor static quantization; fold_mul
// folds by s_j (the weight side) instead of by fl32(1/s_j) (the activation side).
template <int DT, bool HAS_S, int TPR, int CPT, int D, bool STATIC>
__global__ __launch_bounds__(TPR) void k_quant_tok(const void* __restrict__ x, int64_t T, int64_t K,
                                                   const float* __restrict__ s, int8_t* __restrict__ xq,
                                                   float* __restrict__ tok_scale, const float* __restrict__ scale,
                                                   int fold_mul) {
  constexpr int E = Piece<DT>::E, P = Piece<DT>::P;
  __shared__ float red[2][TPR / kWave];
  const int tid = threadIdx.x;
  const int64_t G = gridDim.x;

  // the smoothing factors of this thread's columns are loaded first, so that waiting for them (loads
  // complete in issue order) leaves the first D rows in flight while the reciprocals are computed
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

  float r[CPT][16];
  if constexpr (HAS_S) {
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const bool in = piece_col<DT, TPR>(m, p, tid) < K;
#pragma unroll
        for (int h = 0; h < E / 4; ++h) {
          const uint4 w = sv[m][p * (E / 4) + h];
          const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float sj = __uint_as_float(u[i]);
            r[m][p * E + 4 * h + i] = in ? (fold_mul ? sj : 1.0f / sj) : 1.0f;
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int m = 0; m < CPT; ++m)
#pragma unroll
      for (int e = 0; e < 16; ++e) r[m][e] = 1.0f;
  }
  float static_delta = 1.0f, static_inv = 1.0f;
  if constexpr (STATIC) {
    static_delta = scale[0];
    static_inv = 1.0f / static_delta;
  }
  int parity = 0;
  for (int64_t base = blockIdx.x; base < T; base += D * G) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int64_t t = base + d * G;
      quant_row<DT, HAS_S, TPR, CPT, STATIC>(ring[d], r, t, T, K, tid, xq, tok_scale, red, parity, static_delta,
                                             static_inv);
      parity ^= 1;
      load_raw<DT, TPR, CPT>(x, t + D * G, T, K, tid, ring[d]);
    }
  }
}

template <int DT, bool HAS_S, int TPR, int CPT, bool STATIC>
void launch_one(const void* x, int64_t T, int64_t K, const float* s, int8_t* xq, float* ts, const float* scale,
                int fold_mul, int64_t blocks, hipStream_t stream) {
  constexpr int D = CPT >= 4 ? 1 : 4 / CPT;  // rows in flight per block: about 4 groups of 16 elements per thread
  k_quant_tok<DT, HAS_S, TPR, CPT, D, STATIC><<<(unsigned)blocks, TPR, 0, stream>>>(x, T, K, s, xq, ts, scale,
                                                                                    fold_mul);
}

template <int DT, bool HAS_S, bool STATIC>
hipError_t dispatch(const void* x, int64_t T, int64_t K, const float* s, int8_t* xq, float* ts, const float* scale,
                    int fold_mul, int64_t rows_per_block, hipStream_t stream) {
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
    launch_one<DT, HAS_S, TPR_, CPT_, STATIC>(x, T, K, s, xq, ts, scale, fold_mul, blocks, stream); \
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

// rows_per_block <= 0 picks the default
hipError_t launch_quant_per_token_rpb(const void* x, int dtype, int64_t T, int64_t K, const float* s, int8_t* xq,
                                      float* tok_scale, int64_t rows_per_block, hipStream_t stream) {
  if (rows_per_block <= 0) rows_per_block = default_rows_per_block(T, K);
  if (dtype == PTQ_BF16)
    return s ? dispatch<PTQ_BF16, true, false>(x, T, K, s, xq, tok_scale, nullptr, 0, rows_per_block, stream)
             : dispatch<PTQ_BF16, false, false>(x, T, K, s, xq, tok_scale, nullptr, 0, rows_per_block, stream);
  return s ? dispatch<PTQ_F32, true, false>(x, T, K, s, xq, tok_scale, nullptr, 0, rows_per_block, stream)
           : dispatch<PTQ_F32, false, false>(x, T, K, s, xq, tok_scale, nullptr, 0, rows_per_block, stream);
}

hipError_t launch_quant_static(const void* x, int dtype, int64_t rows, int64_t cols, const float* s, int fold_mul,
                               const float* scale, int8_t* q, float* row_scale, hipStream_t stream) {
  const int64_t rpb = default_rows_per_block(rows, cols);
  if (dtype == PTQ_BF16)
    return s ? dispatch<PTQ_BF16, true, true>(x, rows, cols, s, q, row_scale, scale, fold_mul, rpb, stream)
             : dispatch<PTQ_BF16, false, true>(x, rows, cols, s, q, row_scale, scale, fold_mul, rpb, stream);
  return s ? dispatch<PTQ_F32, true, true>(x, rows, cols, s, q, row_scale, scale, fold_mul, rpb, stream)
           : dispatch<PTQ_F32, false, true>(x, rows, cols, s, q, row_scale, scale, fold_mul, rpb, stream);
}

hipError_t launch_quant_per_token(const void* x, int dtype, int64_t T, int64_t K, const float* s, int8_t* xq,
                                  float* tok_scale, hipStream_t stream) {
  return launch_quant_per_token_rpb(x, dtype, T, K, s, xq, tok_scale, 0, stream);
}

}  // namespace ptq
