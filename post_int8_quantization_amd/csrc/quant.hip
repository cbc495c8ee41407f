// quant.hip -- per-token int8 activation quantization with the smoothing fold (gfx950).
//
// One block of TPR threads owns one token row at a time and walks rows with a
// grid stride, loading the next row while it quantizes the current one.  Each
// thread holds CPT chunks of 16 consecutive elements in registers, so a row is
// read from HBM once (16-byte loads, [INT8] 3.1) and written once as int8 (one
// 16-byte store per chunk).  The smoothing fold x_hat = fl32(x * fl32(1/s_j))
// ([SQ] X diag(s)^-1) uses per-column reciprocals that each thread computes
// once (IEEE division) for its own columns and keeps in registers across the
// rows it visits; the grid size trades that reuse against rows in flight.
//
// Per row: a = max|x_hat| (wave butterfly + LDS across waves),
// delta = a > 0 ? fl32(a/127) : 1, inv = fl32(1/delta),
// code = clamp(rne(fl32(x_hat * inv)), -127, 127)   ([INT8] 2.1).
#include "ptq_dev.hpp"
#include "ptq_launch.hpp"

namespace ptq {

namespace {

template <int DT>
struct Raw {
  static constexpr int kVecs = DT == PTQ_BF16 ? 2 : 4;  // 16-byte vectors per 16-element chunk
};

template <int DT, int TPR, int CPT>
__device__ __forceinline__ void load_raw(const void* x, int64_t t, int64_t K, int tid, int64_t nchunk,
                                         uint4 (&raw)[CPT][Raw<DT>::kVecs]) {
  constexpr int NV = Raw<DT>::kVecs;
  const uint4* row = reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(x) +
                                                    t * K * (DT == PTQ_BF16 ? 2 : 4));
#pragma unroll
  for (int m = 0; m < CPT; ++m) {
    const int64_t c = tid + (int64_t)TPR * m;
#pragma unroll
    for (int q = 0; q < NV; ++q) raw[m][q] = c < nchunk ? load_once(row + c * NV + q) : make_uint4(0, 0, 0, 0);
  }
}

template <int DT>
__device__ __forceinline__ void unpack16(const uint4 (&raw)[Raw<DT>::kVecs], float (&v)[16]) {
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

// One row: fold, absmax (wave butterfly + LDS across waves), codes, store.
template <int DT, bool HAS_S, int TPR, int CPT>
__device__ __forceinline__ void quant_row(const uint4 (&raw)[CPT][Raw<DT>::kVecs], const float (&r)[CPT][16],
                                          int64_t t, int64_t K, int tid, int64_t nchunk, int8_t* __restrict__ xq,
                                          float* __restrict__ tok_scale, float (*red)[TPR / kWave], int parity) {
  constexpr int NW = TPR / kWave;
  float v[CPT][16];
  float amax = 0.0f;
#pragma unroll
  for (int m = 0; m < CPT; ++m) {
    unpack16<DT>(raw[m], v[m]);
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if constexpr (HAS_S) v[m][e] = v[m][e] * r[m][e];
      amax = fmaxf(amax, fabsf(v[m][e]));
    }
  }
  amax = wave_max(amax);
  if constexpr (NW > 1) {
    if ((tid & (kWave - 1)) == 0) red[parity][tid / kWave] = amax;
    __syncthreads();
    amax = red[parity][0];
#pragma unroll
    for (int w = 1; w < NW; ++w) amax = fmaxf(amax, red[parity][w]);
  }
  const float delta = amax > 0.0f ? amax / 127.0f : 1.0f;
  const float inv = 1.0f / delta;
#pragma unroll
  for (int m = 0; m < CPT; ++m) {
    const int64_t c = tid + (int64_t)TPR * m;
    if (c < nchunk) {
      float q[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) q[e] = code_f(v[m][e], inv, 127.0f);
      uint4 o;
      o.x = pack4_i8(q[0], q[1], q[2], q[3]);
      o.y = pack4_i8(q[4], q[5], q[6], q[7]);
      o.z = pack4_i8(q[8], q[9], q[10], q[11]);
      o.w = pack4_i8(q[12], q[13], q[14], q[15]);
      *reinterpret_cast<uint4*>(xq + t * K + c * 16) = o;
    }
  }
  if (tid == 0) tok_scale[t] = delta;
}

// Grid-stride over rows; the next row's raw data is loaded while the current one is processed.
template <int DT, bool HAS_S, int TPR, int CPT>
__global__ __launch_bounds__(TPR) void k_quant_tok(const void* __restrict__ x, int64_t T, int64_t K,
                                                   const float* __restrict__ s, int8_t* __restrict__ xq,
                                                   float* __restrict__ tok_scale) {
  constexpr int NV = Raw<DT>::kVecs;
  __shared__ float red[2][TPR / kWave];
  const int tid = threadIdx.x;
  const int64_t nchunk = K / 16;

  int64_t t = blockIdx.x;
  if (t >= T) return;
  uint4 ra[CPT][NV], rb[CPT][NV];
  load_raw<DT, TPR, CPT>(x, t, K, tid, nchunk, ra);  // in flight while the reciprocals are computed

  float r[CPT][16];
#pragma unroll
  for (int m = 0; m < CPT; ++m) {
    const int64_t c = tid + (int64_t)TPR * m;
#pragma unroll
    for (int e = 0; e < 16; ++e) r[m][e] = (HAS_S && c < nchunk) ? 1.0f / s[c * 16 + e] : 1.0f;
  }
  int parity = 0;
  for (;;) {
    int64_t tn = t + gridDim.x;
    if (tn < T) load_raw<DT, TPR, CPT>(x, tn, K, tid, nchunk, rb);
    quant_row<DT, HAS_S, TPR, CPT>(ra, r, t, K, tid, nchunk, xq, tok_scale, red, parity);
    parity ^= 1;
    if (tn >= T) break;
    t = tn;
    tn = t + gridDim.x;
    if (tn < T) load_raw<DT, TPR, CPT>(x, tn, K, tid, nchunk, ra);
    quant_row<DT, HAS_S, TPR, CPT>(rb, r, t, K, tid, nchunk, xq, tok_scale, red, parity);
    parity ^= 1;
    if (tn >= T) break;
    t = tn;
  }
}

template <int DT, bool HAS_S, int TPR, int CPT>
void launch_one(const void* x, int64_t T, int64_t K, const float* s, int8_t* xq, float* ts, int64_t blocks,
                hipStream_t stream) {
  k_quant_tok<DT, HAS_S, TPR, CPT><<<(unsigned)blocks, TPR, 0, stream>>>(x, T, K, s, xq, ts);
}

template <int DT, bool HAS_S>
hipError_t dispatch(const void* x, int64_t T, int64_t K, const float* s, int8_t* xq, float* ts, int64_t rows_per_block,
                    hipStream_t stream) {
  const int64_t nchunk = K / 16;
  int tpr = nchunk >= 256 ? 256 : 64;
  int64_t cpt = (nchunk + tpr - 1) / tpr;
  while (cpt > 4 && tpr < 1024) {
    tpr *= 2;
    cpt = (nchunk + tpr - 1) / tpr;
  }
  // rows per block: the per-column reciprocals are computed once per block and reused for its rows
  int64_t blocks = (T + rows_per_block - 1) / rows_per_block;
  if (blocks < 1) blocks = 1;
#define PTQ_Q(TPR_, CPT_)                                                           \
  if (tpr == TPR_ && cpt <= CPT_) {                                                 \
    launch_one<DT, HAS_S, TPR_, CPT_>(x, T, K, s, xq, ts, blocks, stream);          \
    return hipGetLastError();                                                       \
  }
  PTQ_Q(64, 1) PTQ_Q(64, 2) PTQ_Q(64, 4)
  PTQ_Q(256, 1) PTQ_Q(256, 2) PTQ_Q(256, 4)
  PTQ_Q(512, 4) PTQ_Q(1024, 4) PTQ_Q(1024, 8)
#undef PTQ_Q
  return hipErrorInvalidValue;
}

}  // namespace

// rows_per_block <= 0 picks the default
hipError_t launch_quant_per_token_rpb(const void* x, int dtype, int64_t T, int64_t K, const float* s, int8_t* xq,
                                      float* tok_scale, int64_t rows_per_block, hipStream_t stream) {
  if (rows_per_block <= 0) {
    // enough blocks to keep rows in flight on every CU, enough rows per block to reuse the reciprocals
    rows_per_block = T / (K >= 4096 ? 512 : 1024);
    rows_per_block = rows_per_block < 1 ? 1 : (rows_per_block > 16 ? 16 : rows_per_block);
  }
  if (dtype == PTQ_BF16)
    return s ? dispatch<PTQ_BF16, true>(x, T, K, s, xq, tok_scale, rows_per_block, stream)
             : dispatch<PTQ_BF16, false>(x, T, K, s, xq, tok_scale, rows_per_block, stream);
  return s ? dispatch<PTQ_F32, true>(x, T, K, s, xq, tok_scale, rows_per_block, stream)
           : dispatch<PTQ_F32, false>(x, T, K, s, xq, tok_scale, rows_per_block, stream);
}

hipError_t launch_quant_per_token(const void* x, int dtype, int64_t T, int64_t K, const float* s, int8_t* xq,
                                  float* tok_scale, hipStream_t stream) {
  return launch_quant_per_token_rpb(x, dtype, T, K, s, xq, tok_scale, 0, stream);
}

}  // namespace ptq
