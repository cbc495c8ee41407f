// quant.hip -- per-token int8 activation quantization with the smoothing fold (gfx950).
//
// One block of TPR threads owns one token row at a time and walks rows with a
// grid stride.  Each thread holds CPT chunks of 16 consecutive elements in
// registers, so a row is read from HBM once (16-byte loads, [INT8] 3.1) and
// written once as int8 (one 16-byte store per chunk).  The smoothing fold
// x_hat = fl32(x * fl32(1/s_j)) ([SQ] X diag(s)^-1) uses per-column
// reciprocals that each thread computes once for its own columns and keeps in
// registers across the rows it visits.
//
// Per row: a = max|x_hat| (wave butterfly + LDS across waves),
// delta = a > 0 ? fl32(a/127) : 1, inv = fl32(1/delta),
// code = clamp(rne(fl32(x_hat * inv)), -127, 127)   ([INT8] 2.1).
#include "ptq_dev.hpp"
#include "ptq_launch.hpp"

namespace ptq {

namespace {

template <int DT, bool HAS_S, int TPR, int CPT>
__global__ __launch_bounds__(TPR) void k_quant_tok(const void* __restrict__ x, int64_t T, int64_t K,
                                                   const float* __restrict__ s, int8_t* __restrict__ xq,
                                                   float* __restrict__ tok_scale) {
  constexpr int NW = TPR / kWave;
  __shared__ float red[2][NW];
  const int tid = threadIdx.x;
  const int64_t nchunk = K / 16;

  float r[CPT][16];
  if constexpr (HAS_S) {
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
      const int64_t c = tid + (int64_t)TPR * m;
#pragma unroll
      for (int e = 0; e < 16; ++e) r[m][e] = c < nchunk ? 1.0f / s[c * 16 + e] : 1.0f;
    }
  }

  int parity = 0;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x, parity ^= 1) {
    float v[CPT][16];
    float amax = 0.0f;
#pragma unroll
    for (int m = 0; m < CPT; ++m) {
      const int64_t c = tid + (int64_t)TPR * m;
      if (c < nchunk) {
        float a8[8], b8[8];
        load8<DT>(x, t * K + c * 16, a8);
        load8<DT>(x, t * K + c * 16 + 8, b8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          v[m][e] = a8[e];
          v[m][e + 8] = b8[e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) v[m][e] = 0.0f;
      }
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
}

template <int DT, bool HAS_S, int TPR, int CPT>
void launch_one(const void* x, int64_t T, int64_t K, const float* s, int8_t* xq, float* ts, int64_t blocks,
                hipStream_t stream) {
  k_quant_tok<DT, HAS_S, TPR, CPT><<<(unsigned)blocks, TPR, 0, stream>>>(x, T, K, s, xq, ts);
}

template <int DT, bool HAS_S>
hipError_t dispatch(const void* x, int64_t T, int64_t K, const float* s, int8_t* xq, float* ts,
                    hipStream_t stream) {
  const int64_t nchunk = K / 16;
  int tpr = nchunk >= 256 ? 256 : 64;
  int64_t cpt = (nchunk + tpr - 1) / tpr;
  while (cpt > 4 && tpr < 1024) {
    tpr *= 2;
    cpt = (nchunk + tpr - 1) / tpr;
  }
  // about 4096 waves in flight; the per-column reciprocals are reused over T/blocks rows
  int64_t blocks = (int64_t)4096 * kWave / tpr;
  if (blocks > T) blocks = T;
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

hipError_t launch_quant_per_token(const void* x, int dtype, int64_t T, int64_t K, const float* s, int8_t* xq,
                                  float* tok_scale, hipStream_t stream) {
  if (dtype == PTQ_BF16)
    return s ? dispatch<PTQ_BF16, true>(x, T, K, s, xq, tok_scale, stream)
             : dispatch<PTQ_BF16, false>(x, T, K, s, xq, tok_scale, stream);
  return s ? dispatch<PTQ_F32, true>(x, T, K, s, xq, tok_scale, stream)
           : dispatch<PTQ_F32, false>(x, T, K, s, xq, tok_scale, stream);
}

}  // namespace ptq
