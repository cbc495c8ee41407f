// calib.hip -- column absmax calibration and smoothing factors (gfx950).
//
// Column absmax ([SQ] max|X_j|, max|W_j| along the input channel j; [INT8] 2.1
// range calibration).  HBM-bound: every element is read once with 16-byte
// loads ([INT8] 3.1).  A block covers 16 vector-columns (256 bytes of a row)
// and a chunk of rows; its 16 row-lanes keep running maxima in registers, fold
// them through LDS, and publish one atomic max per column.  Maxima of
// non-negative floats order like their bit patterns, so an unsigned atomic max
// gives the exact result in any order.
#include "ptq_dev.hpp"
#include "ptq_launch.hpp"

#include <math.h>

namespace ptq {

namespace {

constexpr int kCalibThreads = 256;
constexpr int kVecCols = 16;   // vector-columns per block (lanes % 16)
constexpr int kRowLanes = 16;  // row-lanes per block
constexpr int kUnroll = 4;     // rows in flight per thread

template <int DT>
struct Vec {
  static constexpr int kElems = DT == PTQ_BF16 ? 8 : 4;  // elements per 16-byte vector
};

template <int DT>
__global__ __launch_bounds__(kCalibThreads) void k_absmax_cols(const uint4* __restrict__ x, int64_t rows,
                                                                int64_t vecs_per_row, int64_t rows_per_chunk,
                                                                unsigned* __restrict__ amax_bits) {
  constexpr int E = Vec<DT>::kElems;
  __shared__ float red[kRowLanes][kVecCols * E + 1];
  const int tid = threadIdx.x;
  const int vc = tid % kVecCols, rl = tid / kVecCols;
  const int64_t v = (int64_t)blockIdx.x * kVecCols + vc;
  const int64_t r0 = (int64_t)blockIdx.y * rows_per_chunk;
  const int64_t r1 = r0 + rows_per_chunk < rows ? r0 + rows_per_chunk : rows;

  float m[E];
#pragma unroll
  for (int e = 0; e < E; ++e) m[e] = 0.0f;

  if (v < vecs_per_row) {
    for (int64_t r = r0 + rl; r < r1; r += kRowLanes * kUnroll) {
      uint4 d[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int64_t rr = r + (int64_t)u * kRowLanes;
        d[u] = rr < r1 ? x[rr * vecs_per_row + v] : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const uint32_t w[4] = {d[u].x, d[u].y, d[u].z, d[u].w};
        if constexpr (DT == PTQ_BF16) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            m[2 * i] = fmaxf(m[2 * i], fabsf(bf16_lo(w[i])));
            m[2 * i + 1] = fmaxf(m[2 * i + 1], fabsf(bf16_hi(w[i])));
          }
        } else {
#pragma unroll
          for (int i = 0; i < 4; ++i) m[i] = fmaxf(m[i], fabsf(__uint_as_float(w[i])));
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < E; ++e) red[rl][vc * E + e] = m[e];
  __syncthreads();
  if (tid < kVecCols * E) {
    const int c = tid;  // column within the block's 16*E columns
    float mm = red[0][c];
#pragma unroll
    for (int i = 1; i < kRowLanes; ++i) mm = fmaxf(mm, red[i][c]);
    const int64_t vcol = (int64_t)blockIdx.x * kVecCols + c / E;
    if (vcol < vecs_per_row) atomicMax(amax_bits + vcol * E + (c % E), __float_as_uint(mm));
  }
}

__global__ void k_fill_zero(float* __restrict__ p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.0f;
}

// s_j = a_x^alpha / a_w^(1-alpha) in fp64, rounded once; 1 for a dead channel ([SQ] formula).
__global__ void k_smooth(const float* __restrict__ ax, const float* __restrict__ aw, int64_t K, double alpha,
                         float* __restrict__ s) {
  const int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (j >= K) return;
  const float a = ax[j], b = aw[j];
  if (a == 0.0f || b == 0.0f) {
    s[j] = 1.0f;
    return;
  }
  const double v = pow((double)a, alpha) / pow((double)b, 1.0 - alpha);
  s[j] = (float)v;
}

}  // namespace

hipError_t launch_absmax_cols(const void* x, int dtype, int64_t rows, int64_t cols, float* amax, int accumulate,
                              hipStream_t stream) {
  if (!accumulate) {
    k_fill_zero<<<(unsigned)((cols + 255) / 256), 256, 0, stream>>>(amax, cols);
  }
  const int E = dtype == PTQ_BF16 ? 8 : 4;
  const int64_t vecs = cols / E;
  const int64_t gx = (vecs + kVecCols - 1) / kVecCols;
  // aim at ~2048 blocks; at least 64 rows per block so the per-column atomics stay few
  const int64_t step = kRowLanes * kUnroll;
  int64_t chunk = (rows * gx + 2047) / 2048;
  chunk = ((chunk + step - 1) / step) * step;
  if (chunk < step) chunk = step;
  const int64_t gy = (rows + chunk - 1) / chunk;
  dim3 grid((unsigned)gx, (unsigned)gy);
  if (dtype == PTQ_BF16)
    k_absmax_cols<PTQ_BF16><<<grid, kCalibThreads, 0, stream>>>(reinterpret_cast<const uint4*>(x), rows, vecs,
                                                                 chunk, reinterpret_cast<unsigned*>(amax));
  else
    k_absmax_cols<PTQ_F32><<<grid, kCalibThreads, 0, stream>>>(reinterpret_cast<const uint4*>(x), rows, vecs, chunk,
                                                                reinterpret_cast<unsigned*>(amax));
  return hipGetLastError();
}

hipError_t launch_smooth_factors(const float* ax, const float* aw, int64_t K, float alpha, float* s,
                                 hipStream_t stream) {
  k_smooth<<<(unsigned)((K + 255) / 256), 256, 0, stream>>>(ax, aw, K, (double)alpha, s);
  return hipGetLastError();
}

}  // namespace ptq
