// calib.hip -- column absmax calibration and smoothing factors (gfx950).
//
// Column absmax ([SQ] max|X_j|, max|W_j| along the input channel j; [INT8] 2.1
// range calibration).  HBM-bound: every element is read once with 16-byte
// loads ([INT8] 3.1, streaming hint).  A block of 4 waves owns a strip of 64
// 16-byte vector columns (1 KB of every row) and a run of rows; each wave
// streams its own contiguous rows with 8 to 16 loads in flight per lane,
// keeping running maxima in registers; 2 to 4 blocks per CU keep up to
// ~256 KB in flight per CU.  The waves merge through LDS and the block publishes one atomic max
// per column.  Maxima of non-negative floats order like their bit
// patterns, so an unsigned atomic max gives the exact result in any order.
#include "ptq_dev.hpp"
#include "ptq_launch.hpp"

#include <math.h>

namespace ptq {

namespace {

constexpr int kWaves = 4;                // waves per block (default)
constexpr int64_t kMaxRowBlocks = 64;     // row blocks per column strip (atomics per column)
constexpr int kVecs = kWave;              // 16-byte vector columns per block strip
constexpr int kBatch = 8;                 // row loads per batch; two batches in flight per lane

template <int DT>
struct Vec {
  static constexpr int kElems = DT == PTQ_BF16 ? 8 : 4;  // elements per 16-byte vector
};

template <int DT>
__device__ __forceinline__ void fold_max(float (&m)[Vec<DT>::kElems], const uint4& d) {
  const uint32_t w[4] = {d.x, d.y, d.z, d.w};
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

// grid: x = column strips, y = row runs of rows_per_block rows (split evenly over the waves).
// Each wave keeps two batches of kBatch row loads in flight: the next batch is issued before the
// current one is folded.  Rows are read through per-row range-checked descriptors, so rows past
// the wave's run and lanes past the row's end read zeros (neutral for a max of magnitudes) with no
// branch around any load.
template <int DT, int NWV = kWaves, int KB = kBatch>
__global__ __launch_bounds__(NWV* kWave) void k_absmax_cols(const uint4* __restrict__ x, int64_t rows,
                                                         int64_t vecs_per_row, int64_t rows_per_block,
                                                         unsigned* __restrict__ amax_bits) {
  constexpr int E = Vec<DT>::kElems;
  __shared__ float red[NWV][kVecs * E];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // wave-uniform: row descriptors in SGPRs
  const int64_t v = (int64_t)blockIdx.x * kVecs + lane;
  const int64_t per_wave = (rows_per_block + NWV - 1) / NWV;
  const int64_t b0 = (int64_t)blockIdx.y * rows_per_block;
  const int64_t b1 = b0 + rows_per_block < rows ? b0 + rows_per_block : rows;
  const int64_t r0 = b0 + wave * per_wave;
  const int64_t r1 = r0 + per_wave < b1 ? r0 + per_wave : b1;
  const uint32_t row_bytes = (uint32_t)(vecs_per_row * 16);
  const uint32_t off = (uint32_t)(v * 16);

  float m[E];
#pragma unroll
  for (int e = 0; e < E; ++e) m[e] = 0.0f;
  auto load_batch = [&](uint4 (&d)[KB], int64_t r) {
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int64_t rr = r + u;
      const bool live = rr < r1;
      d[u] = buf_load16_once(buf_rsrc(x + (live ? rr : 0) * vecs_per_row, live ? row_bytes : 0u), off);
    }
  };
  uint4 da[KB], db[KB];
  load_batch(da, r0);
  // the scheduling barriers keep each batch's loads issued before the previous batch is folded
  for (int64_t r = r0; r < r1; r += 2 * KB) {
    load_batch(db, r + KB);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < KB; ++u) fold_max<DT>(m, da[u]);
    load_batch(da, r + 2 * KB);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < KB; ++u) fold_max<DT>(m, db[u]);
  }
#pragma unroll
  for (int e = 0; e < E; ++e) red[wave][lane * E + e] = m[e];
  __syncthreads();
  for (int c = tid; c < kVecs * E; c += NWV * kWave) {
    float mm = red[0][c];
#pragma unroll
    for (int w = 1; w < NWV; ++w) mm = fmaxf(mm, red[w][c]);
    const int64_t vcol = (int64_t)blockIdx.x * kVecs + c / E;
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

// Static per-tensor scales from column maxima (one block).  For a positive constant c, rounding is
// monotone, so max_t |fl32(x_tj / c)| = fl32(max_t |x_tj| / c) (and likewise for x_tj * c): the maximum of
// the folded tensor is the maximum over columns of the folded column maxima.
//   mode 0 (activation, [INT8] 2.1 moving-average range): a = max_j fl32(colmax_j / s_j);
//          state = first ? a : fl32(fl32(m * state) + fl32(fl32(1 - m) * a));
//          scale = state > 0 ? fl32(state / 127) : 1
//   mode 1 (weight, per-tensor MinMax): a = max_j fl32(colmax_j * s_j);  scale = max(fl32(a / 127), min_scale)
// bcast[0 .. n_bcast) receives the scale too (the per-row / per-channel vector a GEMM reads).
constexpr int kScaleThreads = 1024;

__global__ __launch_bounds__(kScaleThreads) void k_tensor_scale(const float* __restrict__ colmax,
                                                                const float* __restrict__ s, int64_t K, int mode,
                                                                float momentum, int first, float min_scale,
                                                                float* __restrict__ state, float* __restrict__ scale,
                                                                float* __restrict__ bcast, int64_t n_bcast) {
  __shared__ float red[kScaleThreads / kWave];
  __shared__ float s_out;
  const int tid = threadIdx.x;
  float a = 0.0f;
  for (int64_t j = tid; j < K; j += kScaleThreads) {
    float c = colmax[j];
    if (s) c = mode == 0 ? c / s[j] : c * s[j];
    a = fmaxf(a, c);
  }
  a = wave_max(a);
  if ((tid & (kWave - 1)) == 0) red[tid / kWave] = a;
  __syncthreads();
  if (tid == 0) {
    float m = red[0];
    for (int w = 1; w < kScaleThreads / kWave; ++w) m = fmaxf(m, red[w]);
    float S;
    if (mode == 0) {
      float st;
      if (first) {
        st = m;
      } else {
        const float t1 = momentum * state[0];
        const float wgt = 1.0f - momentum;
        const float t2 = wgt * m;
        st = t1 + t2;
      }
      state[0] = st;
      S = st > 0.0f ? st / 127.0f : 1.0f;
    } else {
      S = m / 127.0f;
      S = S < min_scale ? min_scale : S;
    }
    scale[0] = S;
    s_out = S;
  }
  __syncthreads();
  const float S = s_out;
  for (int64_t i = tid; i < n_bcast; i += kScaleThreads) bcast[i] = S;
}

}  // namespace

hipError_t launch_absmax_cols(const void* x, int dtype, int64_t rows, int64_t cols, float* amax, int accumulate,
                              hipStream_t stream) {
  if (!accumulate) {
    k_fill_zero<<<(unsigned)((cols + 255) / 256), 256, 0, stream>>>(amax, cols);
  }
  const int E = dtype == PTQ_BF16 ? 8 : 4;
  const int64_t vecs = cols / E;
  const int64_t gx = (vecs + kVecs - 1) / kVecs;
  // 2 (tall matrices) to 4 blocks per CU (256 CUs) and at least one row per wave; tall matrices stream
  // better from fewer, longer row runs (measured: 6.4-6.6 vs 6.2 TB/s on a 1 GB bf16 stack).  At most 64 row
  // blocks: each adds one atomic per column, and more of them queue on the same addresses -- narrow or short
  // matrices (1024-wide activations, 1024-4096-row weights) ran 1.1-2.3x slower at 128-512 row blocks than at 64
  const int64_t target = rows >= 16384 ? 512 : 1024;
  int64_t gy = (target + gx - 1) / gx;
  const int64_t max_gy = (rows + kWaves - 1) / kWaves;
  if (gy > max_gy) gy = max_gy;
  if (gy > kMaxRowBlocks) gy = kMaxRowBlocks;
  const int64_t rows_per_block = (rows + gy - 1) / gy;
  gy = (rows + rows_per_block - 1) / rows_per_block;
  dim3 grid((unsigned)gx, (unsigned)gy);
  if (dtype == PTQ_BF16)
    k_absmax_cols<PTQ_BF16><<<grid, kWaves * kWave, 0, stream>>>(reinterpret_cast<const uint4*>(x), rows, vecs,
                                                            rows_per_block, reinterpret_cast<unsigned*>(amax));
  else
    k_absmax_cols<PTQ_F32><<<grid, kWaves * kWave, 0, stream>>>(reinterpret_cast<const uint4*>(x), rows, vecs,
                                                           rows_per_block, reinterpret_cast<unsigned*>(amax));
  return hipGetLastError();
}

hipError_t launch_tensor_scale(const float* col_amax, const float* s, int64_t K, int mode, float momentum, int first,
                               float min_scale, float* state, float* scale, float* bcast, int64_t n_bcast,
                               hipStream_t stream) {
  k_tensor_scale<<<1, kScaleThreads, 0, stream>>>(col_amax, s, K, mode, momentum, first, min_scale, state, scale,
                                                  bcast, bcast ? n_bcast : 0);
  return hipGetLastError();
}

hipError_t launch_smooth_factors(const float* ax, const float* aw, int64_t K, float alpha, float* s,
                                 hipStream_t stream) {
  k_smooth<<<(unsigned)((K + 255) / 256), 256, 0, stream>>>(ax, aw, K, (double)alpha, s);
  return hipGetLastError();
}

}  // namespace ptq
