// gemm.hip -- int8 x int8 -> int32 GEMM with fused per-token/per-channel dequantization (gfx950).
//
// acc[t,n] = sum_k xq[t,k] wq[n,k];  y[t,n] = fl32(acc) * fl32(tok_scale[t] * ch_scale[n]).
// Both operands are K-contiguous ([INT8] 3.2 loads both tiles with leading
// dimension K); accumulation is exact int32 ([INT8] 5.1 bounds K); the
// dequantization runs in the epilogue of the same kernel ([INT8] 4.2 fusion).
//
// The only dense contraction of the path, so it runs on the CDNA4 matrix
// cores: v_mfma_i32_16x16x64_i8 (A: 16 rows x 64 k, B: 64 k x 16 cols, each
// lane supplying 16 bytes of one row, i.e. lane%16 selects the row/column and
// lane/16 the 16-byte k-group; C: lane%16 = column, rows 4*(lane/16)+0..3).
// Integer sums are exact, so the order of k inside a group never matters as
// long as A and B use the same one, which they do (both are 16 contiguous k).
//
// Two kernels:
//  * k_gemm_tile  -- prefill: BM x BN block tiles, BK-deep K steps staged
//                    through LDS (double buffer, one barrier per step), each
//                    wave owning a TM x TN sub-tile of 16x16 fragments; LDS
//                    rows are XOR-swizzled in 16-byte chunks so the MFMA
//                    operand reads are bank-conflict free.
//  * k_gemm_skinny -- decode (few tokens): HBM-bound weight streaming; each
//                    block owns 16 output channels, its waves split K, the
//                    weight chunks go straight from HBM to MFMA operand
//                    registers and the int32 partials are summed in LDS.
#include "ptq_dev.hpp"
#include "ptq_launch.hpp"

namespace ptq {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4i mfma16(const uint4& a, const uint4& b, v4i c) {
  v4i av = {(int)a.x, (int)a.y, (int)a.z, (int)a.w};
  v4i bv = {(int)b.x, (int)b.y, (int)b.z, (int)b.w};
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(av, bv, c, 0, 0, 0);
}

// 16-byte chunk position inside an LDS row of KC chunks (XOR swizzle by row)
template <int KC>
__device__ __forceinline__ int swz(int row, int kc) {
  if constexpr (KC == 8) return kc ^ (row & 7);
  else if constexpr (KC == 4) return kc ^ ((row >> 1) & 3);
  else return kc;
}

template <int BM, int BN, int BK, int WM, int WN>
__global__ __launch_bounds__(WM* WN * 64) void k_gemm_tile(const int8_t* __restrict__ A, const int8_t* __restrict__ B,
                                                          const float* __restrict__ ts, const float* __restrict__ cs,
                                                          int M, int N, int K, float* __restrict__ Y,
                                                          int32_t* __restrict__ ACC, int tiles_n) {
  constexpr int NT = WM * WN * 64;
  constexpr int TM = BM / WM, TN = BN / WN;
  constexpr int FM = TM / 16, FN = TN / 16;
  constexpr int KC = BK / 16;
  constexpr int A_PT = BM * KC / NT, B_PT = BN * KC / NT;
  static_assert(A_PT * NT == BM * KC && B_PT * NT == BN * KC, "tile loads must divide evenly");
  __shared__ uint4 sA[2][BM * KC];
  __shared__ uint4 sB[2][BN * KC];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 15, lk = lane >> 4;
  const int tile = blockIdx.x;
  const int m0 = (tile / tiles_n) * BM, n0 = (tile % tiles_n) * BN;

  uint4 ra[A_PT], rb[B_PT];
  auto gload = [&](int k0) {
#pragma unroll
    for (int i = 0; i < A_PT; ++i) {
      const int c = tid + i * NT, row = c / KC, kc = c % KC;
      const int gm = m0 + row, gk = k0 + kc * 16;
      ra[i] = (gm < M && gk < K) ? *reinterpret_cast<const uint4*>(A + (int64_t)gm * K + gk) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int i = 0; i < B_PT; ++i) {
      const int c = tid + i * NT, row = c / KC, kc = c % KC;
      const int gn = n0 + row, gk = k0 + kc * 16;
      rb[i] = (gn < N && gk < K) ? *reinterpret_cast<const uint4*>(B + (int64_t)gn * K + gk) : make_uint4(0, 0, 0, 0);
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < A_PT; ++i) {
      const int c = tid + i * NT, row = c / KC, kc = c % KC;
      sA[buf][row * KC + swz<KC>(row, kc)] = ra[i];
    }
#pragma unroll
    for (int i = 0; i < B_PT; ++i) {
      const int c = tid + i * NT, row = c / KC, kc = c % KC;
      sB[buf][row * KC + swz<KC>(row, kc)] = rb[i];
    }
  };

  v4i acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

  const int nk = (K + BK - 1) / BK;
  gload(0);
  sstore(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) gload((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 64; ++ks) {
      uint4 a[FM], b[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int row = wm * TM + i * 16 + lr;
        a[i] = sA[cur][row * KC + swz<KC>(row, ks * 4 + lk)];
      }
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int row = wn * TN + j * 16 + lr;
        b[j] = sB[cur][row * KC + swz<KC>(row, ks * 4 + lk)];
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j) acc[i][j] = mfma16(a[i], b[j], acc[i][j]);
    }
    if (kt + 1 < nk) sstore(cur ^ 1);
    __syncthreads();
  }

  // epilogue: dequantize and store
#pragma unroll
  for (int j = 0; j < FN; ++j) {
    const int n = n0 + wn * TN + j * 16 + lr;
    const float csn = n < N ? cs[n] : 0.0f;
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int m = m0 + wm * TM + i * 16 + lk * 4 + r;
        if (m < M && n < N) {
          const int a = acc[i][j][r];
          const float sc = ts[m] * csn;
          Y[(int64_t)m * N + n] = (float)a * sc;
          if (ACC) ACC[(int64_t)m * N + n] = a;
        }
      }
    }
  }
}

// Decode: M <= 16*MT tokens, 16 output channels per block, KS waves splitting K.
template <int MT, int KS, int U>
__global__ __launch_bounds__(KS * 64) void k_gemm_skinny(const int8_t* __restrict__ A, const int8_t* __restrict__ B,
                                                        const float* __restrict__ ts, const float* __restrict__ cs,
                                                        int M, int N, int K, float* __restrict__ Y,
                                                        int32_t* __restrict__ ACC) {
  __shared__ v4i part[KS][MT][64];
  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lk = lane >> 4;
  const int n0 = blockIdx.x * 16;
  const int n = n0 + lr;
  const bool nvalid = n < N;
  const int8_t* brow = B + (int64_t)(nvalid ? n : 0) * K;

  v4i acc[MT];
#pragma unroll
  for (int t = 0; t < MT; ++t) acc[t] = v4i{0, 0, 0, 0};

  const int kstep = 64 * KS;
  for (int k0 = wave * 64; k0 < K; k0 += kstep * U) {
    uint4 b[U], a[U][MT];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int gk = k0 + u * kstep + lk * 16;
      const bool kv = gk < K;
      b[u] = (nvalid && kv) ? *reinterpret_cast<const uint4*>(brow + gk) : make_uint4(0, 0, 0, 0);
#pragma unroll
      for (int t = 0; t < MT; ++t) {
        const int m = t * 16 + lr;
        a[u][t] = (m < M && kv) ? *reinterpret_cast<const uint4*>(A + (int64_t)m * K + gk) : make_uint4(0, 0, 0, 0);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[t] = mfma16(a[u][t], b[u], acc[t]);
  }
#pragma unroll
  for (int t = 0; t < MT; ++t) part[wave][t][lane] = acc[t];
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      v4i s = part[0][t][lane];
#pragma unroll
      for (int w = 1; w < KS; ++w) s += part[w][t][lane];
      if (nvalid) {
        const float csn = cs[n];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = t * 16 + lk * 4 + r;
          if (m < M) {
            Y[(int64_t)m * N + n] = (float)s[r] * (ts[m] * csn);
            if (ACC) ACC[(int64_t)m * N + n] = s[r];
          }
        }
      }
    }
  }
}

template <int BM, int BN, int BK, int WM, int WN>
hipError_t launch_tile(const int8_t* xq, const int8_t* wq, const float* ts, const float* cs, int M, int N, int K,
                       float* y, int32_t* acc, hipStream_t stream) {
  const int tm = (M + BM - 1) / BM, tn = (N + BN - 1) / BN;
  k_gemm_tile<BM, BN, BK, WM, WN><<<(unsigned)(tm * tn), WM * WN * 64, 0, stream>>>(xq, wq, ts, cs, M, N, K, y, acc,
                                                                                   tn);
  return hipGetLastError();
}

template <int MT>
hipError_t launch_skinny(const int8_t* xq, const int8_t* wq, const float* ts, const float* cs, int M, int N, int K,
                         float* y, int32_t* acc, hipStream_t stream) {
  const int blocks = (N + 15) / 16;
  k_gemm_skinny<MT, 4, 4><<<(unsigned)blocks, 4 * 64, 0, stream>>>(xq, wq, ts, cs, M, N, K, y, acc);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_dequant(const int8_t* xq, const int8_t* wq, const float* tok_scale, const float* ch_scale,
                               int64_t M, int64_t N, int64_t K, float* y, int32_t* acc, hipStream_t stream) {
  const int m = (int)M, n = (int)N, k = (int)K;
  if (M <= 16) return launch_skinny<1>(xq, wq, tok_scale, ch_scale, m, n, k, y, acc, stream);
  if (M <= 32) return launch_skinny<2>(xq, wq, tok_scale, ch_scale, m, n, k, y, acc, stream);
  if (M <= 64) return launch_skinny<4>(xq, wq, tok_scale, ch_scale, m, n, k, y, acc, stream);
  return launch_tile<256, 256, 64, 2, 4>(xq, wq, tok_scale, ch_scale, m, n, k, y, acc, stream);
}

}  // namespace ptq
