/* Drives every entry point of the oracle (oracle/ptq_oracle.c) on small seeded inputs and on the edge inputs
 * the quantizers meet (zero, subnormal, tiny, huge and mixed rows; extreme scales), built with AddressSanitizer
 * and UndefinedBehaviorSanitizer (float-to-int overflow included) so that an out-of-bounds access, an integer
 * overflow or an out-of-range conversion anywhere in the oracle stops the run.  Results are not checked here
 * (the pins do that); only that every call returns and stays defined.  Exit 0 on success. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int o_absmax_cols(const float* x, int64_t rows, int64_t cols, float* amax, int accumulate);
int o_smooth_factors(const float* ax, const float* aw, int64_t K, float alpha, float* s);
int o_fold_weight(const float* w, const float* s, int64_t N, int64_t K, float* wh);
int o_fold_act(const float* x, const float* s, int64_t T, int64_t K, float* xh);
int o_quant_row(const float* r, int64_t K, float S, int qmax, int8_t* q);
double o_mse_row(const float* wh, const int8_t* q, int64_t K, float S);
double o_lsq_scale(const float* wh, const int8_t* q, int64_t K);
int o_ssz(const float* w, const float* s, int64_t N, int64_t K, int bits, int max_iter, double thr, float min_scale,
          float* S, int8_t* q, int32_t* iters, double* mse, double* hist);
int o_ssz_variant(const float* w, const float* s, int64_t N, int64_t K, int bits, int max_iter, double thr,
                  float min_scale, int conv_and, int err_sum, int global_loop, float* S, int32_t* iters, double* mse);
int o_quant_row_asym(const float* r, int64_t K, float S, int Z, int8_t* q);
double o_mse_row_asym(const float* wh, const int8_t* q, int64_t K, float S, int Z);
int o_lsq_affine(const float* wh, const int8_t* q, int64_t K, int Z, double* a, double* b);
int o_ssz_asym(const float* w, const float* s, int64_t N, int64_t K, int max_iter, double thr, float min_scale,
               float* S, int32_t* Z, int8_t* q, int32_t* iters, double* mse, double* hist);
int o_minmax_per_tensor(const float* w, int64_t N, int64_t K, int bits, float min_scale, float* S_out, int8_t* q);
int o_pack_int4(const int8_t* q, int64_t N, int64_t K, uint8_t* packed);
int o_quant_per_token(const float* x, const float* s, int64_t T, int64_t K, int8_t* xq, float* delta);
int o_gemm_i8(const int8_t* xq, const int8_t* wq, int64_t M, int64_t N, int64_t K, int64_t* acc);
int o_dequant(const int64_t* acc, const float* delta, const float* S, int64_t M, int64_t N, double* y);
uint16_t o_bf16_rne(float f);
int o_epilogue(const int64_t* acc, int64_t M, int64_t N, const float* tok_scale, const float* ch_scale,
               const float* bias, int act, int out_type, const float* next_s, float out_scale, void* out);
int o_absmax_tensor(const float* x, int64_t rows, int64_t cols, const float* s, int fold, float* amax);
int o_ema_update(float* state, float a, float momentum, int first);
float o_act_static_scale(float state);
float o_weight_scale_per_tensor(float amax, float min_scale);
int o_quant_static(const float* x, int64_t rows, int64_t cols, const float* s, int fold, float S, int8_t* q);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;

static double uniform(void) { /* xorshift64*, in [0, 1) */
  g_state ^= g_state >> 12;
  g_state ^= g_state << 25;
  g_state ^= g_state >> 27;
  return (double)((g_state * 0x2545F4914F6CDD1Dull) >> 11) * 0x1p-53;
}

#define R 12 /* rows (tokens / weight rows) */
#define K 48 /* depth, a multiple of 16 */

/* row kinds: 0 random N(0,1)-ish, 1 zeros, 2 subnormal, 3 tiny (1e-30), 4 huge (1e37), 5 one outlier, 6 constant,
 * 7 alternating extreme signs */
static void fill(float* x, int64_t rows, int64_t cols, int variant) {
  for (int64_t r = 0; r < rows; ++r) {
    const int kind = (int)((r + variant) % 8);
    for (int64_t k = 0; k < cols; ++k) {
      const double u = uniform() * 2.0 - 1.0;
      float v;
      switch (kind) {
        case 0: v = (float)(u * 3.0); break;
        case 1: v = 0.0f; break;
        case 2: v = (float)(u * 1e-42); break;
        case 3: v = (float)(u * 1e-30); break;
        case 4: v = (float)(u * 1e37); break;
        case 5: v = k == 3 ? 1e6f : (float)(u * 0.01); break;
        case 6: v = -2.5f; break;
        default: v = (k & 1) ? 3.0e38f : -3.0e38f; break;
      }
      x[r * cols + k] = v;
    }
  }
}

static int g_calls = 0;
#define CALL(expr) do { (void)(expr); ++g_calls; } while (0)

int main(void) {
  float x[R * K], w[R * K], wh[R * K], xh[R * K], s[K], ax[K], aw[K], S[R], delta[R], amax, state;
  int8_t q[R * K], xq[R * K], wq[R * K];
  uint8_t packed[R * K / 2];
  int32_t iters[R], Z[R];
  double mse[R], hist[R * 21], y[R * R], a, b;
  int64_t acc[R * R];
  unsigned char out[R * R * 4];
  float bias[R], next_s[R];

  for (int variant = 0; variant < 8; ++variant) {
    fill(x, R, K, variant);
    fill(w, R, K, variant + 3);
    CALL(o_absmax_cols(x, R, K, ax, 0));
    CALL(o_absmax_cols(x, R, K, ax, 1));
    CALL(o_absmax_cols(w, R, K, aw, 0));
    const float alphas[3] = {0.0f, 0.5f, 1.0f};
    for (int ai = 0; ai < 3; ++ai) {
      CALL(o_smooth_factors(ax, aw, K, alphas[ai], s));
      CALL(o_fold_weight(w, s, R, K, wh));
      CALL(o_fold_act(x, s, R, K, xh));
      for (int bits = 4; bits <= 8; bits += 4) {
        CALL(o_ssz(w, s, R, K, bits, 20, 1e-10, 1e-5f, S, q, iters, mse, hist));
        CALL(o_ssz(w, NULL, R, K, bits, 20, 1e-10, 1e-30f, S, q, iters, mse, NULL));
        CALL(o_ssz(w, s, R, K, bits, 0, 0.0, 1e-5f, S, q, iters, mse, hist));
        for (int v = 0; v < 8; ++v) CALL(o_ssz_variant(w, s, R, K, bits, 20, 1e-10, 1e-5f, v & 1, (v >> 1) & 1,
                                                       (v >> 2) & 1, S, iters, mse));
        CALL(o_minmax_per_tensor(w, R, K, bits, 1e-5f, S, q));
      }
      CALL(o_pack_int4(q, R, K, packed));
      CALL(o_ssz_asym(w, s, R, K, 20, 1e-10, 1e-5f, S, Z, q, iters, mse, hist));
      CALL(o_ssz_asym(w, NULL, R, K, 20, 1e-10, 1e-30f, S, Z, q, iters, mse, NULL));
      CALL(o_quant_per_token(x, s, R, K, xq, delta));
      CALL(o_quant_per_token(x, NULL, R, K, xq, delta));
      CALL(o_ssz(w, s, R, K, 8, 20, 1e-10, 1e-5f, S, wq, iters, mse, NULL));
      CALL(o_gemm_i8(xq, wq, R, R, K, acc));
      CALL(o_dequant(acc, delta, S, R, R, y));
      for (int n = 0; n < R; ++n) {
        bias[n] = (float)(uniform() - 0.5);
        next_s[n] = n == 0 ? 1e-30f : (n == 1 ? 1e30f : (float)(0.5 + uniform()));
      }
      for (int act = 0; act <= 2; ++act)
        for (int ot = 0; ot <= 2; ++ot) {
          CALL(o_epilogue(acc, R, R, delta, S, bias, act, ot, next_s, 0.05f, out));
          CALL(o_epilogue(acc, R, R, delta, S, NULL, act, ot, NULL, 1e-30f, out));
          CALL(o_epilogue(acc, R, R, delta, S, NULL, act, ot, NULL, 1e30f, out));
        }
      for (int fold = 0; fold <= 2; ++fold) {
        CALL(o_absmax_tensor(x, R, K, s, fold, &amax));
        state = 0.0f;
        CALL(o_ema_update(&state, amax, 0.9f, 1));
        CALL(o_ema_update(&state, amax * 0.5f, 0.9f, 0));
        const float Sa = o_act_static_scale(state);
        const float Ss[4] = {Sa, 1e-30f, 1e30f, 0x1p-149f};
        for (int si = 0; si < 4; ++si) CALL(o_quant_static(x, R, K, s, fold, Ss[si], xq));
        CALL(o_weight_scale_per_tensor(amax, 1e-5f));
      }
    }
    /* row-level helpers on every row, and at extreme scales */
    for (int r = 0; r < R; ++r) {
      const float* row = wh + r * K;
      const float scales[5] = {1.0f, 1e-30f, 1e30f, 0x1p-149f, 3.0e38f};
      for (int si = 0; si < 5; ++si) {
        CALL(o_quant_row(row, K, scales[si], 127, q));
        CALL(o_mse_row(row, q, K, scales[si]));
        CALL(o_quant_row(row, K, scales[si], 7, q));
        CALL(o_lsq_scale(row, q, K));
        const int zs[3] = {-128, 0, 127};
        for (int zi = 0; zi < 3; ++zi) {
          CALL(o_quant_row_asym(row, K, scales[si], zs[zi], q));
          CALL(o_mse_row_asym(row, q, K, scales[si], zs[zi]));
          CALL(o_lsq_affine(row, q, K, zs[zi], &a, &b));
        }
      }
    }
    const float specials[8] = {0.0f, -0.0f, 1e-45f, 3.0e38f, -3.0e38f, INFINITY, -INFINITY, NAN};
    for (int i = 0; i < 8; ++i) CALL(o_bf16_rne(specials[i]));
  }
  /* inputs the oracle must refuse, not read out of bounds */
  fill(x, R, K, 0);
  x[5] = NAN;
  CALL(o_absmax_cols(x, R, K, ax, 0));
  CALL(o_quant_per_token(x, NULL, R, K, xq, delta));
  CALL(o_ssz(x, NULL, R, K, 8, 20, 1e-10, 1e-5f, S, q, iters, mse, NULL));
  printf("oracle sanitizer driver: %d calls\n", g_calls);
  return 0;
}
