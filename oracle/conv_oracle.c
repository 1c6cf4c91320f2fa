/*
 * conv_oracle.c -- plain float64 oracle of the short causal convolution whose state is
 * kept in a pool next to the GDN recurrent state, and of its speculative verify and
 * accepted-prefix commit.
 *
 * TEST INFRASTRUCTURE ONLY (see gdn_oracle.h): loaded by the tests and the benchmark's
 * CPU-baseline leg; it shares nothing with the HIP library.
 *
 * What it follows (pages by title, section):
 * - TensorRT-LLM PR 20937 (GB300 Qwen3.8-Flash-Next), What changes: the GDN in_proj
 *   GEMV carries a fused conv1d epilogue for verify and decode rows; Per-File QA
 *   Perspective: the speculative staging and commit kernels handle accepted-prefix
 *   boundaries of the convolution state next to the other per-request state, and the
 *   cache manager keeps the convolution state with the replay bookkeeping.
 * - "Proposal: native BF16 MTP speculative decoding for dense Qwen3.8-27B", What: the
 *   verify keeps GDN recovery records and commits the convolution state with them.
 * The pages do not print the convolution. The oracle takes the plainest standard form
 * of a depthwise causal convolution of width K over the channels of the mixed q/k/v
 * input, per channel c and token t of request row r:
 *     in(tau) = x[r][tau][c]                     for tau >= 0 (this call's tokens)
 *             = state[slot][K-1+tau][c]          for -(K-1) <= tau < 0 (earlier inputs)
 *     y[r][t][c] = act(bias[c] + sum_{i=0}^{K-1} w[i][c] * in(t - (K-1) + i))
 *     act = identity or SiLU(z) = z / (1 + e^-z)
 * The state of a slot is the last K-1 inputs, oldest first. Advancing it over n tokens
 * keeps the last K-1 entries of (state ++ those n inputs): it is made of inputs only,
 * so a commit or a roll-back is an exact selection, never a rounding.
 */
#include "conv_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static int conv_dims_ok(const oracle_conv_dims* d) {
  return d && d->batch >= 0 && d->T >= 0 && d->channels >= 1 && d->width >= 2 && d->pool_slots >= 0 &&
         (d->activation == 0 || d->activation == 1);
}

static double act(int activation, double z) { return activation ? z / (1.0 + exp(-z)) : z; }

/* The history of one row and channel after n more inputs: the last K-1 entries of
 * (hist ++ src[0..n-1]), where src[j] is token j of the row (stride `stride`). */
static void advance(const double* hist, int K, const double* src, int64_t stride, int n, double* out) {
  const int H = K - 1;
  for (int m = 0; m < H; ++m) {
    const int q = n + m;  /* position in the concatenated sequence of length H + n */
    out[m] = q < H ? hist[q] : src[(int64_t)(q - H) * stride];
  }
}

int32_t oracle_conv_update(const oracle_conv_dims* d, const double* x, const double* w, const double* bias,
                           double* pool, const int32_t* idx, const double* prev_x, int32_t T_prev,
                           const int32_t* prev_len, double* y, int32_t write_back) {
  if (!conv_dims_ok(d) || (prev_x && T_prev < 1)) return -1;
  const int B = d->batch, T = d->T, D = d->channels, K = d->width, H = K - 1;
  double* hist = (double*)malloc(sizeof(double) * (size_t)(H + T) * 2);
  if (!hist) return -1;
  double* seq = hist + H + T;
  for (int r = 0; r < B; ++r) {
    const int32_t slot = idx[r];
    const int valid = slot >= 0 && slot < d->pool_slots;
    for (int c = 0; c < D; ++c) {
      if (!valid) {  /* padding row: output zero, no state access */
        for (int t = 0; t < T; ++t) y[((int64_t)r * T + t) * D + c] = 0.0;
        continue;
      }
      double* st = pool + (int64_t)slot * H * D;
      for (int m = 0; m < H; ++m) hist[m] = st[(int64_t)m * D + c];
      /* fused commit of the previous step's accepted prefix */
      const int n = prev_x ? prev_len[r] : 0;
      if (prev_x && n >= 1 && n <= T_prev) {
        advance(hist, K, prev_x + (int64_t)r * T_prev * D + c, D, n, seq);
        for (int m = 0; m < H; ++m) {
          hist[m] = seq[m];
          st[(int64_t)m * D + c] = seq[m];
        }
      }
      /* this call's tokens */
      for (int m = 0; m < H; ++m) seq[m] = hist[m];
      for (int t = 0; t < T; ++t) seq[H + t] = x[((int64_t)r * T + t) * D + c];
      for (int t = 0; t < T; ++t) {
        double z = bias ? bias[c] : 0.0;
        for (int i = 0; i < K; ++i) z += w[(int64_t)i * D + c] * seq[t + i];
        y[((int64_t)r * T + t) * D + c] = act(d->activation, z);
      }
      if (write_back)
        for (int m = 0; m < H; ++m) st[(int64_t)m * D + c] = seq[T + m];
    }
  }
  free(hist);
  return 0;
}

int32_t oracle_conv_commit(const oracle_conv_dims* d, const double* x, double* pool, const int32_t* idx,
                           const int32_t* accept) {
  if (!conv_dims_ok(d)) return -1;
  const int B = d->batch, T = d->T, D = d->channels, K = d->width, H = K - 1;
  double hist[16], out[16];
  if (H > 16) return -1;
  for (int r = 0; r < B; ++r) {
    const int32_t slot = idx[r], n = accept[r];
    if (slot < 0 || slot >= d->pool_slots || n < 1 || n > T) continue;
    double* st = pool + (int64_t)slot * H * D;
    for (int c = 0; c < D; ++c) {
      for (int m = 0; m < H; ++m) hist[m] = st[(int64_t)m * D + c];
      advance(hist, K, x + (int64_t)r * T * D + c, D, n, out);
      for (int m = 0; m < H; ++m) st[(int64_t)m * D + c] = out[m];
    }
  }
  return 0;
}
