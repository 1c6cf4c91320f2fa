/*
 * gdn_oracle.c -- plain, slow, float64 oracle of the Gated DeltaNet (GDN) recurrent
 * state update as used by decode and by MTP / speculative verify with a pooled state.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the benchmark's
 * CPU-baseline leg. It shares no code, header, table or helper with the HIP library.
 *
 * What it follows (pages by title, section):
 * - "[NVIDIA] [GDN] Enable FlashInfer MTP verify on SM100+ (Blackwell)", Summary: the
 *   MTP verify kernel (gated_delta_rule_mtp) reads each request's state from a pool
 *   through initial_state_indices; A_log is taken in fp32.
 * - same page, Requirements: a padding index must never be dereferenced; bf16 state
 *   with more than 4 verify tokens keeps one intermediate state per token.
 * - "[GDN] Honor configured linear-attn verify backend in the kernel dispatcher",
 *   Motivation: the SSM state is fp32 or bf16.
 * - TensorRT-LLM PR 20937 (GB300 Qwen3.8-Flash-Next), Per-File QA Perspective and
 *   Moved out of this PR: recurrent pools in bf16 or fp32; commit of the accepted
 *   prefix (checkpoint-commit contract), in-kernel or separate; the review notes name
 *   GDN replay with bf16 rounding.
 * The pages name the gated delta rule but do not print it. The oracle takes its
 * standard form, in this order per token t of request row r and v-head h
 * (k-head kh = h / (Hv/Hk)):
 *     q^ = q / sqrt(sum q^2 + eps),   k^ = k / sqrt(sum k^2 + eps)
 *     g  = exp(-exp(A_log[h]) * softplus(a + dt_bias[h])),   beta = sigmoid(b)
 *     S <- g S                        (decay)
 *     u <- v - S^T k^                 (prediction error of the decayed state)
 *     S <- S + beta k^ u^T            (delta-rule write)
 *     o  = scale * S^T q^             (read-out from the updated state)
 *     bf16 state: S <- RNE_bf16(S) elementwise, carried forward rounded.
 * Readings where the pages are silent are listed beside each function.
 *
 * Cached replay (TensorRT-LLM PR 20937, What changes: a copy-free cached replay of the
 * GDN verify; Moved out of this PR: replay commits in-kernel or by a separate all-layer
 * commit; the cache manager tracks the previous step's accept count and which token
 * buffer holds it): instead of one state per token, the per-token inputs of a verify are
 * kept, and the accepted prefix is replayed from the slot's checkpoint state later.
 *
 * Pins (tests, CPU): closed forms of the gates; one step from a zero state; decay
 * only; the delta property S'^T k^ = v at beta = 1; associative recall with
 * orthonormal keys; the scalar case worked by hand; brute force against the
 * matrix form S_t = g_t (I - beta_t k k^T) S_{t-1} + beta_t k v^T and a 50-digit
 * evaluation; bf16 rounding against exact rational rounding and torch's fp32->bf16
 * over all 2^32 inputs; verify(T) = T decodes; commit(n) = intermediate n.
 */
#include "gdn_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* softplus(x) = log(1 + e^x), in the overflow-free form max(x,0) + log1p(e^-|x|).
 * Reading: no large-x threshold (exact everywhere). */
double oracle_softplus(double x) {
  double m = x > 0.0 ? x : 0.0;
  return m + log1p(exp(-fabs(x)));
}

/* Gates of one (row, token, v-head): decay g and write strength beta.
 * A_log and dt_bias are per v-head parameters, a and b per token and v-head. */
void oracle_gates(double a, double b, double A_log, double dt_bias, double* g, double* beta) {
  *g = exp(-exp(A_log) * oracle_softplus(a + dt_bias));
  *beta = 1.0 / (1.0 + exp(-b));
}

/* float64 -> nearest bf16 value (8 significant bits, 8 exponent bits as fp32),
 * ties to even, correctly rounded from the float64 value (no double rounding).
 * Subnormal bf16 spacing is 2^-133; magnitudes that round past the largest finite
 * bf16 ((2 - 2^-7) * 2^127) become infinities; NaN stays NaN. */
double oracle_round_bf16(double x) {
  if (isnan(x) || isinf(x) || x == 0.0) return x;
  int e;
  (void)frexp(x, &e);                      /* |x| in [2^(e-1), 2^e) */
  int q_exp = (e - 1 >= -126) ? (e - 8) : -133; /* exponent of one unit in the last place */
  double scaled = ldexp(x, -q_exp);        /* exact: power-of-two scaling */
  double r = ldexp(rint(scaled), q_exp);   /* rint: round half to even (default mode) */
  if (fabs(r) >= ldexp(1.0, 128)) return x > 0 ? INFINITY : -INFINITY;
  return r;
}

/* Batch helper for the exhaustive test: fp32 bit patterns -> bf16 bit patterns,
 * through oracle_round_bf16 (each fp32 value is exact in float64). */
void oracle_round_bf16_f32bits(const uint32_t* in, uint16_t* out, int64_t n, int32_t nthreads) {
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
  for (int64_t i = 0; i < n; ++i) {
    float f;
    memcpy(&f, &in[i], 4);
    double r = oracle_round_bf16((double)f);
    if (isnan(r)) {
      out[i] = (uint16_t)(((in[i] >> 16) & 0x8000u) | 0x7fc0u);
      continue;
    }
    float rf = (float)r; /* exact: r is a bf16 value */
    uint32_t u;
    memcpy(&u, &rf, 4);
    out[i] = (uint16_t)(u >> 16);
  }
}

static int dims_ok(const oracle_dims* d) {
  if (!d) return 0;
  if (d->batch < 0 || d->T < 1 || d->num_k_heads < 1 || d->num_v_heads < 1) return 0;
  if (d->num_v_heads % d->num_k_heads != 0) return 0;
  if (d->d_k < 1 || d->d_v < 1 || d->pool_slots < 0) return 0;
  return 1;
}

/* One token of one (row, v-head) tile, in the order of the definition above.
 * S is d_k x d_v (S[i*dv + j]); q, k have d_k entries, v and o d_v entries. */
static void gdn_token(int dk, int dv, double* S, const double* q, const double* k,
                      const double* v, double a, double b, double A_log, double dt_bias,
                      double scale, double eps, int state_bf16, double* o,
                      double* qh, double* kh, double* u) {
  double qq = 0.0, kk = 0.0;
  for (int i = 0; i < dk; ++i) { qq += q[i] * q[i]; kk += k[i] * k[i]; }
  double qn = sqrt(qq + eps), kn = sqrt(kk + eps);
  for (int i = 0; i < dk; ++i) { qh[i] = q[i] / qn; kh[i] = k[i] / kn; }

  double g, beta;
  oracle_gates(a, b, A_log, dt_bias, &g, &beta);

  /* decay */
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) S[i * dv + j] *= g;
  /* u = v - S^T k^ */
  for (int j = 0; j < dv; ++j) {
    double acc = 0.0;
    for (int i = 0; i < dk; ++i) acc += S[i * dv + j] * kh[i];
    u[j] = v[j] - acc;
  }
  /* S += beta k^ u^T */
  for (int i = 0; i < dk; ++i)
    for (int j = 0; j < dv; ++j) S[i * dv + j] += beta * kh[i] * u[j];
  /* o = scale * S^T q^  (from the updated, not yet rounded state) */
  for (int j = 0; j < dv; ++j) {
    double acc = 0.0;
    for (int i = 0; i < dk; ++i) acc += S[i * dv + j] * qh[i];
    o[j] = scale * acc;
  }
  /* bf16 state: the stored (rounded) value is the one carried forward */
  if (state_bf16)
    for (int i = 0; i < dk * dv; ++i) S[i] = oracle_round_bf16(S[i]);
}

static int slot_valid(int32_t s, int32_t P) { return s >= 0 && s < P; }

/* Accepted-prefix commit: for each row with a valid slot and 1 <= n <= cache_T,
 * the pool slot takes the state cached after the n-th verified token; any other
 * row (padding slot, n = 0, n > cache_T) leaves the pool untouched. */
int32_t oracle_commit(const oracle_dims* d, const double* cache, int32_t cache_T,
                      const int32_t* idx, const int32_t* accept, double* pool,
                      int32_t nthreads) {
  if (!dims_ok(d) || cache_T < 1) return -1;
  const int B = d->batch, Hv = d->num_v_heads;
  const size_t tile = (size_t)d->d_k * d->d_v;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel for schedule(static)
#endif
  for (int r = 0; r < B; ++r) {
    int32_t s = idx[r], n = accept[r];
    if (!slot_valid(s, d->pool_slots) || n < 1 || n > cache_T) continue;
    for (int h = 0; h < Hv; ++h)
      memcpy(pool + ((size_t)s * Hv + h) * tile,
             cache + (((size_t)r * cache_T + (n - 1)) * Hv + h) * tile, tile * sizeof(double));
  }
  return 0;
}

/* Verify: T tokens per row from the row's pool slot.
 * - padding rows (slot outside [0, P)): o = 0, no pool or cache access;
 * - cache (optional, depth cache_T >= T): cache[r][t] holds the state after token t;
 * - write_final: the state after the last token is written back to the slot;
 * - prev_accept (optional): fused commit of the previous step, i.e. exactly
 *   oracle_commit(cache, prev_accept) followed by this verify (reading of the
 *   in-kernel commit of the TensorRT-LLM page, What changes / Moved out of this PR).
 * Reading: the pool is read-only unless write_final or a fused commit asks for it,
 * so that a rejected draft can still be rolled back. */
int32_t oracle_verify(const oracle_dims* d,
                      const double* q, const double* k, const double* v,
                      const double* a, const double* b,
                      const double* A_log, const double* dt_bias,
                      double* pool, const int32_t* idx,
                      double* cache, int32_t cache_T, int32_t write_final,
                      const int32_t* prev_accept, double* o, int32_t nthreads) {
  if (!dims_ok(d)) return -1;
  if (cache && cache_T < d->T) return -1;
  if (prev_accept && !cache) return -1;
  const int B = d->batch, T = d->T, Hk = d->num_k_heads, Hv = d->num_v_heads;
  const int dk = d->d_k, dv = d->d_v, G = Hv / Hk;
  const size_t tile = (size_t)dk * dv;

  if (prev_accept) {
    int32_t rc = oracle_commit(d, cache, cache_T, idx, prev_accept, pool, nthreads);
    if (rc) return rc;
  }

#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
  {
    double* S = (double*)malloc(tile * sizeof(double));
    double* qh = (double*)malloc((size_t)dk * sizeof(double));
    double* kh = (double*)malloc((size_t)dk * sizeof(double));
    double* u = (double*)malloc((size_t)dv * sizeof(double));
#ifdef _OPENMP
#pragma omp for schedule(dynamic)
#endif
    for (int64_t th = 0; th < (int64_t)B * Hv; ++th) {
      const int r = (int)(th / Hv), h = (int)(th % Hv), kh_i = h / G;
      const int32_t s = idx[r];
      if (!slot_valid(s, d->pool_slots)) {
        for (int t = 0; t < T; ++t)
          memset(o + (((size_t)r * T + t) * Hv + h) * dv, 0, (size_t)dv * sizeof(double));
        continue;
      }
      memcpy(S, pool + ((size_t)s * Hv + h) * tile, tile * sizeof(double));
      for (int t = 0; t < T; ++t) {
        const size_t rt = (size_t)r * T + t;
        gdn_token(dk, dv, S, q + (rt * Hk + kh_i) * dk, k + (rt * Hk + kh_i) * dk,
                  v + (rt * Hv + h) * dv, a[rt * Hv + h], b[rt * Hv + h], A_log[h],
                  dt_bias[h], d->scale, d->eps, d->state_bf16, o + (rt * Hv + h) * dv,
                  qh, kh, u);
        if (cache)
          memcpy(cache + (((size_t)r * cache_T + t) * Hv + h) * tile, S, tile * sizeof(double));
      }
      if (write_final) memcpy(pool + ((size_t)s * Hv + h) * tile, S, tile * sizeof(double));
    }
    free(S); free(qh); free(kh); free(u);
  }
  return 0;
}

/* Decode: one token per row, the state updated in place in its pool slot. */
int32_t oracle_decode(const oracle_dims* d,
                      const double* q, const double* k, const double* v,
                      const double* a, const double* b,
                      const double* A_log, const double* dt_bias,
                      double* pool, const int32_t* idx, double* o, int32_t nthreads) {
  if (!dims_ok(d) || d->T != 1) return -1;
  const int B = d->batch, Hk = d->num_k_heads, Hv = d->num_v_heads;
  const int dk = d->d_k, dv = d->d_v, G = Hv / Hk;
  const size_t tile = (size_t)dk * dv;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
  {
    double* qh = (double*)malloc((size_t)dk * sizeof(double));
    double* kh = (double*)malloc((size_t)dk * sizeof(double));
    double* u = (double*)malloc((size_t)dv * sizeof(double));
#ifdef _OPENMP
#pragma omp for schedule(dynamic)
#endif
    for (int64_t th = 0; th < (int64_t)B * Hv; ++th) {
      const int r = (int)(th / Hv), h = (int)(th % Hv), kh_i = h / G;
      const int32_t s = idx[r];
      double* orow = o + ((size_t)r * Hv + h) * dv;
      if (!slot_valid(s, d->pool_slots)) {
        memset(orow, 0, (size_t)dv * sizeof(double));
        continue;
      }
      gdn_token(dk, dv, pool + ((size_t)s * Hv + h) * tile, q + ((size_t)r * Hk + kh_i) * dk,
                k + ((size_t)r * Hk + kh_i) * dk, v + ((size_t)r * Hv + h) * dv,
                a[(size_t)r * Hv + h], b[(size_t)r * Hv + h], A_log[h], dt_bias[h],
                d->scale, d->eps, d->state_bf16, orow, qh, kh, u);
    }
    free(qh); free(kh); free(u);
  }
  return 0;
}

/* Replay rlen[r] cached tokens of row r from its slot's state; optionally commit the
 * result to the slot; then run this call's T tokens (outputs only, no state stored).
 * Reading: the replayed tokens produce no output; a replay length outside [0, rT]
 * replays nothing; the commit writes only when at least one token was replayed. */
int32_t oracle_verify_replay(const oracle_dims* d,
                             const double* q, const double* k, const double* v,
                             const double* a, const double* b,
                             const double* A_log, const double* dt_bias,
                             double* pool, const int32_t* idx,
                             const double* rk, const double* rv, const double* ra, const double* rb,
                             int32_t rT, const int32_t* rlen, int32_t commit, double* o,
                             int32_t nthreads) {
  if (!dims_ok(d) || rT < 0) return -1;
  const int B = d->batch, T = d->T, Hk = d->num_k_heads, Hv = d->num_v_heads;
  const int dk = d->d_k, dv = d->d_v, G = Hv / Hk;
  const size_t tile = (size_t)dk * dv;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
  {
    double* S = (double*)malloc(tile * sizeof(double));
    double* qh = (double*)malloc((size_t)dk * sizeof(double));
    double* kh = (double*)malloc((size_t)dk * sizeof(double));
    double* u = (double*)malloc((size_t)dv * sizeof(double));
    double* qz = (double*)calloc((size_t)dk, sizeof(double));
    double* oz = (double*)malloc((size_t)dv * sizeof(double));
#ifdef _OPENMP
#pragma omp for schedule(dynamic)
#endif
    for (int64_t th = 0; th < (int64_t)B * Hv; ++th) {
      const int r = (int)(th / Hv), h = (int)(th % Hv), kh_i = h / G;
      const int32_t s = idx[r];
      if (!slot_valid(s, d->pool_slots)) {
        for (int t = 0; t < T; ++t)
          memset(o + (((size_t)r * T + t) * Hv + h) * dv, 0, (size_t)dv * sizeof(double));
        continue;
      }
      memcpy(S, pool + ((size_t)s * Hv + h) * tile, tile * sizeof(double));
      const int32_t n = (rlen && rlen[r] >= 0 && rlen[r] <= rT) ? rlen[r] : 0;
      for (int t = 0; t < n; ++t) {
        const size_t rt = (size_t)r * rT + t;
        gdn_token(dk, dv, S, qz, rk + (rt * Hk + kh_i) * dk, rv + (rt * Hv + h) * dv, ra[rt * Hv + h],
                  rb[rt * Hv + h], A_log[h], dt_bias[h], d->scale, d->eps, d->state_bf16, oz, qh, kh, u);
      }
      if (commit && n > 0) memcpy(pool + ((size_t)s * Hv + h) * tile, S, tile * sizeof(double));
      for (int t = 0; t < T; ++t) {
        const size_t rt = (size_t)r * T + t;
        gdn_token(dk, dv, S, q + (rt * Hk + kh_i) * dk, k + (rt * Hk + kh_i) * dk, v + (rt * Hv + h) * dv,
                  a[rt * Hv + h], b[rt * Hv + h], A_log[h], dt_bias[h], d->scale, d->eps, d->state_bf16,
                  o + (rt * Hv + h) * dv, qh, kh, u);
      }
    }
    free(S); free(qh); free(kh); free(u); free(qz); free(oz);
  }
  return 0;
}

/* Separate replay commit: every row with a valid slot and 1 <= rlen[r] <= rT gets the
 * state after replaying its rlen[r] cached tokens from the slot written back to it. */
int32_t oracle_commit_replay(const oracle_dims* d, const double* A_log, const double* dt_bias,
                             double* pool, const int32_t* idx,
                             const double* rk, const double* rv, const double* ra, const double* rb,
                             int32_t rT, const int32_t* rlen, int32_t nthreads) {
  if (!dims_ok(d) || rT < 0) return -1;
  const int B = d->batch, Hk = d->num_k_heads, Hv = d->num_v_heads;
  const int dk = d->d_k, dv = d->d_v, G = Hv / Hk;
  const size_t tile = (size_t)dk * dv;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
  {
    double* qh = (double*)malloc((size_t)dk * sizeof(double));
    double* kh = (double*)malloc((size_t)dk * sizeof(double));
    double* u = (double*)malloc((size_t)dv * sizeof(double));
    double* qz = (double*)calloc((size_t)dk, sizeof(double));
    double* oz = (double*)malloc((size_t)dv * sizeof(double));
#ifdef _OPENMP
#pragma omp for schedule(dynamic)
#endif
    for (int64_t th = 0; th < (int64_t)B * Hv; ++th) {
      const int r = (int)(th / Hv), h = (int)(th % Hv), kh_i = h / G;
      const int32_t s = idx[r], n = rlen[r];
      if (!slot_valid(s, d->pool_slots) || n < 1 || n > rT) continue;
      double* S = pool + ((size_t)s * Hv + h) * tile;
      for (int t = 0; t < n; ++t) {
        const size_t rt = (size_t)r * rT + t;
        gdn_token(dk, dv, S, qz, rk + (rt * Hk + kh_i) * dk, rv + (rt * Hv + h) * dv, ra[rt * Hv + h],
                  rb[rt * Hv + h], A_log[h], dt_bias[h], d->scale, d->eps, d->state_bf16, oz, qh, kh, u);
      }
    }
    free(qh); free(kh); free(u); free(qz); free(oz);
  }
  return 0;
}

/* Gated RMS normalisation of the output, per (row, token, v-head) over its d_v values:
 *     y[j] = weight[j] * o[j] / sqrt(mean_j o[j]^2 + eps) * silu(z[j]),
 *     silu(z) = z / (1 + e^-z).
 * TensorRT-LLM PR 20937, Per-File QA Perspective: the decode-rows GDN kernel carries a
 * gated norm; the dense-FP8 notes name a token-major gated RMS norm. The pages do not
 * print it; this is the standard form (normalise, scale, then gate), with one weight
 * vector over d_v shared by the heads. o, z, y: [n][dv] (n = B*T*Hv vectors). */
void oracle_gated_norm(int64_t n, int32_t dv, const double* o, const double* z, const double* weight,
                       double eps, double* y) {
  for (int64_t v = 0; v < n; ++v) {
    const double* ov = o + v * dv;
    double ss = 0.0;
    for (int j = 0; j < dv; ++j) ss += ov[j] * ov[j];
    const double inv = 1.0 / sqrt(ss / dv + eps);
    for (int j = 0; j < dv; ++j) {
      const double zj = z[v * dv + j];
      y[v * dv + j] = weight[j] * ov[j] * inv * (zj / (1.0 + exp(-zj)));
    }
  }
}

/* Prefill of variable-length sequences with pooled initial states.
 * TensorRT-LLM PR 20937, Per-File QA Perspective: the chunked gated-delta-rule prefill
 * takes a bf16 state and an initial-state mask that zeroes fresh states. The pages do not
 * print the chunked form; the oracle follows the definition token by token:
 * for sequence r (tokens cu_seqlens[r] .. cu_seqlens[r+1]-1, packed along the first axis
 * of q, k, v, a, b, o) and v-head h, S starts at pool[idx[r]] (zero when fresh[r] != 0),
 * every token runs through the update above with no rounding between tokens, o is
 * written for every token, and the final state is stored back to the slot (rounded to
 * bf16 once, for a bf16 pool). A row whose slot is outside [0, P) gets o = 0 and no
 * state access. */
int32_t oracle_prefill(const oracle_dims* d, const int32_t* cu_seqlens, const double* q, const double* k,
                       const double* v, const double* a, const double* b, const double* A_log,
                       const double* dt_bias, double* pool, const int32_t* idx, const int32_t* fresh,
                       double* o, int32_t nthreads) {
  if (!d || d->batch < 0 || d->num_k_heads < 1 || d->num_v_heads % d->num_k_heads != 0 || d->d_k < 1 ||
      d->d_v < 1)
    return -1;
  const int B = d->batch, Hk = d->num_k_heads, Hv = d->num_v_heads, dk = d->d_k, dv = d->d_v, G = Hv / Hk;
  const size_t tile = (size_t)dk * dv;
  for (int r = 0; r < B; ++r)
    if (cu_seqlens[r + 1] < cu_seqlens[r]) return -1;
#ifdef _OPENMP
  if (nthreads > 0) omp_set_num_threads(nthreads);
#pragma omp parallel
#endif
  {
    double* qh = (double*)malloc((size_t)dk * sizeof(double));
    double* kh = (double*)malloc((size_t)dk * sizeof(double));
    double* u = (double*)malloc((size_t)dv * sizeof(double));
    double* S = (double*)malloc(tile * sizeof(double));
#ifdef _OPENMP
#pragma omp for schedule(dynamic)
#endif
    for (int64_t th = 0; th < (int64_t)B * Hv; ++th) {
      const int r = (int)(th / Hv), h = (int)(th % Hv), kh_i = h / G;
      const int32_t s = idx[r];
      const int32_t t0 = cu_seqlens[r], t1 = cu_seqlens[r + 1];
      if (!slot_valid(s, d->pool_slots)) {
        for (int32_t t = t0; t < t1; ++t)
          for (int j = 0; j < dv; ++j) o[((size_t)t * Hv + h) * dv + j] = 0.0;
        continue;
      }
      double* slot = pool + ((size_t)s * Hv + h) * tile;
      for (size_t e = 0; e < tile; ++e) S[e] = (fresh && fresh[r]) ? 0.0 : slot[e];
      for (int32_t t = t0; t < t1; ++t)
        gdn_token(dk, dv, S, q + ((size_t)t * Hk + kh_i) * dk, k + ((size_t)t * Hk + kh_i) * dk,
                  v + ((size_t)t * Hv + h) * dv, a[(size_t)t * Hv + h], b[(size_t)t * Hv + h], A_log[h],
                  dt_bias[h], d->scale, d->eps, 0, o + ((size_t)t * Hv + h) * dv, qh, kh, u);
      for (size_t e = 0; e < tile; ++e) slot[e] = d->state_bf16 ? oracle_round_bf16(S[e]) : S[e];
    }
    free(qh); free(kh); free(u); free(S);
  }
  return 0;
}
