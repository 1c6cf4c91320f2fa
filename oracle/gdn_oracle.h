/*
 * gdn_oracle.h -- plain float64 CPU oracle of the Gated DeltaNet (GDN) state update
 * for single-token decode, multi-token (MTP / speculative) verify and accepted-prefix
 * commit.
 *
 * TEST INFRASTRUCTURE. Only the tests, the smoke check and the benchmark's CPU
 * baseline may load this library. The product path (the HIP library) shares no code
 * with it and never calls it.
 *
 * Every array is a row-major float64 (or int32) host array; states are in the
 * logical layout S[i][j] with i the key index (d_k) and j the value index (d_v):
 *   q, k      [B][T][Hk][dk]         v, o   [B][T][Hv][dv]
 *   a, b      [B][T][Hv]             A_log, dt_bias [Hv]
 *   pool      [P][Hv][dk][dv]        cache  [B][cache_T][Hv][dk][dv]
 *   idx, accept, prev_accept  [B] int32
 * Functions return 0 on success, -1 on invalid dimensions.
 */
#ifndef GDN_ORACLE_H
#define GDN_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t batch, T, num_k_heads, num_v_heads, d_k, d_v, pool_slots;
  int32_t state_bf16;   /* 1: every stored state is rounded to bf16 (RNE) */
  double scale;         /* output scale, d_k^-1/2 in the workloads */
  double eps;           /* L2-norm epsilon: x / sqrt(sum x^2 + eps) */
} oracle_dims;

double oracle_softplus(double x);
void oracle_gates(double a, double b, double A_log, double dt_bias, double* g, double* beta);
double oracle_round_bf16(double x);
void oracle_round_bf16_f32bits(const uint32_t* in, uint16_t* out, int64_t n, int32_t nthreads);

int32_t oracle_verify(const oracle_dims* d,
                      const double* q, const double* k, const double* v,
                      const double* a, const double* b,
                      const double* A_log, const double* dt_bias,
                      double* pool, const int32_t* idx,
                      double* cache, int32_t cache_T, int32_t write_final,
                      const int32_t* prev_accept, double* o, int32_t nthreads);

int32_t oracle_decode(const oracle_dims* d,
                      const double* q, const double* k, const double* v,
                      const double* a, const double* b,
                      const double* A_log, const double* dt_bias,
                      double* pool, const int32_t* idx, double* o, int32_t nthreads);

int32_t oracle_commit(const oracle_dims* d, const double* cache, int32_t cache_T,
                      const int32_t* idx, const int32_t* accept, double* pool,
                      int32_t nthreads);

/* Cached replay. rk, rv, ra, rb hold the per-token inputs of an earlier verify
 * ([B][rT][Hk][dk], [B][rT][Hv][dv], [B][rT][Hv], [B][rT][Hv]); rlen[r] tokens of row r
 * are replayed from its pool slot (rlen outside [0, rT] replays nothing). */
int32_t oracle_verify_replay(const oracle_dims* d,
                             const double* q, const double* k, const double* v,
                             const double* a, const double* b,
                             const double* A_log, const double* dt_bias,
                             double* pool, const int32_t* idx,
                             const double* rk, const double* rv, const double* ra, const double* rb,
                             int32_t rT, const int32_t* rlen, int32_t commit, double* o,
                             int32_t nthreads);

int32_t oracle_commit_replay(const oracle_dims* d, const double* A_log, const double* dt_bias,
                             double* pool, const int32_t* idx,
                             const double* rk, const double* rv, const double* ra, const double* rb,
                             int32_t rT, const int32_t* rlen, int32_t nthreads);

/* Prefill of d->batch variable-length sequences (cu_seqlens [B+1]; q, k [N][Hk][dk],
 * v, o [N][Hv][dv], a, b [N][Hv] with N = cu_seqlens[B]) from pooled initial states
 * (zero where fresh[r] != 0; fresh may be NULL), no rounding between tokens, final state
 * stored to the slot (rounded once for a bf16 pool). d->T is not used. */
int32_t oracle_prefill(const oracle_dims* d, const int32_t* cu_seqlens, const double* q, const double* k,
                       const double* v, const double* a, const double* b, const double* A_log,
                       const double* dt_bias, double* pool, const int32_t* idx, const int32_t* fresh,
                       double* o, int32_t nthreads);

/* Gated RMS normalisation of n output vectors of length dv:
 * y[j] = weight[j] * o[j] / sqrt(mean(o^2) + eps) * silu(z[j]). */
void oracle_gated_norm(int64_t n, int32_t dv, const double* o, const double* z, const double* weight,
                       double eps, double* y);

#ifdef __cplusplus
}
#endif
#endif
