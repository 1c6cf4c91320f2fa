/*
 * conv_oracle.h -- float64 CPU oracle of the short causal convolution kept next to the
 * GDN state (verify, decode, accepted-prefix commit).
 *
 * TEST INFRASTRUCTURE, like gdn_oracle.h: only the tests and the benchmark's CPU
 * baseline load it.
 *
 * Row-major float64 (or int32) host arrays:
 *   x, y          [B][T][D]          (D = channels)
 *   w             [K][D]             (tap i multiplies the input K-1-i tokens back)
 *   bias          [D] or NULL
 *   pool          [P][K-1][D]        (per slot: the last K-1 inputs, oldest first)
 *   prev_x        [B][T_prev][D]     (the previous call's inputs, for a fused commit)
 *   idx, accept, prev_len  [B] int32
 * Functions return 0 on success, -1 on invalid dimensions.
 */
#ifndef CONV_ORACLE_H
#define CONV_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
  int32_t batch, T, channels, width, pool_slots;
  int32_t activation;  /* 0: identity, 1: SiLU */
} oracle_conv_dims;

/* For each valid row: first, when prev_x is given and 1 <= prev_len[r] <= T_prev, the
 * slot's state advances over the first prev_len[r] tokens of prev_x and is written back
 * (fused commit); then y of this call's T tokens; then, when write_back, the state
 * advanced over all T tokens is written back. Padding rows (slot outside [0, P)) get
 * y = 0 and no state access. */
int32_t oracle_conv_update(const oracle_conv_dims* d, const double* x, const double* w, const double* bias,
                           double* pool, const int32_t* idx, const double* prev_x, int32_t T_prev,
                           const int32_t* prev_len, double* y, int32_t write_back);

/* Accepted-prefix commit: for each valid row with 1 <= accept[r] <= T, the slot's state
 * advances over the first accept[r] tokens of x ([B][T][D]); other rows are untouched. */
int32_t oracle_conv_commit(const oracle_conv_dims* d, const double* x, double* pool, const int32_t* idx,
                           const int32_t* accept);

#ifdef __cplusplus
}
#endif
#endif
