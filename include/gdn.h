/*
 * gdn.h -- C ABI of the MI355X (gfx950) Gated DeltaNet (GDN) state-update library:
 * pooled-state decode, multi-token (MTP / speculative) verify with an intermediate-
 * state cache, and accepted-prefix commit.
 *
 * Sources (pages by title, section):
 * [P1] "[NVIDIA] [GDN] Enable FlashInfer MTP verify on SM100+ (Blackwell)" (SGLang PR
 *      23273): Summary -- the verify kernel addresses each request's recurrent state in
 *      a pool through initial_state_indices, and A_log is passed as fp32; Requirements
 *      -- padding index guard for bf16 decode, bf16-state MTP beyond 4 tokens with
 *      intermediate caching.
 * [P2] "[GDN] Honor configured linear-attn verify backend in the kernel dispatcher"
 *      (SGLang PR 34592): Motivation -- fp32 and bf16 SSM state must both work with MTP.
 * [P3] TensorRT-LLM PR 20937, GB300 Qwen3.8-Flash-Next NVFP4 target: Per-File QA
 *      Perspective and Moved out of this PR -- bf16 or fp32 recurrent pools, commit of
 *      the accepted prefix in-kernel (below 16 requests) or by a separate all-layer
 *      commit, duplicate rows, graph capture and replay.
 * [P4] "Proposal: native BF16 MTP speculative decoding for dense Qwen3.8-27B
 *      (qwen38_dense), with results on SM120": What -- recovery records and the
 *      convolution state committed with them.
 *
 * The update (the pages name the gated delta rule without printing it; this is its
 * standard form). For request row r, v-head h, k-head kh = h / (Hv/Hk), token t:
 *     q^ = q / sqrt(|q|^2 + eps),  k^ = k / sqrt(|k|^2 + eps)
 *     g = exp(-exp(A_log[h]) * softplus(a + dt_bias[h])),  beta = sigmoid(b)
 *     S <- g S;  S <- S + beta k^ (v - S^T k^)^T;  o = scale * S^T q^
 * S is a d_k x d_v matrix per (slot, v-head). With a bf16 state every stored state is
 * rounded to nearest even and the rounded value is carried to the next token, so a
 * T-token verify equals T single-token decodes and commit(n) equals intermediate n.
 *
 * Layouts (row-major, every pointer a device pointer owned by the caller):
 *   q, k           [B][T][Hk][d_k]      io dtype
 *   v, o           [B][T][Hv][d_v]      io dtype
 *   a, b           [B][T][Hv]           io dtype
 *   A_log, dt_bias [Hv]                 fp32
 *   state_pool     [P][Hv][d_v][d_k]    state dtype: element [s][h][j][i] holds S[i][j]
 *                                       (each value column of S is a contiguous row)
 *   inter_cache    [B][cache_T][Hv][d_v][d_k]   state dtype, same per-tile layout
 *   state_indices, accept lengths       [B] int32
 *
 * Conventions shared by every entry point:
 * - A slot index outside [0, P) (the padding index -1 included) marks a padding row:
 *   no state is read or written for it and its o rows are zeroed.
 * - batch == 0 is a no-op that returns GDN_OK once the sizes and dtypes are valid;
 *   the pointers are not examined then (empty tensors may have NULL data).
 * - Host-checkable faults return an error before anything is launched; nothing is
 *   written. A failed launch returns GDN_ERR_LAUNCH.
 * - The library allocates nothing, never synchronises, keeps no global state (but for
 *   the per-GPU address of gdn_prefill_noalloc's fixed array) and launches its kernels
 *   (one per call; two to four for gdn_prefill) on `stream` (a hipStream_t; NULL is the
 *   default stream). Calls are therefore thread-safe and may be captured in a HIP graph.
 * - Supported geometry: d_k in {16, 32, 64, 128, 256}; d_v a multiple of 16 in
 *   [16, 256]; Hv a multiple of Hk; 1 <= T <= GDN_MAX_T.
 * - Alignment: q, k, v, o, state_pool and inter_cache 16-byte aligned; the others
 *   aligned to their element size.
 * - Writing calls (decode, verify with write_final or a fused commit, commit) need
 *   the valid indices of one call to be distinct; read-only verify allows repeats.
 */
#ifndef GDN_H
#define GDN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GDN_ABI_VERSION 3
#define GDN_API __attribute__((visibility("default")))
#define GDN_MAX_T 16

typedef enum { GDN_DTYPE_F32 = 0, GDN_DTYPE_BF16 = 1 } gdn_dtype;

typedef enum {
  GDN_OK = 0,
  GDN_ERR_NULL = 1,        /* a required pointer is NULL */
  GDN_ERR_SHAPE = 2,       /* inconsistent or negative sizes */
  GDN_ERR_DTYPE = 3,       /* unknown dtype value */
  GDN_ERR_ALIGN = 4,       /* a pointer misses its alignment */
  GDN_ERR_UNSUPPORTED = 5, /* valid but outside the supported geometry */
  GDN_ERR_LAUNCH = 6,      /* the kernel launch failed */
  GDN_ERR_TOO_LARGE = 7    /* the call needs more than the library's fixed prefill array */
} gdn_status;

typedef struct {
  int32_t batch;        /* B: request rows of this call (padding rows included) */
  int32_t T;            /* tokens per row (1 for decode) */
  int32_t num_k_heads;  /* Hk */
  int32_t num_v_heads;  /* Hv, a multiple of Hk; v-head h uses k-head h / (Hv/Hk) */
  int32_t d_k;          /* key dimension */
  int32_t d_v;          /* value dimension */
  int32_t pool_slots;   /* P */
  gdn_dtype state_dtype;
  gdn_dtype io_dtype;
  float scale;          /* output scale, normally d_k^-1/2 */
  float l2norm_eps;     /* q and k are L2-normalised in-kernel: x / sqrt(|x|^2 + eps) */
} gdn_dims;

typedef struct {
  const void* q;
  const void* k;
  const void* v;
  const void* a;
  const void* b;
  const float* A_log;
  const float* dt_bias;
  void* o;
} gdn_io;

/* Single-token decode [P1, Summary; Requirements]: for each row, the state of its
 * slot is advanced by one token and written back in place; o receives the read-out.
 * Needs dims->T == 1. Identical arithmetic to gdn_verify with T = 1, no cache and
 * write_final = 1. */
GDN_API gdn_status gdn_decode(const gdn_dims* dims, const gdn_io* io, void* state_pool,
                      const int32_t* state_indices, void* stream);

/* Multi-token verify [P1, Summary; Requirements; P2, Motivation]: T draft tokens per
 * row run through the update, starting from the row's pool slot.
 * inter_cache  NULL, or a cache of depth cache_T >= T: entry [r][t] receives the
 *              state after token t (the intermediate-state cache that lets any
 *              accepted prefix be restored). Entries t >= T and padding rows are
 *              left untouched.
 * write_final  1: the state after the last token is written back to the slot.
 *              0: the pool is only read, so a rejected draft needs no rollback.
 * prev_accept_len  NULL, or [B] accept lengths of the previous verify whose
 *              intermediates are in inter_cache [P3, in-kernel commit]: for rows with
 *              1 <= n <= cache_T the state starts from inter_cache[r][n-1], which is
 *              also committed to the slot; other rows start from the slot. Exactly
 *              gdn_commit(prev) followed by gdn_verify. Needs inter_cache; row r must
 *              be the same request as in the previous verify. */
GDN_API gdn_status gdn_verify(const gdn_dims* dims, const gdn_io* io, void* state_pool,
                      const int32_t* state_indices, void* inter_cache, int32_t cache_T,
                      int32_t write_final, const int32_t* prev_accept_len, void* stream);

/* Accepted-prefix commit [P3, Per-File QA Perspective; Moved out of this PR]:
 * state_pool[idx[r]] <- inter_cache[r][n-1] for every row with a valid slot and
 * 1 <= n = accept_len[r] <= cache_T; all other rows leave the pool untouched.
 * Reads dims->batch, num_v_heads, d_k, d_v, pool_slots and state_dtype only. */
GDN_API gdn_status gdn_commit(const gdn_dims* dims, const void* inter_cache, int32_t cache_T,
                      const int32_t* state_indices, const int32_t* accept_len,
                      void* state_pool, void* stream);

/* Chunked prefill from pooled initial states [P3] (Per-File QA Perspective: the chunked
 * gated delta rule prefill with a bf16 state and an initial-state mask that zeroes fresh
 * states). dims->batch sequences of variable length; their tokens are packed along the
 * first axis: q, k [N][Hk][d_k], v, o [N][Hv][d_v], a, b [N][Hv] (N = cu_seqlens[B];
 * sequence r holds tokens cu_seqlens[r] .. cu_seqlens[r+1]-1, offsets non-decreasing);
 * dims->T is ignored. Per valid row r and v-head h the state starts at
 * state_pool[idx[r]] (zero where fresh[r] != 0; fresh may be NULL), every token runs
 * through the update, o is written for every token, and the final state is stored back
 * to the slot. Between tokens the state stays fp32 and is not rounded; a bf16 pool
 * receives the final state rounded to nearest even once. Padding rows get o = 0 and no
 * state access. The chunked form runs on the bf16 matrix cores: io must be bf16, d_k 128,
 * d_v a multiple of 32 (GDN_ERR_UNSUPPORTED otherwise). Valid slots must be distinct.
 *
 * Precision, whatever the pool dtype: every product takes bf16 operands with fp32
 * accumulation -- the stored keys, queries and values exactly, and the state at each chunk
 * start, the chunk's triangular inverse and derived matrices, and U rounded to bf16 (2^-9
 * relative each). o and the final state come out within a few bf16 roundings of the
 * token-by-token result relative to their magnitude (tested to 2^-5 of each head's largest
 * |o| and |S|; measured 0.2-1.1 %), not to fp32 precision: an fp32 pool keeps its state in
 * fp32 between calls, but a prefill call is bf16-grade. For an fp32-grade prefill of an fp32
 * pool, run the tokens through gdn_verify with write_final = 1 in calls of up to GDN_MAX_T
 * tokens: it is the same update, token by token in fp32 (tested against this call's float64
 * definition to 1e-4), at the cost of one call per GDN_MAX_T tokens.
 *
 * num_tokens is the length of the packed token axis of q, k, v, a, b and o;
 * cu_seqlens[B] <= num_tokens is required (not checked: the offsets live on the device),
 * and num_tokens * Hv * d_v and num_tokens * Hk * d_k must stay below 2^30 elements
 * (GDN_ERR_UNSUPPORTED otherwise).
 * The first kernel prepares, for every 16-token chunk and v-head, the state-independent
 * products in `workspace` (device memory owned by the caller, 256-byte aligned, at least
 * gdn_prefill_workspace_bytes(dims, num_tokens) bytes, GDN_ERR_SHAPE if smaller). Then each
 * sequence's chunks are walked in order, in segments (their length is chosen from the
 * geometry, as under gdn_prefill_workspace_bytes): one more kernel when every sequence is
 * one segment; otherwise the first segments and the maps of the middle ones, a kernel that
 * composes the maps into each segment's starting state, and the remaining segments (up to
 * four kernels per call). The workspace holds nothing between calls; calls that overlap in
 * time need their own. */
GDN_API gdn_status gdn_prefill(const gdn_dims* dims, const gdn_io* io, void* state_pool,
                               const int32_t* state_indices, const int32_t* cu_seqlens,
                               const int32_t* fresh, int64_t num_tokens, void* workspace,
                               size_t workspace_bytes, void* stream);

/* gdn_prefill without allocation, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). The
 * workspace is not the caller's but a fixed device array inside the library of
 * GDN_PREFILL_NOALLOC_BYTES (128 MiB), one copy per GPU, held from the first call on that
 * GPU until the process ends. Everything else -- arguments, layouts, results, bit for bit,
 * and errors -- is gdn_prefill's. Calls whose workspace (gdn_prefill_workspace_bytes) would
 * exceed the array return GDN_ERR_TOO_LARGE before anything runs (at Hk = 4, Hv = 8, d_v =
 * 128: about 34,000 packed tokens in one sequence). The array's device address is looked up
 * on the first call for a GPU (the GPU of `stream`, or the current one for the NULL stream), so a caller
 * that captures graphs makes one call before capturing; a failed lookup returns
 * GDN_ERR_LAUNCH. No call allocates, frees or synchronises. Every call on one GPU shares
 * that GPU's array, which keeps the last call's contents (nothing in it needs to start at
 * zero): calls that overlap in time on one GPU, on different streams or threads, race and
 * must be ordered by the caller. */
#define GDN_PREFILL_NOALLOC_BYTES ((size_t)128 << 20)
GDN_API gdn_status gdn_prefill_noalloc(const gdn_dims* dims, const gdn_io* io, void* state_pool,
                                       const int32_t* state_indices, const int32_t* cu_seqlens,
                                       const int32_t* fresh, int64_t num_tokens, void* stream);

/* Workspace size of gdn_prefill, in three parts:
 * - per 16-token chunk, (floor(num_tokens / 16) + batch) of them, one 5376-byte record per
 *   v-head (a 4096-byte bf16 chunk x d_k operand -- or, when the chain runs in segments, the
 *   512-byte 16 x 16 factor it is formed from -- two 512-byte 16 x 16 bf16 matrices, the
 *   per-token factors, padding) and one 4096-byte record per k-head (the chunk's
 *   transposed keys, shared by the k-head's v-heads);
 * - a table of the segments of the chunk chain, 4 bytes each, padded to 256 bytes;
 * - per segment and v-head, a slot of 128 * d_v * 4 + 128 * 128 * 2 bytes (a state and a
 *   segment map).
 * Segments hold 2^s tokens and number floor(num_tokens / 2^s) + batch. s is the smallest
 * s >= 8 with 2^s > num_tokens (one segment per sequence) when 2 * batch * num_v_heads *
 * d_v / 16 >= 512; otherwise the smallest s >= 8 with 2^s >= num_tokens * num_v_heads *
 * (d_v / 16) * 2 / 2048 (integer division), but no more than the first. Writes the size to
 * *bytes; GDN_ERR_SHAPE for a negative num_tokens, the gdn_prefill geometry checks
 * otherwise. */
GDN_API gdn_status gdn_prefill_workspace_bytes(const gdn_dims* dims, int64_t num_tokens, size_t* bytes);

/* The gated RMS normalisation of the output, fused into verify or decode [P3] (Per-File QA
 * Perspective: the decode-rows GDN kernel carries a gated norm; the dense-FP8 notes name
 * a token-major gated RMS norm). The pages do not print it; this is the standard form,
 * per (row, token, v-head) vector of d_v outputs o:
 *     y[j] = weight[j] * o[j] / sqrt(mean_j o[j]^2 + eps) * silu(z[j]),
 *     silu(x) = x / (1 + e^-x),  one weight vector over d_v shared by the heads. */
typedef struct {
  const void* z;        /* [B][T][Hv][d_v] io dtype, 16-byte aligned: the gate input */
  const float* weight;  /* [d_v] fp32, 16-byte aligned */
  float eps;            /* >= 0 */
} gdn_out_gate;

/* gdn_verify whose io->o receives y (above) instead of o; everything else (cache, write-
 * back, fused commit, padding rows with y = 0) is as in gdn_verify. T = 1 with
 * write_final = 1 and no cache is the gated decode. One workgroup then holds a head's
 * whole d_v: d_v <= 128 is required for d_k >= 128 (GDN_ERR_UNSUPPORTED otherwise). */
GDN_API gdn_status gdn_verify_gated(const gdn_dims* dims, const gdn_io* io, const gdn_out_gate* gate,
                                    void* state_pool, const int32_t* state_indices, void* inter_cache,
                                    int32_t cache_T, int32_t write_final, const int32_t* prev_accept_len,
                                    void* stream);

/* Per-token inputs of an earlier verify, kept by the caller for cached replay: the k,
 * v, a, b arrays that verify consumed (typically the previous step's io buffers, used
 * alternately with the current ones). io dtype, 16-byte aligned k and v. */
typedef struct {
  const void* k;    /* [B][T_src][Hk][d_k] */
  const void* v;    /* [B][T_src][Hv][d_v] */
  const void* a;    /* [B][T_src][Hv] */
  const void* b;    /* [B][T_src][Hv] */
  int32_t T_src;    /* tokens per row in these arrays, >= 1 */
} gdn_tokens;

/* Cached-replay verify [P3, What changes: a copy-free cached replay of the GDN verify;
 * Moved out of this PR: commit in-kernel or by the separate all-layer commit; the cache
 * manager tracks the previous step's accept count and which token buffer holds it].
 * Instead of one stored state per token, the accepted prefix of the previous verify is
 * replayed: for each valid row, with n = replay_len[r] (n outside [0, T_src] replays
 * nothing), the state of the slot advances through tokens 0..n-1 of `replay`; with
 * commit = 1 and n >= 1 that state is written back to the slot; then this call's T
 * tokens run from it and write o. No per-token state is stored. Replayed and new tokens
 * use the same arithmetic as gdn_verify, so the replayed state equals, bit for bit, the
 * intermediate state gdn_verify would have cached after n tokens. Needs
 * T + T_src <= GDN_MAX_T. `replay` must not alias io's k, v, a, b. */
GDN_API gdn_status gdn_verify_replay(const gdn_dims* dims, const gdn_io* io, void* state_pool,
                                     const int32_t* state_indices, const gdn_tokens* replay,
                                     const int32_t* replay_len, int32_t commit, void* stream);

/* Replay commit (the separate all-layer commit of the same contract): for each valid row
 * with 1 <= n = replay_len[r] <= T_src, the slot's state advanced through tokens 0..n-1
 * of `replay` is written back to the slot; other rows are untouched. Reads dims->batch,
 * num_k_heads, num_v_heads, d_k, d_v, pool_slots, state_dtype, io_dtype, l2norm_eps;
 * needs T_src <= GDN_MAX_T. */
GDN_API gdn_status gdn_commit_replay(const gdn_dims* dims, const float* A_log, const float* dt_bias,
                                     void* state_pool, const int32_t* state_indices,
                                     const gdn_tokens* replay, const int32_t* replay_len, void* stream);

/* ---- Short causal convolution state, pooled next to the GDN state ------------------
 * [P3] What changes: the GDN in_proj GEMV carries a fused conv1d epilogue for verify and
 * decode rows; Per-File QA Perspective: the speculative staging and commit kernels keep
 * accepted-prefix boundaries of the convolution state along with the other per-request
 * state. [P4] "Proposal: native BF16 MTP speculative decoding for dense Qwen3.8-27B",
 * What: the verify keeps recovery records and commits the convolution state with them.
 * The pages do not print the convolution; this is the standard depthwise causal form of
 * width K, per request row r and channel c:
 *     in(tau) = x[r][tau][c] (tau >= 0),   state[slot][K-1+tau][c] (-(K-1) <= tau < 0)
 *     y[r][t][c] = act(bias[c] + sum_{i<K} w[i][c] * in(t-(K-1)+i)),   act = id | SiLU
 * The state of a slot is its last K-1 inputs, oldest first. Advancing it over n tokens
 * keeps the last K-1 entries of (state ++ those tokens): an exact selection, so a commit
 * or a rejected draft never rounds it.
 * Layouts: x, y [B][T][D] and prev_x [B][T_prev][D] and conv_pool [P][K-1][D] in the
 * dims' dtype; weight [K][D] fp32 (tap i multiplies the input K-1-i tokens back); bias
 * [D] fp32 or NULL; state_indices, prev_len, accept_len [B] int32.
 * Geometry: D a multiple of 8 (bf16) or 4 (fp32); 2 <= K <= GDN_CONV_MAX_WIDTH;
 * 1 <= T <= GDN_MAX_T; B <= 65535. x, y, prev_x, conv_pool, weight and bias are
 * 16-byte aligned. Padding rows get y = 0 and no state access. The conventions above
 * (batch 0, errors before launch, one launch, no allocation, distinct indices in
 * writing calls) apply. */
#define GDN_CONV_MAX_WIDTH 8
typedef enum { GDN_CONV_ACT_NONE = 0, GDN_CONV_ACT_SILU = 1 } gdn_conv_act;

typedef struct {
  int32_t batch;
  int32_t T;           /* tokens per row of x */
  int32_t channels;    /* D */
  int32_t width;       /* K */
  int32_t pool_slots;  /* P */
  int32_t dtype;       /* gdn_dtype of x, y, prev_x and conv_pool */
  int32_t activation;  /* gdn_conv_act */
} gdn_conv_dims;

/* Verify or decode of the convolution. For each valid row: (1) when prev_x is given and
 * 1 <= prev_len[r] <= T_prev, the slot's state advances over the first prev_len[r]
 * tokens of prev_x and is written back (the fused commit of the previous step's
 * accepted prefix); (2) y of this call's T tokens from that state; (3) when write_back,
 * the state advanced over all T tokens is written back (decode). Without prev_x and
 * write_back the pool is read-only. prev_x needs prev_len and 1 <= T_prev <= GDN_MAX_T,
 * and must not alias x. */
GDN_API gdn_status gdn_conv_update(const gdn_conv_dims* dims, const void* x, const float* weight,
                                   const float* bias, void* conv_pool, const int32_t* state_indices,
                                   const void* prev_x, int32_t T_prev, const int32_t* prev_len,
                                   void* y, int32_t write_back, void* stream);

/* Accepted-prefix commit of the convolution state: for each valid row with
 * 1 <= accept_len[r] <= T, the slot's state advances over the first accept_len[r]
 * tokens of x; other rows are untouched. Reads dims->batch, T, channels, width,
 * pool_slots and dtype. */
GDN_API gdn_status gdn_conv_commit(const gdn_conv_dims* dims, const void* x, void* conv_pool,
                                   const int32_t* state_indices, const int32_t* accept_len, void* stream);

/* Static text for a status code (never NULL). */
GDN_API const char* gdn_status_string(gdn_status status);

/* GDN_ABI_VERSION of the built library. */
GDN_API int32_t gdn_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GDN_H */
