// gdn_api.cpp -- the C ABI of include/gdn.h: argument validation, kernel choice and
// launch. No allocation and no synchronisation; one launch per call (two to four for the
// prefill). The only global state is the per-device address of the fixed prefill array
// that gdn_prefill_noalloc uses (gdn_noalloc.hip).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/gdn.h"
#include "gdn_internal.h"

namespace {

using gdn::Dt;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool dtype_ok(gdn_dtype d) { return d == GDN_DTYPE_F32 || d == GDN_DTYPE_BF16; }

size_t dsize(gdn_dtype d) { return d == GDN_DTYPE_F32 ? 4 : 2; }

bool dk_supported(int dk) { return dk == 16 || dk == 32 || dk == 64 || dk == 128 || dk == 256; }

// Checks shared by decode, verify and commit: sizes, dtypes, geometry.
gdn_status check_dims(const gdn_dims* d, bool need_tokens) {
  if (!d) return GDN_ERR_NULL;
  if (d->batch < 0 || d->num_k_heads < 1 || d->num_v_heads < 1 || d->d_k < 1 || d->d_v < 1 ||
      d->pool_slots < 0)
    return GDN_ERR_SHAPE;
  if (need_tokens && d->T < 1) return GDN_ERR_SHAPE;
  if (d->num_v_heads % d->num_k_heads != 0) return GDN_ERR_SHAPE;
  if (!dtype_ok(d->state_dtype) || !dtype_ok(d->io_dtype)) return GDN_ERR_DTYPE;
  if (!dk_supported(d->d_k) || d->d_v % 16 != 0 || d->d_v > 256) return GDN_ERR_UNSUPPORTED;
  if (need_tokens && d->T > GDN_MAX_T) return GDN_ERR_UNSUPPORTED;
  // grid limits (heads in y, rows in z) and 32-bit row offsets inside the kernels
  if (d->batch > 65535 || d->num_v_heads > 65535) return GDN_ERR_UNSUPPORTED;
  if (int64_t(d->batch) * d->num_v_heads * 16 > int64_t(INT32_MAX)) return GDN_ERR_UNSUPPORTED;
  if (need_tokens && int64_t(d->batch) * d->T * d->num_v_heads > int64_t(INT32_MAX) / 256)
    return GDN_ERR_UNSUPPORTED;
  return GDN_OK;
}

// Launch shape of the recurrent kernel at d_k = 128 (other d_k use one shape).
// One value row per lane and 4 waves (32 value rows per workgroup) measured fastest
// on the decode and bf16 workloads: more, smaller workgroups reach their state
// sooner and start storing earlier. Large fp32-state grids (a 64 KiB tile, many
// rounds of workgroups) measured faster with 2-wave workgroups (16 value rows).
// Single-token calls (decode) measured fastest with a whole head per workgroup (four rows
// per lane, 4 waves): 13.7 -> 11.3 us on the fp32 decode batch (B = 64, 8 v-heads; two rows
// and 8 waves: 11.6 us), as the per-workgroup work before the state arrives (q and k loads,
// norms, LDS staging) is then done once per head instead of once per 32 value rows; with
// T >= 4 whole-head shapes were 10-16 % slower on every workload.
int pick_shape(const gdn_dims* d) {
  const int64_t tiles = int64_t(d->batch) * d->num_v_heads;
  if (d->state_dtype == GDN_DTYPE_F32 && tiles >= 4096) return 12;
  if (d->T == 1) return 44;
  return 1;
}

// Load policy of the initial state. Nontemporal loads do not keep the state's lines in
// the XCD's L2. That matters where the same lines are stored to later, by the launch
// itself (decode's write-back, an in-kernel commit) or by the commit launch that
// follows a verify: the stores then no longer hit resident lines, which appears to
// spare a write-back of dirty L2 lines at the end of the launch. Measured (plain ->
// nontemporal, cold pools): decode fp32 B=64 15.1 -> 13.7 us, B=256 51.2 -> 46.4 us;
// verify + commit on the MTP T=4 bf16 batch 27.1 -> 22.4 us per step, verify alone
// 1-2 % faster at B = 64..512; cached replay 19.3 -> 16.2 us; gated verify + commit
// 29.3 -> 26.3 us. Slower: T = 8 with 32 v-heads (fused 227 -> 247 us at B = 128, plain
// 205 -> 216 us, 2-6 % at B = 32..96) and the 2-wave fp32 shape (T = 4, 8192 tiles:
// 468 -> 482 us). Replay calls always take them.
bool pick_nt_loads(const gdn_dims* d, bool replay) {
  if (replay) return true;
  const int shape = pick_shape(d);
  return d->T <= 4 && (shape == 1 || shape == 44);
}

gdn_status run_recurrent(const gdn_dims* d, const gdn_io* io, void* pool, const int32_t* idx,
                         void* cache, int32_t cache_T, int32_t write_final,
                         const int32_t* prev_accept, void* stream, const gdn_out_gate* gate = nullptr) {
  if (gate) {
    if (!(gate->eps >= 0.f)) return GDN_ERR_SHAPE;
    if (d->d_k >= 128 && d->d_v > 128) return GDN_ERR_UNSUPPORTED;  // one workgroup holds a head's d_v
  }
  if (d->batch == 0) return GDN_OK;
  if (gate && (!gate->z || !gate->weight)) return GDN_ERR_NULL;
  if (gate && (!aligned(gate->z, 16) || !aligned(gate->weight, 16))) return GDN_ERR_ALIGN;
  if (!io || !io->q || !io->k || !io->v || !io->a || !io->b || !io->A_log || !io->dt_bias || !io->o ||
      !pool || !idx)
    return GDN_ERR_NULL;
  if (prev_accept && !cache) return GDN_ERR_NULL;
  if (cache && cache_T < d->T) return GDN_ERR_SHAPE;
  const uintptr_t isz = dsize(d->io_dtype);
  if (!aligned(io->q, 16) || !aligned(io->k, 16) || !aligned(io->v, 16) || !aligned(io->o, 16) ||
      !aligned(pool, 16) || (cache && !aligned(cache, 16)) || !aligned(io->a, isz) || !aligned(io->b, isz) ||
      !aligned(io->A_log, 4) || !aligned(io->dt_bias, 4) || !aligned(idx, 4) ||
      (prev_accept && !aligned(prev_accept, 4)))
    return GDN_ERR_ALIGN;

  gdn::RecurrentArgs p;
  p.q = io->q; p.k = io->k; p.v = io->v; p.a = io->a; p.b = io->b;
  p.A_log = io->A_log; p.dt_bias = io->dt_bias; p.o = io->o;
  p.pool = pool; p.idx = idx; p.cache = cache; p.prev_accept = prev_accept;
  p.B = d->batch; p.T = d->T; p.Hk = d->num_k_heads; p.Hv = d->num_v_heads;
  p.DK = d->d_k; p.DV = d->d_v; p.P = d->pool_slots; p.cache_T = cache ? cache_T : 0;
  p.G = d->num_v_heads / d->num_k_heads;
  p.write_final = write_final ? 1 : 0;
  p.scale = d->scale; p.eps = d->l2norm_eps;
  p.rk = p.rv = p.ra = p.rb = nullptr;
  p.rlen = nullptr;
  p.rT = 0;
  p.rcommit = 0;
  p.z = gate ? gate->z : nullptr;
  p.gw = gate ? gate->weight : nullptr;
  p.geps = gate ? gate->eps : 0.f;
  const hipError_t e = gdn::launch_recurrent(static_cast<Dt>(d->state_dtype), static_cast<Dt>(d->io_dtype),
                                             pick_shape(d), gate ? 3 : 0, pick_nt_loads(d, false), p,
                                             static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

// Checks of the replay token arrays (pointers, alignment, depth).
gdn_status check_replay(const gdn_dims* d, const gdn_tokens* rep, const int32_t* rlen) {
  if (!rep || !rep->k || !rep->v || !rep->a || !rep->b || !rlen) return GDN_ERR_NULL;
  const uintptr_t isz = dsize(d->io_dtype);
  if (!aligned(rep->k, 16) || !aligned(rep->v, 16) || !aligned(rep->a, isz) || !aligned(rep->b, isz) ||
      !aligned(rlen, 4))
    return GDN_ERR_ALIGN;
  return GDN_OK;
}

void set_replay(gdn::RecurrentArgs& p, const gdn_tokens* rep, const int32_t* rlen, int32_t commit) {
  p.rk = rep->k; p.rv = rep->v; p.ra = rep->a; p.rb = rep->b;
  p.rlen = rlen;
  p.rT = rep->T_src;
  p.rcommit = commit ? 1 : 0;
}

// Checks of the convolution dims: sizes, dtype, geometry, grid limits.
gdn_status check_conv_dims(const gdn_conv_dims* d) {
  if (!d) return GDN_ERR_NULL;
  if (d->batch < 0 || d->T < 1 || d->channels < 1 || d->width < 2 || d->pool_slots < 0) return GDN_ERR_SHAPE;
  if (!dtype_ok(static_cast<gdn_dtype>(d->dtype))) return GDN_ERR_DTYPE;
  if (d->activation != GDN_CONV_ACT_NONE && d->activation != GDN_CONV_ACT_SILU) return GDN_ERR_UNSUPPORTED;
  const int ve = 16 / int(dsize(static_cast<gdn_dtype>(d->dtype)));
  if (d->channels % ve != 0 || d->width > GDN_CONV_MAX_WIDTH || d->T > GDN_MAX_T) return GDN_ERR_UNSUPPORTED;
  if (d->batch > 65535) return GDN_ERR_UNSUPPORTED;
  return GDN_OK;
}

gdn::ConvArgs conv_args(const gdn_conv_dims* d) {
  gdn::ConvArgs p;
  p.x = nullptr; p.w = nullptr; p.bias = nullptr; p.pool = nullptr; p.idx = nullptr;
  p.prev_x = nullptr; p.prev_len = nullptr; p.y = nullptr;
  p.B = d->batch; p.T = d->T; p.D = d->channels; p.K = d->width; p.P = d->pool_slots; p.T_prev = 0;
  p.write_back = 0; p.activation = d->activation;
  return p;
}

// Records of the prefill workspace: chunk j of sequence r takes record
// floor(cu[r] / 16) + j + r, below floor(N / 16) + B for N tokens.
int64_t prefill_records(const gdn_dims* d, int64_t num_tokens) { return num_tokens / 16 + d->batch; }

// Segment length of the chunk chain, as log2 of its tokens. The chain of one (sequence,
// v-head, 16 value columns) is a state wave and an output wave; a chunk step keeps a SIMD
// busy (two chains on one SIMD take twice as long per step), so splitting sequences into
// segments, whose maps are composed afterwards, pays only when those waves leave most of
// the chip's 1024 SIMDs idle. Then segments are sized so that about 2048 waves run (one
// 16384-token prompt with 8 v-heads: 16 segments; 4096 waves, 32 segments, and 1024
// waves, 8 segments, measured 8 % and 6 % slower); else a
// segment is longer than any sequence (N < 2^shift: every sequence is one segment, and
// segment ids are the row numbers, with no gaps in the grid).
int32_t prefill_seg_shift(const gdn_dims* d, int64_t num_tokens) {
  int32_t whole = 8;
  while ((int64_t(1) << whole) <= num_tokens) ++whole;
  const int64_t waves = int64_t(d->batch) * d->num_v_heads * (d->d_v / 16) * 2;
  if (waves >= 512) return whole;
  const int64_t target = num_tokens * d->num_v_heads * (d->d_v / 16) * 2 / 2048;  // tokens per segment
  int32_t shift = 8;
  while ((int64_t(1) << shift) < target) ++shift;
  return std::min(shift, whole);
}

// Segments of the chunk chain: segment g of sequence r takes id floor(cu[r] / 2^shift) + g + r.
int64_t prefill_segments(const gdn_dims* d, int64_t num_tokens) {
  return (num_tokens >> prefill_seg_shift(d, num_tokens)) + d->batch;
}

size_t prefill_workspace(const gdn_dims* d, int64_t num_tokens) {
  const int64_t segs = prefill_segments(d, num_tokens);
  return size_t(gdn::prefill_records_bytes(prefill_records(d, num_tokens), d->num_k_heads, d->num_v_heads) +
                gdn::prefill_table_bytes(segs) + segs * d->num_v_heads * gdn::prefill_slot_bytes(d->d_v));
}

gdn_status check_prefill(const gdn_dims* d, int64_t num_tokens) {
  const gdn_status s = check_dims(d, false);
  if (s != GDN_OK) return s;
  if (num_tokens < 0) return GDN_ERR_SHAPE;
  if (d->io_dtype != GDN_DTYPE_BF16) return GDN_ERR_UNSUPPORTED;  // the matrix cores take bf16 tokens
  if (d->d_k != 128 || d->d_v % 32 != 0) return GDN_ERR_UNSUPPORTED;
  // 32-bit byte offsets inside the token tensors
  if (num_tokens * d->num_v_heads * d->d_v >= (int64_t(1) << 30) ||
      num_tokens * d->num_k_heads * d->d_k >= (int64_t(1) << 30))
    return GDN_ERR_UNSUPPORTED;
  return GDN_OK;
}

// Pointer and alignment checks of a prefill call (the workspace aside).
gdn_status check_prefill_ptrs(const gdn_io* io, const void* pool, const int32_t* idx, const int32_t* cu,
                              const int32_t* fresh) {
  if (!io || !io->q || !io->k || !io->v || !io->a || !io->b || !io->A_log || !io->dt_bias || !io->o || !pool ||
      !idx || !cu)
    return GDN_ERR_NULL;
  if (!aligned(io->q, 16) || !aligned(io->k, 16) || !aligned(io->v, 16) || !aligned(io->o, 16) ||
      !aligned(pool, 16) || !aligned(io->a, 2) || !aligned(io->b, 2) || !aligned(io->A_log, 4) ||
      !aligned(io->dt_bias, 4) || !aligned(idx, 4) || !aligned(cu, 4) || (fresh && !aligned(fresh, 4)))
    return GDN_ERR_ALIGN;
  return GDN_OK;
}

// Launch of a checked prefill call with a workspace of sufficient size.
gdn_status run_prefill(const gdn_dims* dims, const gdn_io* io, void* state_pool, const int32_t* state_indices,
                       const int32_t* cu_seqlens, const int32_t* fresh, int64_t num_tokens, void* workspace,
                       void* stream) {
  const int64_t records = prefill_records(dims, num_tokens);
  gdn::PrefillArgs p;
  p.q = io->q; p.k = io->k; p.v = io->v; p.a = io->a; p.b = io->b;
  p.A_log = io->A_log; p.dt_bias = io->dt_bias; p.o = io->o;
  p.pool = state_pool; p.idx = state_indices; p.fresh = fresh; p.cu = cu_seqlens;
  p.work = workspace; p.records = records;
  p.segments = prefill_segments(dims, num_tokens); p.tokens = num_tokens;
  p.seg_shift = prefill_seg_shift(dims, num_tokens);
  p.B = dims->batch; p.Hk = dims->num_k_heads; p.Hv = dims->num_v_heads; p.DV = dims->d_v;
  p.P = dims->pool_slots; p.G = dims->num_v_heads / dims->num_k_heads;
  p.scale = dims->scale; p.eps = dims->l2norm_eps;
  const hipError_t e = gdn::launch_prefill(static_cast<Dt>(dims->state_dtype), p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

}  // namespace

extern "C" {

gdn_status gdn_decode(const gdn_dims* dims, const gdn_io* io, void* state_pool,
                      const int32_t* state_indices, void* stream) {
  const gdn_status s = check_dims(dims, true);
  if (s != GDN_OK) return s;
  if (dims->T != 1) return GDN_ERR_SHAPE;
  return run_recurrent(dims, io, state_pool, state_indices, nullptr, 0, 1, nullptr, stream);
}

gdn_status gdn_verify(const gdn_dims* dims, const gdn_io* io, void* state_pool,
                      const int32_t* state_indices, void* inter_cache, int32_t cache_T,
                      int32_t write_final, const int32_t* prev_accept_len, void* stream) {
  const gdn_status s = check_dims(dims, true);
  if (s != GDN_OK) return s;
  return run_recurrent(dims, io, state_pool, state_indices, inter_cache, cache_T, write_final,
                       prev_accept_len, stream);
}

gdn_status gdn_verify_gated(const gdn_dims* dims, const gdn_io* io, const gdn_out_gate* gate, void* state_pool,
                            const int32_t* state_indices, void* inter_cache, int32_t cache_T, int32_t write_final,
                            const int32_t* prev_accept_len, void* stream) {
  const gdn_status s = check_dims(dims, true);
  if (s != GDN_OK) return s;
  if (!gate) return GDN_ERR_NULL;
  return run_recurrent(dims, io, state_pool, state_indices, inter_cache, cache_T, write_final,
                       prev_accept_len, stream, gate);
}


gdn_status gdn_prefill_workspace_bytes(const gdn_dims* dims, int64_t num_tokens, size_t* bytes) {
  const gdn_status s = check_prefill(dims, num_tokens);
  if (s != GDN_OK) return s;
  if (!bytes) return GDN_ERR_NULL;
  *bytes = prefill_workspace(dims, num_tokens);
  return GDN_OK;
}

gdn_status gdn_prefill(const gdn_dims* dims, const gdn_io* io, void* state_pool, const int32_t* state_indices,
                       const int32_t* cu_seqlens, const int32_t* fresh, int64_t num_tokens, void* workspace,
                       size_t workspace_bytes, void* stream) {
  gdn_status s = check_prefill(dims, num_tokens);
  if (s != GDN_OK) return s;
  if (dims->batch == 0) return GDN_OK;
  if (workspace_bytes < prefill_workspace(dims, num_tokens)) return GDN_ERR_SHAPE;
  if ((s = check_prefill_ptrs(io, state_pool, state_indices, cu_seqlens, fresh)) != GDN_OK) return s;
  if (!workspace) return GDN_ERR_NULL;
  if (!aligned(workspace, 256)) return GDN_ERR_ALIGN;
  return run_prefill(dims, io, state_pool, state_indices, cu_seqlens, fresh, num_tokens, workspace, stream);
}

gdn_status gdn_prefill_noalloc(const gdn_dims* dims, const gdn_io* io, void* state_pool,
                               const int32_t* state_indices, const int32_t* cu_seqlens, const int32_t* fresh,
                               int64_t num_tokens, void* stream) {
  gdn_status s = check_prefill(dims, num_tokens);
  if (s != GDN_OK) return s;
  if (prefill_workspace(dims, num_tokens) > GDN_PREFILL_NOALLOC_BYTES) return GDN_ERR_TOO_LARGE;
  if (dims->batch == 0) return GDN_OK;
  if ((s = check_prefill_ptrs(io, state_pool, state_indices, cu_seqlens, fresh)) != GDN_OK) return s;
  // the fixed array of the GPU the kernels run on: the stream's, or the current one
  int device = 0;
  const hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &device) : hipGetDevice(&device);
  if (e != hipSuccess) return GDN_ERR_LAUNCH;
  void* work = nullptr;
  if (gdn::noalloc_scratch(device, &work) != hipSuccess) return GDN_ERR_LAUNCH;
  return run_prefill(dims, io, state_pool, state_indices, cu_seqlens, fresh, num_tokens, work, stream);
}

gdn_status gdn_commit(const gdn_dims* dims, const void* inter_cache, int32_t cache_T,
                      const int32_t* state_indices, const int32_t* accept_len, void* state_pool,
                      void* stream) {
  const gdn_status s = check_dims(dims, false);
  if (s != GDN_OK) return s;
  if (cache_T < 1) return GDN_ERR_SHAPE;
  if (dims->batch == 0) return GDN_OK;
  if (!inter_cache || !state_indices || !accept_len || !state_pool) return GDN_ERR_NULL;
  if (!aligned(inter_cache, 16) || !aligned(state_pool, 16) || !aligned(state_indices, 4) ||
      !aligned(accept_len, 4))
    return GDN_ERR_ALIGN;
  gdn::CommitArgs p;
  p.cache = inter_cache; p.pool = state_pool; p.idx = state_indices; p.accept = accept_len;
  p.B = dims->batch; p.Hv = dims->num_v_heads; p.P = dims->pool_slots; p.cache_T = cache_T;
  p.tile_bytes = int64_t(dims->d_k) * dims->d_v * int64_t(dsize(dims->state_dtype));
  const int64_t per_block = int64_t(gdn::kThreads) * gdn::kCommitChunksPerThread * 16;
  p.blocks_per_tile = int32_t((p.tile_bytes + per_block - 1) / per_block);
  const hipError_t e = gdn::launch_commit(p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

gdn_status gdn_verify_replay(const gdn_dims* dims, const gdn_io* io, void* state_pool,
                             const int32_t* state_indices, const gdn_tokens* replay,
                             const int32_t* replay_len, int32_t commit, void* stream) {
  gdn_status s = check_dims(dims, true);
  if (s != GDN_OK) return s;
  if (replay && replay->T_src < 1) return GDN_ERR_SHAPE;
  if (replay && dims->T + replay->T_src > GDN_MAX_T) return GDN_ERR_UNSUPPORTED;
  if (dims->batch == 0) return GDN_OK;
  if (!io || !io->q || !io->k || !io->v || !io->a || !io->b || !io->A_log || !io->dt_bias || !io->o ||
      !state_pool || !state_indices)
    return GDN_ERR_NULL;
  if ((s = check_replay(dims, replay, replay_len)) != GDN_OK) return s;
  const uintptr_t isz = dsize(dims->io_dtype);
  if (!aligned(io->q, 16) || !aligned(io->k, 16) || !aligned(io->v, 16) || !aligned(io->o, 16) ||
      !aligned(state_pool, 16) || !aligned(io->a, isz) || !aligned(io->b, isz) || !aligned(io->A_log, 4) ||
      !aligned(io->dt_bias, 4) || !aligned(state_indices, 4))
    return GDN_ERR_ALIGN;
  gdn::RecurrentArgs p;
  p.q = io->q; p.k = io->k; p.v = io->v; p.a = io->a; p.b = io->b;
  p.A_log = io->A_log; p.dt_bias = io->dt_bias; p.o = io->o;
  p.pool = state_pool; p.idx = state_indices; p.cache = nullptr; p.prev_accept = nullptr;
  p.B = dims->batch; p.T = dims->T; p.Hk = dims->num_k_heads; p.Hv = dims->num_v_heads;
  p.DK = dims->d_k; p.DV = dims->d_v; p.P = dims->pool_slots; p.cache_T = 0;
  p.G = dims->num_v_heads / dims->num_k_heads;
  p.write_final = 0;
  p.scale = dims->scale; p.eps = dims->l2norm_eps;
  set_replay(p, replay, replay_len, commit);
  p.z = nullptr; p.gw = nullptr; p.geps = 0.f;
  const hipError_t e = gdn::launch_recurrent(static_cast<Dt>(dims->state_dtype), static_cast<Dt>(dims->io_dtype),
                                             1, 1, pick_nt_loads(dims, true), p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

gdn_status gdn_commit_replay(const gdn_dims* dims, const float* A_log, const float* dt_bias,
                             void* state_pool, const int32_t* state_indices,
                             const gdn_tokens* replay, const int32_t* replay_len, void* stream) {
  gdn_status s = check_dims(dims, false);
  if (s != GDN_OK) return s;
  if (replay && replay->T_src < 1) return GDN_ERR_SHAPE;
  if (replay && replay->T_src > GDN_MAX_T) return GDN_ERR_UNSUPPORTED;
  if (dims->batch == 0) return GDN_OK;
  if (!A_log || !dt_bias || !state_pool || !state_indices) return GDN_ERR_NULL;
  if ((s = check_replay(dims, replay, replay_len)) != GDN_OK) return s;
  if (!aligned(state_pool, 16) || !aligned(A_log, 4) || !aligned(dt_bias, 4) || !aligned(state_indices, 4))
    return GDN_ERR_ALIGN;
  gdn::RecurrentArgs p;
  p.q = p.k = p.v = p.a = p.b = nullptr;
  p.A_log = A_log; p.dt_bias = dt_bias; p.o = nullptr;
  p.pool = state_pool; p.idx = state_indices; p.cache = nullptr; p.prev_accept = nullptr;
  p.B = dims->batch; p.T = 0; p.Hk = dims->num_k_heads; p.Hv = dims->num_v_heads;
  p.DK = dims->d_k; p.DV = dims->d_v; p.P = dims->pool_slots; p.cache_T = 0;
  p.G = dims->num_v_heads / dims->num_k_heads;
  p.write_final = 0;
  p.scale = dims->scale; p.eps = dims->l2norm_eps;
  set_replay(p, replay, replay_len, 1);
  p.z = nullptr; p.gw = nullptr; p.geps = 0.f;
  const hipError_t e = gdn::launch_recurrent(static_cast<Dt>(dims->state_dtype), static_cast<Dt>(dims->io_dtype),
                                             1, 2, pick_nt_loads(dims, true), p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

gdn_status gdn_conv_update(const gdn_conv_dims* dims, const void* x, const float* weight, const float* bias,
                           void* conv_pool, const int32_t* state_indices, const void* prev_x, int32_t T_prev,
                           const int32_t* prev_len, void* y, int32_t write_back, void* stream) {
  gdn_status s = check_conv_dims(dims);
  if (s != GDN_OK) return s;
  if (prev_x && (T_prev < 1 || T_prev > GDN_MAX_T)) return GDN_ERR_SHAPE;
  if (dims->batch == 0) return GDN_OK;
  if (!x || !weight || !conv_pool || !state_indices || !y || (prev_x && !prev_len)) return GDN_ERR_NULL;
  if (!aligned(x, 16) || !aligned(y, 16) || !aligned(conv_pool, 16) || !aligned(weight, 16) ||
      (bias && !aligned(bias, 16)) || (prev_x && !aligned(prev_x, 16)) || !aligned(state_indices, 4) ||
      (prev_len && !aligned(prev_len, 4)))
    return GDN_ERR_ALIGN;
  gdn::ConvArgs p = conv_args(dims);
  p.x = x; p.w = weight; p.bias = bias; p.pool = conv_pool; p.idx = state_indices; p.y = y;
  p.prev_x = prev_x; p.prev_len = prev_x ? prev_len : nullptr; p.T_prev = prev_x ? T_prev : 0;
  p.write_back = write_back ? 1 : 0;
  const hipError_t e = gdn::launch_conv(static_cast<Dt>(dims->dtype), false, p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

gdn_status gdn_conv_commit(const gdn_conv_dims* dims, const void* x, void* conv_pool,
                           const int32_t* state_indices, const int32_t* accept_len, void* stream) {
  gdn_status s = check_conv_dims(dims);
  if (s != GDN_OK) return s;
  if (dims->batch == 0) return GDN_OK;
  if (!x || !conv_pool || !state_indices || !accept_len) return GDN_ERR_NULL;
  if (!aligned(x, 16) || !aligned(conv_pool, 16) || !aligned(state_indices, 4) || !aligned(accept_len, 4))
    return GDN_ERR_ALIGN;
  gdn::ConvArgs p = conv_args(dims);
  p.pool = conv_pool; p.idx = state_indices;
  p.prev_x = x; p.prev_len = accept_len; p.T_prev = dims->T;
  const hipError_t e = gdn::launch_conv(static_cast<Dt>(dims->dtype), true, p, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDN_OK : GDN_ERR_LAUNCH;
}

const char* gdn_status_string(gdn_status status) {
  switch (status) {
    case GDN_OK: return "GDN_OK: success";
    case GDN_ERR_NULL: return "GDN_ERR_NULL: a required pointer is NULL";
    case GDN_ERR_SHAPE: return "GDN_ERR_SHAPE: inconsistent or negative sizes";
    case GDN_ERR_DTYPE: return "GDN_ERR_DTYPE: unknown dtype";
    case GDN_ERR_ALIGN: return "GDN_ERR_ALIGN: a pointer is not aligned as required";
    case GDN_ERR_UNSUPPORTED: return "GDN_ERR_UNSUPPORTED: geometry outside the supported set";
    case GDN_ERR_LAUNCH: return "GDN_ERR_LAUNCH: kernel launch failed";
    case GDN_ERR_TOO_LARGE:
      return "GDN_ERR_TOO_LARGE: the call needs more than the library's fixed prefill array";
  }
  return "GDN: unknown status";
}

int32_t gdn_abi_version(void) { return GDN_ABI_VERSION; }

}  // extern "C"
