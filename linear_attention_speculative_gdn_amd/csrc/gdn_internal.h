// gdn_internal.h -- launch descriptors shared by the host entry points (gdn_api.cpp)
// and the gfx950 kernels (gdn_kernels.hip, gdn_conv.hip, gdn_prefill.hip). Not part of
// the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace gdn {

enum class Dt : int { F32 = 0, BF16 = 1 };

// One launch of the recurrent kernel (decode, verify, verify with fused commit).
struct RecurrentArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* a;
  const void* b;
  const float* A_log;
  const float* dt_bias;
  void* o;
  void* pool;
  const int32_t* idx;
  void* cache;                 // nullptr: no intermediate states
  const int32_t* prev_accept;  // nullptr: no fused commit
  int32_t B, T, Hk, Hv, DK, DV, P, cache_T;
  int32_t G;                   // v-heads per k-head (Hv / Hk)
  int32_t write_final;
  float scale, eps;
  // cached replay (modes 1 and 2)
  const void* rk;              // [B][rT][Hk][DK] io dtype
  const void* rv;              // [B][rT][Hv][DV]
  const void* ra;              // [B][rT][Hv]
  const void* rb;              // [B][rT][Hv]
  const int32_t* rlen;         // [B] tokens to replay per row
  int32_t rT;                  // tokens per row in the replay arrays (>= 1)
  int32_t rcommit;             // 1: write the replayed state to the slot
  // gated-norm output epilogue (mode 3)
  const void* z;               // [B][T][Hv][DV] io dtype
  const float* gw;             // [DV] norm weights
  float geps;                  // RMS epsilon
};

// One launch of the accepted-prefix commit copy.
struct CommitArgs {
  const void* cache;
  void* pool;
  const int32_t* idx;
  const int32_t* accept;
  int32_t B, Hv, P, cache_T;
  int32_t blocks_per_tile;
  int64_t tile_bytes;
};

// shape: 1 = one value row per lane, 4 waves; 2 = two rows per lane, 4 waves;
// 12 = one row per lane, 2 waves; 14 = one row per lane, 8 waves; 44 = four rows per lane,
// 4 waves (a whole head of d_v = 128 per workgroup) (d_k = 128 only).
// mode: 0 decode / verify, 1 cached-replay verify, 2 replay commit, 3 decode / verify
// with the gated-norm output epilogue (modes 1-3 use their own fixed shapes).
// Mode 3 needs d_v <= 256 for d_k <= 64 and d_v <= 128 for d_k >= 128.
// nt_loads: read the initial state with nontemporal loads (d_k = 128, shape 1 and the
// fixed shapes of modes 1-3; ignored elsewhere).
hipError_t launch_recurrent(Dt state, Dt io, int shape, int mode, bool nt_loads, const RecurrentArgs& p,
                            hipStream_t stream);
hipError_t launch_commit(const CommitArgs& p, hipStream_t stream);

// One launch of the short causal convolution (update, or commit only).
struct ConvArgs {
  const void* x;               // [B][T][D] io dtype (commit only: the tokens to commit)
  const float* w;              // [K][D] taps
  const float* bias;           // [D] or nullptr
  void* pool;                  // [P][K-1][D] io dtype
  const int32_t* idx;          // [B]
  const void* prev_x;          // [B][T_prev][D] or nullptr (commit only: = x)
  const int32_t* prev_len;     // [B] tokens of prev_x to commit (nullptr: none)
  void* y;                     // [B][T][D] io dtype (unused for commit only)
  int32_t B, T, D, K, P, T_prev;
  int32_t write_back;          // 1: store the state advanced over all T tokens
  int32_t activation;          // 0: identity, 1: SiLU
};

// commit_only: advance each valid slot over prev_len tokens of prev_x and stop.
hipError_t launch_conv(Dt io, bool commit_only, const ConvArgs& p, hipStream_t stream);

// The prefill workspace holds, per 16-token chunk, one record per v-head (the products
// that involve the gates) and then one per k-head (its transposed keys, shared
// by the k-head's v-heads). Both sizes are multiples of 256 bytes.
constexpr int kPrefillRecordBytes = 5376;
constexpr int kPrefillKeyRecordBytes = 4096;
// The chunk chain runs in segments of 2^seg_shift tokens (seg_shift >= 8); after the
// records the workspace holds a table of segment ids and, per (segment, v-head), a slot of
// a d_k x d_v fp32 state and a d_k x d_k bf16 map.
constexpr int64_t prefill_records_bytes(int64_t records, int Hk, int Hv) {
  return records * (int64_t(Hv) * kPrefillRecordBytes + int64_t(Hk) * kPrefillKeyRecordBytes);
}
constexpr int64_t prefill_table_bytes(int64_t segments) { return (segments * 4 + 255) / 256 * 256; }
constexpr int64_t prefill_slot_bytes(int dv) { return int64_t(dv) * 128 * 4 + 128 * 128 * 2; }

// One launch of the chunked prefill (bf16 io, d_k = 128, d_v a multiple of 32).
struct PrefillArgs {
  const void* q;               // [N][Hk][128]
  const void* k;
  const void* v;               // [N][Hv][DV]
  const void* a;               // [N][Hv]
  const void* b;
  const float* A_log;          // [Hv]
  const float* dt_bias;
  void* o;                     // [N][Hv][DV]
  void* pool;                  // [P][Hv][DV][128] state dtype
  const int32_t* idx;          // [B]
  const int32_t* fresh;        // [B] or nullptr
  const int32_t* cu;           // [B+1] token offsets
  void* work;                  // [records][Hv] records of kPrefillRecordBytes, then
                               // [records][Hk] of kPrefillKeyRecordBytes
  int64_t records;             // floor(N / 16) + B for N tokens
  int64_t segments;            // floor(N / 2^seg_shift) + B
  int64_t tokens;              // N
  int32_t seg_shift;           // log2 of the tokens per segment of the chunk chain
  int32_t B, Hk, Hv, DV, P, G;
  float scale, eps;
};

hipError_t launch_prefill(Dt state, const PrefillArgs& p, hipStream_t stream);

// Device address of the library's fixed prefill array on `device` (gdn_noalloc.hip),
// resolved with hipGetSymbolAddress on the first call for that device.
hipError_t noalloc_scratch(int device, void** out);

// Commit launch: 1024-thread workgroups of 4 16-byte chunks per thread (one tile of up
// to 64 KiB per workgroup). Measured against 256 threads: verify + commit on the MTP T=4
// bf16 batch 22.5 -> 21.9 us, on the T=4 fp32 B=256 batch 674 -> 662 us; 8 chunks per
// thread, 64-thread workgroups and plain (not nontemporal) loads were slower.
constexpr int kCommitChunksPerThread = 4;
constexpr int kThreads = 1024;

}  // namespace gdn
