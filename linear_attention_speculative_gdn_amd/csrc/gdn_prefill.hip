// gdn_prefill.hip -- gfx950 chunked prefill of the Gated DeltaNet state from pooled initial
// states, on the bf16 matrix cores, in two passes.
//
// The operation: TensorRT-LLM PR 20937, Per-File QA Perspective -- the chunked gated
// delta rule prefill with a bf16 state and an initial-state mask that zeroes fresh
// states. Per sequence r and v-head h the state starts at pool[idx[r]] (zero when
// fresh[r]), every token runs through the gated delta rule, o is written for every token
// and the final state is stored back to the slot.
//
// Chunked form (C tokens per chunk, S_0 the state at the chunk start, Gam_t the product
// of the chunk's decays up to token t, k^ and q^ the L2-normalised keys and queries):
//     A_ts = beta_t (Gam_t / Gam_s) k^_t . k^_s  (s < t),   Tm = (I + A)^-1
//     U = Tm diag(beta) V - Tm diag(beta Gam) K^ S_0          (the per-token deltas)
//     O = scale (diag(Gam) Q^ S_0 + (M o Q^ K^T) U),  M_ts = Gam_t / Gam_s  (s <= t)
//     S_C = Gam_C S_0 + K^T diag(Gam_C / Gam) U
// which equals the token-by-token recurrence up to rounding. Every product is a dense
// contraction, on the 16x16x16 and 16x16x32 bf16 matrix-core products with fp32
// accumulation.
//
// Design for gfx950:
// - Pass 1 (chunk_kernel) computes, for every (chunk, v-head) in parallel, everything that
//   does not depend on the state -- W = Tm diag(beta Gam rk) K, Tm diag(beta), the output
//   mask P, K^T and the per-token factors -- into workspace records. That is most of a
//   chunk's instructions, and none of it is sequential. K^T does not depend on the gates:
//   it goes to one record per k-head, written by its first v-head, which the other
//   v-heads of the group read too.
// - Pass 2 walks each sequence's chunks in order with the state in MFMA accumulators:
//   U~ = Tm diag(beta) V, W S_0, Q S_0, P U and the state update only. group_chain_kernel
//   runs two or four chains per workgroup on records one wave copies into LDS ahead of
//   use, for whole sequences or in segments whose maps are composed; scan_kernel's waves
//   of two column tiles serve wide grids of whole sequences whose d_v is not a multiple
//   of 64, loading their records themselves.
// - One chain per (sequence or segment, v-head, block of 16 value columns): columns are
//   independent given the record. A 16 x 16 accumulator tile holds, per lane, four
//   consecutive rows of one column -- the B-operand layout -- so S_0 feeds W S_0 after a
//   bf16 conversion in registers, and goes to the output product through LDS.
// - Keys and queries enter the products as their stored bf16 values; norms, gates and
//   decays are fp32 diagonal scalings of the 16 x 16 chunk matrices.
// - Records are numbered floor(cu[r] / 16) + j + r for chunk j of sequence r: distinct, and
//   below floor(N / 16) + B, with no prefix sum over the sequences. Both passes bound every
//   record access by the workspace's capacity.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "../../include/gdn.h"
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16v8 __attribute__((ext_vector_type(8)));

constexpr int kC = 16;        // tokens per chunk
constexpr int kDK = 128;      // key dimension
constexpr int kKT = kDK / 16; // 16-row tiles of the key dimension

// Workspace records: byte offsets. Every matrix is stored in the lane layout of the
// matrix-core operand that reads it, so a pass-2 lane fetches its part with 16-byte loads
// of contiguous 1 KiB blocks. Per (chunk, v-head), kPrefillRecordBytes in total:
constexpr int kRecW = 0;       // -W, A operand of 16x16x32: [32-key block m][lane][8 bf16]; for a chain in
                               // segments the 16 x 16 factor -Tm diag(beta Gam rk) instead, A operand of
                               // 16x16x16: [lane][4 bf16] (the chain forms -W from it and K^T)
constexpr int kRecTP = 4096;   // Tm diag(beta) and P = M o (rq rk) Q K^T, A operands: [lane][2 x 4 bf16]
constexpr int kRecF = 5120;    // f_t = rk_t Gam_C / Gam_t [16] fp32
constexpr int kRecGQ = 5184;   // Gam_t rq_t [16] fp32
constexpr int kRecGC = 5248;   // Gam_C fp32
static_assert(kRecGC + 4 <= kPrefillRecordBytes && kPrefillRecordBytes % 256 == 0, "record layout");
// per (chunk, k-head), kPrefillKeyRecordBytes in total, after all the v-head records:
constexpr int kKeyKT = 0;      // K^T, A operand of 16x16x16, tiles 2m, 2m+1: [m][lane][2 x 4 bf16]
static_assert(kKeyKT + 4096 == kPrefillKeyRecordBytes, "key record layout");

// The chain's output product (Q S_0)^T = S_0^T Q^T takes its queries straight from the q
// tensor: the 32 keys 32 m .. 32 m + 31 of a 16x16x32 product sit as key 32 m + 8 g + e in
// slot e of lane group g, so a lane's eight queries are 16 consecutive bytes of a row. The
// state wave hands S_0 over in the same key order (the products with -W keep theirs).
// s16x4 (4 bf16) of state tile kt (rows 16 kt + 4 l4 + i, column l16) into the handover
// block of keys 32 (kt / 2) .. + 31, as the B operand in that key order
__device__ __forceinline__ void hand_tile(s16x8* blk, int kt, int l16, int l4, const s16x4& x) {
  char* b = reinterpret_cast<char*>(blk);
  *reinterpret_cast<s16x4*>(b + 16 * (l16 + 16 * (2 * (kt & 1) + (l4 >> 1))) + 8 * (l4 & 1)) = x;
}

__device__ __forceinline__ f32x4 mfma(const s16x4& a, const s16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

// 16x16x32: A lane (row l16, group l4) slot e pairs with B lane (column l16, group l4)
// slot e. Any assignment of the 32 contraction indices to (group, slot) that both
// operands share gives the same product.
__device__ __forceinline__ f32x4 mfma32(const s16x8& a, const s16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16v8, a), __builtin_bit_cast(bf16v8, b), c, 0,
                                                  0, 0);
}

__device__ __forceinline__ s16x8 cat8(const s16x4& lo, const s16x4& hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ s16x4 bf16x4(float a, float b, float c, float d) {
  const uint64_t lo = pack_bf16x2(a, b), hi = pack_bf16x2(c, d);
  return __builtin_bit_cast(s16x4, (hi << 32) | lo);
}

__device__ __forceinline__ float bf(uint16_t x) { return __uint_as_float(uint32_t(x) << 16); }

__device__ __forceinline__ uint16_t to_bf(float x) { return uint16_t(pack_bf16x2(x, 0.f)); }

// Phase boundary of a one-wave workgroup: a wave's LDS operations complete in order, so
// it is enough that its own LDS accesses have retired (and that the compiler does not move
// memory accesses across). A __syncthreads() here would also wait for global loads still
// in flight.
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// four bf16 of one row at column c (8-byte aligned)
__device__ __forceinline__ s16x4 ld4(const uint16_t* base, int row, int stride, int c) {
  return *reinterpret_cast<const s16x4*>(base + row * stride + c);
}

__device__ __forceinline__ int64_t record_id(int32_t cu_r, int row, int j) { return (cu_r >> 4) + j + row; }

// Segments of 2^seg_shift tokens (a power of two >= 256, chosen on the host):
// segment g of sequence r takes id floor(cu[r] / 2^seg_shift) + g + r, distinct and below
// floor(N / 2^seg_shift) + B, like the records. An empty sequence has one.
__device__ __forceinline__ int64_t segment_id(const PrefillArgs& p, int32_t cu_r, int row, int g) {
  return (cu_r >> p.seg_shift) + g + row;
}
__device__ __forceinline__ int seg_chunks(const PrefillArgs& p) { return 1 << (p.seg_shift - 4); }
__device__ __forceinline__ int seg_count(const PrefillArgs& p, int nchunks) {
  return max(1, (nchunks + seg_chunks(p) - 1) >> (p.seg_shift - 4));
}
// after the records: the segment table ([segments] int32: (g << 16) | r, or -1), then a
// slot per (segment, v-head)
__device__ __forceinline__ int32_t* segment_table(const PrefillArgs& p) {
  return reinterpret_cast<int32_t*>(static_cast<char*>(p.work) + prefill_records_bytes(p.records, p.Hk, p.Hv));
}
__device__ __forceinline__ char* segment_slot(const PrefillArgs& p, int64_t sid, int h) {
  return reinterpret_cast<char*>(segment_table(p)) + prefill_table_bytes(p.segments) +
         (sid * p.Hv + h) * prefill_slot_bytes(p.DV);
}

// record of (chunk record rid, v-head h) and of (rid, k-head kh)
__device__ __forceinline__ char* head_record(const PrefillArgs& p, int64_t rid, int h) {
  return static_cast<char*>(p.work) + (rid * p.Hv + h) * kPrefillRecordBytes;
}
__device__ __forceinline__ char* key_record(const PrefillArgs& p, int64_t rid, int kh) {
  return static_cast<char*>(p.work) + p.records * p.Hv * kPrefillRecordBytes + (rid * p.Hk + kh) * kPrefillKeyRecordBytes;
}

// B operand of the 16x16 identity: multiplying an A-layout tile X (lane (row r, group g)
// holding X[r][4g .. 4g+3]) by it gives X itself in the accumulator layout (lane (g, n)
// holding X[4g .. 4g+3][n]), i.e. X^T in the A layout: an exact transpose through the
// matrix core (each sum has a single 1.0 * x term).
__device__ __forceinline__ s16x4 identity_b(int l16, int l4) {
  const int e = l16 - 4 * l4;  // the lane's 1.0, if in its four rows
  return s16x4{short(e == 0 ? 0x3F80 : 0), short(e == 1 ? 0x3F80 : 0), short(e == 2 ? 0x3F80 : 0),
               short(e == 3 ? 0x3F80 : 0)};
}

__device__ __forceinline__ s16x4 bf16x4(const f32x4& x) { return bf16x4(x.x, x.y, x.z, x.w); }

__device__ __forceinline__ s16x4 lo4(const s16x8& x) { return __builtin_shufflevector(x, x, 0, 1, 2, 3); }
__device__ __forceinline__ s16x4 hi4(const s16x8& x) { return __builtin_shufflevector(x, x, 4, 5, 6, 7); }

// ============================================================ pass 1: chunk records
struct __attribute__((aligned(16))) ChunkLds {
  float a[kC * kC];        // A (fp32) for the triangular solve, by column: a[s * kC + t] = A_ts
  uint16_t tw[kC * kC];    // -Tm diag(beta Gam rk), bf16
  uint16_t tv[kC * kC];    // Tm diag(beta), bf16
};

// Pass 1 is bound by vector-instruction issue and memory latency (about 1200 instructions
// per chunk and v-head), so the gates, decay ratios and norms use the hardware's approximate
// exp, log, reciprocal and reciprocal square root (a few ulp; every product it feeds is
// rounded to bf16): 1500 instructions and 35.7 us with the library functions on 8 x 2048
// tokens, 33.9 us then.
// One wave per (chunk stride x, group of VH v-heads, sequence); wave x handles chunks x, x + the
// stride count, ... of its sequence for VH v-heads of one k-head (WF: with -W's factor in its
// record; CHUNK_SLOW: the grid's order, below). Every product takes its
// operands straight from registers: keys and queries are loaded in the operand layout, K^T
// comes from the identity product, and W^T = K^T TW^T and (Q K^T)^T = K Q^T come out of the
// matrix core already in the layout their A operands need. LDS holds only the 16 x 16 solves.
// With VH = 2 the keys, queries, their norms, K K^T, K Q^T and K^T serve both v-heads, and
// the two triangular solves run side by side, one per 16 lanes.
template <int VH, bool WF, bool CHUNK_SLOW>
__global__ __launch_bounds__(64) void chunk_kernel(const PrefillArgs p) {
  __shared__ ChunkLds L[VH];
  // grid (chunk strides, head groups, sequences), or with CHUNK_SLOW (head groups, sequences,
  // chunk strides): the chunk index then varies slowest, so the waves that have a chunk are
  // dispatched before those past their sequence's end
  const int h0 = (CHUNK_SLOW ? blockIdx.x : blockIdx.y) * VH, row = CHUNK_SLOW ? blockIdx.y : blockIdx.z;
  const int x0 = CHUNK_SLOW ? blockIdx.z : blockIdx.x, nx = CHUNK_SLOW ? gridDim.z : gridDim.x;
  const int l = threadIdx.x, l16 = l & 15, l4 = l >> 4;
  const int32_t slot = p.idx[row];
  const int32_t t0 = p.cu[row], t1 = p.cu[row + 1];
  const int nchunks = (t1 - t0 + kC - 1) / kC;
  if (x0 == 0 && h0 == 0) {
    // the segment table entries from this sequence's first segment id up to the next
    // sequence's (to the table's end for the last; from 0 for the first): each entry is
    // written by exactly one wave
    const int64_t s0 = segment_id(p, t0, row, 0);
    const int64_t s1 = row + 1 < p.B ? segment_id(p, t1, row + 1, 0) : p.segments;
    const int nseg = seg_count(p, nchunks);
    int32_t* table = segment_table(p);
    for (int64_t sidx = (row == 0 ? 0 : s0) + l; sidx < min(s1, p.segments); sidx += 64) {
      const int64_t g = sidx - s0;
      table[sidx] = (g >= 0 && g < nseg) ? int32_t((g << 16) | row) : -1;
    }
  }
  if (slot < 0 || slot >= p.P) return;  // padding rows have no chunks to prepare
  const int kh = h0 / p.G;              // VH divides G: the group shares its k-head
  const bool key_writer = h0 == kh * p.G;  // the k-head's first v-head writes its key record
  const uint16_t* qg = static_cast<const uint16_t*>(p.q) + size_t(kh) * kDK + 4 * l4;
  const uint16_t* kg = static_cast<const uint16_t*>(p.k) + size_t(kh) * kDK + 4 * l4;
  const uint16_t* ag = static_cast<const uint16_t*>(p.a);
  const uint16_t* bg = static_cast<const uint16_t*>(p.b);
  float A_neg[VH], dtb[VH];
#pragma unroll
  for (int vh = 0; vh < VH; ++vh) {
    A_neg[vh] = -expf(p.A_log[h0 + vh]);
    dtb[vh] = p.dt_bias[h0 + vh];
  }
  const s16x4 eye = identity_b(l16, l4);
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  // the solving lanes: 16 per v-head, lane 16 vh + c solves column c of v-head vh
  const int sv = VH == 2 ? (l >> 4) & 1 : 0;

  for (int j = x0; j < nchunks; j += nx) {
    const int64_t rid = record_id(t0, row, j);
    if (rid >= p.records) return;  // workspace too small for the tokens: write nothing
    char* krec = key_record(p, rid, kh);
    const int cs = t0 + j * kC, n = min(kC, t1 - cs), last = t1 - 1;
    const bool live = l16 < n;  // token t = l16 of the chunk exists
    // ---- 1. keys and queries of token l16 in the A layout of 16x16x32 (lane (t, g):
    //         keys 32m + 4g .. +3 and 32m + 16 + 4g .. +3), zero past the end; gates
    s16x8 kA[kKT / 2], qA[kKT / 2];
    {
      const size_t rowoff = size_t(min(cs + l16, last)) * p.Hk * kDK;
#pragma unroll
      for (int m = 0; m < kKT / 2; ++m) {
        const s16x4 k0 = *reinterpret_cast<const s16x4*>(kg + rowoff + 32 * m);
        const s16x4 k1 = *reinterpret_cast<const s16x4*>(kg + rowoff + 32 * m + 16);
        const s16x4 q0 = *reinterpret_cast<const s16x4*>(qg + rowoff + 32 * m);
        const s16x4 q1 = *reinterpret_cast<const s16x4*>(qg + rowoff + 32 * m + 16);
        const s16x8 z8 = {0, 0, 0, 0, 0, 0, 0, 0};
        kA[m] = live ? cat8(k0, k1) : z8;
        qA[m] = live ? cat8(q0, q1) : z8;
      }
    }
    float G[VH], beta[VH];
#pragma unroll
    for (int vh = 0; vh < VH; ++vh) {
      const size_t tg = size_t(min(cs + l16, last)) * p.Hv + h0 + vh;
      const float x = bf(ag[tg]) + dtb[vh];
      G[vh] = live ? A_neg[vh] * (fmaxf(x, 0.f) + __logf(1.f + __expf(-fabsf(x)))) : 0.f;  // log-decay
      beta[vh] = live ? __fdividef(1.f, 1.f + __expf(-bf(bg[tg]))) : 0.f;
    }
#pragma unroll
    for (int d = 1; d < kC; d *= 2) {  // inclusive prefix sums over the 16 tokens (per group)
#pragma unroll
      for (int vh = 0; vh < VH; ++vh) {
        const float y = __shfl_up(G[vh], d, 16);
        if (l16 >= d) G[vh] += y;
      }
    }
    // ---- 2. inverse L2 norms of token l16: each group holds 32 of its 128 keys
    float sk = 0.f, sq = 0.f;
#pragma unroll
    for (int m = 0; m < kKT / 2; ++m)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float kv = bf(uint16_t(kA[m][e])), qv = bf(uint16_t(qA[m][e]));
        sk = fmaf(kv, kv, sk);
        sq = fmaf(qv, qv, sq);
      }
    sk += __shfl_xor(sk, 16); sk += __shfl_xor(sk, 32);
    sq += __shfl_xor(sq, 16); sq += __shfl_xor(sq, 32);
    const float rk = rsqrtf(sk + p.eps), rq = rsqrtf(sq + p.eps);
    // per-token values of the lane's four accumulator rows 4g + i (from group 0's lanes)
    float Gr[VH][4], br[VH][4], rkr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
      for (int vh = 0; vh < VH; ++vh) {
        Gr[vh][i] = __shfl(G[vh], 4 * l4 + i);
        br[vh][i] = __shfl(beta[vh], 4 * l4 + i);
      }
      rkr[i] = __shfl(rk, 4 * l4 + i);
    }
    // ---- 3. K K^T (rows t = 4g + i, column s = l16) and K Q^T = (Q K^T)^T (rows s,
    //         column t = l16: the A layout of Q K^T)
    f32x4 KK = zero4, KQ = zero4;
#pragma unroll
    for (int m = 0; m < kKT / 2; ++m) {
      KK = mfma32(kA[m], kA[m], KK);
      KQ = mfma32(kA[m], qA[m], KQ);
    }
    // A_ts = beta_t (Gam_t / Gam_s) rk_t rk_s k_t.k_s (s < t) -> LDS for the solve;
    // P_ts = (Gam_t / Gam_s) rq_t rk_s q_t.k_s (s <= t) in its A layout (t = l16, s = 4g + i)
    s16x4 pA[VH];
#pragma unroll
    for (int vh = 0; vh < VH; ++vh) {
      float pv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * l4 + i, s_ = l16;
        L[vh].a[s_ * kC + t] = (s_ < t) ? br[vh][i] * rkr[i] * rk * __expf(Gr[vh][i] - G[vh]) * KK[i] : 0.f;
        const int sp = 4 * l4 + i, tp = l16;
        pv[i] = (sp <= tp) ? rq * rkr[i] * __expf(G[vh] - Gr[vh][i]) * KQ[i] : 0.f;
      }
      pA[vh] = bf16x4(pv[0], pv[1], pv[2], pv[3]);
    }
    // ---- 5a. K^T tiles by the identity product (lane (g, key 16kt + l16): tokens 4g ..),
    //          and the k-head's record of K^T, before the solve: the keys and queries then
    //          need no registers across it
    s16x4 ktA[kKT];
#pragma unroll
    for (int m = 0; m < kKT / 2; ++m) {
      ktA[2 * m] = bf16x4(mfma(lo4(kA[m]), eye, zero4));
      ktA[2 * m + 1] = bf16x4(mfma(hi4(kA[m]), eye, zero4));
      if (key_writer) *reinterpret_cast<s16x8*>(krec + kKeyKT + m * 1024 + l * 16) = cat8(ktA[2 * m], ktA[2 * m + 1]);
    }
    lds_sync();
    // ---- 4. Tm = (I + A)^-1 by forward substitution, one column per lane (lanes < 16 VH),
    //         column-oriented: once x[s] is final it updates every later row at once. Column
    //         s + 1 of A (a broadcast LDS read per v-head) loads while step s computes, and
    //         no column earlier: read all ahead, A took registers that limited pass 1 to
    //         three waves per SIMD.
    if (l < kC * VH) {
      const int c = l16;
      const float* a_v = L[sv].a;
      float xs[kC];
#pragma unroll
      for (int t = 0; t < kC; ++t) xs[t] = (t == c) ? 1.f : 0.f;
      f32x4 cur[kC / 4], nxt[kC / 4];
#pragma unroll
      for (int q4 = 0; q4 < kC / 4; ++q4) cur[q4] = reinterpret_cast<const f32x4*>(a_v)[q4];
#pragma unroll
      for (int s_ = 0; s_ < kC - 1; ++s_) {
        if (s_ + 1 < kC - 1) {
#pragma unroll
          for (int q4 = (s_ + 2) / 4; q4 < kC / 4; ++q4)
            nxt[q4] = reinterpret_cast<const f32x4*>(a_v + (s_ + 1) * kC)[q4];
        }
#pragma unroll
        for (int t = s_ + 1; t < kC; ++t) xs[t] = fmaf(-cur[t / 4][t % 4], xs[s_], xs[t]);
        asm volatile("" ::: "memory");
#pragma unroll
        for (int q4 = 0; q4 < kC / 4; ++q4) cur[q4] = nxt[q4];
      }
      // lane 16 vh + c holds token c's values of v-head vh
      const float bs = (VH == 2 && sv) ? beta[VH - 1] : beta[0];
      const float Gs = (VH == 2 && sv) ? G[VH - 1] : G[0];
      const float cw = -bs * __expf(Gs) * rk, cv = bs;
      uint16_t* tw = L[sv].tw;
      uint16_t* tvp = L[sv].tv;
#pragma unroll
      for (int t = 0; t < kC; ++t) {
        tw[t * kC + c] = to_bf(xs[t] * cw);
        tvp[t * kC + c] = to_bf(xs[t] * cv);
      }
    }
    lds_sync();
    const float Gl0 = __shfl(G[0], kC - 1);
#pragma unroll
    for (int vh = 0; vh < VH; ++vh) {
      char* rec = head_record(p, rid, h0 + vh);
      const s16x4 twA = ld4(L[vh].tw, l16, kC, 4 * l4), tvA = ld4(L[vh].tv, l16, kC, 4 * l4);
      // ---- 5b. -W^T = K^T (-TW)^T gives -W in the A layout (lane (t, g): keys 16kt + 4g ..),
      //          stored by 32-key blocks; WF: the factor -TW alone, from which the chain
      //          forms the same -W with the same product (a eighth of the bytes)
      if constexpr (WF) {
        *reinterpret_cast<s16x4*>(rec + kRecW + l * 8) = twA;
      } else {
#pragma unroll
        for (int m = 0; m < kKT / 2; ++m) {
          const s16x4 w0 = bf16x4(mfma(ktA[2 * m], twA, zero4));
          const s16x4 w1 = bf16x4(mfma(ktA[2 * m + 1], twA, zero4));
          *reinterpret_cast<s16x8*>(rec + kRecW + m * 1024 + l * 16) = cat8(w0, w1);
        }
      }
      // ---- 6. Tm diag(beta) and P, the per-token factors
      *reinterpret_cast<s16x8*>(rec + kRecTP + l * 16) = cat8(tvA, pA[vh]);
      const float Gl = vh == 0 ? Gl0 : __shfl(G[vh], kC - 1);
      if (l < kC) {
        reinterpret_cast<float*>(rec + kRecF)[l] = rk * __expf(Gl - G[vh]);
        reinterpret_cast<float*>(rec + kRecGQ)[l] = __expf(G[vh]) * rq;
        if (l == 0) *reinterpret_cast<float*>(rec + kRecGC) = __expf(Gl);
      }
    }
    lds_sync();  // LDS is reused by the next chunk
  }
}

// ============================================================ pass 2: the chunk chain
template <typename ST>
__device__ __forceinline__ f32x4 load_state(const ST* src);
template <>
__device__ __forceinline__ f32x4 load_state<float>(const float* src) {
  return *reinterpret_cast<const f32x4*>(src);
}
template <>
__device__ __forceinline__ f32x4 load_state<bf16s>(const bf16s* src) {
  const uint2 u = *reinterpret_cast<const uint2*>(src);
  return f32x4{bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y)};
}
__device__ __forceinline__ void store_state(float* dst, const f32x4& s) { *reinterpret_cast<f32x4*>(dst) = s; }
__device__ __forceinline__ void store_state(bf16s* dst, const f32x4& s) {
  *reinterpret_cast<uint2*>(dst) = uint2{pack_bf16x2(s.x, s.y), pack_bf16x2(s.z, s.w)};
}

// What the state wave hands to the output wave per chunk, double-buffered by chunk parity:
// one barrier per chunk suffices, since a wave writes buffer j & 1 only after the barrier
// of chunk j - 1, which the output wave reaches after its reads of chunk j - 2 completed.
// (Meeting every second chunk, with four buffers, measured the same.)
// NCB 16-column tiles per wave.
template <int NCB>
struct __attribute__((aligned(16))) ScanLds {
  s16x8 s[2][NCB][kKT / 2][64];  // bf16 S_0 in the B layout of 16x16x32, by 32-key block
  s16x4 u[2][NCB][64];           // bf16 U in the accumulator layout
};

// Operands of one chunk, loaded kDepth chunks ahead: the state wave's and the output wave's.
template <int NCB>
struct StateOps {
  s16x8 w[kKT / 2];   // -W, A layout of 16x16x32
  s16x8 kt[kKT / 2];  // K^T tiles 2m, 2m+1, A layout of 16x16x16
  s16x4 tv;           // Tm diag(beta), A layout
  s16x4 v[NCB];       // V of token l16, columns 16 ct + 4 l4 .. + 3 (A layout; transposed in use)
  f32x4 f;            // f of tokens 4 l4 .. 4 l4 + 3
  float gc;           // Gam_C
};
struct OutOps {
  s16x8 q[kKT / 2];   // Q (stored values), A layout of 16x16x32
  s16x4 pm;           // P, A layout
  float gq;           // Gam_t rq_t of token l16
};

constexpr int kXcds = 8;  // workgroups go to the chip's 8 XCDs round-robin by linear id

// Keeps a chunk's loads after the step that frees their registers: the empty asm takes
// the given values (so the step's last products are done) and clobbers memory (so no
// load moves above it). Hoisted above the step, the loads would need fresh registers and
// copies at the loop's back edge, and a copy waits for its load.
template <typename T>
__device__ __forceinline__ void keep_after(T& x) {
  asm volatile("" : "+v"(x)::"memory");
}

// Runs chunks ja .. jb-1 through step(ops, j) with the operands of chunk j + D loading
// while chunk j computes: D operand sets, each keeping its registers (no copies between
// them: the loop is unrolled D times), D chunks per trip with no exit inside (nothing sinks
// into the next trip), then the last chunks alone; nothing is in flight at the loop's start
// (the wait counts inside the loop then follow from its own loads alone). With two chunks
// in flight a chain waited for its records (8 x 2048 tokens: 117.5 us per call); three
// measured 109.5 us, four 110.7 us.
constexpr int kDepth = 3;  // chunks of operands in flight in the chain

template <int D, typename Ops, typename Fetch, typename Step, typename After>
__device__ __forceinline__ void run_chunks(int ja, int jb, Fetch fetch, Step step, After after) {
  if (jb <= ja) return;
  Ops c[D];
#pragma unroll
  for (int i = 0; i < D; ++i) c[i] = fetch(ja + i);
  __builtin_amdgcn_s_waitcnt(0);
  int j = ja;
  for (; j + D - 1 < jb; j += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      step(c[i], j + i);
      after();
      c[i] = fetch(j + i + D);
    }
  }
#pragma unroll
  for (int i = 0; i < D - 1; ++i)
    if (j + i < jb) step(c[i], j + i);
}

// The workgroup barrier of the chains, as builtins rather than asm: the compiler then knows
// that every LDS access of the wave has completed (lgkmcnt(0)) and does not wait again for
// loads issued before it when their values are used after loads issued since.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0); vmcnt and expcnt left alone
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Everything a chain needs about its (sequence, v-head) and value-column block.
struct ChainArgs {
  int64_t rid0;  // record of chunk 0
  int t0, t1;    // token range of the sequence
  int h, kh;     // v-head, k-head
  int c0;        // first value column of the block (V and o)
};

// The state chain over chunks [ja, jb) with S in MFMA accumulators (tile kt of column tile
// ct of lane l holds S[16kt + 4 l4 + i][column 16 ct + l16 of the block]): U = Tm diag(beta)
// V - W S_0, then the update. The NCB column tiles share every record load.
// WITH_V: the Tm diag(beta) V term (off for a segment map, whose values are zero).
// HANDOFF: bf16 S_0 and U go to the output wave through LDS, one barrier per chunk.
template <bool WITH_V, bool HANDOFF, int NCB>
__device__ __forceinline__ void state_chain(const PrefillArgs& p, ScanLds<NCB>& L, const ChainArgs& a,
                                            f32x4 (&S)[NCB][kKT], int ja, int jb) {
  const int l = threadIdx.x & 63, l16 = l & 15, l4 = l >> 4;
  const uint32_t o_l = uint32_t(l * 16);
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  const int last = max(a.t1 - 1, 0);
  const char* vbase = reinterpret_cast<const char*>(static_cast<const uint16_t*>(p.v) + size_t(a.h) * p.DV + a.c0);
  const uint32_t vrow_b = uint32_t(p.Hv) * uint32_t(p.DV) * 2u;
  const uint32_t o_f = uint32_t(kRecF + 16 * l4);
  const s16x4 eye = identity_b(l16, l4);
  auto fetch = [&](int j) -> StateOps<NCB> {
    StateOps<NCB> c;
    const int64_t rid = min(a.rid0 + j, p.records - 1);
    const char* rec = head_record(p, rid, a.h);
    const char* krec = key_record(p, rid, a.kh);
#pragma unroll
    for (int m = 0; m < kKT / 2; ++m) {
      c.w[m] = *reinterpret_cast<const s16x8*>(rec + kRecW + m * 1024 + o_l);
      c.kt[m] = *reinterpret_cast<const s16x8*>(krec + kKeyKT + m * 1024 + o_l);
    }
    c.f = *reinterpret_cast<const f32x4*>(rec + o_f);
    c.gc = *reinterpret_cast<const float*>(rec + kRecGC);
    if constexpr (WITH_V) {
      c.tv = *reinterpret_cast<const s16x4*>(rec + kRecTP + o_l);  // the lower half
      const uint32_t tok = uint32_t(min(a.t0 + j * kC + l16, last));
#pragma unroll
      for (int ct = 0; ct < NCB; ++ct)
        c.v[ct] = *reinterpret_cast<const s16x4*>(vbase + tok * vrow_b + 8u * l4 + 32u * ct);
    }
    return c;
  };
  auto step = [&](const StateOps<NCB>& c, int j) {
    const int buf = j & 1;
    f32x4 tvv[NCB];
#pragma unroll
    for (int ct = 0; ct < NCB; ++ct) tvv[ct] = zero4;
    if constexpr (WITH_V) {
      // Tm diag(beta) V (V transposed by the identity product). The asm pins the
      // state-independent products to this step: hoisted to the loop's start, they would
      // wait for loads issued just before.
#pragma unroll
      for (int ct = 0; ct < NCB; ++ct) {
        s16x4 v = c.v[ct], tv = c.tv;
        asm volatile("" : "+v"(v), "+v"(tv));
        tvv[ct] = mfma(tv, bf16x4(mfma(v, eye, zero4)), zero4);
      }
    }
    // -W S_0 in two interleaved accumulators per column tile (half the dependent chain).
    // The 16x16x16 product above joins them through a vector add, not as an accumulator:
    // a 16x16x32 product reading the result of a 16x16x16 one needs five wait states, and
    // the compiler does not always place them.
    f32x4 u0[NCB], u1[NCB];
#pragma unroll
    for (int ct = 0; ct < NCB; ++ct) u0[ct] = u1[ct] = zero4;
#pragma unroll
    for (int m = 0; m < kKT / 2; ++m)
#pragma unroll
      for (int ct = 0; ct < NCB; ++ct) {
        const s16x8 sB = cat8(bf16x4(S[ct][2 * m]), bf16x4(S[ct][2 * m + 1]));
        if constexpr (HANDOFF) {
          hand_tile(L.s[buf][ct][m], 2 * m, l16, l4, bf16x4(S[ct][2 * m]));
          hand_tile(L.s[buf][ct][m], 2 * m + 1, l16, l4, bf16x4(S[ct][2 * m + 1]));
        }
        if (m & 1)
          u1[ct] = mfma32(c.w[m], sB, u1[ct]);
        else
          u0[ct] = mfma32(c.w[m], sB, u0[ct]);
      }
    f32x4 u[NCB];
#pragma unroll
    for (int ct = 0; ct < NCB; ++ct) {
      u[ct] = (u0[ct] + u1[ct]) + tvv[ct];
      if constexpr (HANDOFF) L.u[buf][ct][l] = bf16x4(u[ct]);
    }
    if constexpr (HANDOFF) barrier_lds();
    // S <- Gam_C S_0 + K^T diag(rk Gam_C / Gam) U
#pragma unroll
    for (int ct = 0; ct < NCB; ++ct) {
      const s16x4 uB = bf16x4(c.f[0] * u[ct][0], c.f[1] * u[ct][1], c.f[2] * u[ct][2], c.f[3] * u[ct][3]);
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt)
        S[ct][kt] = mfma((kt & 1) ? hi4(c.kt[kt / 2]) : lo4(c.kt[kt / 2]), uB, S[ct][kt] * c.gc);
    }
  };
  auto after = [&]() {
#pragma unroll
    for (int ct = 0; ct < NCB; ++ct)
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt) keep_after(S[ct][kt]);
  };
  run_chunks<kDepth, StateOps<NCB>>(ja, jb, fetch, step, after);
}

// The outputs of chunks [ja, jb), one chunk behind the state chain that hands them over:
// O^T = scale ((Q S_0)^T diag(Gam rq) + U^T P^T) with (Q S_0)^T = S_0^T Q^T: lane (g, t)
// holds columns 4g .. 4g+3 of token t, per column tile.
template <int NCB>
__device__ __forceinline__ void output_chain(const PrefillArgs& p, ScanLds<NCB>& L, const ChainArgs& a, int ja,
                                             int jb) {
  const int l = threadIdx.x & 63, l16 = l & 15, l4 = l >> 4;
  const uint32_t o_l = uint32_t(l * 16);
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  uint16_t* og = static_cast<uint16_t*>(p.o);
  const uint32_t o_gq = uint32_t(kRecGQ + 4 * l16);
  const int last = max(a.t1 - 1, 0);
  const uint16_t* qg = static_cast<const uint16_t*>(p.q) + size_t(a.kh) * kDK + 8 * l4;
  auto fetch = [&](int j) -> OutOps {
    OutOps c;
    const int64_t rid = min(a.rid0 + j, p.records - 1);
    const char* rec = head_record(p, rid, a.h);
    // queries of token l16 (clamped: rows past the end only reach outputs not stored)
    const uint16_t* qrow = qg + size_t(min(a.t0 + j * kC + l16, last)) * p.Hk * kDK;
#pragma unroll
    for (int m = 0; m < kKT / 2; ++m) c.q[m] = *reinterpret_cast<const s16x8*>(qrow + 32 * m);
    c.pm = *reinterpret_cast<const s16x4*>(rec + kRecTP + o_l + 8);  // the upper half
    c.gq = *reinterpret_cast<const float*>(rec + o_gq);
    return c;
  };
  auto step = [&](const OutOps& c, int j) {
    const int buf = j & 1, cs = a.t0 + j * kC, n = min(kC, a.t1 - cs);
    barrier_lds();  // chunk j's S_0 and U are in buffer j & 1
    // Every operand read from LDS, for all column tiles, gets its own registers and has
    // arrived before the first product: no LDS return lands in a register a pending
    // product still reads.
    s16x8 sA[NCB][kKT / 2];
    s16x4 uA[NCB];
#pragma unroll
    for (int ct = 0; ct < NCB; ++ct) {
#pragma unroll
      for (int m = 0; m < kKT / 2; ++m) sA[ct][m] = L.s[buf][ct][m][l];
      uA[ct] = L.u[buf][ct][l];
    }
    if constexpr (NCB == 1) {
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(sA[0][0]), "+v"(sA[0][1]), "+v"(sA[0][2]), "+v"(sA[0][3]),
                   "+v"(uA[0]));
    } else {
      static_assert(NCB == 2, "one or two column tiles per wave");
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(sA[0][0]), "+v"(sA[0][1]), "+v"(sA[0][2]), "+v"(sA[0][3]), "+v"(uA[0]),
                     "+v"(sA[1][0]), "+v"(sA[1][1]), "+v"(sA[1][2]), "+v"(sA[1][3]), "+v"(uA[1]));
    }
#pragma unroll
    for (int ct = 0; ct < NCB; ++ct) {
      f32x4 qs = zero4;
#pragma unroll
      for (int m = 0; m < kKT / 2; ++m) qs = mfma32(sA[ct][m], c.q[m], qs);
      const f32x4 pu = mfma(uA[ct], c.pm, zero4);
      float ov[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ov[i] = p.scale * fmaf(c.gq, qs[i], pu[i]);
      if (l16 < n)
        *reinterpret_cast<uint2*>(og + (size_t(cs + l16) * p.Hv + a.h) * p.DV + a.c0 + 16 * ct + 4 * l4) =
            uint2{pack_bf16x2(ov[0], ov[1]), pack_bf16x2(ov[2], ov[3])};
    }
  };
  // the step ends in its store, so a memory clobber keeps the next loads after it
  auto after = [&]() { asm volatile("" ::: "memory"); };
  run_chunks<kDepth, OutOps>(ja, jb, fetch, step, after);
}

// fp32 state block cb of a segment slot, in the accumulator layout: [kt][lane][4]
__device__ __forceinline__ f32x4* slot_block(const PrefillArgs& p, int64_t sid, int h, int cb) {
  return reinterpret_cast<f32x4*>(segment_slot(p, sid, h)) + (cb * kKT) * 64 + (threadIdx.x & 63);
}
// bf16 segment map of a slot, in the A layout of 16x16x32: [row tile kt][32-column block m][lane][8]
__device__ __forceinline__ s16x8* slot_map(const PrefillArgs& p, int64_t sid, int h) {
  return reinterpret_cast<s16x8*>(segment_slot(p, sid, h) + size_t(p.DV) * kDK * 4);
}

// Whole sequences on chain waves of NCB 16-column tiles that load their own records, a state
// wave and an output wave per block of 16 NCB value columns: kept for batches with two or
// more chains per SIMD whose d_v is not a multiple of 64, where the staged groups of four
// chains do not apply. 1-D grid, XCD-aware: the column blocks of a (sequence, v-head) read
// the same records, so they get ids on one XCD (id % 8 equal) and share its L2. Unit u
// (= sequence * Hv + h) and column block cb take id (u % 8) + 8 (cb + nb (u / 8)).
template <typename ST, int NCB>
__global__ __launch_bounds__(128) void scan_kernel(const PrefillArgs p) {
  __shared__ ScanLds<NCB> L;
  const int l = threadIdx.x & 63, l16 = l & 15, l4 = l >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // 0: the state wave, 1: the output wave
  const int nb = p.DV / (16 * NCB);  // blocks of 16 NCB value columns
  const int rest = int(blockIdx.x) / kXcds, cb = rest % nb;
  const int64_t unit = int64_t(rest / nb) * kXcds + int(blockIdx.x) % kXcds;
  if (unit >= p.segments * p.Hv) return;  // the padding of the last group of 8 units
  const int h = int(unit % p.Hv);
  const int32_t entry = segment_table(p)[unit / p.Hv];
  if (entry < 0 || (entry >> 16) != 0) return;  // no segment has this id (one per sequence here)
  const int row = entry & 0xFFFF;
  if (row >= p.B) return;  // (only a table left by inconsistent cu_seqlens)
  const int32_t slot = p.idx[row];
  ChainArgs a;
  a.t0 = p.cu[row];
  a.t1 = p.cu[row + 1];
  a.h = h;
  a.kh = h / p.G;
  a.c0 = cb * 16 * NCB;

  if (slot < 0 || slot >= p.P) {  // padding row: o = 0 for its tokens, no state access
    uint16_t* og = static_cast<uint16_t*>(p.o);
    const int n16 = (a.t1 - a.t0) * 2 * NCB;  // 16-byte pieces of the block's outputs
    for (int e = wave * 64 + l; e < n16; e += 128) {
      const int t = a.t0 + e / (2 * NCB), c = e % (2 * NCB);
      *reinterpret_cast<u32x4*>(og + (size_t(t) * p.Hv + h) * p.DV + a.c0 + 8 * c) = u32x4{0u, 0u, 0u, 0u};
    }
    return;
  }

  const int nchunks = (a.t1 - a.t0 + kC - 1) / kC;
  a.rid0 = record_id(a.t0, row, 0);
  // chunks with a record (all of them unless the workspace is too small for the tokens).
  // Every load is unconditional: the record index and the tokens are clamped into range (a
  // load in a branch is waited on at the branch end). Operands of tokens past the end meet
  // zero columns of Tm diag(beta) and of P, zero rows of K^T, or outputs not stored.
  const int jb = int(max<int64_t>(0, min<int64_t>(nchunks, p.records - a.rid0)));
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  if (wave == 0) {
    // column tile ct of the block: value rows c0 + 16 ct + l16 of the slot's state
    ST* const my_state =
        static_cast<ST*>(p.pool) + ((size_t(slot) * p.Hv + h) * p.DV + a.c0 + l16) * kDK + 4 * l4;
    const int32_t fresh = p.fresh ? p.fresh[row] : 0;
    f32x4 S[NCB][kKT];
#pragma unroll
    for (int ct = 0; ct < NCB; ++ct)
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt) {
        const f32x4 s = load_state<ST>(my_state + 16 * ct * kDK + 16 * kt);  // unconditional, then masked
        S[ct][kt] = fresh ? zero4 : s;
      }
    state_chain<true, true, NCB>(p, L, a, S, 0, jb);
    // the final state back to the slot (rounded once for a bf16 pool)
#pragma unroll
    for (int ct = 0; ct < NCB; ++ct)
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt) store_state(my_state + 16 * ct * kDK + 16 * kt, S[ct][kt]);
  } else {
    output_chain<NCB>(p, L, a, 0, jb);
  }
}

// ============================================================ pass 2: the chains in groups of
// two or four per workgroup, with their records staged in LDS
//
// A workgroup of 2 CH + 1 waves runs the chains of CH neighbouring 16-column blocks of one
// (sequence or segment, v-head): waves 0 .. CH-1 are their state waves, CH .. 2CH-1 their output
// waves, and wave 2CH copies each chunk's records and the group's 16 CH value columns from
// the workspace into a ring of LDS slots with direct-to-LDS loads (global_load_lds_dwordx4),
// once for all the chains. The chains read their operands out of LDS, so each record byte
// crosses the CU's vector-memory path once, not once per wave that uses it (the state waves
// read the same -W, K^T and Tm diag(beta), the output waves the same Q and P): that path,
// with its texture units busy four fifths of the time, bound the chain step when every
// wave loaded its own operands. Only the copying wave issues direct-to-LDS loads, so the
// other waves' LDS reads need no wait on vector memory; it waits for its own loads with
// explicit vmcnt counts before the barrier that publishes them.
// CH = 2 (one chain wave per SIMD) while two-chain workgroups fit one per CU (one fits in LDS
// at a time); CH = 4 (two chain waves per SIMD, four chains sharing each record read) when
// there are more: 4 x 4096 tokens with 32 v-heads, pass 2 231 -> 177 us against waves of two
// column tiles loading their own records; two-chain workgroups there, one per CU at a time,
// took 232 us, and two per CU (a ring of four slots to fit LDS) 274 us.
//
// Schedule, with B(j) the barrier of chunk j that all the waves reach once per chunk
// (B(-1) before the first chunk). Chunk c is published at B(c - 2), so that every wave reads
// its operands of a chunk one step ahead, off the chain's dependent path:
// - state waves, step j (between B(j-1) and B(j)): the operands of chunk j + 1 are read
//   while U of chunk j is computed from those read in step j - 1; S_0 and U go to the
//   output wave's buffer j & 1; B(j); the update.
// - output waves, after B(j): the outputs of chunk j from buffer j & 1 and the Q, P and
//   factors read in the previous step; then those of chunk j + 1 are read.
// - copying wave, after B(j): chunk j + RING into the slot of chunk j, which the state
//   waves finished reading before B(j - 1) and the output waves before B(j); then a wait
//   until chunk j + 3 has landed (the two later chunks may still be in flight), so that
//   B(j + 1) publishes it.
constexpr int kStW = 0;          // -W: 4 x 1 KiB, as in the v-head record
constexpr int kStKT = 4096;      // K^T: 4 x 1 KiB, as in the k-head record
constexpr int kStQ = 8192;       // Q: 4 x 1 KiB, from q, keys in the order of the handover
constexpr int kStTP = 12288;     // Tm diag(beta) and P: 1 KiB
constexpr int kStSmall = 13312;  // record bytes kRecF .. kRecF + 255: f, Gam rq, Gam_C
constexpr int kStV = 13568;      // V of the group's 16 CH columns, token t at byte 32 CH t
static_assert(kRecF + 256 <= kPrefillRecordBytes && kRecGQ - kRecF == 64 && kRecGC - kRecF == 128, "small fields");
// bytes of a slot and direct-to-LDS loads per chunk for CH chains
constexpr int st_bytes(int CH) { return kStV + 512 * CH; }
constexpr int st_loads(int CH, bool WF) { return (WF ? 11 : 14) + CH / 2; }

// RING slots: chunks j .. j + RING - 1 around chunk j
template <int CH, int RING>
struct __attribute__((aligned(16))) GroupLds {
  char ring[RING][st_bytes(CH)];
  ScanLds<1> hand[CH];
};

typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) void lds_void;
template <typename T>
__device__ __forceinline__ T lds_ld(const lds_char* p) {
  return *reinterpret_cast<const __attribute__((address_space(3))) T*>(p);
}
// lane l's 16 (4) bytes at g land at LDS bytes dst + 16 l (dst + 4 l); dst is wave-uniform
__device__ __forceinline__ void to_lds16(const void* g, lds_char* dst) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)dst, 16, 0, 0);
}
__device__ __forceinline__ void to_lds4(const void* g, lds_char* dst) {
  __builtin_amdgcn_global_load_lds(g, (lds_void*)dst, 4, 0, 0);
}
// s_waitcnt vmcnt(N), the other counters left alone (gfx9 encoding: vmcnt bits 3:0 and
// 15:14, expcnt 6:4, lgkmcnt 11:8)
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
  asm volatile("" ::: "memory");
}

// The state wave's operands of one chunk, read from its slot.
struct StOps {
  s16x8 w[kKT / 2];   // -W, A layout of 16x16x32
  s16x8 kt[kKT / 2];  // K^T tiles 2m, 2m+1, A layout of 16x16x16
  s16x4 tw;           // WF: -Tm diag(beta Gam rk), A layout of 16x16x16
  s16x4 tv;           // Tm diag(beta), A layout
  s16x4 v;            // V of token l16, columns 4 l4 .. + 3 of the chain's block
  f32x4 f;            // f of tokens 4 l4 .. 4 l4 + 3
  float gc;           // Gam_C
};
template <int CH, bool WF>
__device__ __forceinline__ StOps read_state_ops(const lds_char* s, int chain, int l, int l16, int l4) {
  StOps c;
#pragma unroll
  for (int m = 0; m < kKT / 2; ++m) {
    if constexpr (!WF) c.w[m] = lds_ld<s16x8>(s + kStW + m * 1024 + 16 * l);
    c.kt[m] = lds_ld<s16x8>(s + kStKT + m * 1024 + 16 * l);
  }
  if constexpr (WF) c.tw = lds_ld<s16x4>(s + kStW + 8 * l);
  c.tv = lds_ld<s16x4>(s + kStTP + 16 * l);  // the lower half
  c.v = lds_ld<s16x4>(s + kStV + 32 * CH * l16 + 32 * chain + 8 * l4);
  c.f = lds_ld<f32x4>(s + kStSmall + 16 * l4);
  c.gc = lds_ld<float>(s + kStSmall + (kRecGC - kRecF));
  return c;
}

// -W from K^T and the factor: pass 1's own product of the same bf16 operands, so the same bits.
// Halves h0 .. h1 - 1 of two 32-key blocks each, so that at most four products' fp32 results
// are live (all eight at once pushed four-chain workgroups past their register budget, and
// those spills had made 4 x 4096 take 291 us instead of 253 with -W records).
__device__ __forceinline__ void build_w(StOps& c, int h0, int h1) {
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int h = h0; h < h1; ++h) {
#pragma unroll
    for (int m = 2 * h; m < 2 * h + 2; ++m)
      c.w[m] = cat8(bf16x4(mfma(lo4(c.kt[m]), c.tw, zero4)), bf16x4(mfma(hi4(c.kt[m]), c.tw, zero4)));
    __builtin_amdgcn_sched_barrier(0);
  }
}

// The chain of one column block over the staged chunks 0 .. jb - 1 (chunk j in slot j % RING),
// with S in MFMA accumulators: U = Tm diag(beta) V - W S_0 (WITH_V: the values term, off for
// a segment map), then S <- Gam_C S_0 + K^T diag(rk Gam_C / Gam) U. HANDOFF: bf16 S_0 and U
// go to the chain's output wave through buffer j & 1 before B(j). One barrier per chunk,
// B(-1) first, as every wave of the workgroup.
template <int CH, int RING, bool WITH_V, bool HANDOFF, bool WF>
__device__ __forceinline__ void staged_chain(GroupLds<CH, RING>& L, f32x4 (&S)[kKT], int chain, int jb) {
  const int l = threadIdx.x & 63, l16 = l & 15, l4 = l >> 4;
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  auto slot_of = [&](int j) -> lds_char* { return (lds_char*)&L.ring[j % RING][0]; };
  ScanLds<1>& H = L.hand[chain];
  const s16x4 eye = identity_b(l16, l4);
  // the next chunk's operands, U of chunk j, the handover, B(j), the update
  auto step = [&](const StOps& c, StOps& next, int j) {
    const int buf = j & 1;
    next = read_state_ops<CH, WF>(slot_of(j + 1), chain, l, l16, l4);  // published at B(j - 1)
    __builtin_amdgcn_sched_barrier(0);  // they go out first
    f32x4 tvv = zero4;
    if constexpr (WITH_V) {
      // Tm diag(beta) V (V transposed by the identity product); the asm keeps the
      // state-independent products in this step
      s16x4 v = c.v, tv = c.tv;
      asm volatile("" : "+v"(v), "+v"(tv));
      tvv = mfma(tv, bf16x4(mfma(v, eye, zero4)), zero4);
    }
    // -W S_0 in two interleaved accumulators (half the dependent chain); the 16x16x16
    // product above joins them through a vector add
    f32x4 u0 = zero4, u1 = zero4;
#pragma unroll
    for (int m = 0; m < kKT / 2; ++m) {
      const s16x8 sB = cat8(bf16x4(S[2 * m]), bf16x4(S[2 * m + 1]));
      if constexpr (HANDOFF) {
        hand_tile(H.s[buf][0][m], 2 * m, l16, l4, bf16x4(S[2 * m]));
        hand_tile(H.s[buf][0][m], 2 * m + 1, l16, l4, bf16x4(S[2 * m + 1]));
      }
      if (m & 1)
        u1 = mfma32(c.w[m], sB, u1);
      else
        u0 = mfma32(c.w[m], sB, u0);
    }
    const f32x4 u = (u0 + u1) + tvv;
    if constexpr (HANDOFF) H.u[buf][0][l] = bf16x4(u);
    // WF: the next chunk's -W, half here, where the matrix core has finished -W S_0, and
    // half after the barrier, ahead of the update's products (all of it here, the long
    // prompt took 114 us instead of 111)
    if constexpr (WF) build_w(next, 0, 1);
    // Gam_C S_0 before the barrier, where it overlaps the products and the wait; placed
    // after it, between the update's products, it measured slower
#pragma unroll
    for (int kt = 0; kt < kKT; ++kt) S[kt] = S[kt] * c.gc;
    asm volatile("" : "+v"(S[0]), "+v"(S[1]), "+v"(S[2]), "+v"(S[3]), "+v"(S[4]), "+v"(S[5]), "+v"(S[6]), "+v"(S[7]));
    barrier_lds();  // B(j)
    // S <- Gam_C S_0 + K^T diag(rk Gam_C / Gam) U
    const s16x4 uB = bf16x4(c.f[0] * u[0], c.f[1] * u[1], c.f[2] * u[2], c.f[3] * u[3]);
    if constexpr (WF) build_w(next, 1, 2);
#pragma unroll
    for (int kt = 0; kt < kKT; ++kt) S[kt] = mfma((kt & 1) ? hi4(c.kt[kt / 2]) : lo4(c.kt[kt / 2]), uB, S[kt]);
  };
  barrier_lds();  // B(-1)
  StOps ca = read_state_ops<CH, WF>(slot_of(0), chain, l, l16, l4), cb;
  if constexpr (WF) build_w(ca, 0, 2);
  for (int j = 0; j < jb; j += 2) {
    step(ca, cb, j);
    if (j + 1 >= jb) break;
    step(cb, ca, j + 1);
  }
}

// A wave of the workgroup with no chain to run still takes part in every barrier.
__device__ __forceinline__ void barriers_only(int jb) {
  barrier_lds();  // B(-1)
  for (int j = 0; j < jb; ++j) barrier_lds();
}

// MODE 0: whole sequences, from the pool. MODE 1: the first phase of a segmented chain:
// segment 0 from the pool with outputs (its end state to the segment's slot, or to the pool
// when it is the only segment), and for every middle segment the map F(S) = M S + N: the
// state waves run N (the value columns, from zero), the waves that would be output waves
// run M (d_k columns, from the identity, without the values), neither with outputs. MODE 2:
// the later segments, each from the start state that the maps composed into its
// predecessor's slot, with outputs, the last one storing the final state.
template <typename ST, int CH, int RING, int MODE, bool WF>
__global__ __launch_bounds__(64 * (2 * CH + 1)) void group_chain_kernel(const PrefillArgs p) {
  // WF: the chains form -W from its factor (pass 1 wrote the factor in its place)
  constexpr int kStLoads = st_loads(CH, WF);
  // the copying wave's loads newer than chunk j + 3's when it waits: RING - 3 chunks'. Its
  // counter of vector-memory operations in flight holds at most 63, so it never has more
  // than RING - 2 chunks' loads in flight.
  constexpr int kStNewer = (RING - 3) * kStLoads;
  static_assert((CH == 2 || CH == 4) && RING >= 4 && kStNewer + kStLoads <= 63, "two or four chains, ring of 4 to 6");
  constexpr int kThreads = 64 * (2 * CH + 1);
  __shared__ GroupLds<CH, RING> L;
  const int l = threadIdx.x & 63, l16 = l & 15, l4 = l >> 4;
  const int wid = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int chain = wid % CH;
  // groups of column blocks per (segment, v-head); the first phase also covers the d_k
  // columns of the maps
  const int per = (MODE == 1 ? max(p.DV, kDK) : p.DV) / (16 * CH);
  const int rest = int(blockIdx.x) / kXcds, grp = rest % per;
  const int64_t unit = int64_t(rest / per) * kXcds + int(blockIdx.x) % kXcds;
  if (unit >= p.segments * p.Hv) return;  // the padding of the last group of 8 units
  const int h = int(unit % p.Hv), kh = h / p.G;
  const int64_t sid = unit / p.Hv;
  const int32_t entry = segment_table(p)[sid];
  if (entry < 0) return;  // no segment has this id
  const int row = entry & 0xFFFF, g = entry >> 16;
  if (MODE == 0 ? g != 0 : MODE == 2 ? g == 0 : false) return;
  if (row >= p.B) return;  // (only a table left by inconsistent cu_seqlens)
  const int32_t slot = p.idx[row];
  const int t0 = p.cu[row], t1 = p.cu[row + 1];
  const int c0 = (CH * grp + chain) * 16;  // the chain's first column
  const int nchunks = (t1 - t0 + kC - 1) / kC;
  const int nseg = seg_count(p, nchunks);
  if (MODE == 1 && g > 0 && g == nseg - 1) return;  // the last segment has no map to compose
  const bool outputs = MODE != 1 || g == 0;         // state and output waves, as opposed to N and M
  if (outputs && 16 * CH * grp >= p.DV) return;     // (map columns past the value columns)

  if (slot < 0 || slot >= p.P) {  // padding row: o = 0 for its tokens, no state access
    if (g != 0) return;           // zeroed once, by segment 0's groups (of value columns only)
    uint16_t* og = static_cast<uint16_t*>(p.o);
    for (int e = int(threadIdx.x); e < (t1 - t0) * 2 * CH; e += kThreads) {
      const int t = t0 + e / (2 * CH);
      *reinterpret_cast<u32x4*>(og + (size_t(t) * p.Hv + h) * p.DV + 16 * CH * grp + 8 * (e % (2 * CH))) =
          u32x4{0u, 0u, 0u, 0u};
    }
    return;
  }
  // chunks with a record (all of them unless the workspace is too small for the tokens)
  const int nrun = int(max<int64_t>(0, min<int64_t>(nchunks, p.records - record_id(t0, row, 0))));
  // this workgroup's chunks: ja .. ja + jb - 1 of the sequence, j = 0 .. jb - 1 below
  const int ja = MODE == 0 ? 0 : g * seg_chunks(p);
  const int jb = max(0, (MODE == 0 ? nrun : min(ja + seg_chunks(p), nrun)) - ja);
  const int64_t rid0 = record_id(t0, row, ja);
  const int ts = t0 + ja * kC;  // the first token of chunk ja
  const f32x4 zero4 = {0.f, 0.f, 0.f, 0.f};
  auto slot_of = [&](int j) -> lds_char* { return (lds_char*)&L.ring[j % RING][0]; };

  if (MODE == 1 && !outputs && wid < 2 * CH) {  // ---- N (waves 0 .. CH-1) and M of a middle segment
    const bool is_map = wid >= CH;
    if (c0 >= (is_map ? kDK : p.DV)) {  // no such column block
      if (jb > 0) barriers_only(jb);
      return;
    }
    f32x4 S[kKT];
    if (!is_map) {
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt) S[kt] = zero4;
      if (jb > 0) staged_chain<CH, RING, true, false, WF>(L, S, chain, jb);
      f32x4* dst = slot_block(p, sid, h, c0 / 16);
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt) dst[kt * 64] = S[kt];
    } else {
      const int J = c0 / 16;  // columns 16 J .. 16 J + 15 of M
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
        for (int i = 0; i < 4; ++i) S[kt][i] = (16 * kt + 4 * l4 + i == 16 * J + l16) ? 1.f : 0.f;
      if (jb > 0) staged_chain<CH, RING, false, false, WF>(L, S, chain, jb);
      // Tile (kt, J) read as an A operand is its transpose; the identity product turns that
      // back into the tile itself in the A layout, exactly (bf16 in, single terms).
      const s16x4 eye = identity_b(l16, l4);
      char* dst = reinterpret_cast<char*>(slot_map(p, sid, h));
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt) {
        const s16x4 tA = bf16x4(mfma(bf16x4(S[kt]), eye, zero4));
        *reinterpret_cast<s16x4*>(dst + ((kt * (kKT / 2) + (J >> 1)) * 64 + l) * 16 + (J & 1) * 8) = tA;
      }
    }
    return;
  }

  if (wid < CH) {  // ---- the state waves
    ST* const my_state = static_cast<ST*>(p.pool) + ((size_t(slot) * p.Hv + h) * p.DV + c0 + l16) * kDK + 4 * l4;
    f32x4 S[kKT];
    if constexpr (MODE == 2) {
      const f32x4* src = slot_block(p, sid - 1, h, c0 / 16);  // the segment's start state
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt) S[kt] = src[kt * 64];
    } else {
      const int32_t fresh = p.fresh ? p.fresh[row] : 0;
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt) {
        const f32x4 s = load_state<ST>(my_state + 16 * kt);  // unconditional, then masked
        S[kt] = fresh ? zero4 : s;
      }
    }
    if (jb > 0) staged_chain<CH, RING, true, true, WF>(L, S, chain, jb);
    if (MODE == 1 && nseg > 1) {  // segment 0's end state, for the maps to carry forward
      f32x4* dst = slot_block(p, sid, h, c0 / 16);
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt) dst[kt * 64] = S[kt];
    } else if (MODE != 2 || g == nseg - 1) {
      // the final state back to the slot (rounded once for a bf16 pool), by the sequence's
      // last segment
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt) store_state(my_state + 16 * kt, S[kt]);
    }
    return;
  }
  if (jb == 0) return;

  if (wid < 2 * CH) {  // ---- the output waves: O^T = scale ((Q S_0)^T diag(Gam rq) + U^T P^T)
    ScanLds<1>& H = L.hand[chain];
    uint16_t* og = static_cast<uint16_t*>(p.o);
    struct OutSt {
      s16x8 q[kKT / 2];  // Q (stored values), A layout of 16x16x32
      s16x4 pm;          // P, A layout
      float gq;          // Gam_t rq_t of token l16
    };
    auto read_out = [&](int j) {
      const lds_char* s = slot_of(j);
      OutSt c;
#pragma unroll
      for (int m = 0; m < kKT / 2; ++m) c.q[m] = lds_ld<s16x8>(s + kStQ + m * 1024 + 16 * l);
      c.pm = lds_ld<s16x4>(s + kStTP + 16 * l + 8);  // the upper half
      c.gq = lds_ld<float>(s + kStSmall + (kRecGQ - kRecF) + 4 * l16);
      return c;
    };
    barrier_lds();  // B(-1)
    OutSt c = read_out(0);
    for (int j = 0; j < jb; ++j) {
      const int buf = j & 1, cs = ts + j * kC, n = min(kC, t1 - cs);
      barrier_lds();  // B(j): chunk j's S_0 and U are in buffer j & 1
      s16x8 sA[kKT / 2];
#pragma unroll
      for (int m = 0; m < kKT / 2; ++m) sA[m] = H.s[buf][0][m][l];
      s16x4 uA = H.u[buf][0][l];
      // every operand has arrived before the first product
      asm volatile("s_waitcnt lgkmcnt(0)"
                   : "+v"(sA[0]), "+v"(sA[1]), "+v"(sA[2]), "+v"(sA[3]), "+v"(uA), "+v"(c.q[0]), "+v"(c.q[1]),
                     "+v"(c.q[2]), "+v"(c.q[3]), "+v"(c.pm), "+v"(c.gq));
      f32x4 qs = zero4;
#pragma unroll
      for (int m = 0; m < kKT / 2; ++m) qs = mfma32(sA[m], c.q[m], qs);
      const f32x4 pu = mfma(uA, c.pm, zero4);
      float ov[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ov[i] = p.scale * fmaf(c.gq, qs[i], pu[i]);
      if (l16 < n)
        *reinterpret_cast<uint2*>(og + (size_t(cs + l16) * p.Hv + h) * p.DV + c0 + 4 * l4) =
            uint2{pack_bf16x2(ov[0], ov[1]), pack_bf16x2(ov[2], ov[3])};
      c = read_out(j + 1);  // published at B(j - 1)
    }
    return;
  }

  // ---- the copying wave
  const int last = t1 - 1;
  // value columns: lane l loads 16 bytes (piece l % 2CH) of token l / 2CH of each 1 KiB block
  // (a group of map columns only, past the value columns, loads the last group's values)
  const char* vg = reinterpret_cast<const char*>(static_cast<const uint16_t*>(p.v) + size_t(h) * p.DV +
                                                 min(16 * CH * grp, p.DV - 16 * CH)) +
                   16 * (l % (2 * CH));
  const size_t vrow_b = size_t(p.Hv) * p.DV * 2;
  const uint16_t* qg = static_cast<const uint16_t*>(p.q) + size_t(kh) * kDK + 8 * (l >> 4);
  // chunk c (records clamped into the workspace, tokens to the sequence: the chunks past
  // the end that the ring reaches are loaded but never used)
  auto issue = [&](int c) {
    lds_char* s = slot_of(c);
    const int64_t rid = min(rid0 + c, p.records - 1);
    const char* rec = head_record(p, rid, h);
    const char* krec = key_record(p, rid, kh) + 16 * l;
    // queries of token l % 16, keys 32 m + 8 (l / 16) .. + 7 (clamped: rows past the end only
    // reach outputs not stored)
    const uint16_t* qrow = qg + size_t(min(ts + c * kC + (l & 15), last)) * p.Hk * kDK;
#pragma unroll
    for (int m = 0; m < kKT / 2; ++m) {
      if constexpr (!WF) to_lds16(rec + kRecW + m * 1024 + 16 * l, s + kStW + m * 1024);
      to_lds16(krec + kKeyKT + m * 1024, s + kStKT + m * 1024);
      to_lds16(qrow + 32 * m, s + kStQ + m * 1024);
    }
    if constexpr (WF) to_lds16(rec + kRecW + 16 * l, s + kStW);  // the factor: the first 512 bytes
    to_lds16(rec + kRecTP + 16 * l, s + kStTP);
    to_lds4(rec + kRecF + 4 * l, s + kStSmall);
#pragma unroll
    for (int vo = 0; vo < CH / 2; ++vo) {
      const int tok = min(ts + c * kC + vo * (32 / CH) + l / (2 * CH), last);
      to_lds16(vg + size_t(tok) * vrow_b, s + kStV + 1024 * vo);
    }
  };
  // chunks 0 .. RING - 1, never more than four chunks' loads in flight
#pragma unroll
  for (int c = 0; c < RING - 2; ++c) issue(c);
  wait_vm<kStNewer>();  // chunk 0 has landed
  issue(RING - 2);
  wait_vm<kStNewer>();  // chunk 1 has landed
  barrier_lds();        // B(-1)
  issue(RING - 1);
  wait_vm<kStNewer>();  // chunk 2 has landed
  for (int j = 0; j < jb; ++j) {
    barrier_lds();  // B(j)
    issue(j + RING);
    wait_vm<kStNewer>();  // chunk j + 3 has landed
  }
  wait_vm<0>();  // nothing lands in LDS after the workgroup ends
}

// The start states of the segments after the first: S_1 is segment 0's end state, and
// S_{g+1} = M_g S_g + N_g for g = 1 .. n-2, stored over N_g in the slot of segment g. One
// workgroup of eight waves per (sequence, v-head, 16 value columns): wave r computes row tile
// r (16 rows) of each S_{g+1}, from row tile r of M_g and all of S_g, which the waves share
// in bf16 through LDS (double-buffered, one barrier per composition). S_g and M_g enter the
// products in bf16, as the chain's own S_0 does; each row tile sums N_g and the four 32-key
// blocks in that order. With one wave per column block doing all eight row tiles, the 14
// compositions of one 16384-token prompt took 16 us. 1-D grid, XCD-aware as in the chains
// (unit = row * Hv + h).
__global__ __launch_bounds__(512) void combine_kernel(const PrefillArgs p) {
  __shared__ s16x8 sh[2][kKT / 2][64];  // S_g in the B layout of 16x16x32, by 32-key block
  const int nb = p.DV / 16;
  const int rest = int(blockIdx.x) / kXcds, cb = rest % nb;
  const int64_t unit = int64_t(rest / nb) * kXcds + int(blockIdx.x) % kXcds;
  if (unit >= int64_t(p.B) * p.Hv) return;
  const int h = int(unit % p.Hv), row = int(unit / p.Hv);
  const int32_t slot = p.idx[row];
  if (slot < 0 || slot >= p.P) return;
  const int32_t t0 = p.cu[row], t1 = p.cu[row + 1];
  const int nchunks = (t1 - t0 + kC - 1) / kC;
  const int nseg = seg_count(p, nchunks);
  if (nseg < 3) return;
  const int l = threadIdx.x & 63;
  const int r = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // the wave's row tile
  const int64_t sid0 = segment_id(p, t0, row, 0);
  // row tile r of S_g holds rows 32 (r / 2) + 16 (r % 2) + 4 l4 + i: the low or high half
  // of B-operand block r / 2
  auto share = [&](int buf, const f32x4& s) {
    reinterpret_cast<s16x4*>(&sh[buf][r / 2][l])[r & 1] = bf16x4(s);
  };
  share(1, slot_block(p, min(sid0, p.segments - 1), h, cb)[r * 64]);  // S_1
  // the map's row tiles and N of the next four compositions load while one computes (one
  // ahead, each composition waited for its loads: 14.2 us for the 14 of one 16384-token
  // prompt)
  struct Ops {
    s16x8 map[kKT / 2];
    f32x4 n;
  };
  auto fetch = [&](int g) -> Ops {
    Ops o;
    const int64_t sid = min(sid0 + min(g, nseg - 2), p.segments - 1);
    const s16x8* map = slot_map(p, sid, h) + l;
#pragma unroll
    for (int m = 0; m < kKT / 2; ++m) o.map[m] = map[(r * (kKT / 2) + m) * 64];
    o.n = slot_block(p, sid, h, cb)[r * 64];
    return o;
  };
  auto step = [&](const Ops& c, int g) {
    s16x8 sB[kKT / 2];
#pragma unroll
    for (int m = 0; m < kKT / 2; ++m) sB[m] = sh[g & 1][m][l];
    f32x4 acc = c.n;
#pragma unroll
    for (int m = 0; m < kKT / 2; ++m) acc = mfma32(c.map[m], sB[m], acc);
    slot_block(p, min(sid0 + g, p.segments - 1), h, cb)[r * 64] = acc;
    share((g + 1) & 1, acc);
    barrier_lds();  // S_{g+1} shared; every read of buffer g & 1 done
  };
  constexpr int D = 4;
  barrier_lds();
  Ops c[D];  // a ring indexed at compile time (the loop is unrolled D times): no copies
#pragma unroll
  for (int i = 0; i < D; ++i) c[i] = fetch(1 + i);  // clamped to the last map past the end
  int g = 1;
  for (; g + D - 1 <= nseg - 2; g += D) {
#pragma unroll
    for (int i = 0; i < D; ++i) {
      step(c[i], g + i);
      c[i] = fetch(g + i + D);
    }
  }
#pragma unroll
  for (int i = 0; i < D - 1; ++i)
    if (g + i <= nseg - 2) step(c[i], g + i);
}

template <typename ST, int NCB>
hipError_t launch_scan(const PrefillArgs& p, hipStream_t stream) {
  const int64_t units = (p.segments * p.Hv + kXcds - 1) / kXcds * kXcds;
  hipLaunchKernelGGL((scan_kernel<ST, NCB>), dim3(unsigned(units * (p.DV / (16 * NCB)))), dim3(128), 0, stream, p);
  return hipGetLastError();
}

template <typename ST, int CH, int RING, int MODE, bool WF = MODE != 0>
hipError_t launch_group(const PrefillArgs& p, hipStream_t stream) {
  const int64_t units = (p.segments * p.Hv + kXcds - 1) / kXcds * kXcds;
  const int per = (MODE == 1 ? std::max(p.DV, kDK) : p.DV) / (16 * CH);
  hipLaunchKernelGGL((group_chain_kernel<ST, CH, RING, MODE, WF>), dim3(unsigned(units * per)), dim3(64 * (2 * CH + 1)), 0,
                     stream, p);
  return hipGetLastError();
}

// Pass 2. A sequence longer than one segment of 2^seg_shift tokens runs its chain in
// segments: with F_g the map from the state at the start of segment g to the state at its
// end, F_g(S) = M_g S + N_g (N_g the chain from a zero state, M_g, d_k x d_k, the chain from
// the identity with zero values). Three launches then: segment 0 with outputs and the maps of
// the middle segments (MODE 1); combine_kernel, the start states S_{g+1} = M_g S_g + N_g in
// sequence; every later segment again from its start state with outputs (MODE 2). The chain
// is sequential within a segment only.
//
// The chains stage their records in LDS, four per workgroup when two-chain workgroups would
// exceed one per CU (one per CU fits in LDS at a time; 4 x 4096 tokens with 32 v-heads, the
// segments of one long prompt), else two. Chain waves of two 16-column tiles that load their
// own records remain for many whole sequences with a d_v that is not a multiple of 64.
struct Pass2Plan {
  bool whole, wide, quads, quads1;
  // the chains form -W from its factor, which pass 1 then writes in its place: every chain
  // in segments or in four-chain workgroups, and whole sequences in two-chain workgroups
  // that average 1024 tokens or more. With such batches every CU stages records for the
  // whole call and its copying wave, paced by the CU's memory pipeline, takes as long per
  // chunk as the state waves, and pass 1 writes an eighth of -W's bytes: 8 x 2048 80.6 ->
  // 77.8 us, 4 x 4096 252.5 -> 217.3 us (pass 1 76.8 -> 62.2 us, pass 2 178.6 -> 162.6 us).
  // The chains of shorter sequences outlast the others with the chip to themselves, the
  // state waves alone set their step and the products that form -W lengthen it (the mixed
  // batch of 1 .. 1000 tokens 32.4 -> 34.5 us).
  bool factor;
};
inline Pass2Plan plan_pass2(const PrefillArgs& p) {
  Pass2Plan q;
  q.whole = (int64_t(1) << p.seg_shift) > p.tokens;
  q.wide = q.whole && int64_t(p.B) * p.Hv * (p.DV / 16) * 2 >= 2048;
  q.quads = p.DV % 64 == 0 && p.segments * p.Hv * (p.DV / 32) > 256;
  q.quads1 = p.DV % 64 == 0 && p.segments * p.Hv * (std::max(p.DV, kDK) / 32) > 256;
  q.factor = !q.whole || q.quads || (!q.wide && p.tokens >= int64_t(1024) * p.B);
  return q;
}

template <typename ST>
hipError_t launch_pass2(const PrefillArgs& p, hipStream_t stream) {
  const Pass2Plan q = plan_pass2(p);
  const bool whole = q.whole, wide = q.wide, quads = q.quads, quads1 = q.quads1;
  hipError_t e;
  if (whole && quads) {
    e = launch_group<ST, 4, 5, 0, true>(p, stream);
  } else if (wide) {
    e = launch_scan<ST, 2>(p, stream);
  } else if (whole) {
    e = q.factor ? launch_group<ST, 2, 6, 0, true>(p, stream) : launch_group<ST, 2, 6, 0, false>(p, stream);
  } else {
    e = quads1 ? launch_group<ST, 4, 5, 1>(p, stream) : launch_group<ST, 2, 6, 1>(p, stream);
  }
  if (e != hipSuccess) return e;
  // a sequence has at least three segments only if it is longer than two of them
  if (p.tokens > (int64_t(2) << p.seg_shift)) {
    const int64_t units = (int64_t(p.B) * p.Hv + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL(combine_kernel, dim3(unsigned(units * (p.DV / 16))), dim3(512), 0, stream, p);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (p.tokens > (int64_t(1) << p.seg_shift))
    e = quads ? launch_group<ST, 4, 5, 2>(p, stream) : launch_group<ST, 2, 6, 2>(p, stream);
  return e;
}

}  // namespace

// Pass 1 gets enough waves to fill the chip whatever the batch: each (sequence, v-head)
// gets `strides` waves that share its chunks.
hipError_t launch_prefill(Dt state, const PrefillArgs& p, hipStream_t stream) {
  // Two v-heads per wave share their k-head's work and run their solves side by side, but
  // halve the waves: worth it once one wave per (chunk, v-head) exceeds the four per SIMD
  // that the chip holds at once (8 x 2048 tokens: pass 1 30.5 -> 23.3 us; the mixed batch,
  // about 1000 waves, loses 0.8 us).
  const int vh = (p.G % 2 == 0 && p.records * p.Hv > 4096) ? 2 : 1;  // v-heads per wave
  const int64_t heads = int64_t(p.B) * p.Hv;
  const unsigned strides = unsigned(std::min<int64_t>(1024, std::max<int64_t>(1, (8192 + heads - 1) / heads)));
  // Where the chains form -W themselves (plan_pass2), pass 1 writes its 16 x 16 factor
  // instead (pass 2 then stages 11 + CH/2 loads per chunk instead of 14 + CH/2; the long
  // prompt 117.3 -> 110.9 us).
  const bool factor = plan_pass2(p).factor;
  // When most waves would find no chunk (the strides cover more than twice the tokens: short
  // sequences beside long ones), the chunk index varies slowest in the grid, so the waves
  // with work are not queued behind empty ones: the mixed batch of 1 .. 1000 tokens 32.5 ->
  // 29.7 us (a second round of dispatch had held its longest sequences back). Otherwise the
  // grid keeps the chunks of a (sequence, head group) together (4 x 4096: 252 vs 257 us).
  const bool slow = int64_t(strides) * p.B * kC > 2 * p.tokens;
  const dim3 grid = slow ? dim3(unsigned(p.Hv / vh), unsigned(p.B), strides) : dim3(strides, unsigned(p.Hv / vh), unsigned(p.B));
  auto launch = [&](auto kernel) { hipLaunchKernelGGL(kernel, grid, dim3(64), 0, stream, p); };
  if (vh == 2) {
    if (factor) slow ? launch(chunk_kernel<2, true, true>) : launch(chunk_kernel<2, true, false>);
    else slow ? launch(chunk_kernel<2, false, true>) : launch(chunk_kernel<2, false, false>);
  } else {
    if (factor) slow ? launch(chunk_kernel<1, true, true>) : launch(chunk_kernel<1, true, false>);
    else slow ? launch(chunk_kernel<1, false, true>) : launch(chunk_kernel<1, false, false>);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return state == Dt::F32 ? launch_pass2<float>(p, stream) : launch_pass2<bf16s>(p, stream);
}

}  // namespace gdn
