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
// contraction, on v_mfma_f32_16x16x16_bf16 with fp32 accumulation.
//
// Design for gfx950:
// - Pass 1 (chunk_kernel) computes, for every (chunk, v-head) in parallel, everything that
//   does not depend on the state -- W = Tm diag(beta Gam rk) K, Tm diag(beta), the output
//   mask P, K^T and the per-token factors -- into a workspace record. That is most of a
//   chunk's instructions, and none of it is sequential.
// - Pass 2 (scan_kernel) walks each sequence's chunks in order with the state in MFMA
//   accumulators: U~ = Tm diag(beta) V, W S_0, Q S_0, P U and the state update only. The
//   next chunk's record and queries are loaded while the current chunk computes.
// - One pass-2 wave per (sequence, v-head, block of NB value columns): columns are
//   independent given the record. A 16 x 16 accumulator tile holds, per lane, four
//   consecutive rows of one column -- the B-operand layout -- so S_0 feeds W S_0 and
//   Q S_0 after a bf16 conversion in registers.
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
constexpr int kStr = kDK + 8; // LDS row stride (bf16) of 128-wide chunk matrices, padded
constexpr int kTS = kC + 4;   // LDS row stride (bf16) of the transposed chunk matrices

// Workspace record of one (chunk, v-head): byte offsets (prefill_record_bytes(d_v) in total).
// Every matrix is stored in the lane layout of the matrix-core operand that reads it, so
// a pass-2 lane fetches its part with one 8- or 16-byte load.
constexpr int kRecW = 0;       // -W, A operand of 16x16x32: [32-key block m][lane][8 bf16]
constexpr int kRecKT = 4096;   // K^T, A operand of 16x16x16: [16-key tile][lane][4 bf16]
constexpr int kRecTV = 8192;   // Tm diag(beta), A operand: [lane][4 bf16]
constexpr int kRecP = 8704;    // P = M o (rq rk) Q K^T, A operand: [lane][4 bf16]
constexpr int kRecF = 9216;    // f_t = rk_t Gam_C / Gam_t [16] fp32
constexpr int kRecGQ = 9280;   // Gam_t rq_t [16] fp32
constexpr int kRecGC = 9344;   // Gam_C fp32
constexpr int kRecV = 9472;    // V, B operand of 16x16x16 by 16-column blocks: [block][lane][4 bf16]
static_assert(kRecGC + 4 <= kRecV && kRecV == kPrefillRecordFixed && kRecV % 256 == 0, "record layout");
constexpr int kVSegMax = 8;    // 16-byte value segments per lane and chunk (d_v <= 256)

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

// ============================================================ pass 1: chunk records
struct __attribute__((aligned(16))) ChunkLds {
  uint16_t k[kC * kStr];   // the chunk's keys (stored bf16 values; zero rows past the end)
  uint16_t q[kC * kStr];   // queries
  uint16_t w[kC * kStr];   // W, bf16
  uint16_t kt[kDK * kTS];  // K^T
  uint16_t tw[kC * kC];    // Tm diag(beta Gam rk), bf16
  uint16_t tv[kC * kC];    // Tm diag(beta), bf16
  uint16_t pm[kC * kC];    // P, bf16
  float a[kC * kC];        // A (fp32) for the triangular solve
  float rk[kC], rq[kC], beta[kC], G[kC];
};

// grid (chunk strides, v-heads, sequences), one wave each; wave x handles chunks x,
// x + gridDim.x, ... of its sequence.
__global__ __launch_bounds__(64) void chunk_kernel(const PrefillArgs p) {
  __shared__ ChunkLds L;
  const int h = blockIdx.y, row = blockIdx.z;
  const int l = threadIdx.x, l16 = l & 15, l4 = l >> 4;
  const int32_t slot = p.idx[row];
  if (slot < 0 || slot >= p.P) return;  // padding rows have no chunks to prepare
  const int32_t t0 = p.cu[row], t1 = p.cu[row + 1];
  const int nchunks = (t1 - t0 + kC - 1) / kC;
  const int kh = h / p.G;
  const uint16_t* qg = static_cast<const uint16_t*>(p.q);
  const uint16_t* kg = static_cast<const uint16_t*>(p.k);
  const uint16_t* ag = static_cast<const uint16_t*>(p.a);
  const uint16_t* bg = static_cast<const uint16_t*>(p.b);
  const float A_neg = -expf(p.A_log[h]), dtb = p.dt_bias[h];

  for (int j = blockIdx.x; j < nchunks; j += gridDim.x) {
    const int64_t rid = record_id(t0, row, j);
    if (rid >= p.records) return;  // workspace too small for the tokens: write nothing
    char* rec = static_cast<char*>(p.work) + (rid * p.Hv + h) * p.rec_bytes;
    const int cs = t0 + j * kC, n = min(kC, t1 - cs), last = t1 - 1;
    // the chunk's values, 16-byte segments: segment s = l + 64 i is token s / (d_v / 8),
    // columns 8 (s % (d_v / 8)) .. + 7 (rows past the end meet zero columns of Tm diag(beta))
    const int vsegs = p.DV / 8;
    u32x4 vv[kVSegMax];
#pragma unroll
    for (int i = 0; i < kVSegMax; ++i) {
      const int sgi = min(l + 64 * i, kC * vsegs - 1);
      vv[i] = *reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.v) +
                                              (size_t(min(cs + sgi / vsegs, last)) * p.Hv + h) * p.DV +
                                              8 * (sgi % vsegs));
    }
    // ---- 1. stage k and q rows (256 B each, zero past the end), K^T; gates and the
    //         inclusive prefix sum of the log-decays (no decay, no write past the end)
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int t = it * 4 + l4, seg = l16;
      const size_t src = (size_t(min(cs + t, last)) * p.Hk + kh) * kDK + 8 * seg;
      u32x4 kk = *reinterpret_cast<const u32x4*>(kg + src);
      u32x4 qq = *reinterpret_cast<const u32x4*>(qg + src);
      if (t >= n) kk = qq = u32x4{0u, 0u, 0u, 0u};
      *reinterpret_cast<uint2*>(L.k + t * kStr + 8 * seg) = uint2{kk.x, kk.y};
      *reinterpret_cast<uint2*>(L.k + t * kStr + 8 * seg + 4) = uint2{kk.z, kk.w};
      *reinterpret_cast<uint2*>(L.q + t * kStr + 8 * seg) = uint2{qq.x, qq.y};
      *reinterpret_cast<uint2*>(L.q + t * kStr + 8 * seg + 4) = uint2{qq.z, qq.w};
      const uint32_t kw[4] = {kk.x, kk.y, kk.z, kk.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        L.kt[(8 * seg + 2 * e) * kTS + t] = uint16_t(kw[e]);
        L.kt[(8 * seg + 2 * e + 1) * kTS + t] = uint16_t(kw[e] >> 16);
      }
    }
    {
      const bool live = l16 < n;
      const size_t tg = size_t(min(cs + l16, last)) * p.Hv + h;
      const float x = bf(ag[tg]) + dtb;
      float lg = live ? A_neg * (fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)))) : 0.f;
      const float be = live ? 1.f / (1.f + expf(-bf(bg[tg]))) : 0.f;
#pragma unroll
      for (int d = 1; d < kC; d *= 2) {
        const float y = __shfl_up(lg, d);
        if (l16 >= d) lg += y;
      }
      if (l < kC) {
        L.G[l] = lg;
        L.beta[l] = be;
      }
    }
    lds_sync();
    // ---- 2. inverse L2 norms, 4 lanes per token, 16-byte LDS reads
    {
      const int t = l >> 2, part = l & 3;
      float sk = 0.f, sq = 0.f;
#pragma unroll
      for (int e8 = 0; e8 < 4; ++e8) {
        const u32x4 kk = *reinterpret_cast<const u32x4*>(L.k + t * kStr + 32 * part + 8 * e8);
        const u32x4 qq = *reinterpret_cast<const u32x4*>(L.q + t * kStr + 32 * part + 8 * e8);
        float kf[8], qf[8];
        unpack_io(kk, kf, static_cast<const bf16s*>(nullptr));
        unpack_io(qq, qf, static_cast<const bf16s*>(nullptr));
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          sk = fmaf(kf[e], kf[e], sk);
          sq = fmaf(qf[e], qf[e], sq);
        }
      }
      sk += __shfl_xor(sk, 1); sk += __shfl_xor(sk, 2);
      sq += __shfl_xor(sq, 1); sq += __shfl_xor(sq, 2);
      if (part == 0) {
        L.rk[t] = 1.f / sqrtf(sk + p.eps);
        L.rq[t] = 1.f / sqrtf(sq + p.eps);
      }
    }
    lds_sync();
    // ---- 3. K K^T and Q K^T (contraction over d_k); A (strict lower) and P (lower)
    f32x4 KK = {0.f, 0.f, 0.f, 0.f}, QK = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kt = 0; kt < kKT; ++kt) {
      const s16x4 kA = ld4(L.k, l16, kStr, 16 * kt + 4 * l4);
      const s16x4 qA = ld4(L.q, l16, kStr, 16 * kt + 4 * l4);
      KK = mfma(kA, kA, KK);
      QK = mfma(qA, kA, QK);
    }
    {
      const int s = l16;
      const float rks = L.rk[s], Gs = L.G[s];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int t = 4 * l4 + i;
        const float dec = (s <= t) ? expf(L.G[t] - Gs) : 0.f;
        L.a[t * kC + s] = (s < t) ? L.beta[t] * L.rk[t] * rks * dec * KK[i] : 0.f;
        L.pm[t * kC + s] = to_bf(L.rq[t] * rks * dec * QK[i]);
      }
    }
    lds_sync();
    // ---- 4. Tm = (I + A)^-1 by forward substitution, one column per lane (lanes < 16),
    //         column-oriented: once x[s] is final it updates every later row at once
    if (l < kC) {
      const int c = l;
      float x[kC];
#pragma unroll
      for (int t = 0; t < kC; ++t) x[t] = (t == c) ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < kC - 1; ++s)
#pragma unroll
        for (int t = s + 1; t < kC; ++t) x[t] = fmaf(-L.a[t * kC + s], x[s], x[t]);
      const float cw = -L.beta[c] * expf(L.G[c]) * L.rk[c], cv = L.beta[c];
#pragma unroll
      for (int t = 0; t < kC; ++t) {
        L.tw[t * kC + c] = to_bf(x[t] * cw);
        L.tv[t * kC + c] = to_bf(x[t] * cv);
      }
    }
    lds_sync();
    // ---- 5. -W = -Tm diag(beta Gam rk) K (16 x 128); the K^T operands are the record's
    {
      const s16x4 twA = ld4(L.tw, l16, kC, 4 * l4);
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt) {
        const s16x4 kB = ld4(L.kt, 16 * kt + l16, kTS, 4 * l4);
        *reinterpret_cast<s16x4*>(rec + kRecKT + kt * 512 + l * 8) = kB;
        const f32x4 W = mfma(twA, kB, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) L.w[(4 * l4 + i) * kStr + 16 * kt + l16] = to_bf(W[i]);
      }
    }
    lds_sync();
    // ---- 6. the rest of the record: -W by 32-key blocks (lane (t, g) holds keys
    //         32m + 4g .. 4g+3 and 32m + 16 + 4g .. 4g+3 of row t), Tm diag(beta), P, factors
#pragma unroll
    for (int m = 0; m < kKT / 2; ++m) {
      const s16x4 lo = ld4(L.w, l16, kStr, 32 * m + 4 * l4), hi = ld4(L.w, l16, kStr, 32 * m + 16 + 4 * l4);
      *reinterpret_cast<s16x8*>(rec + kRecW + m * 1024 + l * 16) = cat8(lo, hi);
    }
    *reinterpret_cast<s16x4*>(rec + kRecTV + l * 8) = ld4(L.tv, l16, kC, 4 * l4);
    *reinterpret_cast<s16x4*>(rec + kRecP + l * 8) = ld4(L.pm, l16, kC, 4 * l4);
    // V^T blocks through the K^T buffer (free after step 5), 128 columns at a time
    for (int c128 = 0; c128 < p.DV; c128 += kDK) {
#pragma unroll
      for (int i = 0; i < kVSegMax; ++i) {
        const int sgi = l + 64 * i, t = sgi / vsegs, col = 8 * (sgi % vsegs) - c128;
        if (sgi < kC * vsegs && col >= 0 && col < kDK) {
          const uint32_t w4[4] = {vv[i].x, vv[i].y, vv[i].z, vv[i].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            L.kt[(col + 2 * e) * kTS + t] = uint16_t(w4[e]);
            L.kt[(col + 2 * e + 1) * kTS + t] = uint16_t(w4[e] >> 16);
          }
        }
      }
      lds_sync();
      const int nb = min(kDK, p.DV - c128) / 16;
      for (int b = 0; b < nb; ++b)
        *reinterpret_cast<s16x4*>(rec + kRecV + (c128 / 16 + b) * 512 + l * 8) = ld4(L.kt, 16 * b + l16, kTS, 4 * l4);
      lds_sync();
    }
    if (l < kC) {
      const float Gl = L.G[kC - 1], Gt = L.G[l];
      reinterpret_cast<float*>(rec + kRecF)[l] = L.rk[l] * expf(Gl - Gt);
      reinterpret_cast<float*>(rec + kRecGQ)[l] = expf(Gt) * L.rq[l];
      if (l == 0) *reinterpret_cast<float*>(rec + kRecGC) = expf(Gl);
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

// Partial products of the KS waves of a workgroup, double-buffered by chunk parity (one
// barrier per chunk: a wave writes buffer j & 1 only after the barrier of chunk j - 1,
// which every wave passes after its reads of chunk j - 2), and the output tile.
template <int KS>
struct __attribute__((aligned(16))) ScanLds {
  f32x4 u[2][KS][64];   // U partials: wave 0 holds Tm diag(beta) V - W S_0 over its keys
  f32x4 qs[2][KS][64];  // Q S_0 partials
  uint16_t o[kC * 16];  // the chunk's 16 x 16 output tile, bf16
};

// One chunk's operands for wave `wk` (keys 128/KS * wk ..), loaded one to two chunks ahead.
template <int KS>
struct ChunkOps {
  static constexpr int KT = kKT / KS, KM = KT / 2;
  s16x8 w[KM];   // -W, A layout of 16x16x32
  s16x8 q[KM];   // Q (stored values), same layout
  s16x4 kt[KT];  // K^T, A layout of 16x16x16
  s16x4 tv, pm;  // Tm diag(beta) and P, A layout
  s16x4 v;       // V, B layout (tokens 4 l4 .. of column l16)
  f32x4 f, gq;   // factors of tokens 4 l4 .. 4 l4 + 3
  float gc;
};

constexpr int kXcds = 8;  // workgroups go to the chip's 8 XCDs round-robin by linear id

// One workgroup per (sequence, v-head, block of 16 value columns); KS waves per workgroup
// split the key dimension: wave wk holds S rows 128/KS * wk .. as 16-key tiles. io is bf16.
// 1-D grid, XCD-aware: the column blocks of a (sequence, v-head) read the same records,
// so they are given ids on one XCD (id % 8 equal) and share its L2. Head unit u (=
// row * Hv + h) and column block cb take id (u % 8) + 8 (cb + nb (u / 8)).
template <typename ST, int KS>
__global__ __launch_bounds__(64 * KS) void scan_kernel(const PrefillArgs p) {
  constexpr int KT = kKT / KS, KM = KT / 2;
  static_assert(KM >= 1, "at least one 32-key block per wave");
  __shared__ ScanLds<KS> L;
  const int l = threadIdx.x & 63, l16 = l & 15, l4 = l >> 4;
  const int wk = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nb = p.DV / 16;
  const int rest = int(blockIdx.x) / kXcds, cb = rest % nb;
  const int u = (rest / nb) * kXcds + int(blockIdx.x) % kXcds;
  if (u >= p.B * p.Hv) return;  // the padding of the last group of 8 head units
  const int c0 = cb * 16, h = u % p.Hv, row = u / p.Hv;
  const int32_t slot = p.idx[row];
  const int32_t fresh = p.fresh ? p.fresh[row] : 0;
  const int32_t t0 = p.cu[row], t1 = p.cu[row + 1];
  const int kh = h / p.G;
  const uint16_t* qg = static_cast<const uint16_t*>(p.q);
  uint16_t* og = static_cast<uint16_t*>(p.o);

  if (slot < 0 || slot >= p.P) {  // padding row: o = 0 for its tokens, no state access
    for (int t = t0 + wk * 32 + (l >> 1); t < t1; t += 32 * KS)
      *reinterpret_cast<u32x4*>(og + (size_t(t) * p.Hv + h) * p.DV + c0 + 8 * (l & 1)) = u32x4{0u, 0u, 0u, 0u};
    return;
  }

  // the state: tile kt of lane l holds S[key0 + 16kt + 4 l4 + i][c0 + l16]
  const int key0 = wk * (kDK / KS);
  ST* const pool_tile = static_cast<ST*>(p.pool) + (size_t(slot) * p.Hv + h) * size_t(p.DV) * kDK;
  ST* const my_state = pool_tile + size_t(c0 + l16) * kDK + key0 + 4 * l4;
  f32x4 S[KT];
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) {
    const f32x4 s = load_state<ST>(my_state + 16 * kt);  // unconditional, then masked
    S[kt] = fresh ? f32x4{0.f, 0.f, 0.f, 0.f} : s;
  }

  const int nchunks = (t1 - t0 + kC - 1) / kC;
  const int64_t rid0 = record_id(t0, row, 0);
  const int last = max(t1 - 1, 0);
  // Uniform bases and 32-bit lane byte offsets (the host bounds every token tensor below
  // 2^31 elements), so the loads take a scalar base and keep their lane offsets in VGPRs
  // that do not change from chunk to chunk.
  const char* qbase = reinterpret_cast<const char*>(qg + size_t(kh) * kDK + key0);
  const uint32_t qrow_b = uint32_t(p.Hk) * kDK * 2u;
  const uint32_t o_w = uint32_t(kRecW + wk * KM * 1024 + l * 16), o_kt = uint32_t(kRecKT + wk * KT * 512 + l * 8);
  const uint32_t o_ab = uint32_t(l * 8), o_fg = uint32_t(16 * l4), o_v = uint32_t(kRecV + cb * 512 + l * 8);
  // Every load is unconditional: the record index and the tokens are clamped into range
  // (a load in a branch is waited on at the branch end). Operands of tokens past the end
  // meet zero columns of Tm diag(beta) and of P, zero rows of K^T, or outputs not stored.
  auto fetch = [&](int j) -> ChunkOps<KS> {
    ChunkOps<KS> c;
    const int64_t rid = min(rid0 + j, p.records - 1);
    const char* rec = static_cast<const char*>(p.work) + (rid * p.Hv + h) * p.rec_bytes;
    const int cs = t0 + j * kC;
    const uint32_t oq = uint32_t(min(cs + l16, last)) * qrow_b + 8u * l4;
#pragma unroll
    for (int m = 0; m < KM; ++m) {
      c.w[m] = *reinterpret_cast<const s16x8*>(rec + o_w + m * 1024);
      c.q[m] = cat8(*reinterpret_cast<const s16x4*>(qbase + oq + 64 * m),
                    *reinterpret_cast<const s16x4*>(qbase + oq + 64 * m + 32));
    }
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) c.kt[kt] = *reinterpret_cast<const s16x4*>(rec + o_kt + kt * 512);
    c.tv = *reinterpret_cast<const s16x4*>(rec + kRecTV + o_ab);
    c.pm = *reinterpret_cast<const s16x4*>(rec + kRecP + o_ab);
    c.f = *reinterpret_cast<const f32x4*>(rec + kRecF + o_fg);
    c.gq = *reinterpret_cast<const f32x4*>(rec + kRecGQ + o_fg);
    c.gc = *reinterpret_cast<const float*>(rec + kRecGC);
    c.v = *reinterpret_cast<const s16x4*>(rec + o_v);
    return c;
  };

  auto step = [&](const ChunkOps<KS>& c, int j) {
    const int cs = t0 + j * kC, n = min(kC, t1 - cs), buf = j & 1;
    // ---- U partial = [wave 0: Tm diag(beta) V] - W S_0 and Q S_0 over the wave's keys
    f32x4 u = (wk == 0) ? mfma(c.tv, c.v, f32x4{0.f, 0.f, 0.f, 0.f}) : f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 qs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < KM; ++m) {
      const f32x4 a = S[2 * m], b = S[2 * m + 1];
      const s16x8 sB = cat8(bf16x4(a.x, a.y, a.z, a.w), bf16x4(b.x, b.y, b.z, b.w));
      u = mfma32(c.w[m], sB, u);
      qs = mfma32(c.q[m], sB, qs);
    }
    if constexpr (KS > 1) {  // sum the partials in wave order (every wave gets the same U)
      L.u[buf][wk][l] = u;
      L.qs[buf][wk][l] = qs;
      asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
      u = L.u[buf][0][l];
#pragma unroll
      for (int w = 1; w < KS; ++w) u += L.u[buf][w][l];
      if (wk == KS - 1) {
        qs = L.qs[buf][0][l];
#pragma unroll
        for (int w = 1; w < KS; ++w) qs += L.qs[buf][w][l];
      }
    }
    // ---- O = scale (diag(Gam rq) Q S_0 + P U), by the last wave, 16-byte stores from LDS
    if (wk == KS - 1) {
      const f32x4 pu = mfma(c.pm, bf16x4(u.x, u.y, u.z, u.w), f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int i = 0; i < 4; ++i) L.o[(4 * l4 + i) * 16 + l16] = to_bf(p.scale * (c.gq[i] * qs[i] + pu[i]));
      lds_sync();
      if (l < 2 * kC) {
        const int t = l >> 1, half = l & 1;
        const u32x4 ov = *reinterpret_cast<const u32x4*>(L.o + t * 16 + 8 * half);
        if (t < n) *reinterpret_cast<u32x4*>(og + (size_t(cs + t) * p.Hv + h) * p.DV + c0 + 8 * half) = ov;
      }
      lds_sync();
    }
    // ---- S <- Gam_C S_0 + K^T diag(rk Gam_C / Gam) U over the wave's keys
    const s16x4 uB = bf16x4(c.f[0] * u[0], c.f[1] * u[1], c.f[2] * u[2], c.f[3] * u[3]);
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) S[kt] = mfma(c.kt[kt], uB, S[kt] * c.gc);
  };

  // two chunks in flight: the operands of chunk j + 2 load while chunk j computes. The
  // loads are kept after the step that frees their registers: the empty asm takes the
  // updated state (so the step's last products are done) and clobbers memory (so no load
  // moves above it). Hoisted above the step, the loads would need fresh registers and
  // copies at the loop's back edge, and a copy waits for its load.
  auto fence = [&]() {
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) asm volatile("" : "+v"(S[kt])::"memory");
  };
  // chunks with a record (all of them unless the workspace is too small for the tokens)
  const int nrun = int(max<int64_t>(0, min<int64_t>(nchunks, p.records - rid0)));
  if (nrun > 0) {
    ChunkOps<KS> c0p = fetch(0), c1p = fetch(1);
    int j = 0;
    if (nrun & 1) {  // an odd count: the first chunk alone, then pairs
      step(c0p, 0);
      c0p = c1p;
      c1p = fetch(2);
      j = 1;
    }
    // Start the loop with nothing in flight (the first step needs its operands anyway):
    // the wait counts inside the loop then follow from its own loads alone.
    __builtin_amdgcn_s_waitcnt(0);
    for (; j < nrun; j += 2) {  // no exit inside the pair: nothing sinks into the next one
      step(c0p, j);
      fence();
      c0p = fetch(j + 2);
      step(c1p, j + 1);
      fence();
      c1p = fetch(j + 3);
    }
  }

  // ---- the final state back to the slot (rounded once for a bf16 pool)
#pragma unroll
  for (int kt = 0; kt < KT; ++kt) store_state(my_state + 16 * kt, S[kt]);
}

template <typename ST, int KS>
hipError_t launch_scan(const PrefillArgs& p, hipStream_t stream) {
  const int64_t units = (int64_t(p.B) * p.Hv + kXcds - 1) / kXcds * kXcds;
  const dim3 grid(unsigned(units * (p.DV / 16)));
  hipLaunchKernelGGL((scan_kernel<ST, KS>), grid, dim3(64 * KS), 0, stream, p);
  return hipGetLastError();
}

// One wave per 16 value columns measured fastest down to 512 such tiles (half a wave per
// SIMD), the key split's partial sums costing more than its shorter chain saves; the split
// is kept for grids too small to give every SIMD work.
template <typename ST>
hipError_t launch_scan_split(const PrefillArgs& p, hipStream_t stream) {
  const int64_t tiles = int64_t(p.B) * p.Hv * (p.DV / 16);
  if (tiles >= 256) return launch_scan<ST, 1>(p, stream);
  if (tiles >= 128) return launch_scan<ST, 2>(p, stream);
  return launch_scan<ST, 4>(p, stream);
}

}  // namespace

// Pass 1 gets enough waves to fill the chip whatever the batch: each (sequence, v-head)
// gets `strides` waves that share its chunks. Pass 2 splits the key dimension over 2 or 4
// waves only when one wave per 16 value columns would leave most SIMDs idle.
hipError_t launch_prefill(Dt state, const PrefillArgs& p, hipStream_t stream) {
  const int64_t heads = int64_t(p.B) * p.Hv;
  const unsigned strides = unsigned(std::min<int64_t>(1024, std::max<int64_t>(1, (4096 + heads - 1) / heads)));
  hipLaunchKernelGGL(chunk_kernel, dim3(strides, unsigned(p.Hv), unsigned(p.B)), dim3(64), 0, stream, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return state == Dt::F32 ? launch_scan_split<float>(p, stream) : launch_scan_split<bf16s>(p, stream);
}

}  // namespace gdn
