// gdn_prefill.hip -- gfx950 chunked prefill of the Gated DeltaNet state from pooled initial
// states, on the bf16 matrix cores.
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
// contraction, so it runs on v_mfma_f32_16x16x16_bf16 with fp32 accumulation.
//
// Design for gfx950:
// - one wave64 per (sequence, v-head, block of 32 value columns): the value columns of the
//   delta rule are independent given K, beta and the decays, so column blocks need no
//   communication; the k-side matrices (K K^T, Q K^T, Tm, W) are recomputed per block;
// - the 128 x 32 fp32 state lives in MFMA accumulators for the whole sequence (16 tiles of
//   16 x 16, 64 floats per lane). A 16 x 16 accumulator tile holds, per lane, four
//   consecutive rows of one column -- exactly the B-operand layout of the next MFMA -- so
//   S_0 feeds W S_0 and Q S_0 after a bf16 conversion in registers, with no data movement;
// - keys and queries enter the products as their stored bf16 values; the L2 norms, gates
//   and decays are applied as fp32 diagonal scalings of the small chunk matrices;
// - 16-token chunks keep the unit-triangular solve to 16 sequential steps per column in
//   registers; chunk staging and layout changes go through a wave-private LDS area.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gdn.h"
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kC = 16;        // tokens per chunk
constexpr int kDK = 128;      // key dimension
constexpr int kKT = kDK / 16; // 16-row tiles of the key dimension
constexpr int kStr = kDK + 8; // LDS row stride (bf16) of 128-wide chunk matrices, padded
constexpr int kTS = kC + 4;   // LDS row stride (bf16) of the transposed chunk matrices

__device__ __forceinline__ f32x4 mfma(const s16x4& a, const s16x4& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ s16x4 bf16x4(float a, float b, float c, float d) {
  const uint64_t lo = pack_bf16x2(a, b), hi = pack_bf16x2(c, d);
  return __builtin_bit_cast(s16x4, (hi << 32) | lo);
}

__device__ __forceinline__ float bf(uint16_t x) { return __uint_as_float(uint32_t(x) << 16); }

// Phase boundary of the one-wave workgroup: a wave's LDS operations complete in order, so
// it is enough that its own LDS accesses have retired (and that the compiler does not move
// memory accesses across). A __syncthreads() here would also wait for the next chunk's
// global loads still in flight.
__device__ __forceinline__ void lds_sync() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

__device__ __forceinline__ uint16_t to_bf(float x) { return uint16_t(pack_bf16x2(x, 0.f)); }

// four bf16 of one row at column c (8-byte aligned)
__device__ __forceinline__ s16x4 ld4(const uint16_t* base, int row, int stride, int c) {
  return *reinterpret_cast<const s16x4*>(base + row * stride + c);
}

template <int kNB>
struct __attribute__((aligned(16))) PrefillLds {
  uint16_t k[kC * kStr];   // the chunk's keys (stored bf16 values; zero rows past the end)
  uint16_t q[kC * kStr];   // queries
  uint16_t w[kC * kStr];   // W = Tm diag(beta Gam rk) K, bf16
  uint16_t kt[kDK * kTS];  // K^T: the keys by dimension, for column operands
  uint16_t vt[kNB * kTS];  // V^T: the wave's value columns by column
  uint16_t tw[kC * kC];    // Tm diag(beta Gam rk), bf16
  uint16_t tv[kC * kC];    // Tm diag(beta), bf16
  uint16_t pm[kC * kC];    // P = M o (rq rk) Q K^T, bf16
  uint16_t o[kC * kNB];    // the chunk's outputs, bf16, for 16-byte stores
  float a[kC * kC];        // A (fp32) for the triangular solve
  float rk[kC], rq[kC], beta[kC], G[kC];
};

template <typename ST>
__device__ __forceinline__ void load_state(const ST* src, f32x4& s);
template <>
__device__ __forceinline__ void load_state<float>(const float* src, f32x4& s) {
  s = *reinterpret_cast<const f32x4*>(src);
}
template <>
__device__ __forceinline__ void load_state<bf16s>(const bf16s* src, f32x4& s) {
  const uint2 u = *reinterpret_cast<const uint2*>(src);
  s = f32x4{bf16_lo(u.x), bf16_hi(u.x), bf16_lo(u.y), bf16_hi(u.y)};
}
__device__ __forceinline__ void store_state(float* dst, const f32x4& s) { *reinterpret_cast<f32x4*>(dst) = s; }
__device__ __forceinline__ void store_state(bf16s* dst, const f32x4& s) {
  *reinterpret_cast<uint2*>(dst) = uint2{pack_bf16x2(s.x, s.y), pack_bf16x2(s.z, s.w)};
}

// grid (value blocks of kNB columns, v-heads, sequences), one wave each. io is bf16.
template <typename ST, int kNB>
__global__ __launch_bounds__(64) void prefill_kernel(const PrefillArgs p) {
  constexpr int kNT = kNB / 16;  // 16-column tiles of the wave's value block
  __shared__ PrefillLds<kNB> L;
  const int vb = blockIdx.x, h = blockIdx.y, row = blockIdx.z;
  const int l = threadIdx.x, l16 = l & 15, l4 = l >> 4;
  const int c0 = vb * kNB;
  const int32_t slot = p.idx[row];
  const int32_t fresh = p.fresh ? p.fresh[row] : 0;
  const int32_t t0 = p.cu[row], t1 = p.cu[row + 1];
  const int kh = h / p.G;
  const uint16_t* qg = static_cast<const uint16_t*>(p.q);
  const uint16_t* kg = static_cast<const uint16_t*>(p.k);
  const uint16_t* vg = static_cast<const uint16_t*>(p.v);
  const uint16_t* ag = static_cast<const uint16_t*>(p.a);
  const uint16_t* bg = static_cast<const uint16_t*>(p.b);
  uint16_t* og = static_cast<uint16_t*>(p.o);

  if (slot < 0 || slot >= p.P) {  // padding row: o = 0 for its tokens, no state access
    for (int t = t0 + l / (kNB / 8); t < t1; t += 64 / (kNB / 8))
      *reinterpret_cast<u32x4*>(og + (size_t(t) * p.Hv + h) * p.DV + c0 + 8 * (l % (kNB / 8))) =
          u32x4{0u, 0u, 0u, 0u};
    return;
  }

  // ---- the state block: tile (kt, nt) of lane l holds S[16kt + 4 l4 + i][c0 + 16nt + l16]
  ST* const pool_tile = static_cast<ST*>(p.pool) + (size_t(slot) * p.Hv + h) * size_t(p.DV) * kDK;
  f32x4 S[kKT][kNT];
#pragma unroll
  for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      S[kt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (!fresh) load_state<ST>(pool_tile + size_t(c0 + 16 * nt + l16) * kDK + 16 * kt + 4 * l4, S[kt][nt]);
    }

  const float A_neg = -expf(p.A_log[h]), dtb = p.dt_bias[h];

  // The chunk's raw inputs, loaded one chunk ahead: the loads of chunk i+1 are in flight
  // while chunk i computes. Token indices are clamped into the sequence, so every load
  // is unconditional (a load in a branch is waited on at the branch end).
  u32x4 kr[4], qr[4], vr;
  uint16_t ar, br;
  auto fetch = [&](int cs_) {
    const int last = t1 - 1;
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const size_t src = (size_t(min(cs_ + it * 4 + l4, last)) * p.Hk + kh) * kDK + 8 * l16;
      kr[it] = *reinterpret_cast<const u32x4*>(kg + src);
      qr[it] = *reinterpret_cast<const u32x4*>(qg + src);
    }
    vr = *reinterpret_cast<const u32x4*>(vg + (size_t(min(cs_ + l / (kNB / 8), last)) * p.Hv + h) * p.DV + c0 +
                                          8 * (l % (kNB / 8)));
    const size_t tg = size_t(min(cs_ + l16, last)) * p.Hv + h;
    ar = ag[tg];
    br = bg[tg];
  };
  if (t1 > t0) fetch(t0);

  for (int cs = t0; cs < t1; cs += kC) {
    const int n = min(kC, t1 - cs);
    // ---- 1. stage the chunk: k and q rows (256 B each), the wave's 32 value columns;
    //         gates of token l (l < 16); tokens past the end: zero inputs, no decay, no write
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int t = it * 4 + l4, seg = l16;
      const u32x4 kk = (t < n) ? kr[it] : u32x4{0u, 0u, 0u, 0u};
      const u32x4 qq = (t < n) ? qr[it] : u32x4{0u, 0u, 0u, 0u};
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
    if (l < kC * (kNB / 8)) {
      const int t = l / (kNB / 8), seg = l % (kNB / 8);
      const u32x4 vv = (t < n) ? vr : u32x4{0u, 0u, 0u, 0u};
      const uint32_t vw[4] = {vv.x, vv.y, vv.z, vv.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        L.vt[(8 * seg + 2 * e) * kTS + t] = uint16_t(vw[e]);
        L.vt[(8 * seg + 2 * e + 1) * kTS + t] = uint16_t(vw[e] >> 16);
      }
    }
    {  // gates of token l (lanes < 16) and the inclusive prefix sum of the log-decays
      const bool live = l < n;
      const float x = bf(ar) + dtb;
      float lg = live ? A_neg * (fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)))) : 0.f;
#pragma unroll
      for (int d = 1; d < kC; d *= 2) {
        const float y = __shfl_up(lg, d);
        if (l16 >= d) lg += y;
      }
      if (l < kC) {
        L.G[l] = lg;
        L.beta[l] = live ? 1.f / (1.f + expf(-bf(br))) : 0.f;
      }
    }
    fetch(cs + kC);  // the next chunk (clamped: harmless past the end)
    lds_sync();
    // ---- 2. inverse L2 norms (4 lanes per token) and the cumulative log-decay
    {  // inverse L2 norms, 4 lanes per token, 16-byte LDS reads
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
    // ---- 3. K K^T and Q K^T (16 x 16, contraction over d_k = 128)
    f32x4 KK = {0.f, 0.f, 0.f, 0.f}, QK = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < kKT; ++j) {
      const s16x4 kA = ld4(L.k, l16, kStr, 16 * j + 4 * l4);
      const s16x4 qA = ld4(L.q, l16, kStr, 16 * j + 4 * l4);
      KK = mfma(kA, kA, KK);
      QK = mfma(qA, kA, QK);
    }
    // entries (t = 4 l4 + i, s = l16): A (strict lower) and P (lower with diagonal)
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
    //         column-oriented: once x[s] is final it is applied to every later row at once,
    //         so the dependent chain is 15 steps deep instead of 120
    if (l < kC) {
      const int c = l;
      float x[kC];
#pragma unroll
      for (int t = 0; t < kC; ++t) x[t] = (t == c) ? 1.f : 0.f;
#pragma unroll
      for (int s = 0; s < kC - 1; ++s)
#pragma unroll
        for (int t = s + 1; t < kC; ++t) x[t] = fmaf(-L.a[t * kC + s], x[s], x[t]);
      const float cw = L.beta[c] * expf(L.G[c]) * L.rk[c], cv = L.beta[c];
#pragma unroll
      for (int t = 0; t < kC; ++t) {
        L.tw[t * kC + c] = to_bf(x[t] * cw);
        L.tv[t * kC + c] = to_bf(x[t] * cv);
      }
    }
    lds_sync();
    // ---- 5. W = Tm diag(beta Gam rk) K  (16 x 128) and U~ = Tm diag(beta) V  (16 x 32)
    {
      const s16x4 twA = ld4(L.tw, l16, kC, 4 * l4);
#pragma unroll
      for (int j = 0; j < kKT; ++j) {
        const f32x4 W = mfma(twA, ld4(L.kt, 16 * j + l16, kTS, 4 * l4), f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) L.w[(4 * l4 + i) * kStr + 16 * j + l16] = to_bf(W[i]);
      }
    }
    f32x4 U[kNT];
    {
      const s16x4 tvA = ld4(L.tv, l16, kC, 4 * l4);
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt)
        U[nt] = mfma(tvA, ld4(L.vt, 16 * nt + l16, kTS, 4 * l4), f32x4{0.f, 0.f, 0.f, 0.f});
    }
    lds_sync();
    // ---- 6. U = U~ - W S_0 and Q S_0, with S_0 converted to bf16 B operands in place
    f32x4 QS[kNT];
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt) {
      f32x4 ws = {0.f, 0.f, 0.f, 0.f}, qs = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt) {
        const f32x4 s = S[kt][nt];
        const s16x4 sB = bf16x4(s.x, s.y, s.z, s.w);
        ws = mfma(ld4(L.w, l16, kStr, 16 * kt + 4 * l4), sB, ws);
        qs = mfma(ld4(L.q, l16, kStr, 16 * kt + 4 * l4), sB, qs);
      }
      U[nt] = U[nt] - ws;
      QS[nt] = qs;
    }
    // ---- 7. O = scale (diag(Gam rq) Q S_0 + P U), staged in LDS for 16-byte stores
    {
      const s16x4 pA = ld4(L.pm, l16, kC, 4 * l4);
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        const f32x4 pu = mfma(pA, bf16x4(U[nt].x, U[nt].y, U[nt].z, U[nt].w), f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 4 * l4 + i;
          const float ov = p.scale * (expf(L.G[t]) * L.rq[t] * QS[nt][i] + pu[i]);
          L.o[t * kNB + 16 * nt + l16] = to_bf(ov);
        }
      }
    }
    // ---- 8. S <- Gam_C S_0 + K^T diag(rk Gam_C / Gam) U
    {
      const float Gl = L.G[kC - 1];
      const float gC = expf(Gl);
      s16x4 uB[kNT];
#pragma unroll
      for (int nt = 0; nt < kNT; ++nt) {
        float f[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 4 * l4 + i;
          f[i] = L.rk[t] * expf(Gl - L.G[t]) * U[nt][i];
        }
        uB[nt] = bf16x4(f[0], f[1], f[2], f[3]);
      }
#pragma unroll
      for (int kt = 0; kt < kKT; ++kt) {
        const s16x4 kT = ld4(L.kt, 16 * kt + l16, kTS, 4 * l4);
#pragma unroll
        for (int nt = 0; nt < kNT; ++nt) S[kt][nt] = mfma(kT, uB[nt], S[kt][nt] * gC);
      }
    }
    lds_sync();
    {
      const int t = l / (kNB / 8), seg = l % (kNB / 8);
      if (t < n && l < kC * (kNB / 8))
        *reinterpret_cast<u32x4*>(og + (size_t(cs + t) * p.Hv + h) * p.DV + c0 + 8 * seg) =
            *reinterpret_cast<const u32x4*>(L.o + t * kNB + 8 * seg);
    }
    lds_sync();
  }

  // ---- the final state back to the slot (rounded once for a bf16 pool)
#pragma unroll
  for (int kt = 0; kt < kKT; ++kt)
#pragma unroll
    for (int nt = 0; nt < kNT; ++nt)
      store_state(pool_tile + size_t(c0 + 16 * nt + l16) * kDK + 16 * kt + 4 * l4, S[kt][nt]);
}

template <typename ST, int NB>
hipError_t launch_nb(const PrefillArgs& p, hipStream_t stream) {
  const dim3 grid(unsigned(p.DV / NB), unsigned(p.Hv), unsigned(p.B));
  hipLaunchKernelGGL((prefill_kernel<ST, NB>), grid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

// The chunks of a sequence run one after another in one wave, so a launch is bound by
// that chain; 16-column waves give twice the waves of 32-column ones, for grids that
// would leave SIMDs idle.
hipError_t launch_prefill(Dt state, const PrefillArgs& p, hipStream_t stream) {
  const bool narrow = int64_t(p.B) * p.Hv * (p.DV / 32) < 1024;
  if (state == Dt::F32) return narrow ? launch_nb<float, 16>(p, stream) : launch_nb<float, 32>(p, stream);
  return narrow ? launch_nb<bf16s, 16>(p, stream) : launch_nb<bf16s, 32>(p, stream);
}

}  // namespace gdn
