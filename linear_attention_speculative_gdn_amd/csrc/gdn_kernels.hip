// gdn_kernels.hip -- gfx950 (CDNA4) kernels of the Gated DeltaNet state update for
// pooled decode, multi-token (MTP / speculative) verify and accepted-prefix commit.
//
// The operation: the pages "[NVIDIA] [GDN] Enable FlashInfer MTP verify on SM100+
// (Blackwell)" (Summary, Requirements) and TensorRT-LLM PR 20937 (Per-File QA
// Perspective; Moved out of this PR) -- a per-request recurrent state gathered from a
// pool by slot index, padding slots skipped, T draft tokens through the gated delta
// rule, one cached state per token, fp32 or bf16 pools, commit of the accepted prefix.
// Per token, with q^ and k^ the L2-normalised q and k:
//     g = exp(-exp(A_log) softplus(a + dt_bias)), beta = sigmoid(b)
//     S <- g S;  S <- S + beta k^ (v - S^T k^)^T;  o = scale S^T q^
// evaluated here in the equivalent single-pass order
//     rk = S^T k^, rq = S^T q^            (one pass over the old state)
//     w  = beta (v - g rk)
//     S  <- g S + k^ w^T                  (second pass, fused with the store)
//     o  = scale (g rq + (k^.q^) w)
// which needs no second reduction over the updated state.
//
// The work is rank-1 updates and matrix-vector products: about 3 flop per byte of
// state traffic, far below the MI355X ridge, so the kernels are HBM-bound and use no
// MFMA. Design for gfx950:
// - the state of a (row, v-head) tile is stored value-column-major ([d_v][d_k], key
//   index contiguous), so each value index j owns a contiguous row and the two
//   reductions run along contiguous memory;
// - a workgroup (4 wave64) covers one (row, v-head, block of value rows); each value
//   row is spread over L = d_k/16 lanes holding 16 elements each, as 16-byte chunks
//   l, l+L, l+2L, ... so one wave64 load/store instruction moves whole 128-byte lines;
// - every global load (per-token inputs, then the state) is issued before the first
//   store, so the in-order vector memory counter never makes a load wait on stores;
// - the state stays in VGPRs across all T tokens; rk and rq are summed over the L
//   lanes of a row with DPP (quad_perm, row_half_mirror, row_mirror), no LDS trip;
// - every state store (intermediates, write-back, commit) is a nontemporal 16-byte
//   store: nothing reads the data again within the call, and streaming stores
//   measured 5-20 % faster than plain ones here;
// - bf16 states are rounded to nearest even with v_cvt_pk_bf16_f32 after every token
//   and the rounded value is carried, so verify(T) equals T decodes bit for bit.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gdn.h"
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

// ---------------------------------------------------------------- state chunks
// A chunk is 16 bytes of a state row: 4 fp32 or 8 bf16 elements.
template <typename ST>
struct Chunk;

template <>
struct Chunk<float> {
  static constexpr int CE = 4;
  __device__ __forceinline__ static void unpack(const u32x4& u, float* f) {
    f[0] = __uint_as_float(u.x); f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z); f[3] = __uint_as_float(u.w);
  }
  // fp32 state: storing is exact, nothing to round.
  __device__ __forceinline__ static u32x4 pack_round(float* f) {
    return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]),
                 __float_as_uint(f[3])};
  }
};

template <>
struct Chunk<bf16s> {
  static constexpr int CE = 8;
  __device__ __forceinline__ static void unpack(const u32x4& u, float* f) {
    f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x); f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
    f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z); f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
  }
  // bf16 state: round to nearest even and carry the rounded value in f.
  __device__ __forceinline__ static u32x4 pack_round(float* f) {
    u32x4 u;
    u.x = pack_bf16x2(f[0], f[1]); u.y = pack_bf16x2(f[2], f[3]);
    u.z = pack_bf16x2(f[4], f[5]); u.w = pack_bf16x2(f[6], f[7]);
    unpack(u, f);
    return u;
  }
};

// ---------------------------------------------------------------- cross-lane sums
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int kQuadXor1 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int kQuadXor2 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int kRowHalfMirror = 0x141;
constexpr int kRowMirror = 0x140;

// Sum over aligned groups of L lanes (L in {1,2,4,8,16}); every lane of a group gets
// the same, bit-identical total (each step adds the same two partial sums).
template <int L>
__device__ __forceinline__ float group_sum(float x) {
  if constexpr (L >= 2) x += dpp<kQuadXor1>(x);
  if constexpr (L >= 4) x += dpp<kQuadXor2>(x);
  if constexpr (L >= 8) x += dpp<kRowHalfMirror>(x);
  if constexpr (L >= 16) x += dpp<kRowMirror>(x);
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
  x = group_sum<16>(x);
  const int i = __float_as_int(x);
  return (__int_as_float(__builtin_amdgcn_readlane(i, 0)) + __int_as_float(__builtin_amdgcn_readlane(i, 16))) +
         (__int_as_float(__builtin_amdgcn_readlane(i, 32)) + __int_as_float(__builtin_amdgcn_readlane(i, 48)));
}

// ---------------------------------------------------------------- recurrent kernel
// Lane map: L = DK/16 lanes per value row, RW = 64/L rows per wave and slot, R slots
// per lane; a workgroup of NW waves covers RPW = NW*R*RW value rows of one
// (request row, v-head). Lane (grp = lane/L, l = lane%L) of wave w holds, for slot r,
// value row jl = (w*R + r)*RW + grp and the chunks l + c*L (c < 16/CE) of that row.
//
// MODE 0: decode / verify. T tokens from the slot's state (or, with a fused commit,
//         from the previous step's accepted intermediate), optional intermediate
//         cache and write-back.
// MODE 1: cached-replay verify. n = rlen[row] tokens of an earlier verify (their k, v,
//         a, b kept by the caller) are replayed from the slot's state, the result is
//         optionally committed to the slot, then the T new tokens run; no state is
//         stored per token.
// MODE 2: replay commit. The n replayed tokens' state is written back to the slot; no
//         new tokens, no outputs.
// Replayed and new tokens go through the same per-token code, in one sequence (the
// replayed ones first), so a replay reproduces the states a verify computed bit for bit.
//
// GATE (MODE 0 only, one workgroup per (row, v-head): RPW >= DV): the outputs are not
// stored as o but as the gated RMS normalisation y = w * o / sqrt(mean_j o^2 + eps) *
// silu(z) of each (row, token, v-head) vector. The outputs of all tokens collect in LDS;
// after the token loop one wave per token sums the squares, and every thread writes its
// 16-byte slice of y.
//
// Every global load is unconditional, from an address clamped into its buffer, and
// out-of-range lanes discard the value afterwards: a load inside a branch would be
// waited on at the end of the branch, which serialises the memory round trips.
template <typename ST, typename IT, int DK, int R, int NW, int MODE, bool GATE = false, bool NTL = false>
__global__ __launch_bounds__(NW * 64) void recurrent_kernel(const RecurrentArgs p) {
  constexpr bool NEW = MODE != 2;        // this call has its own tokens (and outputs)
  constexpr bool REPLAY = MODE != 0;
  constexpr int NT = NW * 64;
  constexpr int L = DK / 16;
  constexpr int RW = 64 / L;
  constexpr int RPW = NW * R * RW;
  constexpr int CE = Chunk<ST>::CE;
  constexpr int NCH = 16 / CE;           // chunks per lane and row
  constexpr int VE = 16 / sizeof(IT);    // io elements per 16-byte vector
  constexpr int QVEC = DK / VE;          // vectors of one token's q (or k)
  constexpr int VVEC = RPW / VE;         // vectors of one token's v rows of this block
  constexpr int NQ = (GDN_MAX_T * QVEC + NT - 1) / NT;
  constexpr int NV = (GDN_MAX_T * VVEC + NT - 1) / NT;

  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int T = NEW ? p.T : 0;
  const int TMAX = T + (REPLAY ? p.rT : 0);  // token capacity of the LDS buffers
  float* s_q = smem;                // [TMAX][DK]  q, then q^ (zero for replayed tokens)
  float* s_k = s_q + TMAX * DK;     // [TMAX][DK]  k, then k^
  float* s_v = s_k + TMAX * DK;     // [TMAX][RPW] v of this block's rows
  float* s_g = s_v + TMAX * RPW;    // [TMAX] decay
  float* s_beta = s_g + TMAX;       // [TMAX] write strength
  float* s_kq = s_beta + TMAX;      // [TMAX] k^.q^
  float* s_o = s_kq + TMAX;         // [NW][R*RW] outputs of one token, per wave
  float* s_og = s_o + NW * R * RW;  // GATE: [T][RPW] outputs of all tokens
  float* s_rs = s_og + T * RPW;     // GATE: [T] 1 / rms of each token's outputs

  // grid (v-block, v-head, row): no integer division on the way to the first loads.
  // Workgroups are dealt to the 8 XCDs round-robin by linear id, so the v-blocks of
  // one tile sit on different XCDs and read that row's q and k separately (about 5 %
  // extra read traffic at d = 128); ordering the grid by row instead, so that a row's
  // workgroups share one L2, measured 10 % slower: the workgroups in flight then touch
  // scattered tiles instead of neighbouring blocks of the same tiles.
  const int vb = blockIdx.x;
  const int h = blockIdx.y;
  const int row = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int grp = lane / L, l = lane % L;
  const int DV = p.DV;
  const size_t tile = size_t(DK) * DV;

  const IT* qp = static_cast<const IT*>(p.q);
  const IT* kp = static_cast<const IT*>(p.k);
  const IT* vp = static_cast<const IT*>(p.v);
  const IT* ap = static_cast<const IT*>(p.a);
  const IT* bp = static_cast<const IT*>(p.b);
  IT* op = static_cast<IT*>(p.o);

  // The per-row scalars first, as scalar loads issued together (the compiler reads
  // memory with scalar loads only before anything that might write it, hence the
  // barrier after them), so that one wait on the slot index covers them all.
  const int32_t slot = p.idx[row];
  const int32_t n_prev = (MODE == 0 && p.prev_accept) ? p.prev_accept[row] : 0;
  int32_t n_rep = 0;
  float a_log = 0.f, dtb = 0.f;  // replay modes: the gate parameters, read up front
  if constexpr (REPLAY) {
    const int32_t x = p.rlen[row];
    n_rep = (x >= 0 && x <= p.rT) ? x : 0;
    a_log = p.A_log[h];
    dtb = p.dt_bias[h];
  }
  asm volatile("" ::: "memory");
  const int kh = h / p.G;

  // ---- 1. this call's per-token inputs (do not depend on the slot): q, k, v as
  //         16-byte vectors, a and b of token tid
  const int nq = T * QVEC, nv = T * VVEC;
  u32x4 qraw[NQ], kraw[NQ], vraw[NV];
  float a_in = 0.f, b_in = 0.f;
  if constexpr (NEW) {
#pragma unroll
    for (int it = 0; it < NQ; ++it) {
      const int e = min(tid + it * NT, nq - 1);
      const int t = e / QVEC, c = e - t * QVEC;
      const size_t off = (size_t(row * T + t) * p.Hk + kh) * DK + c * VE;
      qraw[it] = *reinterpret_cast<const u32x4*>(qp + off);
      kraw[it] = *reinterpret_cast<const u32x4*>(kp + off);
    }
#pragma unroll
    for (int it = 0; it < NV; ++it) {
      const int e = min(tid + it * NT, nv - 1);
      const int t = e / VVEC, c = e - t * VVEC;
      const int j = min(vb * RPW + c * VE, DV - VE);
      vraw[it] = *reinterpret_cast<const u32x4*>(vp + (size_t(row * T + t) * p.Hv + h) * DV + j);
    }
    const int tg = min(tid, T - 1);
    a_in = ld_io(ap + size_t(row * T + tg) * p.Hv + h);
    b_in = ld_io(bp + size_t(row * T + tg) * p.Hv + h);
  }
  // GATE: the gate input z (laid out like v) and the norm weights of the same vectors
  u32x4 zraw[GATE ? NV : 1];
  f32x4 gwr[GATE ? NV : 1][VE / 4];
  if constexpr (GATE) {
    const IT* zp = static_cast<const IT*>(p.z);
#pragma unroll
    for (int it = 0; it < NV; ++it) {
      const int e = min(tid + it * NT, nv - 1);
      const int t = e / VVEC, c = e - t * VVEC;
      const int j = min(c * VE, DV - VE);
      zraw[it] = *reinterpret_cast<const u32x4*>(zp + (size_t(row * T + t) * p.Hv + h) * DV + j);
#pragma unroll
      for (int u = 0; u < VE / 4; ++u) gwr[it][u] = *reinterpret_cast<const f32x4*>(p.gw + j + 4 * u);
    }
  }
  // keep the loads above issued before the wait on the slot index (they must not
  // be sunk into the non-padding branch)
  asm volatile("" ::: "memory");

  if (slot < 0 || slot >= p.P || (MODE == 2 && n_rep == 0)) {  // nothing to do but o = 0
    if constexpr (NEW) {
      for (int e = tid; e < nv; e += NT) {
        const int t = e / VVEC, j = vb * RPW + (e - t * VVEC) * VE;
        if (j < DV) *reinterpret_cast<u32x4*>(op + (size_t(row * T + t) * p.Hv + h) * DV + j) = u32x4{0u, 0u, 0u, 0u};
      }
    }
    return;
  }

  // ---- 2. the replayed tokens' k, v, a, b (the caller guarantees at least one token
  //         per row in the replay arrays, so the clamped addresses stay inside them)
  const int nrq = n_rep * QVEC, nrv = n_rep * VVEC;
  u32x4 rkraw[NQ], rvraw[NV];
  float ra_in = 0.f, rb_in = 0.f;
  if constexpr (REPLAY) {
    const IT* rkp = static_cast<const IT*>(p.rk);
    const IT* rvp = static_cast<const IT*>(p.rv);
#pragma unroll
    for (int it = 0; it < NQ; ++it) {
      const int e = min(tid + it * NT, max(nrq, 1) - 1);
      const int t = e / QVEC, c = e - t * QVEC;
      rkraw[it] = *reinterpret_cast<const u32x4*>(rkp + (size_t(row * p.rT + t) * p.Hk + kh) * DK + c * VE);
    }
#pragma unroll
    for (int it = 0; it < NV; ++it) {
      const int e = min(tid + it * NT, max(nrv, 1) - 1);
      const int t = e / VVEC, c = e - t * VVEC;
      const int j = min(vb * RPW + c * VE, DV - VE);
      rvraw[it] = *reinterpret_cast<const u32x4*>(rvp + (size_t(row * p.rT + t) * p.Hv + h) * DV + j);
    }
    const int tg = min(tid, max(n_rep, 1) - 1);
    ra_in = ld_io(static_cast<const IT*>(p.ra) + size_t(row * p.rT + tg) * p.Hv + h);
    rb_in = ld_io(static_cast<const IT*>(p.rb) + size_t(row * p.rT + tg) * p.Hv + h);
  }

  // ---- 3. the initial state: the pool slot, or the previous step's accepted
  //         intermediate for a fused commit
  const bool commit_prev = n_prev >= 1 && n_prev <= p.cache_T;
  const ST* src = commit_prev
                      ? static_cast<const ST*>(p.cache) + ((size_t(row) * p.cache_T + (n_prev - 1)) * p.Hv + h) * tile
                      : static_cast<const ST*>(p.pool) + (size_t(slot) * p.Hv + h) * tile;
  int jrow[R];
  bool rv[R];
  u32x4 raw[R][NCH];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    jrow[r] = vb * RPW + (wave * R + r) * RW + grp;
    rv[r] = jrow[r] < DV;
    const int jr = min(jrow[r], DV - 1);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const u32x4* at = reinterpret_cast<const u32x4*>(src + size_t(jr) * DK + (l + c * L) * CE);
      raw[r][c] = NTL ? __builtin_nontemporal_load(at) : *at;
    }
  }

  // ---- 4. token inputs -> LDS (replayed tokens first, then this call's); gates.
  //         In mode 0, A_log and dt_bias are read only by the lanes that compute a
  //         gate, after the state loads: reading them earlier, in every wave or in
  //         wave 0 only, as scalar or as vector loads, measured 15-20 % slower on the
  //         small MTP verify batch (B = 64, one wave of workgroups), though decode
  //         gained 5 %. The replay modes, bound by arithmetic, gain 2-7 % from the
  //         early read.
  if constexpr (REPLAY) {
#pragma unroll
    for (int it = 0; it < NQ; ++it) {
      const int e = tid + it * NT;
      if (e < nrq) {
        float f[VE];
        unpack_io(rkraw[it], f, kp);
#pragma unroll
        for (int m = 0; m < VE; ++m) {
          s_k[e * VE + m] = f[m];
          s_q[e * VE + m] = 0.f;
        }
      }
    }
#pragma unroll
    for (int it = 0; it < NV; ++it) {
      const int e = tid + it * NT;
      if (e < nrv) {
        float f[VE];
        unpack_io(rvraw[it], f, vp);
        const int t = e / VVEC, c = e - t * VVEC;
        const bool ok = vb * RPW + c * VE < DV;
#pragma unroll
        for (int m = 0; m < VE; ++m) s_v[t * RPW + c * VE + m] = ok ? f[m] : 0.f;
      }
    }
    if (tid < n_rep) {
      const float x = ra_in + dtb;
      s_g[tid] = expf(-expf(a_log) * (fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)))));
      s_beta[tid] = 1.f / (1.f + expf(-rb_in));
    }
  }
  if constexpr (NEW) {
    float* const sq_new = s_q + n_rep * DK;
    float* const sk_new = s_k + n_rep * DK;
    float* const sv_new = s_v + n_rep * RPW;
#pragma unroll
    for (int it = 0; it < NQ; ++it) {
      const int e = tid + it * NT;
      if (e < nq) {
        float f[VE];
        unpack_io(qraw[it], f, qp);
#pragma unroll
        for (int m = 0; m < VE; ++m) sq_new[e * VE + m] = f[m];
        unpack_io(kraw[it], f, kp);
#pragma unroll
        for (int m = 0; m < VE; ++m) sk_new[e * VE + m] = f[m];
      }
    }
#pragma unroll
    for (int it = 0; it < NV; ++it) {
      const int e = tid + it * NT;
      if (e < nv) {
        float f[VE];
        unpack_io(vraw[it], f, vp);
        const int t = e / VVEC, c = e - t * VVEC;
        const bool ok = vb * RPW + c * VE < DV;
#pragma unroll
        for (int m = 0; m < VE; ++m) sv_new[t * RPW + c * VE + m] = ok ? f[m] : 0.f;
      }
    }
    if (tid < T) {
      const float x = a_in + (REPLAY ? dtb : p.dt_bias[h]);
      s_g[n_rep + tid] = expf(-expf(REPLAY ? a_log : p.A_log[h]) * (fmaxf(x, 0.f) + log1pf(expf(-fabsf(x)))));
      s_beta[n_rep + tid] = 1.f / (1.f + expf(-b_in));
    }
  }
  __syncthreads();

  // ---- 5. L2 normalisation of q and k, and k^.q^, one wave per token
  const int NTOK = n_rep + T;
  constexpr int PL = (DK + 63) / 64;  // elements per lane
  for (int t = wave; t < NTOK; t += NW) {
    float qv[PL], kv[PL];
    float sq = 0.f, sk = 0.f, skq = 0.f;
#pragma unroll
    for (int u = 0; u < PL; ++u) {
      const int i = lane + u * 64;
      qv[u] = (DK >= 64 || i < DK) ? s_q[t * DK + i] : 0.f;
      kv[u] = (DK >= 64 || i < DK) ? s_k[t * DK + i] : 0.f;
      sq = fmaf(qv[u], qv[u], sq);
      sk = fmaf(kv[u], kv[u], sk);
      skq = fmaf(qv[u], kv[u], skq);
    }
    sq = wave_sum(sq);
    sk = wave_sum(sk);
    skq = wave_sum(skq);
    const float rq = 1.f / sqrtf(sq + p.eps), rk = 1.f / sqrtf(sk + p.eps);
#pragma unroll
    for (int u = 0; u < PL; ++u) {
      const int i = lane + u * 64;
      if (DK >= 64 || i < DK) {
        s_q[t * DK + i] = qv[u] * rq;
        s_k[t * DK + i] = kv[u] * rk;
      }
    }
    if (lane == 0) s_kq[t] = skq * rq * rk;
  }
  __syncthreads();

  // ---- 6. state to registers; fused commit of the gathered state
  float S[R][16];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int c = 0; c < NCH; ++c) Chunk<ST>::unpack(raw[r][c], &S[r][c * CE]);

  ST* const pool_tile = static_cast<ST*>(p.pool) + (size_t(slot) * p.Hv + h) * tile;
  if (commit_prev) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (rv[r])
#pragma unroll
        for (int c = 0; c < NCH; ++c)
          st_nt(pool_tile + size_t(jrow[r]) * DK + (l + c * L) * CE, raw[r][c]);
  }

  // ---- 7. the tokens: n_rep replayed ones, then this call's T
  ST* const cache_row = p.cache ? static_cast<ST*>(p.cache) + size_t(row) * p.cache_T * p.Hv * tile : nullptr;
  const size_t cache_t_stride = size_t(p.Hv) * tile;
  const float scale = p.scale;
  const f32x4* s_k4 = reinterpret_cast<const f32x4*>(s_k);
  const f32x4* s_q4 = reinterpret_cast<const f32x4*>(s_q);
  for (int tau = 0; tau < NTOK; ++tau) {
    float kh_[16], qh_[16];
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
      for (int m4 = 0; m4 < CE / 4; ++m4) {
        const int i4 = (tau * DK + (l + c * L) * CE) / 4 + m4;
        const f32x4 kk = s_k4[i4], qq = s_q4[i4];
        kh_[c * CE + m4 * 4 + 0] = kk.x; kh_[c * CE + m4 * 4 + 1] = kk.y;
        kh_[c * CE + m4 * 4 + 2] = kk.z; kh_[c * CE + m4 * 4 + 3] = kk.w;
        qh_[c * CE + m4 * 4 + 0] = qq.x; qh_[c * CE + m4 * 4 + 1] = qq.y;
        qh_[c * CE + m4 * 4 + 2] = qq.z; qh_[c * CE + m4 * 4 + 3] = qq.w;
      }
    const float gt = s_g[tau], bt = s_beta[tau], kqt = s_kq[tau];
    float rk[R], rq[R];
    if (!REPLAY || tau >= n_rep) {  // a token with an output: S^T k and S^T q
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float pk0 = 0.f, pk1 = 0.f, pq0 = 0.f, pq1 = 0.f;
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          pk0 = fmaf(S[r][e], kh_[e], pk0);
          pk1 = fmaf(S[r][e + 1], kh_[e + 1], pk1);
          pq0 = fmaf(S[r][e], qh_[e], pq0);
          pq1 = fmaf(S[r][e + 1], qh_[e + 1], pq1);
        }
        rk[r] = group_sum<L>(pk0 + pk1);
        rq[r] = group_sum<L>(pq0 + pq1);
      }
    } else {  // a replayed token has no output: S^T k only
#pragma unroll
      for (int r = 0; r < R; ++r) {
        float pk0 = 0.f, pk1 = 0.f;
#pragma unroll
        for (int e = 0; e < 16; e += 2) {
          pk0 = fmaf(S[r][e], kh_[e], pk0);
          pk1 = fmaf(S[r][e + 1], kh_[e + 1], pk1);
        }
        rk[r] = group_sum<L>(pk0 + pk1);
        rq[r] = 0.f;
      }
    }
    const int t = tau - n_rep;  // index among this call's tokens (negative: replayed)
    ST* const cache_t = (cache_row && t >= 0) ? cache_row + t * cache_t_stride + h * tile : nullptr;
    const bool commit_now = REPLAY && p.rcommit && tau == n_rep - 1;
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int jl = (wave * R + r) * RW + grp;
      const float w = bt * (s_v[tau * RPW + jl] - gt * rk[r]);
      const float ov = (gt * rq[r] + kqt * w) * scale;
#pragma unroll
      for (int e = 0; e < 16; ++e) S[r][e] = fmaf(gt, S[r][e], kh_[e] * w);
      u32x4 packed[NCH];
#pragma unroll
      for (int c = 0; c < NCH; ++c) packed[c] = Chunk<ST>::pack_round(&S[r][c * CE]);
      if (rv[r]) {
        if (cache_t) {
#pragma unroll
          for (int c = 0; c < NCH; ++c)
            st_nt(cache_t + size_t(jrow[r]) * DK + (l + c * L) * CE, packed[c]);
        }
        if (commit_now) {
#pragma unroll
          for (int c = 0; c < NCH; ++c)
            st_nt(pool_tile + size_t(jrow[r]) * DK + (l + c * L) * CE, packed[c]);
        }
        if (NEW && l == 0) {
          if constexpr (GATE) {
            if (t >= 0) s_og[t * RPW + (wave * R + r) * RW + grp] = ov;
          } else {
            s_o[wave * (R * RW) + r * RW + grp] = ov;
          }
        }
      }
    }
    if constexpr (NEW && !GATE) {
      if (t >= 0) {
        // o of this wave's R*RW consecutive value rows, as whole 16-byte vectors. The
        // strip in LDS is private to the wave, and a wave's LDS accesses complete in
        // order, so no barrier is needed.
        IT* const o_t = op + (size_t(row * T + t) * p.Hv + h) * DV + vb * RPW + wave * (R * RW);
        if constexpr ((R * RW) % VE == 0) {
          if (lane < (R * RW) / VE && vb * RPW + wave * (R * RW) + lane * VE < DV) {
            float f[VE];
#pragma unroll
            for (int m = 0; m < VE; ++m) f[m] = s_o[wave * (R * RW) + lane * VE + m];
            *reinterpret_cast<u32x4*>(o_t + lane * VE) = pack_io(f, op);
          }
        } else {  // fewer rows per wave than one vector holds (d_k = 256)
          if (lane < R * RW && vb * RPW + wave * (R * RW) + lane < DV)
            st_io(o_t + lane, s_o[wave * (R * RW) + lane]);
        }
      }
    }
  }

  // ---- 8. GATE: y = w * o / sqrt(mean o^2 + eps) * silu(z) for every token
  if constexpr (GATE) {
    __syncthreads();
    constexpr int PV = (RPW + 63) / 64;
    for (int t = wave; t < T; t += NW) {
      float ss = 0.f;
#pragma unroll
      for (int u = 0; u < PV; ++u) {
        const int j = lane + u * 64;
        const float x = (j < DV) ? s_og[t * RPW + j] : 0.f;
        ss = fmaf(x, x, ss);
      }
      ss = wave_sum(ss);
      if (lane == 0) s_rs[t] = 1.f / sqrtf(ss / float(DV) + p.geps);
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < NV; ++it) {
      const int e = tid + it * NT;
      const int t = e / VVEC, c = e - t * VVEC;
      if (e < nv && c * VE < DV) {
        float zf[VE], y[VE];
        unpack_io(zraw[it], zf, op);
        const float rs = s_rs[t];
#pragma unroll
        for (int u = 0; u < VE / 4; ++u) {
          const float wv[4] = {gwr[it][u].x, gwr[it][u].y, gwr[it][u].z, gwr[it][u].w};
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            const int mm = 4 * u + m;
            const float zz = zf[mm];
            y[mm] = (s_og[t * RPW + c * VE + mm] * rs) * wv[m] * (zz / (1.f + expf(-zz)));
          }
        }
        *reinterpret_cast<u32x4*>(op + (size_t(row * T + t) * p.Hv + h) * DV + c * VE) = pack_io(y, op);
      }
    }
  }

  // ---- 9. final state back to the slot
  if (MODE == 0 && p.write_final) {
#pragma unroll
    for (int r = 0; r < R; ++r)
      if (rv[r])
#pragma unroll
        for (int c = 0; c < NCH; ++c)
          st_nt(pool_tile + size_t(jrow[r]) * DK + (l + c * L) * CE, Chunk<ST>::pack_round(&S[r][c * CE]));
  }
}

// ---------------------------------------------------------------- commit kernel
// pool[idx[r], h] <- cache[r, n-1, h] for 1 <= n <= cache_T and a valid slot.
// blocks_per_tile workgroups per (row, v-head), each copying kThreads*CPT chunks;
// a tile is read once and written once, both nontemporal (no reuse within the call).
template <int CPT>
__global__ __launch_bounds__(kThreads) void commit_kernel(const CommitArgs p) {
  const int blk = blockIdx.x, h = blockIdx.y, row = blockIdx.z;  // grid (blocks, Hv, B)
  // both per-row scalars in flight together: with the tests short-circuited the accept
  // length was read only after the slot had arrived (one more round trip; 21.85 -> 21.66 us
  // per verify + commit step on the MTP T=4 batch)
  const int32_t slot = p.idx[row], n = p.accept[row];
  asm volatile("" ::: "memory");
  if ((slot < 0) | (slot >= p.P) | (n < 1) | (n > p.cache_T)) return;
  const char* src = static_cast<const char*>(p.cache) + ((size_t(row) * p.cache_T + (n - 1)) * p.Hv + h) * p.tile_bytes;
  char* dst = static_cast<char*>(p.pool) + (size_t(slot) * p.Hv + h) * p.tile_bytes;
  const int64_t nchunks = p.tile_bytes / 16;
  u32x4 buf[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int64_t e = (int64_t(blk) * CPT + c) * kThreads + threadIdx.x;
    if (e < nchunks) buf[c] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src) + e);
  }
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int64_t e = (int64_t(blk) * CPT + c) * kThreads + threadIdx.x;
    if (e < nchunks) __builtin_nontemporal_store(buf[c], reinterpret_cast<u32x4*>(dst) + e);
  }
}

template <typename ST, typename IT, int DK, int R, int NW = 4, int MODE = 0, bool GATE = false, bool NTL = false>
hipError_t launch_rec(const RecurrentArgs& p, hipStream_t stream) {
  constexpr int RPW = NW * R * (64 / (DK / 16));
  const int nvb = (p.DV + RPW - 1) / RPW;
  if (GATE && nvb != 1) return hipErrorInvalidValue;  // the norm needs a head's d_v in one workgroup
  const dim3 grid(unsigned(nvb), unsigned(p.Hv), unsigned(p.B));
  const size_t tmax = size_t(MODE == 2 ? 0 : p.T) + size_t(MODE == 0 ? 0 : p.rT);
  const size_t lds = sizeof(float) * (2 * tmax * DK + tmax * RPW + 3 * tmax + RPW +
                                      (GATE ? size_t(p.T) * (RPW + 1) : 0));
  hipLaunchKernelGGL((recurrent_kernel<ST, IT, DK, R, NW, MODE, GATE, NTL>), grid, dim3(NW * 64), lds, stream, p);
  return hipGetLastError();
}

// Plain calls choose among the measured launch shapes. Replay calls are bound by
// vector ALU and LDS reads rather than HBM (up to twice the tokens per state pass, no
// per-token stores): at d_k = 128 two rows per lane halve the k^/q^ reads from LDS
// per state element, and 8 waves per workgroup keep more of them in flight.
template <typename ST, typename IT>
hipError_t launch_dk(int shape, int mode, bool ntl, const RecurrentArgs& p, hipStream_t stream) {
  if (mode == 1) {
    switch (p.DK) {
      case 16: return launch_rec<ST, IT, 16, 1, 4, 1>(p, stream);
      case 32: return launch_rec<ST, IT, 32, 1, 4, 1>(p, stream);
      case 64: return launch_rec<ST, IT, 64, 1, 4, 1>(p, stream);
      case 128:
        return ntl ? launch_rec<ST, IT, 128, 2, 8, 1, false, true>(p, stream)
                   : launch_rec<ST, IT, 128, 2, 8, 1>(p, stream);
      case 256: return launch_rec<ST, IT, 256, 1, 4, 1>(p, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (mode == 3) {  // verify with the gated-norm epilogue: one workgroup covers d_v
    switch (p.DK) {
      case 16: return launch_rec<ST, IT, 16, 1, 4, 0, true>(p, stream);    // 256 value rows
      case 32: return launch_rec<ST, IT, 32, 1, 8, 0, true>(p, stream);    // 256
      case 64: return launch_rec<ST, IT, 64, 2, 8, 0, true>(p, stream);    // 256
      case 128:  // 128 value rows in every shape, chosen by T as measured: one row per
                 // lane and 16 waves above 4 tokens (T = 8: 255 -> 241 us against two rows
                 // and 8 waves), four rows and 4 waves for 2-4 tokens (T = 4: 17.3 us; 18.1
                 // with one row and 16 waves, 18.0 with two rows and 8), two rows and 8 waves
                 // for one token (11.0 us; 11.7 with four)
        if (p.T > 4) return launch_rec<ST, IT, 128, 1, 16, 0, true>(p, stream);
        if (p.T > 1)
          return ntl ? launch_rec<ST, IT, 128, 4, 4, 0, true, true>(p, stream)
                     : launch_rec<ST, IT, 128, 4, 4, 0, true>(p, stream);
        return ntl ? launch_rec<ST, IT, 128, 2, 8, 0, true, true>(p, stream)
                   : launch_rec<ST, IT, 128, 2, 8, 0, true>(p, stream);
      case 256: return launch_rec<ST, IT, 256, 4, 8, 0, true>(p, stream);  // 128
      default: return hipErrorInvalidValue;
    }
  }
  if (mode == 2) {
    switch (p.DK) {
      case 16: return launch_rec<ST, IT, 16, 1, 4, 2>(p, stream);
      case 32: return launch_rec<ST, IT, 32, 1, 4, 2>(p, stream);
      case 64: return launch_rec<ST, IT, 64, 1, 4, 2>(p, stream);
      case 128:
        return ntl ? launch_rec<ST, IT, 128, 2, 8, 2, false, true>(p, stream)
                   : launch_rec<ST, IT, 128, 2, 8, 2>(p, stream);
      case 256: return launch_rec<ST, IT, 256, 1, 4, 2>(p, stream);
      default: return hipErrorInvalidValue;
    }
  }
  switch (p.DK) {
    case 16: return launch_rec<ST, IT, 16, 1>(p, stream);
    case 32: return launch_rec<ST, IT, 32, 1>(p, stream);
    case 64: return launch_rec<ST, IT, 64, 1>(p, stream);
    case 128:
      if (shape == 2) return launch_rec<ST, IT, 128, 2>(p, stream);
      if (shape == 12) return launch_rec<ST, IT, 128, 1, 2>(p, stream);
      if (shape == 14) return launch_rec<ST, IT, 128, 1, 8>(p, stream);
      if (shape == 44)
        return ntl ? launch_rec<ST, IT, 128, 4, 4, 0, false, true>(p, stream) : launch_rec<ST, IT, 128, 4, 4>(p, stream);
      return ntl ? launch_rec<ST, IT, 128, 1, 4, 0, false, true>(p, stream) : launch_rec<ST, IT, 128, 1>(p, stream);
    case 256: return launch_rec<ST, IT, 256, 1>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_recurrent(Dt state, Dt io, int shape, int mode, bool nt_loads, const RecurrentArgs& p,
                            hipStream_t stream) {
  if (state == Dt::F32 && io == Dt::F32) return launch_dk<float, float>(shape, mode, nt_loads, p, stream);
  if (state == Dt::F32 && io == Dt::BF16) return launch_dk<float, bf16s>(shape, mode, nt_loads, p, stream);
  if (state == Dt::BF16 && io == Dt::F32) return launch_dk<bf16s, float>(shape, mode, nt_loads, p, stream);
  return launch_dk<bf16s, bf16s>(shape, mode, nt_loads, p, stream);
}

hipError_t launch_commit(const CommitArgs& p, hipStream_t stream) {
  const dim3 grid(unsigned(p.blocks_per_tile), unsigned(p.Hv), unsigned(p.B));
  hipLaunchKernelGGL((commit_kernel<kCommitChunksPerThread>), grid, dim3(kThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gdn
