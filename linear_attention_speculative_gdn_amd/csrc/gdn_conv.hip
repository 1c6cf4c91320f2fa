// gdn_conv.hip -- gfx950 kernel of the short causal convolution whose state is pooled
// next to the GDN recurrent state: speculative verify (read-only state), decode
// (state written back), the fused commit of the previous step's accepted prefix, and
// the separate accepted-prefix commit.
//
// The operation: TensorRT-LLM PR 20937 (What changes: the in_proj GEMV carries a fused
// conv1d epilogue for verify and decode rows; Per-File QA Perspective: the staging and
// commit kernels keep accepted-prefix boundaries of the convolution state next to the
// other per-request state) and the dense-Qwen BF16 MTP proposal (What: GDN recovery
// records committed together with the convolution state). The pages do not print the
// convolution; this is the standard depthwise causal form of width K, per channel c:
//     y[t] = act(bias[c] + sum_{i<K} w[i][c] * in(t - (K-1) + i)),  act = id or SiLU,
// where in(tau < 0) are the K-1 inputs kept in the slot's state, oldest first.
//
// Design for gfx950: the work is a K-tap FIR over D channels per token, a few flops
// per byte, so the kernel is HBM- and latency-bound and uses no MFMA.
// - one lane owns a 16-byte chunk of channels (8 bf16 or 4 fp32) of one request row for
//   all tokens; a wave64 moves 1 KiB per load instruction along the channel axis;
// - the pool is laid out [P][K-1][D] and the taps [K][D], so every access of a lane
//   (state row, token, tap) is one 16-byte load, coalesced across the wave;
// - every load that does not depend on the slot (tokens, taps, bias) is issued before
//   the wait on the slot index; all loads are unconditional from clamped addresses;
// - the history is held right-aligned in registers (position p is the input at time
//   p - (KMAX-1)), so the unrolled FIR indexes registers statically for any K <= KMAX;
// - a commit is a selection of inputs, so the state moves as raw 16-byte chunks and is
//   exact; a decode write-back, whose source position depends on T and K at run time,
//   goes through a lane-private LDS strip instead of dynamically indexed registers.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gdn.h"
#include "gdn_device.h"
#include "gdn_internal.h"

namespace gdn {
namespace {

constexpr int kConvThreads = 64;

__device__ __forceinline__ float silu(float z) { return z / (1.f + expf(-z)); }

// IT: element type of x, y, the pool and prev_x. KMAX >= K, TMAX >= T (T ignored with
// COMMIT_ONLY, which advances the state over prev_len tokens of prev_x and stops).
template <typename IT, int KMAX, int TMAX, bool COMMIT_ONLY>
__global__ __launch_bounds__(kConvThreads) void conv_kernel(const ConvArgs p) {
  constexpr int VE = 16 / sizeof(IT);  // channels per 16-byte chunk
  constexpr int H = KMAX - 1;          // history registers
  extern __shared__ __attribute__((aligned(16))) u32x4 s_seq[];  // [H + T][kConvThreads]

  const int row = blockIdx.y;
  const int tid = threadIdx.x;
  const int ch = blockIdx.x * kConvThreads + tid;
  const int32_t slot = p.idx[row];
  const int32_t n_raw = p.prev_len ? p.prev_len[row] : 0;
  // the two per-row scalars are issued before the input loads below, which the compiler
  // otherwise places first, delaying the slot -> state chain (MTP T=4 batch: 5.47 -> 5.40 us)
  asm volatile("" ::: "memory");
  if (ch >= p.D / VE) return;
  const int K = p.K, T = COMMIT_ONLY ? 0 : p.T;
  const size_t D = size_t(p.D), c0 = size_t(ch) * VE;
  const IT* xp = static_cast<const IT*>(p.x);
  const IT* pxp = static_cast<const IT*>(p.prev_x);
  IT* yp = static_cast<IT*>(p.y);

  // ---- 1. inputs that do not depend on the slot: this call's tokens, taps, bias
  u32x4 xr[TMAX];
  f32x4 wr[KMAX][VE / 4];  // wr[j]: the tap applied to the input j tokens back
  f32x4 br[VE / 4];
  if constexpr (!COMMIT_ONLY) {
#pragma unroll
    for (int t = 0; t < TMAX; ++t)
      xr[t] = *reinterpret_cast<const u32x4*>(xp + (size_t(row) * T + min(t, T - 1)) * D + c0);
#pragma unroll
    for (int j = 0; j < KMAX; ++j)
#pragma unroll
      for (int v = 0; v < VE / 4; ++v)
        wr[j][v] = *reinterpret_cast<const f32x4*>(p.w + size_t(max(K - 1 - j, 0)) * D + c0 + 4 * v);
    const float* bp = p.bias ? p.bias : p.w;  // any readable address when there is no bias
#pragma unroll
    for (int v = 0; v < VE / 4; ++v) br[v] = *reinterpret_cast<const f32x4*>(bp + c0 + 4 * v);
  }
  // keep the loads above issued before the wait on the slot index
  asm volatile("" ::: "memory");

  if (slot < 0 || slot >= p.P) {  // padding row: y = 0, no state access
    if constexpr (!COMMIT_ONLY) {
#pragma unroll
      for (int t = 0; t < TMAX; ++t)
        if (t < T) *reinterpret_cast<u32x4*>(yp + (size_t(row) * T + t) * D + c0) = u32x4{0u, 0u, 0u, 0u};
    }
    return;
  }

  // ---- 2. the history before this call's first token, right-aligned: hr[q] is the
  //         input at time q - H (q >= KMAX - K; lower entries are never used). With a
  //         commit of n tokens of prev_x it is the slot's state advanced over them.
  const bool commit_prev = pxp && n_raw >= 1 && n_raw <= p.T_prev;
  const int n = commit_prev ? n_raw : 0;
  IT* const st = static_cast<IT*>(p.pool) + size_t(slot) * (K - 1) * D + c0;
  u32x4 hr[H];
#pragma unroll
  for (int q = 0; q < H; ++q) {
    const int m = max(q - (KMAX - K), 0);  // row of the new state
    const int tau = n + m - (K - 1);       // its time before the commit
    const IT* src = tau >= 0 ? pxp + (size_t(row) * p.T_prev + tau) * D + c0 : st + size_t(tau + K - 1) * D;
    hr[q] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src));
  }
  // State rows are read and written with nontemporal accesses: plain ones leave the rows
  // in L2, where the in-place stores dirty them for a write-back at the end of the launch
  // (measured 3-6 % slower on the MTP T=4, decode and T=8 workloads).
  if (commit_prev) {  // every source was read above, so the in-place stores are safe
#pragma unroll
    for (int q = 0; q < H; ++q)
      if (q >= KMAX - K)
        __builtin_nontemporal_store(hr[q], reinterpret_cast<u32x4*>(st + size_t(q - (KMAX - K)) * D));
  }
  if constexpr (COMMIT_ONLY) return;

  // ---- 3. outputs: y[t] = act(bias + sum over lags j < K of wr[j] * in(t - j)),
  //         oldest input first
  float bias[VE];
#pragma unroll
  for (int v = 0; v < VE / 4; ++v) {
    const float hb = p.bias ? 1.f : 0.f;
    bias[4 * v + 0] = hb * br[v].x; bias[4 * v + 1] = hb * br[v].y;
    bias[4 * v + 2] = hb * br[v].z; bias[4 * v + 3] = hb * br[v].w;
  }
#pragma unroll
  for (int t = 0; t < TMAX; ++t) {
    float acc[VE];
#pragma unroll
    for (int e = 0; e < VE; ++e) acc[e] = bias[e];
#pragma unroll
    for (int j = KMAX - 1; j >= 0; --j) {
      if (j >= K) continue;  // uniform: taps beyond the width
      const int tau = t - j;
      float f[VE];
      unpack_io(tau >= 0 ? xr[tau] : hr[H + tau], f, xp);
#pragma unroll
      for (int v = 0; v < VE / 4; ++v) {
        acc[4 * v + 0] = fmaf(wr[j][v].x, f[4 * v + 0], acc[4 * v + 0]);
        acc[4 * v + 1] = fmaf(wr[j][v].y, f[4 * v + 1], acc[4 * v + 1]);
        acc[4 * v + 2] = fmaf(wr[j][v].z, f[4 * v + 2], acc[4 * v + 2]);
        acc[4 * v + 3] = fmaf(wr[j][v].w, f[4 * v + 3], acc[4 * v + 3]);
      }
    }
    if (p.activation)
#pragma unroll
      for (int e = 0; e < VE; ++e) acc[e] = silu(acc[e]);
    if (t < T) *reinterpret_cast<u32x4*>(yp + (size_t(row) * T + t) * D + c0) = pack_io(acc, yp);
  }

  // ---- 4. decode write-back: the state advanced over all T tokens, i.e. the inputs at
  //         times T-(K-1) .. T-1. Positions depend on T and K at run time, so the lane
  //         stages its sequence in a private LDS strip (a wave's LDS accesses complete
  //         in order; no barrier).
  if (p.write_back) {
#pragma unroll
    for (int q = 0; q < H; ++q) s_seq[q * kConvThreads + tid] = hr[q];
#pragma unroll
    for (int t = 0; t < TMAX; ++t)
      if (t < T) s_seq[(H + t) * kConvThreads + tid] = xr[t];
    for (int m = 0; m < K - 1; ++m)
      __builtin_nontemporal_store(s_seq[(H + T - (K - 1) + m) * kConvThreads + tid],
                                  reinterpret_cast<u32x4*>(st + size_t(m) * D));
  }
}

template <typename IT, int KMAX, bool COMMIT_ONLY>
hipError_t launch_conv_t(const ConvArgs& p, hipStream_t stream) {
  const int nch = p.D / int(16 / sizeof(IT));
  const dim3 grid(unsigned((nch + kConvThreads - 1) / kConvThreads), unsigned(p.B));
  if constexpr (COMMIT_ONLY) {
    hipLaunchKernelGGL((conv_kernel<IT, KMAX, 1, true>), grid, dim3(kConvThreads), 0, stream, p);
    return hipGetLastError();
  }
  const size_t lds = p.write_back ? sizeof(u32x4) * size_t(KMAX - 1 + p.T) * kConvThreads : 0;
  if (p.T <= 1)
    hipLaunchKernelGGL((conv_kernel<IT, KMAX, 1, false>), grid, dim3(kConvThreads), lds, stream, p);
  else if (p.T <= 4)
    hipLaunchKernelGGL((conv_kernel<IT, KMAX, 4, false>), grid, dim3(kConvThreads), lds, stream, p);
  else if (p.T <= 8)
    hipLaunchKernelGGL((conv_kernel<IT, KMAX, 8, false>), grid, dim3(kConvThreads), lds, stream, p);
  else
    hipLaunchKernelGGL((conv_kernel<IT, KMAX, 16, false>), grid, dim3(kConvThreads), lds, stream, p);
  return hipGetLastError();
}

template <typename IT, bool COMMIT_ONLY>
hipError_t launch_conv_k(const ConvArgs& p, hipStream_t stream) {
  return p.K <= 4 ? launch_conv_t<IT, 4, COMMIT_ONLY>(p, stream) : launch_conv_t<IT, 8, COMMIT_ONLY>(p, stream);
}

}  // namespace

hipError_t launch_conv(Dt io, bool commit_only, const ConvArgs& p, hipStream_t stream) {
  if (io == Dt::F32)
    return commit_only ? launch_conv_k<float, true>(p, stream) : launch_conv_k<float, false>(p, stream);
  return commit_only ? launch_conv_k<bf16s, true>(p, stream) : launch_conv_k<bf16s, false>(p, stream);
}

}  // namespace gdn
