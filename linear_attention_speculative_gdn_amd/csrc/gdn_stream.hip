// gdn_stream.hip -- a measurement kernel, not part of the GDN method: a pure streaming copy
// with the memory pattern of the state updates (every block read once, written `writes`
// times, all loads of a thread before its stores), to measure the HBM rate that a kernel
// doing only the data movement of such a call reaches on this chip -- the practical
// ceiling the roofline fractions are read against. The rate of such a copy depends on how
// the work is cut (threads per workgroup, 16-byte chunks per thread), on the load and store
// policy (nontemporal or not) and on the order of the copies (copy-major: the workgroups in
// flight write neighbouring blocks of one copy, as the verify's workgroups write
// neighbouring blocks of one token's states; block-major: the copies of one block are
// neighbours), so the caller times several variants and keeps the best.
//
// A second kernel only waits: it holds the stream for a given time so that the launches
// queued behind it (a timing event, then the timed graph) are all submitted before the
// event's timestamp is taken; the host's submission latency then stays off the clock.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/gdn_stream.h"

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <int TH, int CH, bool NTL, bool NTS, bool CM>
__global__ __launch_bounds__(TH) void stream_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                    int32_t writes) {
  const int64_t blk = blockIdx.x, nblk = gridDim.x, per_block = int64_t(TH) * CH;
  u32x4 v[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const u32x4* a = src + blk * per_block + c * TH + threadIdx.x;
    v[c] = NTL ? __builtin_nontemporal_load(a) : *a;
  }
  for (int w = 0; w < writes; ++w) {
    const int64_t ob = CM ? int64_t(w) * nblk + blk : blk * writes + w;
#pragma unroll
    for (int c = 0; c < CH; ++c) {
      u32x4* a = dst + ob * per_block + c * TH + threadIdx.x;
      if (NTS)
        __builtin_nontemporal_store(v[c], a);
      else
        *a = v[c];
    }
  }
}

// Spins on the constant-rate wall clock until `ticks` have passed, at most 2^24 rounds of
// s_sleep (each a few hundred cycles), so that it ends in any case.
__global__ void wait_kernel(uint64_t ticks) {
  const uint64_t t0 = wall_clock64();
  for (uint32_t i = 0; i < (1u << 24); ++i) {
    if (wall_clock64() - t0 >= ticks) break;
    __builtin_amdgcn_s_sleep(8);
  }
}

template <int TH, int CH>
hipError_t launch(int flags, const void* src, void* dst, int64_t blocks, int32_t writes, hipStream_t s) {
  const dim3 grid{unsigned(blocks), 1, 1}, block{unsigned(TH), 1, 1};
  const u32x4* in = static_cast<const u32x4*>(src);
  u32x4* out = static_cast<u32x4*>(dst);
  switch (flags) {
    case 0: hipLaunchKernelGGL((stream_kernel<TH, CH, false, false, false>), grid, block, 0, s, in, out, writes); break;
    case 1: hipLaunchKernelGGL((stream_kernel<TH, CH, true, false, false>), grid, block, 0, s, in, out, writes); break;
    case 2: hipLaunchKernelGGL((stream_kernel<TH, CH, false, true, false>), grid, block, 0, s, in, out, writes); break;
    case 3: hipLaunchKernelGGL((stream_kernel<TH, CH, true, true, false>), grid, block, 0, s, in, out, writes); break;
    case 4: hipLaunchKernelGGL((stream_kernel<TH, CH, false, false, true>), grid, block, 0, s, in, out, writes); break;
    case 5: hipLaunchKernelGGL((stream_kernel<TH, CH, true, false, true>), grid, block, 0, s, in, out, writes); break;
    case 6: hipLaunchKernelGGL((stream_kernel<TH, CH, false, true, true>), grid, block, 0, s, in, out, writes); break;
    default: hipLaunchKernelGGL((stream_kernel<TH, CH, true, true, true>), grid, block, 0, s, in, out, writes); break;
  }
  return hipGetLastError();
}

}  // namespace

extern "C" {

int32_t gdn_stream_copy(const void* src, void* dst, int64_t bytes, int32_t writes, int32_t threads, int32_t chunks,
                        int32_t flags, void* stream) {
  if (bytes < 0 || writes < 1 || writes > 16 || flags < 0 || flags > 7) return 2;
  if (!((threads == 64 || threads == 256) && (chunks == 1 || chunks == 2 || chunks == 8))) return 2;
  const int64_t block = int64_t(threads) * chunks * 16;
  if (bytes % block != 0 || bytes / block > int64_t(INT32_MAX)) return 2;
  if (bytes == 0) return 0;
  if (!src || !dst) return 1;
  if ((reinterpret_cast<uintptr_t>(src) & 15) || (reinterpret_cast<uintptr_t>(dst) & 15)) return 4;
  const int64_t blocks = bytes / block;
  const hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (threads == 64)
    e = chunks == 1 ? launch<64, 1>(flags, src, dst, blocks, writes, s)
                    : chunks == 2 ? launch<64, 2>(flags, src, dst, blocks, writes, s)
                                  : launch<64, 8>(flags, src, dst, blocks, writes, s);
  else
    e = chunks == 1 ? launch<256, 1>(flags, src, dst, blocks, writes, s)
                    : chunks == 2 ? launch<256, 2>(flags, src, dst, blocks, writes, s)
                                  : launch<256, 8>(flags, src, dst, blocks, writes, s);
  return e == hipSuccess ? 0 : 6;
}

int32_t gdn_stream_wait(int64_t ns, void* stream) {
  if (ns < 0 || ns > 10000000) return 2;
  int device = 0, khz = 0;
  if (hipGetDevice(&device) != hipSuccess ||
      hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, device) != hipSuccess || khz <= 0)
    return 6;
  const uint64_t ticks = uint64_t(ns) * uint64_t(khz) / 1000000u;
  hipLaunchKernelGGL(wait_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream), ticks);
  return hipGetLastError() == hipSuccess ? 0 : 6;
}

}  // extern "C"
