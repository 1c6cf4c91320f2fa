// gdn_device.h -- gfx950 device helpers shared by the kernels (16-byte vectors, bf16
// packing with round to nearest even, io element access). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdn {

typedef float f32x2 __attribute__((ext_vector_type(2)));
// 16 bytes as a native vector (global_load/store_dwordx4, nontemporal builtins).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

struct bf16s {
  uint16_t bits;
};

// fp32 pair -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 f = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// ---------------------------------------------------------------- io elements
__device__ __forceinline__ float ld_io(const float* p) { return *p; }
__device__ __forceinline__ float ld_io(const bf16s* p) { return __uint_as_float(uint32_t(p->bits) << 16); }

// 16 bytes of io elements -> floats
__device__ __forceinline__ void unpack_io(const u32x4& u, float* f, const float*) {
  f[0] = __uint_as_float(u.x); f[1] = __uint_as_float(u.y);
  f[2] = __uint_as_float(u.z); f[3] = __uint_as_float(u.w);
}
__device__ __forceinline__ void unpack_io(const u32x4& u, float* f, const bf16s*) {
  f[0] = bf16_lo(u.x); f[1] = bf16_hi(u.x); f[2] = bf16_lo(u.y); f[3] = bf16_hi(u.y);
  f[4] = bf16_lo(u.z); f[5] = bf16_hi(u.z); f[6] = bf16_lo(u.w); f[7] = bf16_hi(u.w);
}

__device__ __forceinline__ void st_io(float* p, float x) { *p = x; }
__device__ __forceinline__ void st_io(bf16s* p, float x) { p->bits = uint16_t(pack_bf16x2(x, 0.f)); }

// floats -> 16 bytes of io elements (bf16: round to nearest even)
__device__ __forceinline__ u32x4 pack_io(const float* f, const float*) {
  return u32x4{__float_as_uint(f[0]), __float_as_uint(f[1]), __float_as_uint(f[2]), __float_as_uint(f[3])};
}
__device__ __forceinline__ u32x4 pack_io(const float* f, const bf16s*) {
  return u32x4{pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]), pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7])};
}

// 16-byte nontemporal store (data not read again within the call).
__device__ __forceinline__ void st_nt(void* p, const u32x4& u) {
  __builtin_nontemporal_store(u, reinterpret_cast<u32x4*>(p));
}

}  // namespace gdn
