/*
 * gdn_stream.h -- C ABI of libgdn_stream.so, a measurement library beside the GDN state-
 * update library. It computes nothing of the method. Its streaming copy moves data with the
 * memory pattern of the state updates (every block read once and written `writes` times,
 * 16-byte accesses, each thread's loads before its stores); its rate under the same
 * cold-memory timing protocol is the practical ceiling against which the state-update
 * kernels' HBM rates are read. A verify of T tokens that stores every intermediate state
 * reads each state once and writes it T times; a decode or a commit reads it once and
 * writes it once.
 */
#ifndef GDN_STREAM_H
#define GDN_STREAM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming copy of `bytes` bytes (a multiple of the block, threads * chunks * 16 bytes),
 * `writes` times over: workgroup i of `threads` threads (64 or 256) reads block i with
 * `chunks` 16-byte loads per thread (1, 2 or 8), then writes it `writes` (1..16) times.
 * flags: bit 0 nontemporal loads, bit 1 nontemporal stores, bit 2 copy-major order (copy w
 * of block i at dst + (w * blocks + i) * block; otherwise block-major, at (i * writes + w) *
 * block). src holds `bytes`, dst `bytes * writes`; device pointers, 16-byte aligned, owned
 * by the caller; `stream` a hipStream_t (NULL: the default stream). One launch, no
 * allocation, no synchronisation. Returns 0, or before any launch 1 (NULL pointer), 2 (a
 * size or parameter out of range), 4 (misaligned); 6 if the launch failed. */
__attribute__((visibility("default"))) int32_t gdn_stream_copy(const void* src, void* dst, int64_t bytes,
                                                               int32_t writes, int32_t threads, int32_t chunks,
                                                               int32_t flags, void* stream);

/* Holds `stream` for `ns` nanoseconds (0 <= ns <= 10^7) with one spinning wave that reads
 * the wall clock: work queued behind it starts only then, so a timing event queued next is
 * stamped after everything queued in between has been submitted. Returns 0, 2 for ns out of
 * range, 6 if the clock rate cannot be read or the launch failed. */
__attribute__((visibility("default"))) int32_t gdn_stream_wait(int64_t ns, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* GDN_STREAM_H */
