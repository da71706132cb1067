/*
 * fs_bench.h -- measurement aids exported by the same library as fs.h.  They
 * are not steps of the method: the benchmark uses them to measure the HBM
 * streaming ceilings each kernel is compared with, and to scale the hardware
 * traffic counters by a kernel whose traffic is known exactly.  Conventions
 * (device pointers, return codes, fs_last_error) are those of fs.h.
 */
#ifndef FS_BENCH_H
#define FS_BENCH_H

#include "fs.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * fs_copy_bytes -- plain streaming copy of `bytes` bytes (dst, src device,
 * both 16-byte aligned, bytes a multiple of 16).  A measurement aid, not
 * part of the method: it gives the practical copy ceiling of the HBM and the
 * scale of the hardware traffic counters for a kernel of known traffic.
 * Errors: FS_E_INVAL, FS_E_ALIGN, FS_E_HIP.
 */
int fs_copy_bytes(void *dst, const void *src, int64_t bytes, hipStream_t stream);

/*
 * fs_stream_read / fs_stream_fill -- measurement aids beside fs_copy_bytes,
 * not part of the method: the HBM read-only and write-only streaming rates
 * that, with the copy rate, bound each kernel's read/write mix.
 * fs_stream_read reads `bytes` bytes at src and discards them; sink (device,
 * 4 bytes) may receive an unspecified value.  fs_stream_fill writes the
 * 32-bit `value` over `bytes` bytes at dst.  Pointers 16-byte aligned (sink
 * 4-byte), bytes a multiple of 16.  Errors: FS_E_INVAL, FS_E_ALIGN,
 * FS_E_OVERFLOW, FS_E_HIP.
 */
int fs_stream_read(const void *src, int64_t bytes, uint32_t *sink, hipStream_t stream);
int fs_stream_fill(void *dst, int64_t bytes, uint32_t value, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* FS_BENCH_H */
