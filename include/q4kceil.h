/*
 * q4kceil.h -- measurement entry point of libq4kmoe.so: the read ceiling that
 * the hot-path kernels are measured against.  It is not part of the method
 * (cortiq-engine mv_lab.rs: the loads-only kernel `ld`, the ceiling of an
 * access pattern; here the plainest pattern over the same bytes).
 */
#ifndef Q4KCEIL_H
#define Q4KCEIL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads every byte of n_ranges ranges of range_bytes bytes, range i at
 * base + offsets[i] (offsets: a DEVICE array of n_ranges int64 byte offsets),
 * with coalesced 16-byte loads, 16 KB per workgroup, and keeps only a
 * checksum; sink (a device word) is written only when the checksum hits a
 * fixed 32-bit value.  Enqueued on `stream` (a hipStream_t, NULL = default).
 * base 16-byte aligned, every base + offsets[i] 16-byte aligned (caller's
 * precondition), range_bytes >= 16 and a multiple of 16.  Returns 0, 1 (bad
 * size), 2 (null or misaligned pointer) or 5 (launch failed). */
int q4k_ceiling_read(const void *base, const int64_t *offsets, int64_t n_ranges,
                     int64_t range_bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* Q4KCEIL_H */
