/*
 * mtp_probe.h -- measurement helper beside the verify-step library (not part
 * of the verify step): a plain streaming read of device memory, the
 * reference for what a read-only kernel reaches on this device, reported next
 * to the 8 TB/s peak when the verify attention's bandwidth is measured.
 */
#ifndef MTP_PROBE_H
#define MTP_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes at device pointer `src` once (16-byte vector loads,
 * one pass, every byte folded into a checksum so that no load can be
 * dropped) and writes nothing except, with negligible probability, the
 * checksum to sink[0] (a device uint32).  src must be 16-byte aligned and
 * bytes a multiple of 16; returns 0 when launched, 2 for a bad size or
 * alignment, 1 for a NULL pointer, 5 for a launch error.  Asynchronous on
 * `stream` (a hipStream_t). */
int32_t mtp_probe_stream_read(const void* src, size_t bytes, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MTP_PROBE_H */
