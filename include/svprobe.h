/*
 * svprobe.h -- C ABI of libsvprobe, the streaming-read ceiling measured by the
 * benchmark next to the verify step (a measurement kernel, not part of the
 * verify step).
 */
#ifndef SVPROBE_H
#define SVPROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` (rounded down to whole 16-byte vectors) of the DEVICE buffer
 * `buf` (16-byte aligned) in `groups` contiguous chunks, one 256-thread
 * workgroup each, with the row-statistics kernel's load pattern (tiles of 8
 * non-temporal 16-byte loads per thread, two tiles in flight) and no other
 * arithmetic than an XOR fold; writes one word per workgroup to the DEVICE
 * array `out` [groups].  Enqueued on `stream` (a hipStream_t, NULL = default);
 * `events`, if not NULL, holds a hipEvent_t pair recorded around the kernel.
 * Returns 0, -1 for bad arguments (checked on the host, nothing enqueued) or
 * -3 if the launch failed. */
int sv_stream_probe(const void *buf, size_t bytes, int groups, unsigned *out, void *stream, void *events[2]);

#ifdef __cplusplus
}
#endif

#endif /* SVPROBE_H */
