/*
 * csa2_measure.h -- measurement helper exported by libcsa2.so beside the decode
 * path (include/csa2.h).  It is not a step of the method: it gives the plain
 * read rate of the device, the ceiling that the Full scan's key stream (64
 * bytes per cached position, read once) is measured against.
 */
#ifndef CSA2_MEASURE_H
#define CSA2_MEASURE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Words of `sink` that csa2_stream_read needs for `bytes` (one per 64 KiB). */
size_t csa2_stream_read_sink_words(size_t bytes);

/*
 * csa2_stream_read -- read `bytes` bytes at `src` (device memory, 16-byte
 * aligned, bytes a multiple of 16) once, in the scoring kernel's launch shape:
 * one 512-thread workgroup per 64 KiB, each thread issuing eight 16-byte loads
 * before it uses any.  Writes an XOR of the data, one 32-bit word per
 * workgroup, to sink[0 .. csa2_stream_read_sink_words(bytes)) (device).
 * Asynchronous on `stream`.  Errors: INVALID for null or misaligned pointers,
 * WORKSPACE when sink_words is too small.  bytes == 0 is a no-op.
 */
int csa2_stream_read(const void* src, size_t bytes, unsigned int* sink, size_t sink_words,
                     void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_MEASURE_H */
