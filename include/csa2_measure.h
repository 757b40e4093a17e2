/*
 * csa2_measure.h -- measurement helpers exported by libcsa2.so beside the
 * decode path (include/csa2.h).  They are not steps of the method: they give
 * the plain read rate of the device (the ceiling the Full scan's key stream
 * is measured against), the cost of a dependent kernel node, and the cost of
 * handing split partials to a merge inside one kernel instead of in a second
 * one (the choice between one and two kernels per attention layer).
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

/*
 * csa2_empty_kernel -- launch one workgroup of 64 threads that does nothing,
 * on `stream`: a chain of them in a captured graph times the cost of a
 * dependent kernel node.
 */
int csa2_empty_kernel(void* stream);

/* Bytes of scratch csa2_handoff needs for `groups` x `splits` partials (0 on
 * invalid sizes). */
size_t csa2_handoff_scratch_bytes(int groups, int splits);

/*
 * csa2_handoff -- what handing split partial results to a merge costs, the
 * step between the decode path's split attention and its combine.  groups x
 * splits workgroups each write a partial of 8,192 floats (value + split +
 * index * 1e-6), and out[g][i] (8,192 floats per group, device) becomes the
 * sum over group g's splits.  All workgroups of a group run on one XCD.
 *   mode 0: two kernels, the partials then a merge kernel;
 *   mode 1: one kernel: partials stored through to memory (device-scope
 *           relaxed atomic stores), a per-group arrival counter that every
 *           workgroup of the group waits on, then each merges 1/splits of the
 *           outputs with device-scope relaxed loads;
 *   mode 2: one kernel: plain stores, a device-scope release fence, the
 *           counter, an acquire fence, plain loads.
 * Modes 1 and 2 keep at most 256 workgroups (8 * ceil(groups / 8) * splits),
 * so all of them are resident at once; each wait is bounded (2^16 polls) and
 * a workgroup that gives up writes NaN.  scratch: csa2_handoff_scratch_bytes
 * bytes, 256-byte aligned, device memory whose last 8 * groups bytes
 * (the counters) are zero before the first call; every call leaves them
 * zero.  Calls on one scratch must not overlap.
 * Errors: INVALID for bad modes, sizes or pointers; WORKSPACE for a small
 * scratch; UNSUPPORTED for more than 256 workgroups in modes 1 and 2.
 */
int csa2_handoff(int mode, int groups, int splits, float value, void* scratch,
                 size_t scratch_bytes, float* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_MEASURE_H */
