/*
 * kvattn_measure.h -- a measurement aid shipped with libkvattn; not part of
 * the attention path.
 *
 * The decode kernels are bounded by HBM bandwidth.  Besides the published
 * peak, the benchmark reports the streaming-read rate this device actually
 * sustains, measured with the plain read kernel below, so that the decode
 * rate can be read against both.
 */
#ifndef KVATTN_MEASURE_H
#define KVATTN_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueue on `stream` one read of the `bytes` bytes at device address `buf`
 * (bytes > 0 and a multiple of 16; buf 16-byte aligned) by `workgroups`
 * workgroups of 256 threads, each lane streaming 16-byte words with a grid
 * stride.  The words are folded with xor and the fold is written to
 * sink[blockIdx] (a device array of at least `workgroups` uint32) only if it
 * equals an unlikely constant, so the kernel writes almost nothing.  Returns 0,
 * KVATTN_ERR_INVALID_ARG (-1) for a bad argument, or KVATTN_ERR_HIP (-6) if the
 * launch fails.  Time it with events on the same stream. */
int kvattn_measure_stream_read(const void *buf, size_t bytes, int workgroups, uint32_t *sink,
                               void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KVATTN_MEASURE_H */
