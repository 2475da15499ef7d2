/*
 * kvattn_measure.h -- a measurement aid shipped with libkvattn; not part of
 * the attention path.
 *
 * The decode kernels are bounded by HBM bandwidth and the prefill kernel by
 * the matrix cores (at small head dims also by the one exponential each score
 * needs).  Besides the published peaks, the benchmark reports the
 * streaming-read rate, the fp16 MFMA rate and the exp2 rate this device
 * actually sustains, measured with the plain kernels below, so that each
 * kernel's rate can be read against them.
 */
#ifndef KVATTN_MEASURE_H
#define KVATTN_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#include "kvattn.h"

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

/* Enqueue on `stream` one write of the `bytes` bytes at device address `buf`
 * (bytes > 0 and a multiple of 16; buf 16-byte aligned) by `workgroups`
 * workgroups of 256 threads, each lane storing whole 16-byte words with a grid
 * stride (word j holds j, j ^ 0x55555555, j + 1 and ~j in its four uint32, j
 * taken mod 2^32).  Plain coalesced stores, like the attention kernels' output
 * and cache rows: the memory counters' reading for it calibrates their reading
 * for those kernels.  Returns 0, KVATTN_ERR_INVALID_ARG (-1) for a bad
 * argument, or KVATTN_ERR_HIP (-6) if the launch fails. */
int kvattn_measure_stream_write(void *buf, size_t bytes, int workgroups, void *stream);

/* Enqueue on `stream` a plain matrix-core loop: `workgroups` workgroups of four
 * waves, each wave running `iters` rounds of eight independent chains of
 * v_mfma_f32_16x16x32_f16 (fp16 inputs, fp32 accumulation) on register
 * operands, with no memory traffic in the loop.  The sums are written to
 * sink[blockIdx] (a device array of at least `workgroups` floats) only if
 * they equal an unlikely constant.  Returns 0, KVATTN_ERR_INVALID_ARG (-1) or
 * KVATTN_ERR_HIP (-6).  Time it with events on the same stream and divide
 * kvattn_measure_mfma_f16_flops(workgroups, iters) by the time: the fp16
 * MFMA rate the device sustains (the prefill kernel's matrix work is of this
 * instruction). */
int kvattn_measure_mfma_f16(int workgroups, int iters, float *sink, void *stream);

/* Floating-point operations of one such launch (0 for a non-positive
 * argument).  Pure host function. */
double kvattn_measure_mfma_f16_flops(int workgroups, int iters);

/* Enqueue on `stream` a plain exponential loop: `workgroups` workgroups of 256
 * threads, each thread running `iters` rounds of 32 independent chains
 * x <- exp2(-x) (one v_exp_f32 per exponential, fp32), with no memory
 * traffic in the loop.  The sums are written to sink[blockIdx] (a device
 * array of at least `workgroups` floats) only if they equal an unlikely
 * constant.  Returns 0, KVATTN_ERR_INVALID_ARG (-1) or KVATTN_ERR_HIP (-6).
 * Time it with events on the same stream and divide
 * kvattn_measure_exp2_count(workgroups, iters) by the time: the exponential
 * rate the device sustains (the prefill kernel's exponentials are of this
 * instruction). */
int kvattn_measure_exp2(int workgroups, int iters, float *sink, void *stream);

/* Exponentials of one such launch (0 for a non-positive argument).  Pure host
 * function. */
double kvattn_measure_exp2_count(int workgroups, int iters);

/* The sustained shader clock of a prefill: kvattn_prefill (same arguments,
 * same kernels, same result and cache update) with one addition: when the
 * prompt runs on the pipelined 16-bit kernel, workgroup 0 (the heaviest query
 * tile, enqueued first) reads the shader-clock counter (s_memtime) and the
 * 100 MHz real-time counter (s_memrealtime) when it starts and when it ends,
 * and writes the two differences to sample[0] (shader cycles) and sample[1]
 * (real-time ticks), a device array of two uint64.  sample[0] / sample[1] *
 * 0.1 GHz is then the mean shader clock over that workgroup's life, which
 * spans most of the launch.  Other prompts leave `sample` unwritten.  Returns
 * what kvattn_prefill returns, or KVATTN_ERR_INVALID_ARG for a null sample. */
int kvattn_measure_prefill_clock(kvattn_cache *c, int layer, const void *q, const void *k, const void *v,
                                 void *o, int T, float scale, kvattn_dtype o_dtype, uint64_t *sample,
                                 void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KVATTN_MEASURE_H */
