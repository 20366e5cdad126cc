/*
 * qi4_probe.h -- measurement probes exported by libqi4 beside the calls of qi4.h.
 *
 * They measure the two ceilings the library's kernels are held against: the
 * bandwidth of streaming reads from device memory (the decode GEMMs read every
 * weight once per call: the FastLLM page, section 3.1, argues that reading the
 * weights sets the time per token) and the throughput of the fp16 matrix cores
 * (the prefill GEMM is a dense contraction).  Conventions as in qi4.h: device
 * pointers, `stream` a hipStream_t as void*, enqueue only, negative status on
 * error with nothing launched.
 */
#ifndef QI4_PROBE_H
#define QI4_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Words of the `sink` buffer qi4_probe_stream_read writes (one per wave). */
#define QI4_PROBE_READ_SINK_WORDS 8192

/* Read every byte of buf[0, bytes) once (16-byte loads with the non-temporal
 * hint, one contiguous span per workgroup, eight loads in flight per lane).  bytes a positive multiple of 16, buf
 * 16-byte aligned (QI4_ERR_SHAPE otherwise); `sink` receives
 * QI4_PROBE_READ_SINK_WORDS uint32 words (an xor of the data, so the loads are
 * kept).  Time it with events around the call: bytes / time is the achieved
 * read bandwidth. */
int qi4_probe_stream_read(const void *buf, int64_t bytes, uint32_t *sink, void *stream);

/* `workgroups` workgroups of four waves, each wave running `iters` rounds of
 * eight independent fp16 MFMA 16x16x32 chains with no memory traffic; `sink`
 * (one float) is written only in a case that does not arise.  Both counts >= 1
 * (QI4_ERR_SHAPE).  qi4_probe_mfma_flops gives the flops of such a launch (or a
 * negative status); flops / time is the achieved matrix-core throughput. */
int qi4_probe_mfma(int64_t iters, int64_t workgroups, float *sink, void *stream);
int64_t qi4_probe_mfma_flops(int64_t iters, int64_t workgroups);

#ifdef __cplusplus
}
#endif

#endif /* QI4_PROBE_H */
