/*
 * pa_measure.h -- measurement helper of the paged GQA decode library (C ABI).
 *
 * The decode path is bound by HBM bandwidth ("6 Hours of YouTube and 85
 * handtyped pages of notes on LLM Inference - Start here", samir-vllm README:
 * decode is memory-bound; "Building an LLM inference engine from scratch",
 * section 5.1: the KV cache grows with every token).  Beside the device's
 * published peak, a benchmark reports what a plain streaming read achieves on
 * the same device: this entry point is that read.
 */
#ifndef PA_MEASURE_H
#define PA_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Streaming read: every 16-byte word of buf[0 .. bytes) is read once (each
 * work-group takes 16 KiB chunks, 16 bytes per lane per load with the
 * non-temporal cache policy, and strides
 * over the buffer) and folded into one 32-bit word per work-group, written
 * to sink[work-group] so the reads cannot be elided.  buf: device, 16-byte
 * aligned, bytes a positive multiple of 16.  sink: device, at least `groups`
 * uint32 words; groups in [1, 65536] (0 = 4 per compute unit).
 * Enqueued on `stream`; returns PA_OK or a negative pa_status (PA_ERR_NULL,
 * PA_ERR_ALIGN, PA_ERR_VALUE, PA_ERR_DEVICE, PA_ERR_LAUNCH as in pa_decode.h).
 */
int pa_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t groups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_MEASURE_H */
