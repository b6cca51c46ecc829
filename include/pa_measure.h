/*
 * pa_measure.h -- measurement helpers of the paged GQA decode library (C ABI).
 *
 * The decode path is bound by HBM bandwidth ("6 Hours of YouTube and 85
 * handtyped pages of notes on LLM Inference - Start here", samir-vllm README:
 * decode is memory-bound; "Building an LLM inference engine from scratch",
 * section 5.1: the KV cache grows with every token).  Beside the device's
 * published peak, a benchmark reports what a plain streaming read achieves on
 * the same device (pa_stream_read), and what the decode kernels' own page
 * reads achieve when nothing else is computed (pa_page_stream), and where the
 * time of a balanced launch goes (pa_decode_balanced_timeline).
 */
#ifndef PA_MEASURE_H
#define PA_MEASURE_H

#include <stddef.h>
#include <stdint.h>

#include "pa_decode.h"

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

/*
 * Page stream: the page reads of the decode kernels without their
 * arithmetic, so that a benchmark can set a kernel's time beside the time of
 * its own access pattern.  The pages are those the decode attention reads
 * through the block tables ("6 Hours of YouTube ...", samir-vllm README,
 * features completed so far: a page map and an attention length per
 * sequence), in the pools of pa_decode.h (page_format 0, BF16), pa_decode_q8.h
 * (1, INT8 codes and scales) or pa_decode_q4.h (2, INT4 codes and scales).
 *
 * One work-group per sequence b < batch; for each of the 8 KV heads,
 * waves_per_head wavefronts (1 or 2: the first and the second half of the
 * pages) stream the head's blocks of the ceil(seq_lens[b] / 16) pages named
 * by block_tables[b] through a ring of `ring` LDS slots per wavefront (1..3),
 * with the decode kernel's direct-to-LDS loads, cache policy and waits for
 * that format.  Each landed page is read back from LDS and every 32-bit word
 * of the head's blocks (K, V and, for codes, the head's scale line) is folded
 * by XOR into one word per wavefront, stored at
 * sink[b * 8 * waves_per_head + head * waves_per_head + half].
 * A length outside [0, 16 * max_blocks_per_seq] streams nothing (fold 0); a
 * block-table entry outside [0, num_pages) reads page 0.
 *
 * shape: as for the decode entry points, max_blocks_per_seq <= 256.  Pools:
 * device, 16-byte aligned (kv_scales may be NULL for BF16 pages);
 * block_tables, seq_lens: device int32 [batch][max_blocks_per_seq], [batch];
 * sink: device, batch * 8 * waves_per_head uint32 words.  The rings of a
 * work-group (ring x 8 x waves_per_head slots of 4 KiB for BF16, 2304 B for
 * INT8, 1280 B for INT4) must fit the 160 KiB of LDS of a CU, else
 * PA_ERR_VALUE (BF16 pages with 2 wavefronts per head: ring <= 2).
 * Enqueued on `stream`; returns PA_OK or a negative pa_status (PA_ERR_NULL,
 * PA_ERR_SHAPE, PA_ERR_ALIGN, PA_ERR_VALUE, PA_ERR_LAUNCH as in pa_decode.h).
 */
int pa_page_stream(const pa_shape* shape, int32_t batch, const void* k_pool, const void* v_pool,
                   const void* kv_scales, int32_t page_format, const int32_t* block_tables,
                   const int32_t* seq_lens, int32_t waves_per_head, int32_t ring, uint32_t* sink,
                   void* stream);

/*
 * Timeline of a balanced launch: pa_decode_balanced (pa_decode_balanced.h)
 * with FP32 output and no RoPE, the same reads, arithmetic and writes, which
 * also records for every wavefront the device's constant-rate real-time
 * counter (pa_wall_clock_khz ticks per millisecond) at seven points of its
 * work.  A benchmark can then tell a launch's fixed costs (the memory round
 * trips before the first page lands, the output stores at the end) from its
 * page stream, and see how evenly its work-groups finish (the samir-vllm
 * README's decode is memory-bound, so these are what a launch spends beside
 * its reads).
 *
 * stamps: device uint64 [groups][8 wavefronts][8 words], 8-byte aligned,
 * stamp_words >= groups * 64 (else PA_ERR_VALUE; NULL: PA_ERR_NULL).  Per
 * wavefront:
 *   [0] start            [1] its plan descriptor in
 *   [2] lengths, page ids and q rows in
 *   [3] first page in LDS (0 when the wavefront has no pages)
 *   [4] last page consumed
 *   [5] every output store issued   [6] every store acknowledged
 *   [7] bits 0..31 the HW_ID hardware register as read, bits 32..47 the
 *       XCC_ID register (which of the 8 dies the work-group ran on), bits
 *       48..63 the wavefront's page count.
 * The stamps are written once a wavefront's stores are acknowledged, so
 * [6] - [0] covers the wavefront's whole life.  Other arguments, results and
 * errors as for pa_decode_balanced (out: FP32).
 */
int pa_decode_balanced_timeline(const pa_shape* shape, int32_t batch, const void* q,
                                const void* k_new, const void* v_new, void* k_pool, void* v_pool,
                                void* kv_scales, int32_t page_format, const int32_t* block_tables,
                                const int32_t* seq_lens, int32_t max_seq_len, float scale,
                                float* out, const int32_t* plan, int64_t plan_words,
                                int32_t groups, uint64_t* stamps, int64_t stamp_words,
                                void* stream);

/*
 * Rate of the real-time counter that pa_decode_balanced_timeline reads, in
 * kHz, for the current device.  Returns PA_OK, PA_ERR_NULL or PA_ERR_DEVICE.
 */
int pa_wall_clock_khz(int32_t* khz);

#ifdef __cplusplus
}
#endif

#endif /* PA_MEASURE_H */
