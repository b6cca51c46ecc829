/*
 * Balanced launch of paged GQA decode attention: one wavefront per
 * (sequence, KV head) stream, streams packed into work-groups by the host,
 * no split partials in device memory and no merge launch.
 *
 * The decode attention is that of include/pa_decode.h (the samir-vllm
 * README's paged decode attention, "features completed so far": each
 * sequence's query heads read that sequence's pages through its block table
 * with an FP32 online softmax; grouped-query attention, query heads 4g ..
 * 4g+3 read KV head g).  This launch changes only how the work is spread:
 *
 *   - a "stream" is the pages of one sequence's KV head (ceil(L/16) pages);
 *     its 4 query heads are served by the one wavefront that streams it;
 *   - pa_balance_plan (host) packs whole streams into work-groups, the
 *     largest first into the least-loaded group, so that every work-group
 *     gets about the same number of pages; the heads of a sequence go
 *     together in groups of 1, 2, 4 or 8 (one wavefront per head, in
 *     lockstep); within a work-group the units are laid end to end and cut
 *     evenly across its groups of wavefronts, so a stream may be split over
 *     wavefronts of one work-group (never over two work-groups);
 *   - each wavefront streams its pages without a break between streams, and
 *     the pieces of a stream split over wavefronts are merged in LDS by the
 *     work-group after one barrier (log-sum-exp, in wavefront order).
 *
 * Results equal the oracle within the same tolerance as pa_decode_attention;
 * they are deterministic run to run for a given plan but not bitwise equal to
 * the grid launch (the pages are summed in other groups).
 */
#ifndef PA_DECODE_BALANCED_H
#define PA_DECODE_BALANCED_H

#include <stddef.h>
#include <stdint.h>

#include "pa_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Plan of the balanced launch for host lengths (a scheduler knows them).
 *   seq_lens_host  HOST int32 [batch], the lengths the device will hold
 *                  when the plan is used (after the append); each within
 *                  [0, max_seq_len] and the block table's capacity
 *   num_cus        compute units to plan for (0: the current device's)
 *   heads_together 1, 2, 4 or 8: how many KV heads of a sequence one group of
 *                  wavefronts streams in lockstep (so their 128-byte slices of
 *                  each token row are read together).  8 packs whole
 *                  sequences into work-groups and never splits one (best when
 *                  no sequence is longer than a work-group's share of the
 *                  pages); 1 and 2 may split a sequence's heads over the
 *                  wavefronts of a work-group (for batches of few, long
 *                  sequences)
 *   plan           HOST int32 buffer of capacity_words words, or NULL to
 *                  query the size; the caller copies the plan to the device.
 *                  Every word of the plan is written.
 *   *words_out     words the plan takes, 64 + groups * 8 * 64;
 *                  *groups_out work-groups to launch.  Both are set also
 *                  when capacity_words is too small (PA_ERR_VALUE), so a
 *                  caller can offer room for its usual plan (groups = the
 *                  compute units) and call again only when it is short.
 * Planning runs on the host once per batch of lengths, that is once per
 * decode step of a serving loop; it reuses its buffers from call to call
 * (one set per calling thread).  Measured on the host of an MI355X machine
 * (bench.py's plan_host_us): 512 Zipf lengths, 8 heads per lane, 256
 * work-groups, 28 us (the GPU step: about 164 us); 64 uniform lengths, 1 head
 * per lane, 29 us; 512 Zipf lengths, 1 head per lane, 84 us.
 * Returns PA_ERR_VALUE when the batch cannot be planned this way (a
 * wavefront would hold more than 7 stream pieces or 256 pages even with
 * more work-groups; batches of very many one-page sequences, or sequences
 * beyond 32,768 tokens): use pa_decode_attention or the work list then.
 * The plan is valid for these lengths only.  Makes no HIP call when
 * num_cus > 0.
 */
int pa_balance_plan(const pa_shape* shape, int32_t batch, const int32_t* seq_lens_host,
                    int32_t max_seq_len, int32_t num_cus, int32_t heads_together,
                    int32_t* plan, int64_t capacity_words, int64_t* words_out,
                    int32_t* groups_out);

/*
 * Decode step over a balanced plan, for every page format:
 *   page_format 0  BF16 pages (k_pool, v_pool as in pa_decode.h; kv_scales NULL)
 *               1  INT8 pages (codes and scales as in pa_decode_q8.h)
 *               2  INT4 pages (as in pa_decode_q4.h)
 * k_new and v_new: both NULL (attention only) or both given (the fused
 * append of pa_append_decode_attention, quantised for pages 1 and 2: each
 * sequence's new row is written into slot (L-1)%16 of its last page and
 * attended from registers).  rope: NULL, or the tables of
 * pa_append_decode_attention_rope (requires k_new; the tables must cover
 * max_seq_len positions).  plan: DEVICE int32 copy of pa_balance_plan's
 * output, plan_words and groups as it returned them.  No workspace: the
 * pieces of a stream meet in LDS.  The device lengths must be the ones the
 * plan was built from: a sequence whose device length differs gets NaN
 * outputs and no append; one longer than max_seq_len, or with a used
 * block-table entry outside the pool, gets NaN outputs, and its new row is
 * written as pa_append_kv would (when its target page id lies in the pool).
 * A pool of more than 2^28 pages returns PA_ERR_VALUE (a page id travels
 * with its KV head in one 32-bit word).  Enqueues one kernel on `stream`.
 */
int pa_decode_balanced(const pa_shape* shape, int32_t batch, const void* q,
                       const void* k_new, const void* v_new, const pa_rope* rope,
                       void* k_pool, void* v_pool, void* kv_scales, int32_t page_format,
                       const int32_t* block_tables, const int32_t* seq_lens,
                       int32_t max_seq_len, float scale, void* out, int32_t out_dtype,
                       const int32_t* plan, int64_t plan_words, int32_t groups,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_DECODE_BALANCED_H */
