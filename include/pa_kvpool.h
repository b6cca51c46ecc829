/*
 * pa_kvpool.h -- host page allocator and admission control for the shared
 * K/V page pool that feeds the block tables of include/pa_decode.h.
 *
 * Rules ("6 Hours of YouTube and 85 handtyped pages of notes on LLM
 * Inference - Start here", samir-vllm README, section current scope):
 *  - a request reserves credit for its largest processed prefix, prompt +
 *    allowed_new - 1 tokens (the last predicted token is returned without
 *    being processed), rounded up to whole pages, in every layer; the
 *    allowed output budget is min(max_new, context - prompt);
 *  - credit and physical pages are separate: pa_kvpool_grow takes pages
 *    lazily, when a sequence grows into a new page (lowest free page first);
 *  - requests wait in FIFO order while their credit does not fit beside the
 *    active ones (no overtaking); a request whose credit exceeds the whole
 *    pool, or whose prompt leaves no room in the context, is rejected;
 *  - pa_kvpool_finish (early or not) returns the pages and the credit;
 *  - static batching admits the next group only when no request is active.
 *
 * Host memory only: no HIP call is made.  A pool object is not thread-safe;
 * the caller serialises calls on one pool.  Status codes are pa_status
 * values from pa_decode.h (PA_ERR_VALUE for unknown request ids, out-of-order
 * lengths or a too-small output array).
 */
#ifndef PA_KVPOOL_H
#define PA_KVPOOL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pa_kvpool pa_kvpool;            /* opaque */

enum { PA_KV_WAIT = 1, PA_KV_REJECT = 2 };     /* pa_kvpool_submit results */

typedef struct pa_kvpool_stats {               /* the engine's --stats counters */
  int64_t pool_pages;        /* pages in the pool                                   */
  int64_t peak_active;       /* most requests active at once                        */
  int64_t max_batch;         /* largest active set at a pa_kvpool_step (decode step) */
  int64_t peak_allocated;    /* most physical pages held at once                    */
  int64_t admission_waits;   /* requests not admitted by the first pass after submit */
  int64_t free_pages;        /* pages free now                                      */
} pa_kvpool_stats;

/* A pool of num_pages pages of page_tokens tokens, for num_layers layers and a
 * context of context_tokens; static_batching != 0 selects static admission.
 * *out receives the pool (free it with pa_kvpool_destroy). */
int pa_kvpool_create(int32_t num_pages, int32_t num_layers, int32_t page_tokens,
                     int32_t context_tokens, int32_t static_batching, pa_kvpool** out);
int pa_kvpool_destroy(pa_kvpool* pool);

/* Credit of a request: allowed new tokens and reserved pages over all layers. */
int pa_kvpool_credit(const pa_kvpool* pool, int32_t prompt_tokens, int32_t max_new_tokens,
                     int32_t* allowed_new, int64_t* credit_pages);

/* Queue a request: *result = PA_KV_WAIT (queued) or PA_KV_REJECT.
 * request_id must not be in use by a waiting or active request. */
int pa_kvpool_submit(pa_kvpool* pool, int64_t request_id, int32_t prompt_tokens,
                     int32_t max_new_tokens, int32_t* result);

/* One admission pass: admits waiting requests in FIFO order while their credit
 * fits; writes their ids to admitted[0 .. *count) (capacity entries). */
int pa_kvpool_admit(pa_kvpool* pool, int64_t* admitted, int32_t capacity, int32_t* count);

/* Hold pages for tokens 0 .. length-1 of an active request in every layer;
 * length may not shrink nor exceed prompt + allowed_new - 1. */
int pa_kvpool_grow(pa_kvpool* pool, int64_t request_id, int32_t length);

/* Mark a decode step over the current active set (batch-size counter). */
int pa_kvpool_step(pa_kvpool* pool);

/* End an active request: its pages and credit return to the pool. */
int pa_kvpool_finish(pa_kvpool* pool, int64_t request_id);

/* Block-table row of an active request for one layer: row[0 .. *num_pages)
 * are its physical pages in logical order, the rest of row (row_capacity
 * entries) is filled with -1. */
int pa_kvpool_block_table(const pa_kvpool* pool, int64_t request_id, int32_t layer,
                          int32_t* row, int32_t row_capacity, int32_t* num_pages);

/* Allowed new tokens, credit, current length and whether it is active. */
int pa_kvpool_request_info(const pa_kvpool* pool, int64_t request_id, int32_t* allowed_new,
                           int32_t* credit_pages, int32_t* length, int32_t* active);

int pa_kvpool_get_stats(const pa_kvpool* pool, pa_kvpool_stats* out);

#ifdef __cplusplus
}
#endif

#endif /* PA_KVPOOL_H */
