/*
 * pa_decode_q8.h -- INT8 K/V pages for the paged GQA decode library (C ABI).
 *
 * The K/V cache may be stored as INT8 and dequantised back to the compute
 * precision before attention, halving the cache's bytes ("Building an LLM
 * inference engine from scratch: KV cache, operator fusion and quantisation
 * practice", section 5.1); the quantiser is the symmetric one of section
 * 3.4: scale = max|x| / 127, code = clamp(round(x / scale), -128, 127), and
 * a code stands for code * scale.
 *
 * Granularity and arithmetic (where the pages are silent): one FP32 scale per
 * (token, KV head) row of 64 values, separately for K and V; the BF16 input
 * is widened to FP32, scale = max|x| / 127 and x / scale are correctly
 * rounded FP32 divisions, round() is round-half-to-even; an all-zero row
 * stores scale 0 and codes 0.  Inputs must be finite.
 *
 * Layouts (row-major, no padding; 16-byte aligned unless stated):
 *   k_codes/v_codes  int8    [num_pages][8 KV heads][16 slots][64]
 *                    (within a page, each head's 16 code rows are one
 *                    contiguous 1 KiB block)
 *   kv_scales        float32 [num_pages][8 KV heads][2][16 slots]
 *                    ([..][0][s]: K scale of slot s, [..][1][s]: V scale)
 *   one page = 8 KiB of K codes + 8 KiB of V codes + 1 KiB of scales
 *   q, k_new, v_new, k_rows, v_rows, out, block_tables, seq_lens, the
 *   workspace and pa_rope tables: as in pa_decode.h.
 *
 * Memory, ownership, streams and errors are as in pa_decode.h: the caller
 * owns every buffer, calls only enqueue work on `stream`, every call returns
 * PA_OK or a negative pa_status before launching anything, and metadata
 * outside the pool is never followed (NaN outputs, no writes).  The
 * workspace of the decode calls is sized by pa_decode_workspace_bytes with
 * the same arguments (the split partials do not depend on the page format).
 */
#ifndef PA_DECODE_Q8_H
#define PA_DECODE_Q8_H

#include "pa_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Quantised one-token append: for every b with L = seq_lens[b] >= 1, the K
 * row k_new[b] (8 heads x 64 BF16) is quantised head by head into
 * k_codes[page][h][(L-1)%16] and its 8 scales into kv_scales[page][h][0][(L-1)%16],
 * page = block_tables[b][(L-1)/16]; v_new[b] likewise with [..][1][..].
 * Deterministic (the codes and scales are a function of the row alone);
 * nothing else changes.  Idle slots and out-of-range metadata write nothing.
 * Two sequences must not target the same slot in one call.
 */
int pa_append_kv_q8(const pa_shape* shape, int32_t batch,
                    const void* k_new, const void* v_new,
                    void* k_codes, void* v_codes, void* kv_scales,
                    const int32_t* block_tables, const int32_t* seq_lens,
                    void* stream);

/*
 * Quantised append with RoPE: q_out[b] = RoPE(q[b]) and the slot of token
 * L-1 receives the quantised RoPE(k_new[b]) (rotation and BF16 rounding as
 * in pa_append_kv_rope, then quantisation) and the quantised v_new[b].  The
 * tables must cover 16 * max_blocks_per_seq positions.
 */
int pa_append_kv_rope_q8(const pa_shape* shape, int32_t batch,
                         const void* q, const void* k_new, const void* v_new,
                         const pa_rope* rope, void* q_out,
                         void* k_codes, void* v_codes, void* kv_scales,
                         const int32_t* block_tables, const int32_t* seq_lens,
                         void* stream);

/*
 * Quantised prefill fill: tokens start .. start+num_tokens-1 of one sequence
 * (k_rows, v_rows: BF16 [num_tokens][8][64]) quantised into their page slots,
 * token t into page block_table_row[t/16], slot t%16.  Tokens whose page id
 * is outside [0, num_pages) are skipped.
 */
int pa_fill_kv_q8(const pa_shape* shape, const void* k_rows, const void* v_rows,
                  int32_t num_tokens, int32_t start, const int32_t* block_table_row,
                  void* k_codes, void* v_codes, void* kv_scales, void* stream);

/*
 * Decode attention over INT8 pages: pa_decode_attention's result on the
 * dequantised cache (code * scale).  Arguments, planning and workspace as
 * in pa_decode_attention; accuracy against float64 attention over the
 * dequantised cache as for BF16 pages.
 */
int pa_decode_attention_q8(const pa_shape* shape, int32_t batch, const void* q,
                           const void* k_codes, const void* v_codes, const void* kv_scales,
                           const int32_t* block_tables, const int32_t* seq_lens,
                           int32_t max_seq_len, float scale,
                           void* out, int32_t out_dtype, int32_t pages_per_split,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Fused quantised decode step: the effect of pa_append_kv_q8 followed by
 * pa_decode_attention_q8, in one launch (plus the split merge).  The
 * work-group holding a sequence's last page quantises the new rows, writes
 * their codes and scales, and uses the codes in place of what it read for
 * that slot; pools and outputs are identical to the two-call form,
 * including for a sequence longer than max_seq_len (NaN output row; its new
 * row is still quantised and written when 1 <= L <= 16 * max_blocks_per_seq
 * and the page id is valid, as pa_append_kv_q8 does).
 */
int pa_append_decode_attention_q8(const pa_shape* shape, int32_t batch, const void* q,
                                  const void* k_new, const void* v_new,
                                  void* k_codes, void* v_codes, void* kv_scales,
                                  const int32_t* block_tables, const int32_t* seq_lens,
                                  int32_t max_seq_len, float scale,
                                  void* out, int32_t out_dtype, int32_t pages_per_split,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Fused quantised decode step with RoPE: pa_append_kv_rope_q8 followed by
 * pa_decode_attention_q8 on its q_out, in one launch.  The tables must cover
 * max_seq_len positions.
 */
int pa_append_decode_attention_rope_q8(const pa_shape* shape, int32_t batch, const void* q,
                                       const void* k_new, const void* v_new,
                                       const pa_rope* rope,
                                       void* k_codes, void* v_codes, void* kv_scales,
                                       const int32_t* block_tables, const int32_t* seq_lens,
                                       int32_t max_seq_len, float scale,
                                       void* out, int32_t out_dtype, int32_t pages_per_split,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * INT8-page decode step launched from a work list (pa_decode_worklist with
 * page_format 1): as pa_append_decode_attention_worklist, with the pools of
 * this header; k_new/v_new both NULL for decode only.
 */
int pa_append_decode_attention_worklist_q8(const pa_shape* shape, int32_t batch, const void* q,
                                           const void* k_new, const void* v_new,
                                           void* k_codes, void* v_codes, void* kv_scales,
                                           const int32_t* block_tables, const int32_t* seq_lens,
                                           int32_t max_seq_len, float scale,
                                           void* out, int32_t out_dtype, int32_t pages_per_split,
                                           const int32_t* work, int32_t num_work,
                                           void* workspace, size_t workspace_bytes,
                                           void* stream);

/*
 * Split size for INT8 pages from host sequence lengths: pa_decode_plan_lengths
 * with the planner's cost model set for 17 KiB pages.
 */
int pa_decode_plan_lengths_q8(const pa_shape* shape, int32_t batch,
                              const int32_t* seq_lens_host, int32_t max_seq_len,
                              int32_t num_cus, int32_t* pages_out, int32_t* splits_out);

#ifdef __cplusplus
}
#endif

#endif /* PA_DECODE_Q8_H */
