/*
 * pa_decode_q4.h -- INT4 K/V pages for the paged GQA decode library (C ABI).
 *
 * The K/V cache may be held at a lower precision than the compute type, INT8
 * or even INT4, and dequantised before attention ("Building an LLM inference
 * engine from scratch: KV cache, operator fusion and quantisation practice",
 * section 5.1).  These entry points store it at 4 bits with the symmetric
 * quantiser of section 3.4 taken with bits = 4: scale = max|x| / 7, code =
 * clamp(round(x / scale), -8, 7), and a code stands for code * scale.
 *
 * Granularity and arithmetic are those of the INT8 pages (pa_decode_q8.h):
 * one FP32 scale per (token, KV head) row of 64 values, separately for K and
 * V; BF16 widened to FP32, correctly rounded FP32 divisions, round-half-to-
 * even; an all-zero row stores scale 0 and codes 0.  Inputs must be finite.
 *
 * Storage (the pages leave it open): two codes per byte, each stored as
 * code + 8 (0..15); byte j of a row holds dim 2j in its low nibble and dim
 * 2j+1 in its high nibble.
 *
 * Layouts (row-major, no padding; 16-byte aligned unless stated):
 *   k_codes/v_codes  uint8   [num_pages][8 KV heads][16 slots][32]
 *                    (within a page, each head's 16 code rows are one
 *                    contiguous 512-byte block)
 *   kv_scales        float32 [num_pages][8 KV heads][2][16 slots], as for
 *                    INT8 pages
 *   one page = 4 KiB of K codes + 4 KiB of V codes + 1 KiB of scales
 *   q, k_new, v_new, k_rows, v_rows, out, block_tables, seq_lens, the
 *   workspace and pa_rope tables: as in pa_decode.h.
 *
 * Each call behaves as its INT8 namesake in pa_decode_q8.h (same arguments,
 * same checks, same status codes) with the pools above.  Memory, ownership,
 * streams and errors are as in pa_decode.h: the caller owns every buffer,
 * calls only enqueue work on `stream`, every call returns PA_OK or a
 * negative pa_status before launching anything, and metadata outside the
 * pool is never followed (NaN outputs, no writes).  The workspace of the
 * decode calls is sized by pa_decode_workspace_bytes with the same arguments.
 */
#ifndef PA_DECODE_Q4_H
#define PA_DECODE_Q4_H

#include "pa_decode.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Quantised one-token append at 4 bits: for every b with L = seq_lens[b] >= 1,
 * the rows k_new[b] and v_new[b] (8 heads x 64 BF16) are quantised head by
 * head into slot (L-1)%16 of page block_tables[b][(L-1)/16], codes and
 * scales.  Idle slots and out-of-range metadata write nothing.  Two
 * sequences must not target the same slot in one call.
 */
int pa_append_kv_q4(const pa_shape* shape, int32_t batch,
                    const void* k_new, const void* v_new,
                    void* k_codes, void* v_codes, void* kv_scales,
                    const int32_t* block_tables, const int32_t* seq_lens,
                    void* stream);

/*
 * As pa_append_kv_q4 with RoPE: q_out[b] = RoPE(q[b]), and the key is
 * rotated (and rounded to BF16) before it is quantised.  The tables must
 * cover 16 * max_blocks_per_seq positions.
 */
int pa_append_kv_rope_q4(const pa_shape* shape, int32_t batch,
                         const void* q, const void* k_new, const void* v_new,
                         const pa_rope* rope, void* q_out,
                         void* k_codes, void* v_codes, void* kv_scales,
                         const int32_t* block_tables, const int32_t* seq_lens,
                         void* stream);

/*
 * Quantised prefill fill at 4 bits: tokens start .. start+num_tokens-1 of one
 * sequence (k_rows, v_rows: BF16 [num_tokens][8][64]) into their page slots.
 * Tokens whose page id is outside [0, num_pages) are skipped.
 */
int pa_fill_kv_q4(const pa_shape* shape, const void* k_rows, const void* v_rows,
                  int32_t num_tokens, int32_t start, const int32_t* block_table_row,
                  void* k_codes, void* v_codes, void* kv_scales, void* stream);

/*
 * Decode attention over INT4 pages: pa_decode_attention's result on the
 * dequantised cache (code * scale), with its arguments, planning and
 * workspace; accuracy against float64 attention over the dequantised cache
 * as for BF16 pages.  A plan whose grid (batch x splits) fits the device's
 * compute units at once, with splits of 32 pages or more, runs two
 * wavefronts per KV head (each takes half of a split's pages; their states
 * are merged in the work-group): the summation order, and so the last bits
 * of the result, depend on the plan and the device's compute-unit count.
 * Results are deterministic run to run on one device, and the grid and
 * work-list launches of one plan agree bit for bit.
 */
int pa_decode_attention_q4(const pa_shape* shape, int32_t batch, const void* q,
                           const void* k_codes, const void* v_codes, const void* kv_scales,
                           const int32_t* block_tables, const int32_t* seq_lens,
                           int32_t max_seq_len, float scale,
                           void* out, int32_t out_dtype, int32_t pages_per_split,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * Fused decode step over INT4 pages: pa_append_kv_q4 followed by
 * pa_decode_attention_q4 in one launch (plus the split merge); pools and
 * outputs identical to the two-call form, with the same append rule for a
 * sequence longer than max_seq_len as pa_append_decode_attention_q8.
 */
int pa_append_decode_attention_q4(const pa_shape* shape, int32_t batch, const void* q,
                                  const void* k_new, const void* v_new,
                                  void* k_codes, void* v_codes, void* kv_scales,
                                  const int32_t* block_tables, const int32_t* seq_lens,
                                  int32_t max_seq_len, float scale,
                                  void* out, int32_t out_dtype, int32_t pages_per_split,
                                  void* workspace, size_t workspace_bytes, void* stream);

/*
 * Fused decode step with RoPE over INT4 pages: pa_append_kv_rope_q4 followed
 * by pa_decode_attention_q4 on its q_out, in one launch.  The tables must
 * cover max_seq_len positions.
 */
int pa_append_decode_attention_rope_q4(const pa_shape* shape, int32_t batch, const void* q,
                                       const void* k_new, const void* v_new,
                                       const pa_rope* rope,
                                       void* k_codes, void* v_codes, void* kv_scales,
                                       const int32_t* block_tables, const int32_t* seq_lens,
                                       int32_t max_seq_len, float scale,
                                       void* out, int32_t out_dtype, int32_t pages_per_split,
                                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * INT4-page decode step launched from a work list (pa_decode_worklist with
 * page_format 2); k_new/v_new both NULL for decode only.
 */
int pa_append_decode_attention_worklist_q4(const pa_shape* shape, int32_t batch, const void* q,
                                           const void* k_new, const void* v_new,
                                           void* k_codes, void* v_codes, void* kv_scales,
                                           const int32_t* block_tables, const int32_t* seq_lens,
                                           int32_t max_seq_len, float scale,
                                           void* out, int32_t out_dtype, int32_t pages_per_split,
                                           const int32_t* work, int32_t num_work,
                                           void* workspace, size_t workspace_bytes,
                                           void* stream);

/*
 * Split size for INT4 pages from host sequence lengths: pa_decode_plan_lengths
 * with the planner's cost model set for 9 KiB pages.
 */
int pa_decode_plan_lengths_q4(const pa_shape* shape, int32_t batch,
                              const int32_t* seq_lens_host, int32_t max_seq_len,
                              int32_t num_cus, int32_t* pages_out, int32_t* splits_out);

#ifdef __cplusplus
}
#endif

#endif /* PA_DECODE_Q4_H */
