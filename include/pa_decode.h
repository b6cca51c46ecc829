/*
 * pa_decode.h -- C ABI of the MI355X (gfx950) paged GQA decode library.
 *
 * Operations (defined by the pages of the subject, cited by title/section):
 *
 *  - pa_append_kv: decode writes each sequence's new K/V row into its page
 *    slot at the token's absolute position ("6 Hours of YouTube and 85
 *    handtyped pages of notes on LLM Inference - Start here", samir-vllm
 *    README, features completed so far: shared BF16 KV page pool, a block
 *    table per sequence and layer, 16 tokens of K and V per physical page).
 *
 *  - pa_decode_attention: each active sequence's new query, 32 query heads
 *    over 8 KV heads of dimension 64, attends that sequence's cached tokens
 *    through its block table and attention length, with an FP32 online
 *    softmax, never gathering a contiguous prefix and never storing scores
 *    (same page, same section: direct paged decode attention; batched decode
 *    with a page map and attention length per sequence).  The result is the
 *    textbook single-query attention: scores q.K^T scaled by `scale`,
 *    max-subtracted softmax over the sequence, weighted sum of V
 *    ("Building an LLM inference engine from scratch: KV cache, operator
 *    fusion and quantisation practice", section 3.2).
 *
 * Memory and ownership (same README: preallocated device buffers, reused;
 * request count never grows the pool): every buffer is allocated and owned
 * by the caller.  The library allocates no device memory and keeps no
 * mutable global state besides a per-device cache of the compute-unit
 * count and, for pa_append_decode_attention_noalloc, a static device array
 * per GPU (part of the loaded code object) and its address.  All device
 * pointers are HIP device addresses.  Calls only enqueue
 * work on `stream` (a hipStream_t; NULL means the default stream) and
 * return without synchronising, except pa_validate_metadata.
 *
 * Errors (same README, current scope: impossible requests get an explicit
 * error, never a silent one): every call returns PA_OK or a negative
 * pa_status before it launches anything.  Host-checkable mistakes are
 * reported: NULL pointers, unsupported shapes, misaligned pointers, an
 * undersized workspace, out-of-range sizes.  Device-resident metadata
 * (page ids, lengths) cannot be checked without a synchronisation; the
 * kernels never read or write outside the pool for any metadata value: a
 * sequence whose block-table entries fall outside [0, num_pages) or whose
 * length exceeds the capacity gets NaN in every output element, and an
 * append with such metadata writes nothing.  pa_validate_metadata checks
 * metadata explicitly.
 *
 * Supported shape: num_q_heads 32, num_kv_heads 8, head_dim 64, page_size
 * 16 (anything else returns PA_ERR_SHAPE).
 */
#ifndef PA_DECODE_H
#define PA_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_NULL = -1,      /* a required pointer is NULL                          */
  PA_ERR_SHAPE = -2,     /* head counts / head_dim / page_size not supported    */
  PA_ERR_ALIGN = -3,     /* a pointer is not aligned as documented              */
  PA_ERR_WORKSPACE = -4, /* workspace missing or smaller than required          */
  PA_ERR_LAUNCH = -5,    /* HIP reported an error when launching                */
  PA_ERR_VALUE = -6,     /* a size or scalar argument is out of range           */
  PA_ERR_METADATA = -7,  /* pa_validate_metadata found a bad table or length    */
  PA_ERR_DEVICE = -8     /* HIP device query failed                             */
} pa_status;

typedef enum pa_out_dtype {
  PA_OUT_F32 = 0,        /* float32 output (the default for parity)             */
  PA_OUT_BF16 = 1        /* BF16 output, round-to-nearest-even                  */
} pa_out_dtype;

/* Geometry of one layer's pool region.  Passed by pointer, read only. */
typedef struct pa_shape {
  int32_t num_q_heads;        /* Hq = 32                                        */
  int32_t num_kv_heads;       /* Hkv = 8; query head h reads KV head h / 4      */
  int32_t head_dim;           /* D = 64                                         */
  int32_t page_size;          /* P = 16 tokens per page                         */
  int32_t num_pages;          /* pages in the region k_pool / v_pool point at   */
  int32_t max_blocks_per_seq; /* row length (stride) of block_tables, >= 1;
                                 capacity of a sequence = 16 * this             */
} pa_shape;

/*
 * Layouts (all row-major, no padding):
 *   q             BF16  [batch][Hq][D]                 16-byte aligned
 *   k_pool/v_pool BF16  [num_pages][P][Hkv][D]         16-byte aligned
 *                 token t of sequence b lives in page block_tables[b][t/16],
 *                 slot t%16; one page = 16 KiB of K plus 16 KiB of V
 *   k_new/v_new   BF16  [batch][Hkv][D]                16-byte aligned
 *   block_tables  int32 [batch][max_blocks_per_seq]    4-byte aligned;
 *                 entries past ceil(seq_len/16) are never read
 *   seq_lens      int32 [batch]                        4-byte aligned;
 *                 length AFTER the append; 0 marks an idle batch slot
 *   out           [batch][Hq][D], float32 or BF16      16-byte aligned
 */

/*
 * Append one token per sequence: for every b with L = seq_lens[b] >= 1,
 * copy k_new[b] (8 x 64 BF16, 1 KiB) to k_pool[block_tables[b][(L-1)/16]]
 * [(L-1)%16] and v_new[b] likewise.  Bit-exact copy; nothing else in the
 * pools changes.  Idle slots (L == 0) and sequences whose target page id or
 * length is out of range write nothing.  Two sequences must not target the
 * same slot in one call.  batch == 0 is a no-op returning PA_OK.
 */
int pa_append_kv(const pa_shape* shape, int32_t batch,
                 const void* k_new, const void* v_new,
                 void* k_pool, void* v_pool,
                 const int32_t* block_tables, const int32_t* seq_lens,
                 void* stream);

/*
 * Prefill page fill: write tokens start .. start+num_tokens-1 of one
 * sequence into its pages (the prompt's K/V, one prompt at a time, as the
 * engine prefills), token t into page block_table_row[t/16], slot t%16.
 * k_rows, v_rows: BF16 [num_tokens][8][64] (16-byte aligned);
 * block_table_row: int32 device row of that sequence (4-byte aligned).
 * Bit-exact copy; tokens whose page id is outside [0, num_pages) are
 * skipped.  start + num_tokens must not exceed 16 * max_blocks_per_seq.
 */
int pa_fill_kv(const pa_shape* shape, const void* k_rows, const void* v_rows,
               int32_t num_tokens, int32_t start, const int32_t* block_table_row,
               void* k_pool, void* v_pool, void* stream);

/*
 * Workspace needed by pa_decode_attention for these arguments, in bytes
 * (0 when every sequence fits one split).  pages_per_split is 0 to let the
 * library plan (the plan then depends on the current device's compute-unit
 * count) or a fixed split size in pages, 1 .. min(max_blocks_per_seq, 256).
 * Returns PA_OK and stores the size in *bytes.
 */
int pa_decode_workspace_bytes(const pa_shape* shape, int32_t batch,
                              int32_t max_seq_len, int32_t pages_per_split,
                              size_t* bytes);

/*
 * Split size (pages per work-group) the library would use for these
 * arguments; with pages_per_split != 0 it is returned unchanged after
 * validation.  Stores it in *pages_out and the number of splits of the
 * longest sequence in *splits_out (either may be NULL).
 *
 * This plan sees only the batch size and max_seq_len, so it fits batches
 * whose lengths are near max_seq_len.  For a skewed batch it leaves a tail:
 * measured on MI355X, fused step, batch of 512 with lengths clipped
 * Zipf(1.1) in [1, 2048], BF16 pages, cold caches: this plan (one 128-page
 * split per sequence) 205-210 us; pa_decode_plan_lengths 201-208 us; the
 * work list (pa_append_decode_attention_worklist) 166-171 us; the balanced
 * launch (include/pa_decode_balanced.h, 8 heads per lane) 163-166 us.  With
 * lengths at hand, use one of the latter.  For batch 256 x 2048 all four
 * take 163-166 us.  For a batch of a few long sequences among many short
 * ones (512 lengths from Zipf(1.1) truncated to [1, 2048]) the work list
 * is the one that splits the long ones finely enough: 49-50 us, against 96-97 us
 * for pa_decode_plan_lengths and 66-100 us for the balanced launch.
 */
int pa_decode_plan(const pa_shape* shape, int32_t batch, int32_t max_seq_len,
                   int32_t pages_per_split, int32_t* pages_out,
                   int32_t* splits_out);

/*
 * Split size for a batch whose lengths the caller knows on the host (a
 * scheduler does): seq_lens_host is a HOST array of `batch` lengths.  The
 * library simulates how its work-groups would be spread over num_cus
 * compute units (0: the current device's count) for each candidate split
 * size (8 .. 256 pages) and returns the fastest by its cost model; pass the
 * result as pages_per_split.  Useful for skewed batches, where the
 * size-only plan is blind.  Reads nothing on the device; with num_cus > 0
 * it makes no HIP call at all.
 */
int pa_decode_plan_lengths(const pa_shape* shape, int32_t batch,
                           const int32_t* seq_lens_host, int32_t max_seq_len,
                           int32_t num_cus, int32_t* pages_out, int32_t* splits_out);

/*
 * Paged GQA decode attention for one layer.
 *   out[b][h][:] = sum_t w_t V_b[t][h/4][:],  w = softmax_t(scale * q[b][h] . K_b[t][h/4])
 * over tokens t in [0, seq_lens[b]); rows with seq_lens[b] == 0 are zero.
 * max_seq_len is a host-side upper bound of seq_lens (0 .. 16 *
 * max_blocks_per_seq); a sequence longer than it gets NaN outputs.
 * scale must be finite (1/8 for head_dim 64).  out_dtype is a pa_out_dtype.
 * Sequences longer than one split write FP32 partial results (running max,
 * sum, unnormalised output) to the workspace and a second kernel merges them
 * in split order; results are deterministic run to run and do not depend on
 * where pages sit in the pool.  `out` must not alias any input.  One
 * work-group runs per (sequence, split) of the plan, so batch x splits must
 * not exceed 2^31 - 1 (PA_ERR_VALUE otherwise); there is no other limit on
 * batch.
 */
int pa_decode_attention(const pa_shape* shape, int32_t batch,
                        const void* q, const void* k_pool, const void* v_pool,
                        const int32_t* block_tables, const int32_t* seq_lens,
                        int32_t max_seq_len, float scale,
                        void* out, int32_t out_dtype,
                        int32_t pages_per_split,
                        void* workspace, size_t workspace_bytes,
                        void* stream);

/*
 * Fused decode step: the effect of pa_append_kv followed by
 * pa_decode_attention with the same arguments, in one launch (plus the split
 * merge when the plan has several splits).  The work-group that owns each
 * sequence's last page writes the new K/V row (k_new[b], v_new[b]) into slot
 * (L-1)%16 of page block_tables[b][(L-1)/16] and takes that token's K/V from
 * registers.  Pools end bit-identical to the two-call sequence and outputs
 * are identical too.  Same layouts, alignment and error rules as the two
 * calls; k_new and v_new are required when batch > 0.  The append follows
 * pa_append_kv's rule for every sequence: the row is written whenever
 * 1 <= L <= 16 * max_blocks_per_seq and the target page id lies in
 * [0, num_pages), also when L exceeds max_seq_len (whose output row is NaN,
 * as in pa_decode_attention).
 */
int pa_append_decode_attention(const pa_shape* shape, int32_t batch,
                               const void* q, const void* k_new, const void* v_new,
                               void* k_pool, void* v_pool,
                               const int32_t* block_tables, const int32_t* seq_lens,
                               int32_t max_seq_len, float scale,
                               void* out, int32_t out_dtype,
                               int32_t pages_per_split,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

/*
 * Rotary position embedding of the new token (the step before the append in
 * the model: the new K is stored at its absolute RoPE position).  Rotate-half
 * pairing: dims i and i+32 rotate by the angle of position L-1 and frequency
 * i, out[i] = x[i] c - x[i+32] s, out[i+32] = x[i+32] c + x[i] s, each
 * product and sum rounded to FP32 on its own, the result rounded to BF16
 * (RNE).  The angles come as caller tables, so the frequency schedule is the
 * caller's choice.
 */
typedef struct pa_rope {
  const float* cos;    /* device, float32 [positions][head_dim/2], 4-byte aligned */
  const float* sin;    /* device, float32 [positions][head_dim/2]                 */
  int32_t positions;   /* rows of each table; must cover every position used       */
} pa_rope;

/*
 * Append with RoPE: for each b with L = seq_lens[b] >= 1, q_out[b] = RoPE(q[b])
 * and the page slot of token L-1 receives RoPE(k_new[b]) and v_new[b].  Idle
 * slots and out-of-range metadata write no pool bytes and copy q[b] to
 * q_out[b].  q, q_out: BF16 [batch][32][64], 16-byte aligned; the tables
 * must cover 16 * max_blocks_per_seq positions.
 */
int pa_append_kv_rope(const pa_shape* shape, int32_t batch,
                      const void* q, const void* k_new, const void* v_new,
                      const pa_rope* rope, void* q_out,
                      void* k_pool, void* v_pool,
                      const int32_t* block_tables, const int32_t* seq_lens,
                      void* stream);

/*
 * Fused decode step with RoPE: the effect of pa_append_kv_rope followed by
 * pa_decode_attention on its q_out, in one launch (plus the split merge).
 * Every work-group rotates its own query rows; the one holding the last
 * page rotates and writes the new key.  Outputs and pools are identical to
 * the two-call form.  The tables must cover max_seq_len positions.  A
 * sequence longer than max_seq_len (NaN output row) still has its rotated
 * row written, as pa_append_decode_attention does, when the tables hold
 * position L-1; pa_append_kv_rope refuses tables shorter than the block
 * table's capacity, so with such tables both forms write it.
 */
int pa_append_decode_attention_rope(const pa_shape* shape, int32_t batch,
                                    const void* q, const void* k_new, const void* v_new,
                                    const pa_rope* rope,
                                    void* k_pool, void* v_pool,
                                    const int32_t* block_tables, const int32_t* seq_lens,
                                    int32_t max_seq_len, float scale,
                                    void* out, int32_t out_dtype,
                                    int32_t pages_per_split,
                                    void* workspace, size_t workspace_bytes,
                                    void* stream);

/*
 * pa_decode_attention (k_new = v_new = NULL) or pa_append_decode_attention
 * (both non-NULL) plus timing hooks: event_before_main and event_after_main
 * (hipEvent_t handles created by the caller; either may be NULL) are
 * recorded on `stream` immediately before and after the main kernel is
 * enqueued, i.e. before the split merge kernel, so the pair times the main
 * kernel alone and an event after the call times the merge.  Same
 * arguments, checks and results otherwise.
 */
int pa_decode_attention_profiled(const pa_shape* shape, int32_t batch,
                                 const void* q, const void* k_new, const void* v_new,
                                 void* k_pool, void* v_pool,
                                 const int32_t* block_tables, const int32_t* seq_lens,
                                 int32_t max_seq_len, float scale,
                                 void* out, int32_t out_dtype,
                                 int32_t pages_per_split,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream, void* event_before_main,
                                 void* event_after_main);

/*
 * Work list for known sequence lengths (host copy): the (sequence, split)
 * work items of one decode launch, ordered by their page count, largest
 * first, so that long items start first and short ones fill in behind them
 * (the longest-processing-time-first rule).  Items without pages are left
 * out, except split 0 of a sequence without pages (its output row is still
 * written: zeros, or NaN for a length beyond max_seq_len).
 *   pages_per_split: the split size, or 0 to plan it from the lengths (the
 *     cost model of pa_decode_plan_lengths for page_format 0 (BF16 pages),
 *     of pa_decode_plan_lengths_q8 for 1 (INT8 pages), of
 *     pa_decode_plan_lengths_q4 for 2 (INT4 pages); other values are
 *     PA_ERR_VALUE);
 *   num_cus: compute units assumed by the planner (0 = current device);
 *   work: host int32 [2 * capacity]; item k is sequence work[2k], split
 *     work[2k+1]; *count receives the number of items (PA_ERR_VALUE when it
 *     exceeds capacity; batch * splits always suffices);
 *   pages_out, splits_out (may be NULL): the split size and the splits per
 *     sequence of the plan, to be passed with the list.
 * Host cost: planning the split size simulates one launch per candidate
 * size (8 .. 256 pages): on the host of an MI355X machine 50 us for 64
 * sequences of uniform lengths, 0.4 ms for 512 Zipf lengths (bench.py's
 * plan_host_us); building the list for a given size takes tens of
 * microseconds.  A serving loop, whose lengths grow by one token a
 * step, can plan the size once for a batch and pass it (pages_per_split)
 * on the steps that follow, replanning when the batch changes.
 */
int pa_decode_worklist(const pa_shape* shape, int32_t batch, const int32_t* seq_lens_host,
                       int32_t max_seq_len, int32_t pages_per_split, int32_t page_format,
                       int32_t num_cus, int32_t* work, int32_t capacity, int32_t* count,
                       int32_t* pages_out, int32_t* splits_out);

/*
 * Decode step launched from a work list (a copy of pa_decode_worklist's
 * output in device memory, 4-byte aligned; num_work items): one work-group
 * per item, in list order.  k_new and v_new are both given (the fused
 * append, as pa_append_decode_attention) or both NULL (decode only, as
 * pa_decode_attention).  pages_per_split must be the split size the list was
 * built for (0 is refused).  Results are bitwise those of the grid launch.
 * The list must hold every item of the plan exactly once; entries naming a
 * sequence outside [0, batch) or a split outside the plan are skipped.
 */
int pa_append_decode_attention_worklist(const pa_shape* shape, int32_t batch,
                                        const void* q, const void* k_new, const void* v_new,
                                        void* k_pool, void* v_pool,
                                        const int32_t* block_tables, const int32_t* seq_lens,
                                        int32_t max_seq_len, float scale,
                                        void* out, int32_t out_dtype, int32_t pages_per_split,
                                        const int32_t* work, int32_t num_work,
                                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Debug check of device-resident metadata: copies block_tables and
 * seq_lens to the host (synchronising `stream`) and checks that every
 * length lies in [0, max_seq_len], every used block-table entry lies in
 * [0, num_pages) and no page is used twice.  Returns PA_OK or
 * PA_ERR_METADATA and stores the first offending batch index in
 * *bad_index (or -1); bad_index may be NULL.
 */
int pa_validate_metadata(const pa_shape* shape, int32_t batch,
                         const int32_t* block_tables, const int32_t* seq_lens,
                         int32_t max_seq_len, void* stream, int64_t* bad_index);

/* Static, human-readable name of a pa_status value. */
const char* pa_status_string(int status);

/* ABI version of this header (bumped on incompatible changes). */
int pa_abi_version(void);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the fused
 * step of pa_append_decode_attention, same arguments minus the workspace,
 * same results bit for bit.  The split partials go to a scratch array that
 * the library holds in device memory for the life of the process (one per
 * GPU it runs on, PA_NOALLOC_SCRATCH_BYTES bytes); nothing is allocated by
 * the call.  A plan whose partials need more than that (batch x splits x
 * 32 heads x 66 floats, rounded up to 256 bytes, plus 2 floats per row:
 * pa_decode_workspace_bytes) returns PA_ERR_WORKSPACE before any launch.
 * The partials need no clearing: every row read is written first in the same
 * call.  Calls on one GPU share its scratch: calls that overlap in time on one
 * GPU (on different streams, or from several host threads) race and must be
 * serialised by the caller.  The first call on a device looks the scratch up
 * (hipGetSymbolAddress); a failure there returns PA_ERR_DEVICE.
 */
#define PA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int pa_append_decode_attention_noalloc(const pa_shape* shape, int32_t batch,
                                       const void* q, const void* k_new, const void* v_new,
                                       void* k_pool, void* v_pool,
                                       const int32_t* block_tables, const int32_t* seq_lens,
                                       int32_t max_seq_len, float scale,
                                       void* out, int32_t out_dtype,
                                       int32_t pages_per_split, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PA_DECODE_H */
