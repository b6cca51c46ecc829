// Host side of the INT8 and INT4 K/V page entry points (C ABI in
// include/pa_decode_q8.h and include/pa_decode_q4.h): argument checks, the
// quantised append and fill kernels, and launches of the decode kernel.
#include <hip/hip_runtime.h>

#include <cmath>

#include "pa_decode.h"
#include "pa_decode_q4.h"
#include "pa_decode_q8.h"
#include "pa_host.h"
#include "pa_decode_kernel.h"

#define PA_API extern "C" __attribute__((visibility("default")))

namespace pa {

// Quantised one-token append (FMT: INT8 or INT4 codes): one wavefront per
// sequence; lane = 4 * row + c
// with row = 2 * head + (0: K, 1: V) and c the lane's dims {8c..} and
// {32+8c..} of that row.  With ROPE (256 threads) the new query is rotated
// into q_out by all four wavefronts as in append_rope_kernel, and the new key
// is rotated before it is quantised.  Idle slots and out-of-range metadata
// write no pool bytes (q_out still gets q, rotated or copied).
template <int FMT, bool ROPE>
__global__ __launch_bounds__(ROPE ? 256 : 64) void append_quant_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, const float* __restrict__ rope_cos,
    const float* __restrict__ rope_sin, uint16_t* __restrict__ q_out,
    uint8_t* __restrict__ k_codes, uint8_t* __restrict__ v_codes, float* __restrict__ kv_scales,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ seq_lens,
    int32_t max_blocks, int32_t num_pages) {
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int L = seq_lens[b];
  const bool live = L >= 1 && L <= max_blocks * kPage;
  const int pos = live ? L - 1 : 0;
  if (ROPE) {
    const int64_t cs_row = (int64_t)pos * (kD / 2);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int j = t + 256 * r;
      const int64_t base = ((int64_t)b * kHq + (j >> 5)) * kD + (j & 31);
      const uint16_t x1b = q[base], x2b = q[base + 32];
      uint16_t y1b = x1b, y2b = x2b;
      if (live) {
        const float x1 = __uint_as_float((uint32_t)x1b << 16);
        const float x2 = __uint_as_float((uint32_t)x2b << 16);
        const float c = rope_cos[cs_row + (j & 31)], sn = rope_sin[cs_row + (j & 31)];
        y1b = (uint16_t)f32_to_bf16_rne(rope_first(x1, x2, c, sn));
        y2b = (uint16_t)f32_to_bf16_rne(rope_second(x1, x2, c, sn));
      }
      q_out[base] = y1b;
      q_out[base + 32] = y2b;
    }
  }
  if (!live || t >= 64) return;
  const int id = block_tables[(int64_t)b * max_blocks + pos / kPage];
  if ((unsigned)id >= (unsigned)num_pages) return;
  const int row = t >> 2, c = t & 3;
  const int g = row >> 1;
  const bool is_k = (row & 1) == 0;
  const uint16_t* src = (is_k ? k_new : v_new) + ((int64_t)b * kHkv + g) * kD + 8 * c;
  uint4 lo = *reinterpret_cast<const uint4*>(src);
  uint4 hi = *reinterpret_cast<const uint4*>(src + 32);
  if (ROPE && is_k) {
    const int64_t cs = (int64_t)pos * (kD / 2) + 8 * c;
    rope_pairs8(lo, hi, rope_cos + cs, rope_sin + cs);
  }
  using QL = QuantLayout<FMT>;
  u32x2 clo, chi;
  const float sc = quantize_quad_row<FMT>(lo, hi, clo, chi);
  const int slot = pos % kPage;
  store_quad_codes<FMT>((is_k ? k_codes : v_codes) + (int64_t)id * QL::kPageBytes + g * QL::kHead +
                            slot * QL::kRow,
                        c, clo, chi);
  if (c == 0) kv_scales[(int64_t)id * kScalePageFloats + (g * 2 + (is_k ? 0 : 1)) * kPage + slot] = sc;
}

// Quantised prefill fill: tokens start .. start+T-1 of one sequence, one
// wavefront per token (lane mapping of append_quant_kernel), 4 per work-group.
template <int FMT>
__global__ __launch_bounds__(256) void fill_quant_kernel(const uint16_t* __restrict__ k_rows,
                                                         const uint16_t* __restrict__ v_rows,
                                                         int32_t num_tokens, int32_t start,
                                                         const int32_t* __restrict__ bt_row,
                                                         uint8_t* __restrict__ k_codes,
                                                         uint8_t* __restrict__ v_codes,
                                                         float* __restrict__ kv_scales,
                                                         int32_t num_pages) {
  const int tok = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (tok >= num_tokens) return;                    // whole wavefront: quads stay complete
  const int t = start + tok;
  const int id = bt_row[t / kPage];
  if ((unsigned)id >= (unsigned)num_pages) return;
  const int row = lane >> 2, c = lane & 3;
  const int g = row >> 1;
  const bool is_k = (row & 1) == 0;
  const uint16_t* src = (is_k ? k_rows : v_rows) + ((int64_t)tok * kHkv + g) * kD + 8 * c;
  const uint4 lo = *reinterpret_cast<const uint4*>(src);
  const uint4 hi = *reinterpret_cast<const uint4*>(src + 32);
  using QL = QuantLayout<FMT>;
  u32x2 clo, chi;
  const float sc = quantize_quad_row<FMT>(lo, hi, clo, chi);
  const int slot = t % kPage;
  store_quad_codes<FMT>((is_k ? k_codes : v_codes) + (int64_t)id * QL::kPageBytes + g * QL::kHead +
                            slot * QL::kRow,
                        c, clo, chi);
  if (c == 0) kv_scales[(int64_t)id * kScalePageFloats + (g * 2 + (is_k ? 0 : 1)) * kPage + slot] = sc;
}

}  // namespace pa

using namespace pa_host;

namespace pa_host {

// Planner cost model for INT8 pages: 17 KiB per page (8 KiB of K codes,
// 8 KiB of V codes, 1 KiB of scales).  The per-page time of one CU alone, the
// fixed cost per work-group and per empty grid slot were fitted to this
// kernel's measured times on MI355X over batches of 8 to 512 sequences
// (uniform and Zipf lengths) and split sizes 8 .. 128 pages.
PlanModel plan_model_q8() {
  PlanModel m;
  m.page_bytes = 2.0 * pa::kPageCodes + pa::kScalePageFloats * 4.0;
  m.page_us = 0.5;
  m.group_us = 3.0;
  m.empty_us = 0.5;
  return m;
}

// Planner cost model for INT4 pages: 9 KiB per page (4 KiB of K codes, 4 KiB
// of V codes, 1 KiB of scales).  The per-page time of one CU alone and the
// fixed costs were fitted to this kernel's measured times on MI355X over
// batches of 8 to 512 sequences (uniform and Zipf lengths) and split sizes
// 8 .. 128 pages; at this page size the per-page arithmetic, not HBM, sets
// the rate.  Two work-groups fit on a CU (92 VGPRs, 30 KiB of LDS each), and
// two sharing a CU stream 1.3x the pages of one alone: at 256 sequences of
// 2,048 tokens, 64-page splits (two per CU) measured 69.2 us against 74.8 us
// for one 128-page split per CU.
PlanModel plan_model_q4() {
  PlanModel m;
  m.page_bytes = 2.0 * pa::kPageCodes4 + pa::kScalePageFloats * 4.0;
  m.page_us = 0.5;
  m.group_us = 2.0;
  m.empty_us = 0.5;
  m.resident = 2;
  m.shared_gain = 1.3;
  m.two_wave_gain = 1.3;
  return m;
}

}  // namespace pa_host

namespace {

int check_pools_q8(const void* k_codes, const void* v_codes, const void* kv_scales) {
  if (!k_codes || !v_codes || !kv_scales) return PA_ERR_NULL;
  if (!aligned(k_codes, 16) || !aligned(v_codes, 16) || !aligned(kv_scales, 16)) return PA_ERR_ALIGN;
  return PA_OK;
}

template <int FMT>
int append_quant_impl(const pa_shape* shape, int32_t batch, const void* q, const void* k_new,
                   const void* v_new, const pa_rope* rope, void* q_out, void* k_codes,
                   void* v_codes, void* kv_scales, const int32_t* block_tables,
                   const int32_t* seq_lens, void* stream) {
  int rc = check_shape(shape);
  if (rc != PA_OK) return rc;
  if (batch < 0) return PA_ERR_VALUE;
  if (batch == 0) return PA_OK;
  if (!k_new || !v_new || !block_tables || !seq_lens) return PA_ERR_NULL;
  rc = check_pools_q8(k_codes, v_codes, kv_scales);
  if (rc != PA_OK) return rc;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(block_tables, 4) ||
      !aligned(seq_lens, 4))
    return PA_ERR_ALIGN;
  if (rope) {
    if (!q || !q_out) return PA_ERR_NULL;
    if (!aligned(q, 16) || !aligned(q_out, 16)) return PA_ERR_ALIGN;
    rc = check_rope(rope, (int64_t)shape->max_blocks_per_seq * pa::kPage);
    if (rc != PA_OK) return rc;
  }
  if (shape->num_pages < 1) return PA_ERR_VALUE;
  hipStream_t st = (hipStream_t)stream;
  if (rope)
    hipLaunchKernelGGL((pa::append_quant_kernel<FMT, true>), dim3(batch), dim3(256), 0, st,
                       (const uint16_t*)q, (const uint16_t*)k_new, (const uint16_t*)v_new,
                       rope->cos, rope->sin, (uint16_t*)q_out, (uint8_t*)k_codes,
                       (uint8_t*)v_codes, (float*)kv_scales, block_tables, seq_lens,
                       shape->max_blocks_per_seq, shape->num_pages);
  else
    hipLaunchKernelGGL((pa::append_quant_kernel<FMT, false>), dim3(batch), dim3(64), 0, st,
                       nullptr, (const uint16_t*)k_new, (const uint16_t*)v_new, nullptr, nullptr,
                       nullptr, (uint8_t*)k_codes, (uint8_t*)v_codes, (float*)kv_scales,
                       block_tables, seq_lens, shape->max_blocks_per_seq, shape->num_pages);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

// k_new/v_new non-NULL: the quantised append is fused into the main kernel
template <int FMT>
int decode_quant_impl(const pa_shape* shape, int32_t batch, const void* q, const void* k_new,
                   const void* v_new, const pa_rope* rope, const void* k_codes,
                   const void* v_codes, const void* kv_scales, const int32_t* block_tables,
                   const int32_t* seq_lens, int32_t max_seq_len, float scale, void* out,
                   int32_t out_dtype, int32_t pages_per_split, void* workspace,
                   size_t workspace_bytes, void* stream, const int32_t* work = nullptr,
                   int32_t num_work = 0) {
  int rc = check_decode_sizes(shape, batch, max_seq_len);
  if (rc != PA_OK) return rc;
  if (out_dtype != PA_OUT_F32 && out_dtype != PA_OUT_BF16) return PA_ERR_VALUE;
  if (!std::isfinite(scale)) return PA_ERR_VALUE;
  if (batch == 0) return PA_OK;
  if (!q || !block_tables || !seq_lens || !out) return PA_ERR_NULL;
  rc = check_pools_q8(k_codes, v_codes, kv_scales);
  if (rc != PA_OK) return rc;
  const bool fused = k_new != nullptr || v_new != nullptr;
  if (fused && (!k_new || !v_new)) return PA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(out, 16) || !aligned(block_tables, 4) || !aligned(seq_lens, 4) ||
      (fused && (!aligned(k_new, 16) || !aligned(v_new, 16))))
    return PA_ERR_ALIGN;
  if (rope) {
    if (!fused) return PA_ERR_VALUE;
    rc = check_rope(rope, max_seq_len);
    if (rc != PA_OK) return rc;
  }
  if (shape->num_pages < 1 && max_seq_len > 0) return PA_ERR_VALUE;
  if (work) {
    // the list was built for one split size: it must be given, not planned
    if (pages_per_split == 0 || num_work < 1) return PA_ERR_VALUE;
    if (!aligned(work, 4)) return PA_ERR_ALIGN;
  }
  int ps = 0, ns = 0;
  rc = plan_split(shape, batch, max_seq_len, pages_per_split, &ps, &ns);
  if (rc != PA_OK) return rc;
  const size_t need = workspace_for(batch, ns);
  if (need > 0) {
    if (!workspace || workspace_bytes < need) return PA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return PA_ERR_ALIGN;
  }
  if ((int64_t)batch * ns > INT32_MAX) return PA_ERR_VALUE;        // one block per (sequence, split)

  pa::DecodeArgs a = {};
  a.q = (const uint16_t*)q;
  a.k_pool = k_codes;
  a.v_pool = v_codes;
  a.kv_scales = (const float*)kv_scales;
  a.k_new = (const uint16_t*)k_new;
  a.v_new = (const uint16_t*)v_new;
  a.k_pool_w = const_cast<void*>(k_codes);
  a.v_pool_w = const_cast<void*>(v_codes);
  a.kv_scales_w = (float*)const_cast<void*>(kv_scales);
  a.rope_cos = rope ? rope->cos : nullptr;
  a.rope_sin = rope ? rope->sin : nullptr;
  a.rope_positions = rope ? rope->positions : 0;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.out = out;
  a.part_acc = (float*)workspace;
  const size_t rows = (size_t)batch * ns * pa::kHq;
  const size_t acc_bytes = (rows * pa::kD * sizeof(float) + 255) & ~(size_t)255;
  a.part_ml = need ? (float*)((char*)workspace + acc_bytes) : nullptr;
  a.xscale = scale * pa::kLog2e;
  a.num_pages = shape->num_pages;
  a.max_blocks = shape->max_blocks_per_seq;
  a.max_seq_len = max_seq_len;
  a.pages_per_split = ps;
  a.num_splits = ns;
  a.work = work;
  a.num_work = num_work;
  a.batch = batch;
  int cu = 0;
  const bool have_cu = pa_host::current_cu_count(&cu) == PA_OK;
  const bool merge_preload = have_cu && batch <= cu;
  // INT4 pages are bound by their arithmetic: when every work-group of the
  // plan fits the CUs at once and its splits are long, two wavefronts per KV
  // head give each CU the waves of two work-groups without split partials.
  // The choice depends on the plan (batch x splits, split size) alone, so a
  // work-list launch of the same plan sums in the same order as the grid
  // launch and matches it bit for bit.
  const bool two_waves = FMT == pa::kFmtINT4 && have_cu && (int64_t)batch * ns <= cu &&
                         ps >= pa_host::kTwoWaveMinPages;
  const hipError_t e = pa::launch_decode<FMT>(a, batch, out_dtype == PA_OUT_BF16, fused,
                                               rope != nullptr, merge_preload, two_waves, false,
                                               (hipStream_t)stream, nullptr, nullptr);
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

}  // namespace

PA_API int pa_append_kv_q8(const pa_shape* shape, int32_t batch, const void* k_new,
                           const void* v_new, void* k_codes, void* v_codes, void* kv_scales,
                           const int32_t* block_tables, const int32_t* seq_lens, void* stream) {
  return append_quant_impl<pa::kFmtINT8>(shape, batch, nullptr, k_new, v_new, nullptr, nullptr, k_codes,
                                                v_codes, kv_scales, block_tables, seq_lens, stream);
}

PA_API int pa_append_kv_rope_q8(const pa_shape* shape, int32_t batch, const void* q,
                                const void* k_new, const void* v_new, const pa_rope* rope,
                                void* q_out, void* k_codes, void* v_codes, void* kv_scales,
                                const int32_t* block_tables, const int32_t* seq_lens,
                                void* stream) {
  if (batch > 0 && !rope) return PA_ERR_NULL;
  return append_quant_impl<pa::kFmtINT8>(shape, batch, q, k_new, v_new, rope, q_out, k_codes, v_codes, kv_scales,
                        block_tables, seq_lens, stream);
}

namespace {

template <int FMT>
int fill_quant_impl(const pa_shape* shape, const void* k_rows, const void* v_rows,
                    int32_t num_tokens, int32_t start, const int32_t* block_table_row,
                    void* k_codes, void* v_codes, void* kv_scales, void* stream) {
  int rc = check_shape(shape);
  if (rc != PA_OK) return rc;
  if (num_tokens < 0 || start < 0 ||
      (int64_t)start + num_tokens > (int64_t)shape->max_blocks_per_seq * pa::kPage)
    return PA_ERR_VALUE;
  if (num_tokens == 0) return PA_OK;
  if (!k_rows || !v_rows || !block_table_row) return PA_ERR_NULL;
  rc = check_pools_q8(k_codes, v_codes, kv_scales);
  if (rc != PA_OK) return rc;
  if (!aligned(k_rows, 16) || !aligned(v_rows, 16) || !aligned(block_table_row, 4))
    return PA_ERR_ALIGN;
  if (shape->num_pages < 1) return PA_ERR_VALUE;
  hipLaunchKernelGGL(pa::fill_quant_kernel<FMT>, dim3(ceil_div(num_tokens, 4)), dim3(256), 0,
                     (hipStream_t)stream, (const uint16_t*)k_rows, (const uint16_t*)v_rows,
                     num_tokens, start, block_table_row, (uint8_t*)k_codes, (uint8_t*)v_codes,
                     (float*)kv_scales, shape->num_pages);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

template <int FMT>
int plan_lengths_quant(const pa_shape* shape, int32_t batch, const int32_t* seq_lens_host,
                       int32_t max_seq_len, int32_t num_cus, int32_t* pages_out,
                       int32_t* splits_out) {
  int rc = check_decode_sizes(shape, batch, max_seq_len);
  if (rc != PA_OK) return rc;
  if (batch > 0 && !seq_lens_host) return PA_ERR_NULL;
  if (num_cus < 0) return PA_ERR_VALUE;
  int ps = 1, ns = 1;
  if (batch > 0) {
    rc = plan_split_lengths(shape, batch, seq_lens_host, max_seq_len, num_cus,
                            FMT == pa::kFmtINT8 ? plan_model_q8() : plan_model_q4(), &ps, &ns);
    if (rc != PA_OK) return rc;
  }
  if (pages_out) *pages_out = ps;
  if (splits_out) *splits_out = ns;
  return PA_OK;
}

}  // namespace

// INT8 pages (include/pa_decode_q8.h)

PA_API int pa_fill_kv_q8(const pa_shape* shape, const void* k_rows, const void* v_rows,
                         int32_t num_tokens, int32_t start, const int32_t* block_table_row,
                         void* k_codes, void* v_codes, void* kv_scales, void* stream) {
  return fill_quant_impl<pa::kFmtINT8>(shape, k_rows, v_rows, num_tokens, start, block_table_row,
                                       k_codes, v_codes, kv_scales, stream);
}

PA_API int pa_decode_attention_q8(const pa_shape* shape, int32_t batch, const void* q,
                                  const void* k_codes, const void* v_codes,
                                  const void* kv_scales, const int32_t* block_tables,
                                  const int32_t* seq_lens, int32_t max_seq_len, float scale,
                                  void* out, int32_t out_dtype, int32_t pages_per_split,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  return decode_quant_impl<pa::kFmtINT8>(shape, batch, q, nullptr, nullptr, nullptr, k_codes, v_codes, kv_scales,
                        block_tables, seq_lens, max_seq_len, scale, out, out_dtype,
                        pages_per_split, workspace, workspace_bytes, stream);
}

PA_API int pa_append_decode_attention_q8(const pa_shape* shape, int32_t batch, const void* q,
                                         const void* k_new, const void* v_new, void* k_codes,
                                         void* v_codes, void* kv_scales,
                                         const int32_t* block_tables, const int32_t* seq_lens,
                                         int32_t max_seq_len, float scale, void* out,
                                         int32_t out_dtype, int32_t pages_per_split,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  if (batch > 0 && (!k_new || !v_new)) return PA_ERR_NULL;
  return decode_quant_impl<pa::kFmtINT8>(shape, batch, q, k_new, v_new, nullptr, k_codes, v_codes, kv_scales,
                        block_tables, seq_lens, max_seq_len, scale, out, out_dtype,
                        pages_per_split, workspace, workspace_bytes, stream);
}

PA_API int pa_append_decode_attention_rope_q8(const pa_shape* shape, int32_t batch, const void* q,
                                              const void* k_new, const void* v_new,
                                              const pa_rope* rope, void* k_codes, void* v_codes,
                                              void* kv_scales, const int32_t* block_tables,
                                              const int32_t* seq_lens, int32_t max_seq_len,
                                              float scale, void* out, int32_t out_dtype,
                                              int32_t pages_per_split, void* workspace,
                                              size_t workspace_bytes, void* stream) {
  if (batch > 0 && (!k_new || !v_new || !rope)) return PA_ERR_NULL;
  return decode_quant_impl<pa::kFmtINT8>(shape, batch, q, k_new, v_new, rope, k_codes, v_codes, kv_scales,
                        block_tables, seq_lens, max_seq_len, scale, out, out_dtype,
                        pages_per_split, workspace, workspace_bytes, stream);
}

PA_API int pa_append_decode_attention_worklist_q8(
    const pa_shape* shape, int32_t batch, const void* q, const void* k_new, const void* v_new,
    void* k_codes, void* v_codes, void* kv_scales, const int32_t* block_tables,
    const int32_t* seq_lens, int32_t max_seq_len, float scale, void* out, int32_t out_dtype,
    int32_t pages_per_split, const int32_t* work, int32_t num_work, void* workspace,
    size_t workspace_bytes, void* stream) {
  if (batch > 0 && !work) return PA_ERR_NULL;
  return decode_quant_impl<pa::kFmtINT8>(shape, batch, q, k_new, v_new, nullptr, k_codes, v_codes, kv_scales,
                        block_tables, seq_lens, max_seq_len, scale, out, out_dtype,
                        pages_per_split, workspace, workspace_bytes, stream, work, num_work);
}

PA_API int pa_decode_plan_lengths_q8(const pa_shape* shape, int32_t batch,
                                     const int32_t* seq_lens_host, int32_t max_seq_len,
                                     int32_t num_cus, int32_t* pages_out, int32_t* splits_out) {
  return plan_lengths_quant<pa::kFmtINT8>(shape, batch, seq_lens_host, max_seq_len, num_cus,
                                          pages_out, splits_out);
}

// INT4 pages (include/pa_decode_q4.h)

PA_API int pa_append_kv_q4(const pa_shape* shape, int32_t batch, const void* k_new,
                           const void* v_new, void* k_codes, void* v_codes, void* kv_scales,
                           const int32_t* block_tables, const int32_t* seq_lens, void* stream) {
  return append_quant_impl<pa::kFmtINT4>(shape, batch, nullptr, k_new, v_new, nullptr, nullptr, k_codes,
                                                v_codes, kv_scales, block_tables, seq_lens, stream);
}

PA_API int pa_append_kv_rope_q4(const pa_shape* shape, int32_t batch, const void* q,
                                const void* k_new, const void* v_new, const pa_rope* rope,
                                void* q_out, void* k_codes, void* v_codes, void* kv_scales,
                                const int32_t* block_tables, const int32_t* seq_lens,
                                void* stream) {
  if (batch > 0 && !rope) return PA_ERR_NULL;
  return append_quant_impl<pa::kFmtINT4>(shape, batch, q, k_new, v_new, rope, q_out, k_codes, v_codes, kv_scales,
                        block_tables, seq_lens, stream);
}

PA_API int pa_fill_kv_q4(const pa_shape* shape, const void* k_rows, const void* v_rows,
                         int32_t num_tokens, int32_t start, const int32_t* block_table_row,
                         void* k_codes, void* v_codes, void* kv_scales, void* stream) {
  return fill_quant_impl<pa::kFmtINT4>(shape, k_rows, v_rows, num_tokens, start, block_table_row,
                                       k_codes, v_codes, kv_scales, stream);
}

PA_API int pa_decode_attention_q4(const pa_shape* shape, int32_t batch, const void* q,
                                  const void* k_codes, const void* v_codes,
                                  const void* kv_scales, const int32_t* block_tables,
                                  const int32_t* seq_lens, int32_t max_seq_len, float scale,
                                  void* out, int32_t out_dtype, int32_t pages_per_split,
                                  void* workspace, size_t workspace_bytes, void* stream) {
  return decode_quant_impl<pa::kFmtINT4>(shape, batch, q, nullptr, nullptr, nullptr, k_codes, v_codes, kv_scales,
                        block_tables, seq_lens, max_seq_len, scale, out, out_dtype,
                        pages_per_split, workspace, workspace_bytes, stream);
}

PA_API int pa_append_decode_attention_q4(const pa_shape* shape, int32_t batch, const void* q,
                                         const void* k_new, const void* v_new, void* k_codes,
                                         void* v_codes, void* kv_scales,
                                         const int32_t* block_tables, const int32_t* seq_lens,
                                         int32_t max_seq_len, float scale, void* out,
                                         int32_t out_dtype, int32_t pages_per_split,
                                         void* workspace, size_t workspace_bytes, void* stream) {
  if (batch > 0 && (!k_new || !v_new)) return PA_ERR_NULL;
  return decode_quant_impl<pa::kFmtINT4>(shape, batch, q, k_new, v_new, nullptr, k_codes, v_codes, kv_scales,
                        block_tables, seq_lens, max_seq_len, scale, out, out_dtype,
                        pages_per_split, workspace, workspace_bytes, stream);
}

PA_API int pa_append_decode_attention_rope_q4(const pa_shape* shape, int32_t batch, const void* q,
                                              const void* k_new, const void* v_new,
                                              const pa_rope* rope, void* k_codes, void* v_codes,
                                              void* kv_scales, const int32_t* block_tables,
                                              const int32_t* seq_lens, int32_t max_seq_len,
                                              float scale, void* out, int32_t out_dtype,
                                              int32_t pages_per_split, void* workspace,
                                              size_t workspace_bytes, void* stream) {
  if (batch > 0 && (!k_new || !v_new || !rope)) return PA_ERR_NULL;
  return decode_quant_impl<pa::kFmtINT4>(shape, batch, q, k_new, v_new, rope, k_codes, v_codes, kv_scales,
                        block_tables, seq_lens, max_seq_len, scale, out, out_dtype,
                        pages_per_split, workspace, workspace_bytes, stream);
}

PA_API int pa_append_decode_attention_worklist_q4(
    const pa_shape* shape, int32_t batch, const void* q, const void* k_new, const void* v_new,
    void* k_codes, void* v_codes, void* kv_scales, const int32_t* block_tables,
    const int32_t* seq_lens, int32_t max_seq_len, float scale, void* out, int32_t out_dtype,
    int32_t pages_per_split, const int32_t* work, int32_t num_work, void* workspace,
    size_t workspace_bytes, void* stream) {
  if (batch > 0 && !work) return PA_ERR_NULL;
  return decode_quant_impl<pa::kFmtINT4>(shape, batch, q, k_new, v_new, nullptr, k_codes, v_codes, kv_scales,
                        block_tables, seq_lens, max_seq_len, scale, out, out_dtype,
                        pages_per_split, workspace, workspace_bytes, stream, work, num_work);
}

PA_API int pa_decode_plan_lengths_q4(const pa_shape* shape, int32_t batch,
                                     const int32_t* seq_lens_host, int32_t max_seq_len,
                                     int32_t num_cus, int32_t* pages_out, int32_t* splits_out) {
  return plan_lengths_quant<pa::kFmtINT4>(shape, batch, seq_lens_host, max_seq_len, num_cus,
                                          pages_out, splits_out);
}
