// Host side of the paged GQA decode library: argument checks, split planning
// and kernel launches behind the C ABI declared in include/pa_decode.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <queue>
#include <utility>
#include <vector>

#include "pa_decode.h"
#include "pa_host.h"
#include "pa_decode_kernel.h"

#define PA_API extern "C" __attribute__((visibility("default")))

// Kernels launched only from this file (the shared decode and merge kernel
// templates are in pa_kernels.h).
namespace pa {

// One-token append: one wavefront per sequence, each lane copies 16 bytes of
// the 1 KiB K row and 16 bytes of the V row.
__global__ __launch_bounds__(64) void append_kernel(const uint4* __restrict__ k_new,
                                                    const uint4* __restrict__ v_new,
                                                    uint4* __restrict__ k_pool,
                                                    uint4* __restrict__ v_pool,
                                                    const int32_t* __restrict__ block_tables,
                                                    const int32_t* __restrict__ seq_lens,
                                                    int32_t max_blocks, int32_t num_pages) {
  const int b = blockIdx.x;
  const int lane = threadIdx.x;
  const int L = seq_lens[b];
  if (L <= 0 || L > max_blocks * kPage) return;
  const int pos = L - 1;
  const int id = block_tables[(int64_t)b * max_blocks + pos / kPage];
  if ((unsigned)id >= (unsigned)num_pages) return;
  const int64_t row = (int64_t)id * kPage + (pos % kPage);   // 1 KiB rows = 64 x uint4
  k_pool[row * 64 + lane] = k_new[(int64_t)b * 64 + lane];
  v_pool[row * 64 + lane] = v_new[(int64_t)b * 64 + lane];
}

// Prefill page fill: tokens start .. start+T-1 of one sequence (K and V
// rows of 1 KiB each) into their page slots; 4 tokens per work-group, one
// wavefront per token, 16 bytes per lane.  Tokens whose page id is out of
// range are skipped.
__global__ __launch_bounds__(256) void fill_kernel(const uint4* __restrict__ k_rows,
                                                   const uint4* __restrict__ v_rows,
                                                   int32_t num_tokens, int32_t start,
                                                   const int32_t* __restrict__ bt_row,
                                                   uint4* __restrict__ k_pool,
                                                   uint4* __restrict__ v_pool,
                                                   int32_t num_pages) {
  const int tok = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (tok >= num_tokens) return;
  const int t = start + tok;
  const int id = bt_row[t / kPage];
  if ((unsigned)id >= (unsigned)num_pages) return;
  const int64_t row = (int64_t)id * kPage + (t % kPage);
  k_pool[row * 64 + lane] = k_rows[(int64_t)tok * 64 + lane];
  v_pool[row * 64 + lane] = v_rows[(int64_t)tok * 64 + lane];
}

// One-token append with RoPE: one work-group of 256 threads per sequence
// rotates the new query (32 heads x 32 pairs, into q_out) and key (8 x 32
// pairs) at position L-1 and writes the rotated key and the value into the
// page slot.  Idle slots and out-of-range metadata write no pool bytes; their
// q_out row is a copy of q.
__global__ __launch_bounds__(256) void append_rope_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k_new,
    const uint16_t* __restrict__ v_new, const float* __restrict__ rope_cos,
    const float* __restrict__ rope_sin, uint16_t* __restrict__ q_out,
    uint16_t* __restrict__ k_pool, uint16_t* __restrict__ v_pool,
    const int32_t* __restrict__ block_tables, const int32_t* __restrict__ seq_lens,
    int32_t max_blocks, int32_t num_pages) {
  const int b = blockIdx.x;
  const int t = threadIdx.x;
  const int L = seq_lens[b];
  const bool live = L >= 1 && L <= max_blocks * kPage;
  const int pos = live ? L - 1 : 0;
  const int64_t cs_row = (int64_t)pos * (kD / 2);
  // query: thread t rotates pairs j = t, t+256, t+512, t+768 (head j/32, dim j%32)
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
  if (!live) return;
  const int id = block_tables[(int64_t)b * max_blocks + pos / kPage];
  if ((unsigned)id >= (unsigned)num_pages) return;
  const int64_t row = ((int64_t)id * kPage + (pos % kPage)) * kRowElems;   // token row
  {  // key: thread t rotates pair (head t/32, dim t%32)
    const int64_t src = (int64_t)b * kRowElems + (t >> 5) * kD + (t & 31);
    const float x1 = __uint_as_float((uint32_t)k_new[src] << 16);
    const float x2 = __uint_as_float((uint32_t)k_new[src + 32] << 16);
    const float c = rope_cos[cs_row + (t & 31)], sn = rope_sin[cs_row + (t & 31)];
    const int64_t dst = row + (t >> 5) * kD + (t & 31);
    k_pool[dst] = (uint16_t)f32_to_bf16_rne(rope_first(x1, x2, c, sn));
    k_pool[dst + 32] = (uint16_t)f32_to_bf16_rne(rope_second(x1, x2, c, sn));
  }
  if (t < 64)  // value: 64 x 16 bytes
    reinterpret_cast<uint4*>(v_pool + row)[t] =
        reinterpret_cast<const uint4*>(v_new + (int64_t)b * kRowElems)[t];
}

}  // namespace pa

namespace pa_host {

constexpr int kMaxDevices = 64;
int g_cu_count[kMaxDevices];
std::once_flag g_cu_once[kMaxDevices];

// Compute units of the current device, queried once per device.
int current_cu_count(int* cu) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return PA_ERR_DEVICE;
  std::call_once(g_cu_once[dev], [dev] {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
    g_cu_count[dev] = n;
  });
  if (g_cu_count[dev] <= 0) return PA_ERR_DEVICE;
  *cu = g_cu_count[dev];
  return PA_OK;
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_shape(const pa_shape* s) {
  if (!s) return PA_ERR_NULL;
  if (s->num_q_heads != pa::kHq || s->num_kv_heads != pa::kHkv || s->head_dim != pa::kD ||
      s->page_size != pa::kPage)
    return PA_ERR_SHAPE;
  if (s->num_pages < 0 || s->max_blocks_per_seq < 1) return PA_ERR_VALUE;
  // page offsets are formed in 64-bit; the block table row stride in 32-bit
  if ((int64_t)s->max_blocks_per_seq * pa::kPage > INT32_MAX) return PA_ERR_VALUE;
  return PA_OK;
}

int ceil_div(int a, int b) { return (a + b - 1) / b; }

// Split size in pages.  With `fixed` != 0 that size is used as given.
// Otherwise: at least one work-group per compute unit (sequences x splits >=
// CUs; a work-group holds a whole CU's worth of waves and LDS ring), but
// never splits shorter than 8 pages (128 tokens), so the partial results stay
// a small fraction of the bytes.
int plan_split(const pa_shape* s, int batch, int max_seq_len, int fixed, int* pages, int* splits) {
  const int max_pages = ceil_div(max_seq_len, pa::kPage);
  int ps;
  if (fixed != 0) {
    if (fixed < 1 || fixed > s->max_blocks_per_seq || fixed > pa::kMaxSplitPages)
      return PA_ERR_VALUE;
    ps = fixed;
  } else {
    if (max_pages <= 8 || batch <= 0) {
      ps = max_pages > 0 ? max_pages : 1;
    } else {
      int cu = 0;
      const int rc = current_cu_count(&cu);
      if (rc != PA_OK) return rc;
      const int want = ceil_div(cu, batch);                   // splits per sequence wanted
      const int cap = ceil_div(max_pages, 8);                 // >= 8 pages per split
      const int ns = want < 1 ? 1 : (want > cap ? cap : want);
      ps = ceil_div(max_pages, ns);
    }
    if (ps > pa::kMaxSplitPages) ps = pa::kMaxSplitPages;
  }
  *pages = ps;
  *splits = max_pages > 0 ? ceil_div(max_pages, ps) : 1;
  return PA_OK;
}

// Split size for known sequence lengths (host copy).  For each candidate
// size the host simulates one launch: work-groups are dealt round-robin to
// the XCDs (work-group i to XCD i mod 8) and each XCD starts its next one
// when one of its CUs frees up (one resident work-group per CU); a
// work-group spends group_us on fixed costs, then streams its pages, all
// streaming work-groups sharing the HBM bandwidth equally but none faster
// than one CU alone (page_us per page); empty grid slots cost empty_us; a
// multi-split plan adds the merge (merge_us plus its partial traffic).  The
// constants were fitted to measurements of this kernel on MI355X over batch
// 8 .. 512 and split sizes 8 .. 128.  The largest size predicted within 3%
// of the fastest is returned (the model's error is about that size).
double simulate_plan(const int32_t* lens, int batch, int max_seq_len, int ps, int cu, int xcds,
                     const PlanModel& m, bool worklist) {
  const int max_pages = ceil_div(max_seq_len, pa::kPage);
  const int S = ceil_div(max_pages, ps);
  const double chip_rate = m.hbm_bytes_per_us / m.page_bytes;    // pages/us, whole chip
  const double cu_rate = 1.0 / m.page_us;                        // pages/us, one CU alone
  const int per_xcd = (cu / xcds > 0 ? cu / xcds : 1) * (m.resident > 1 ? m.resident : 1);
  struct Item { double fixed, pages; };
  std::vector<Item> items;
  items.reserve((size_t)batch * S);
  double partial_rows = 0;
  for (int b = 0; b < batch; ++b) {
    const int L = lens[b] < 0 ? 0 : (lens[b] > max_seq_len ? max_seq_len : lens[b]);
    const int n = ceil_div(L, pa::kPage);
    const int nsb = n > 0 ? ceil_div(n, ps) : 1;
    if (nsb > 1) partial_rows += nsb;
    for (int k = 0; k < S; ++k) {
      if (k < nsb) items.push_back({m.group_us, (double)((k + 1) * ps <= n ? ps : n - k * ps)});
      else if (!worklist) items.push_back({m.empty_us, 0.0});
    }
  }
  if (worklist)
    std::stable_sort(items.begin(), items.end(),
                     [](const Item& x, const Item& y) { return x.pages > y.pages; });
  // two wavefronts per KV head when the plan's grid (batch x splits) fits the
  // CUs and the splits are long enough
  const bool two_waves = (int64_t)batch * S <= cu && ps >= kTwoWaveMinPages;
  const double cu_rate1 = two_waves ? cu_rate * m.two_wave_gain : cu_rate;
  // Streaming progress is tracked in virtual pages V (every streaming
  // work-group advances by the same rate), so a work-group that starts
  // streaming r pages at V0 ends when V reaches V0 + r.
  typedef std::pair<double, int> Ev;   // (time or V, xcd); payload index in pages_of
  std::priority_queue<std::pair<double, std::pair<int, double>>,
                      std::vector<std::pair<double, std::pair<int, double>>>,
                      std::greater<std::pair<double, std::pair<int, double>>>> fixed_end;
  std::priority_queue<Ev, std::vector<Ev>, std::greater<Ev>> stream_end;
  std::vector<size_t> next(xcds);
  std::vector<int> busy(xcds, 0);
  for (int x = 0; x < xcds; ++x) next[x] = (size_t)x;
  double t = 0, V = 0;
  auto fill = [&](int x) {
    while (busy[x] < per_xcd && next[x] < items.size()) {
      const Item& it = items[next[x]];
      next[x] += (size_t)xcds;
      ++busy[x];
      fixed_end.push({t + it.fixed, {x, it.pages}});
    }
  };
  for (int x = 0; x < xcds; ++x) fill(x);
  while (!fixed_end.empty() || !stream_end.empty()) {
    const int ns = (int)stream_end.size();
    // beyond one streaming work-group per CU, each extra one adds
    // (shared_gain - 1) of a CU's rate (work-groups spread evenly over CUs)
    const double cap = ns <= cu ? cu_rate1
                                : cu_rate * (cu + (ns - cu) * (m.shared_gain - 1.0)) / ns;
    const double r = ns > 0 ? std::min(cap, chip_rate / ns) : cu_rate1;
    const double dt_fixed = fixed_end.empty() ? 1e300 : fixed_end.top().first - t;
    const double dt_stream = stream_end.empty() ? 1e300 : (stream_end.top().first - V) / r;
    if (dt_fixed <= dt_stream) {
      t += dt_fixed;
      V += r * dt_fixed * (ns > 0);
      const auto e = fixed_end.top();
      fixed_end.pop();
      if (e.second.second > 0) {
        stream_end.push({V + e.second.second, e.second.first});
      } else {
        --busy[e.second.first];
        fill(e.second.first);
      }
    } else {
      t += dt_stream;
      V = stream_end.top().first;
      const int x = stream_end.top().second;
      stream_end.pop();
      --busy[x];
      fill(x);
    }
  }
  if (partial_rows > 0)
    t += m.merge_us + 2.0 * partial_rows * pa::kHq * (pa::kD + 2) * 4.0 / m.hbm_bytes_per_us;
  return t;
}

int plan_split_lengths(const pa_shape* s, int batch, const int32_t* lens, int max_seq_len,
                       int num_cus, const PlanModel& model, int* pages, int* splits,
                       bool worklist) {
  int cu = num_cus;
  if (cu <= 0) {
    const int rc = current_cu_count(&cu);
    if (rc != PA_OK) return rc;
  }
  const int max_pages = ceil_div(max_seq_len, pa::kPage);
  if (max_pages <= 0) { *pages = 1; *splits = 1; return PA_OK; }
  const int xcds = (cu % 8 == 0) ? 8 : 1;         // MI300-class parts: 8 XCDs
  std::vector<std::pair<int, double>> cands;
  // A work list balances items of different sizes but needs many of them: at
  // 128-page splits the Zipf batch of 512 measured 7% slower than at 32-64.
  // Work-list plans stop at 64 pages unless the lengths are even (the
  // shortest at least half the longest) and there is a sequence per CU.
  int min_pages = max_pages;
  for (int b = 0; b < batch; ++b) {
    const int L = lens[b] < 0 ? 0 : (lens[b] > max_seq_len ? max_seq_len : lens[b]);
    min_pages = std::min(min_pages, ceil_div(L, pa::kPage));
  }
  const bool even = 2 * min_pages >= max_pages;
  const bool long_splits = !worklist || (batch >= cu && even);
  // The model spreads work-groups that share a CU evenly over the CUs, which
  // holds when they all stream about as long.  In a skewed batch two long
  // work-groups can stay paired on one CU to the end (INT4 pages, 512-sequence
  // Zipf batch, 128-page grid: modelled 68 us, measured 111 us), so such a
  // batch is planned with one work-group per CU.
  PlanModel mm = model;
  if (!even) mm.resident = 1;
  for (int ps : {8, 16, 32, 64, 128, 256}) {
    if (!long_splits && ps > 64) break;
    const int cand = ps < max_pages ? ps : max_pages;
    if (cand > s->max_blocks_per_seq || cand > pa::kMaxSplitPages) break;
    cands.push_back({cand, simulate_plan(lens, batch, max_seq_len, cand, cu, xcds, mm,
                                         worklist)});
    if (cand == max_pages) break;
  }
  if (cands.empty()) { *pages = 1; *splits = max_pages; return PA_OK; }
  double best = 1e300;
  for (auto& c : cands) best = std::min(best, c.second);
  int ps = cands.front().first;
  for (auto& c : cands)
    if (c.second <= best * 1.03) ps = std::max(ps, c.first);
  *pages = ps;
  *splits = ceil_div(max_pages, ps);
  return PA_OK;
}

size_t workspace_for(int batch, int splits) {
  if (splits <= 1) return 0;
  const size_t rows = (size_t)batch * splits * pa::kHq;
  size_t acc = rows * pa::kD * sizeof(float);
  acc = (acc + 255) & ~(size_t)255;
  return acc + rows * 2 * sizeof(float);
}

int check_decode_sizes(const pa_shape* shape, int32_t batch, int32_t max_seq_len) {
  int rc = check_shape(shape);
  if (rc != PA_OK) return rc;
  if (batch < 0) return PA_ERR_VALUE;
  if (max_seq_len < 0 || (int64_t)max_seq_len > (int64_t)shape->max_blocks_per_seq * pa::kPage)
    return PA_ERR_VALUE;
  return PA_OK;
}

int check_rope(const pa_rope* rope, int64_t needed_positions) {
  if (!rope->cos || !rope->sin) return PA_ERR_NULL;
  if (!aligned(rope->cos, 4) || !aligned(rope->sin, 4)) return PA_ERR_ALIGN;
  if (rope->positions < 1 || rope->positions < needed_positions) return PA_ERR_VALUE;
  return PA_OK;
}

int build_worklist(int batch, const int32_t* lens, int max_seq_len, int ps, int32_t* work,
                   int capacity, int* count) {
  struct Item { int pages, b, s; };
  std::vector<Item> items;
  for (int b = 0; b < batch; ++b) {
    const int L = lens[b];
    const int n = (L > 0 && L <= max_seq_len) ? ceil_div(L, pa::kPage) : 0;
    const int nsb = n > 0 ? ceil_div(n, ps) : 1;
    for (int k = 0; k < nsb; ++k) items.push_back({n > 0 ? std::min(ps, n - k * ps) : 0, b, k});
  }
  std::stable_sort(items.begin(), items.end(),
                   [](const Item& x, const Item& y) { return x.pages > y.pages; });
  *count = (int)items.size();
  if ((int)items.size() > capacity) return PA_ERR_VALUE;
  for (size_t k = 0; k < items.size(); ++k) {
    work[2 * k] = items[k].b;
    work[2 * k + 1] = items[k].s;
  }
  return PA_OK;
}

}  // namespace pa_host

using namespace pa_host;

PA_API int pa_abi_version(void) { return 1; }

PA_API const char* pa_status_string(int status) {
  switch (status) {
    case PA_OK: return "PA_OK";
    case PA_ERR_NULL: return "PA_ERR_NULL: a required pointer is NULL";
    case PA_ERR_SHAPE: return "PA_ERR_SHAPE: only 32 query heads, 8 KV heads, head_dim 64, 16-token pages";
    case PA_ERR_ALIGN: return "PA_ERR_ALIGN: pointer not aligned (16 B for tensors, 4 B for metadata)";
    case PA_ERR_WORKSPACE: return "PA_ERR_WORKSPACE: workspace missing or too small";
    case PA_ERR_LAUNCH: return "PA_ERR_LAUNCH: HIP kernel launch failed";
    case PA_ERR_VALUE: return "PA_ERR_VALUE: size or scalar argument out of range";
    case PA_ERR_METADATA: return "PA_ERR_METADATA: block table or sequence length invalid";
    case PA_ERR_DEVICE: return "PA_ERR_DEVICE: HIP device query failed";
    default: return "unknown pa_status";
  }
}

PA_API int pa_append_kv(const pa_shape* shape, int32_t batch, const void* k_new,
                        const void* v_new, void* k_pool, void* v_pool,
                        const int32_t* block_tables, const int32_t* seq_lens, void* stream) {
  int rc = check_shape(shape);
  if (rc != PA_OK) return rc;
  if (batch < 0) return PA_ERR_VALUE;
  if (batch == 0) return PA_OK;
  if (!k_new || !v_new || !k_pool || !v_pool || !block_tables || !seq_lens) return PA_ERR_NULL;
  if (!aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) ||
      !aligned(block_tables, 4) || !aligned(seq_lens, 4))
    return PA_ERR_ALIGN;
  if (shape->num_pages < 1) return PA_ERR_VALUE;
  hipLaunchKernelGGL(pa::append_kernel, dim3(batch), dim3(64), 0, (hipStream_t)stream,
                     (const uint4*)k_new, (const uint4*)v_new, (uint4*)k_pool, (uint4*)v_pool,
                     block_tables, seq_lens, shape->max_blocks_per_seq, shape->num_pages);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

PA_API int pa_fill_kv(const pa_shape* shape, const void* k_rows, const void* v_rows,
                      int32_t num_tokens, int32_t start, const int32_t* block_table_row,
                      void* k_pool, void* v_pool, void* stream) {
  int rc = check_shape(shape);
  if (rc != PA_OK) return rc;
  if (num_tokens < 0 || start < 0 ||
      (int64_t)start + num_tokens > (int64_t)shape->max_blocks_per_seq * pa::kPage)
    return PA_ERR_VALUE;
  if (num_tokens == 0) return PA_OK;
  if (!k_rows || !v_rows || !block_table_row || !k_pool || !v_pool) return PA_ERR_NULL;
  if (!aligned(k_rows, 16) || !aligned(v_rows, 16) || !aligned(k_pool, 16) ||
      !aligned(v_pool, 16) || !aligned(block_table_row, 4))
    return PA_ERR_ALIGN;
  if (shape->num_pages < 1) return PA_ERR_VALUE;
  hipLaunchKernelGGL(pa::fill_kernel, dim3(ceil_div(num_tokens, 4)), dim3(256), 0,
                     (hipStream_t)stream, (const uint4*)k_rows, (const uint4*)v_rows, num_tokens,
                     start, block_table_row, (uint4*)k_pool, (uint4*)v_pool, shape->num_pages);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

PA_API int pa_decode_plan(const pa_shape* shape, int32_t batch, int32_t max_seq_len,
                          int32_t pages_per_split, int32_t* pages_out, int32_t* splits_out) {
  int rc = check_decode_sizes(shape, batch, max_seq_len);
  if (rc != PA_OK) return rc;
  int ps = 0, ns = 0;
  rc = plan_split(shape, batch, max_seq_len, pages_per_split, &ps, &ns);
  if (rc != PA_OK) return rc;
  if (pages_out) *pages_out = ps;
  if (splits_out) *splits_out = ns;
  return PA_OK;
}

PA_API int pa_decode_plan_lengths(const pa_shape* shape, int32_t batch,
                                  const int32_t* seq_lens_host, int32_t max_seq_len,
                                  int32_t num_cus, int32_t* pages_out, int32_t* splits_out) {
  int rc = check_decode_sizes(shape, batch, max_seq_len);
  if (rc != PA_OK) return rc;
  if (batch > 0 && !seq_lens_host) return PA_ERR_NULL;
  if (num_cus < 0) return PA_ERR_VALUE;
  int ps = 1, ns = 1;
  if (batch > 0) {
    rc = plan_split_lengths(shape, batch, seq_lens_host, max_seq_len, num_cus, PlanModel(), &ps,
                            &ns);
    if (rc != PA_OK) return rc;
  }
  if (pages_out) *pages_out = ps;
  if (splits_out) *splits_out = ns;
  return PA_OK;
}

PA_API int pa_decode_workspace_bytes(const pa_shape* shape, int32_t batch, int32_t max_seq_len,
                                     int32_t pages_per_split, size_t* bytes) {
  if (!bytes) return PA_ERR_NULL;
  int ps = 0, ns = 0;
  const int rc = pa_decode_plan(shape, batch, max_seq_len, pages_per_split, &ps, &ns);
  if (rc != PA_OK) return rc;
  *bytes = workspace_for(batch, ns);
  return PA_OK;
}

namespace {
// k_new/v_new non-NULL: the one-token append is fused into the main kernel
int decode_impl(const pa_shape* shape, int32_t batch, const void* q, const void* k_new,
                const void* v_new, const pa_rope* rope, const void* k_pool,
                const void* v_pool, const int32_t* block_tables, const int32_t* seq_lens,
                int32_t max_seq_len, float scale, void* out, int32_t out_dtype,
                int32_t pages_per_split, void* workspace, size_t workspace_bytes,
                void* stream, void* event_before_main, void* event_after_main,
                const int32_t* work = nullptr, int32_t num_work = 0) {
  int rc = check_decode_sizes(shape, batch, max_seq_len);
  if (rc != PA_OK) return rc;
  if (out_dtype != PA_OUT_F32 && out_dtype != PA_OUT_BF16) return PA_ERR_VALUE;
  if (!std::isfinite(scale)) return PA_ERR_VALUE;
  if (batch == 0) return PA_OK;
  if (!q || !k_pool || !v_pool || !block_tables || !seq_lens || !out) return PA_ERR_NULL;
  const bool fused = k_new != nullptr || v_new != nullptr;
  if (fused && (!k_new || !v_new)) return PA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(out, 16) ||
      !aligned(block_tables, 4) || !aligned(seq_lens, 4) ||
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
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.k_new = (const uint16_t*)k_new;
  a.v_new = (const uint16_t*)v_new;
  a.k_pool_w = const_cast<void*>(k_pool);
  a.v_pool_w = const_cast<void*>(v_pool);
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
  // a batch that fits the compute units merges with its partials requested up front
  int cu = 0;
  const bool have_cu = current_cu_count(&cu) == PA_OK;
  const bool merge_preload = have_cu && batch <= cu;
  // One slot per wavefront unless the launch leaves CUs idle, or every
  // work-group runs at once on its own CU with a short split: a busy CU then
  // needs more pages in flight, or the start of each short stream is
  // exposed, and a second slot per wavefront covers it (page order and
  // arithmetic are the same either way).
  const int64_t groups = work ? (int64_t)num_work : (int64_t)batch * ns;
  const bool two_slots =
      have_cu && groups <= cu && (groups < cu || ps < pa_host::kOneSlotMinPages);
  const hipError_t e = pa::launch_decode<pa::kFmtBF16>(a, batch, out_dtype == PA_OUT_BF16, fused,
                                                rope != nullptr, merge_preload, false, two_slots,
                                                (hipStream_t)stream,
                                                (hipEvent_t)event_before_main,
                                                (hipEvent_t)event_after_main);
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}
}  // namespace

PA_API int pa_decode_attention(const pa_shape* shape, int32_t batch, const void* q,
                               const void* k_pool, const void* v_pool,
                               const int32_t* block_tables, const int32_t* seq_lens,
                               int32_t max_seq_len, float scale, void* out, int32_t out_dtype,
                               int32_t pages_per_split, void* workspace, size_t workspace_bytes,
                               void* stream) {
  return decode_impl(shape, batch, q, nullptr, nullptr, nullptr, k_pool, v_pool, block_tables,
                     seq_lens, max_seq_len, scale, out, out_dtype, pages_per_split, workspace,
                     workspace_bytes, stream, nullptr, nullptr);
}

PA_API int pa_append_decode_attention(const pa_shape* shape, int32_t batch, const void* q,
                                      const void* k_new, const void* v_new, void* k_pool,
                                      void* v_pool, const int32_t* block_tables,
                                      const int32_t* seq_lens, int32_t max_seq_len, float scale,
                                      void* out, int32_t out_dtype, int32_t pages_per_split,
                                      void* workspace, size_t workspace_bytes, void* stream) {
  if (batch > 0 && (!k_new || !v_new)) return PA_ERR_NULL;
  return decode_impl(shape, batch, q, k_new, v_new, nullptr, k_pool, v_pool, block_tables,
                     seq_lens, max_seq_len, scale, out, out_dtype, pages_per_split, workspace,
                     workspace_bytes, stream, nullptr, nullptr);
}

PA_API int pa_append_decode_attention_rope(const pa_shape* shape, int32_t batch, const void* q,
                                           const void* k_new, const void* v_new,
                                           const pa_rope* rope, void* k_pool, void* v_pool,
                                           const int32_t* block_tables, const int32_t* seq_lens,
                                           int32_t max_seq_len, float scale, void* out,
                                           int32_t out_dtype, int32_t pages_per_split,
                                           void* workspace, size_t workspace_bytes,
                                           void* stream) {
  if (batch > 0 && (!k_new || !v_new || !rope)) return PA_ERR_NULL;
  return decode_impl(shape, batch, q, k_new, v_new, rope, k_pool, v_pool, block_tables, seq_lens,
                     max_seq_len, scale, out, out_dtype, pages_per_split, workspace,
                     workspace_bytes, stream, nullptr, nullptr);
}

PA_API int pa_append_kv_rope(const pa_shape* shape, int32_t batch, const void* q,
                             const void* k_new, const void* v_new, const pa_rope* rope,
                             void* q_out, void* k_pool, void* v_pool,
                             const int32_t* block_tables, const int32_t* seq_lens,
                             void* stream) {
  int rc = check_shape(shape);
  if (rc != PA_OK) return rc;
  if (batch < 0) return PA_ERR_VALUE;
  if (batch == 0) return PA_OK;
  if (!q || !k_new || !v_new || !rope || !q_out || !k_pool || !v_pool || !block_tables ||
      !seq_lens)
    return PA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k_new, 16) || !aligned(v_new, 16) || !aligned(q_out, 16) ||
      !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(block_tables, 4) ||
      !aligned(seq_lens, 4))
    return PA_ERR_ALIGN;
  if (shape->num_pages < 1) return PA_ERR_VALUE;
  rc = check_rope(rope, (int64_t)shape->max_blocks_per_seq * pa::kPage);
  if (rc != PA_OK) return rc;
  hipLaunchKernelGGL(pa::append_rope_kernel, dim3(batch), dim3(256), 0, (hipStream_t)stream,
                     (const uint16_t*)q, (const uint16_t*)k_new, (const uint16_t*)v_new,
                     rope->cos, rope->sin, (uint16_t*)q_out, (uint16_t*)k_pool,
                     (uint16_t*)v_pool, block_tables, seq_lens, shape->max_blocks_per_seq,
                     shape->num_pages);
  return hipGetLastError() == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

PA_API int pa_decode_attention_profiled(const pa_shape* shape, int32_t batch, const void* q,
                                        const void* k_new, const void* v_new,
                                        void* k_pool, void* v_pool,
                                        const int32_t* block_tables, const int32_t* seq_lens,
                                        int32_t max_seq_len, float scale, void* out,
                                        int32_t out_dtype, int32_t pages_per_split,
                                        void* workspace, size_t workspace_bytes, void* stream,
                                        void* event_before_main, void* event_after_main) {
  return decode_impl(shape, batch, q, k_new, v_new, nullptr, k_pool, v_pool, block_tables,
                     seq_lens, max_seq_len, scale, out, out_dtype, pages_per_split, workspace,
                     workspace_bytes, stream, event_before_main, event_after_main);
}

PA_API int pa_decode_worklist(const pa_shape* shape, int32_t batch, const int32_t* seq_lens_host,
                              int32_t max_seq_len, int32_t pages_per_split, int32_t page_format,
                              int32_t num_cus, int32_t* work, int32_t capacity, int32_t* count,
                              int32_t* pages_out, int32_t* splits_out) {
  int rc = check_decode_sizes(shape, batch, max_seq_len);
  if (rc != PA_OK) return rc;
  if (!count || (batch > 0 && (!seq_lens_host || !work))) return PA_ERR_NULL;
  if (capacity < 0 || num_cus < 0 || page_format < 0 || page_format > 2) return PA_ERR_VALUE;
  int ps = pages_per_split, ns = 1;
  if (batch > 0 && ps == 0) {
    const PlanModel model = page_format == 1   ? plan_model_q8()
                            : page_format == 2 ? plan_model_q4()
                                               : PlanModel();
    rc = plan_split_lengths(shape, batch, seq_lens_host, max_seq_len, num_cus, model, &ps, &ns,
                            true);
    if (rc != PA_OK) return rc;
  }
  rc = plan_split(shape, batch, max_seq_len, ps == 0 ? 1 : ps, &ps, &ns);
  if (rc != PA_OK) return rc;
  *count = 0;
  if (batch > 0) {
    rc = build_worklist(batch, seq_lens_host, max_seq_len, ps, work, capacity, count);
    if (rc != PA_OK) return rc;
  }
  if (pages_out) *pages_out = ps;
  if (splits_out) *splits_out = ns;
  return PA_OK;
}

PA_API int pa_append_decode_attention_worklist(
    const pa_shape* shape, int32_t batch, const void* q, const void* k_new, const void* v_new,
    void* k_pool, void* v_pool, const int32_t* block_tables, const int32_t* seq_lens,
    int32_t max_seq_len, float scale, void* out, int32_t out_dtype, int32_t pages_per_split,
    const int32_t* work, int32_t num_work, void* workspace, size_t workspace_bytes,
    void* stream) {
  if (batch > 0 && !work) return PA_ERR_NULL;
  return decode_impl(shape, batch, q, k_new, v_new, nullptr, k_pool, v_pool, block_tables,
                     seq_lens, max_seq_len, scale, out, out_dtype, pages_per_split, workspace,
                     workspace_bytes, stream, nullptr, nullptr, work, num_work);
}

// Split partials of pa_append_decode_attention_noalloc: a file-scope device
// array, one copy per GPU, held until the process ends.  Host code never
// passes the array's name to a kernel (on the host it is only a stand-in for
// the symbol): each device's address is looked up once, with that device
// current, and kept in g_scratch_ptr.
static __device__ __align__(256) unsigned char scratch[PA_NOALLOC_SCRATCH_BYTES];

namespace pa_host {
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_rc[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

// Device address of the current device's scratch array, or NULL.
void* current_scratch() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    g_scratch_rc[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_rc[dev] == hipSuccess ? ptr : nullptr;
  });
  return g_scratch_ptr[dev];
}
}  // namespace pa_host

PA_API int pa_append_decode_attention_noalloc(const pa_shape* shape, int32_t batch,
                                              const void* q, const void* k_new,
                                              const void* v_new, void* k_pool, void* v_pool,
                                              const int32_t* block_tables,
                                              const int32_t* seq_lens, int32_t max_seq_len,
                                              float scale, void* out, int32_t out_dtype,
                                              int32_t pages_per_split, void* stream) {
  if (batch > 0 && (!k_new || !v_new)) return PA_ERR_NULL;
  int rc = check_decode_sizes(shape, batch, max_seq_len);
  if (rc != PA_OK) return rc;
  if (batch == 0) return PA_OK;
  int ps = 0, ns = 0;
  rc = plan_split(shape, batch, max_seq_len, pages_per_split, &ps, &ns);
  if (rc != PA_OK) return rc;
  if (workspace_for(batch, ns) > PA_NOALLOC_SCRATCH_BYTES) return PA_ERR_WORKSPACE;
  void* ws = current_scratch();
  if (!ws) return PA_ERR_DEVICE;
  return decode_impl(shape, batch, q, k_new, v_new, nullptr, k_pool, v_pool, block_tables,
                     seq_lens, max_seq_len, scale, out, out_dtype, pages_per_split, ws,
                     PA_NOALLOC_SCRATCH_BYTES, stream, nullptr, nullptr);
}

PA_API int pa_validate_metadata(const pa_shape* shape, int32_t batch,
                                const int32_t* block_tables, const int32_t* seq_lens,
                                int32_t max_seq_len, void* stream, int64_t* bad_index) {
  if (bad_index) *bad_index = -1;
  int rc = check_decode_sizes(shape, batch, max_seq_len);
  if (rc != PA_OK) return rc;
  if (batch == 0) return PA_OK;
  if (!block_tables || !seq_lens) return PA_ERR_NULL;
  const int mb = shape->max_blocks_per_seq;
  std::vector<int32_t> bt((size_t)batch * mb), lens(batch);
  hipStream_t st = (hipStream_t)stream;
  if (hipMemcpyAsync(bt.data(), block_tables, bt.size() * 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipMemcpyAsync(lens.data(), seq_lens, lens.size() * 4, hipMemcpyDeviceToHost, st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return PA_ERR_LAUNCH;
  std::vector<int32_t> owner(shape->num_pages > 0 ? shape->num_pages : 0, -1);
  for (int b = 0; b < batch; ++b) {
    const int L = lens[b];
    if (L < 0 || L > max_seq_len) { if (bad_index) *bad_index = b; return PA_ERR_METADATA; }
    const int n = ceil_div(L, pa::kPage);
    for (int i = 0; i < n; ++i) {
      const int id = bt[(size_t)b * mb + i];
      if (id < 0 || id >= shape->num_pages || owner[id] != -1) {
        if (bad_index) *bad_index = b;
        return PA_ERR_METADATA;
      }
      owner[id] = b;
    }
  }
  return PA_OK;
}
