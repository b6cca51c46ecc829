// Host page allocator and admission control for the shared K/V page pool
// (C ABI in include/pa_kvpool.h).
//
// The rules are those of the engine's README ("6 Hours of YouTube and 85
// handtyped pages of notes on LLM Inference", current scope): a request
// reserves credit for prompt + allowed new tokens - 1 (the last predicted
// token is never processed), rounded up to whole pages in every layer, with
// the output budget capped by the context; physical pages are taken lazily
// as a sequence grows; requests wait in FIFO order while their credit does
// not fit and are rejected outright when it exceeds the whole pool; finishing
// returns pages and credit; static batching admits the next group only when
// the current one is done.  A new page is the lowest-numbered free page.
#include <cstdint>
#include <deque>
#include <new>
#include <functional>
#include <queue>
#include <unordered_map>
#include <vector>

#include "pa_decode.h"
#include "pa_kvpool.h"

#define PA_API extern "C" __attribute__((visibility("default")))

struct pa_kvpool {
  struct Request {
    int32_t prompt = 0, allowed_new = 0, credit = 0, length = 0;
    bool active = false, waited = false;
    std::vector<std::vector<int32_t>> pages;   // per layer
  };
  int32_t num_pages = 0, layers = 0, page_tokens = 0, context = 0;
  bool static_batching = false;
  int64_t reserved = 0;
  std::priority_queue<int32_t, std::vector<int32_t>, std::greater<int32_t>> free_pages;
  std::unordered_map<int64_t, Request> requests;   // waiting or active
  std::deque<int64_t> waiting;
  int64_t active_count = 0;
  pa_kvpool_stats stats = {};

  int64_t pages_for(int64_t tokens) const { return (tokens + page_tokens - 1) / page_tokens; }
};

PA_API int pa_kvpool_create(int32_t num_pages, int32_t num_layers, int32_t page_tokens,
                            int32_t context_tokens, int32_t static_batching, pa_kvpool** out) {
  if (!out) return PA_ERR_NULL;
  *out = nullptr;
  if (num_pages < 1 || num_layers < 1 || page_tokens < 1 || context_tokens < 2)
    return PA_ERR_VALUE;
  pa_kvpool* p = new (std::nothrow) pa_kvpool;
  if (!p) return PA_ERR_VALUE;
  p->num_pages = num_pages;
  p->layers = num_layers;
  p->page_tokens = page_tokens;
  p->context = context_tokens;
  p->static_batching = static_batching != 0;
  std::vector<int32_t> ids(num_pages);
  for (int32_t i = 0; i < num_pages; ++i) ids[i] = i;
  p->free_pages = std::priority_queue<int32_t, std::vector<int32_t>, std::greater<int32_t>>(
      std::greater<int32_t>(), std::move(ids));
  p->stats.pool_pages = num_pages;
  p->stats.free_pages = num_pages;
  *out = p;
  return PA_OK;
}

PA_API int pa_kvpool_destroy(pa_kvpool* pool) {
  delete pool;
  return PA_OK;
}

PA_API int pa_kvpool_credit(const pa_kvpool* pool, int32_t prompt_tokens, int32_t max_new_tokens,
                            int32_t* allowed_new, int64_t* credit_pages) {
  if (!pool || !allowed_new || !credit_pages) return PA_ERR_NULL;
  if (prompt_tokens < 1 || prompt_tokens >= pool->context || max_new_tokens < 1)
    return PA_ERR_VALUE;
  const int32_t room = pool->context - prompt_tokens;
  *allowed_new = max_new_tokens < room ? max_new_tokens : room;
  *credit_pages = (int64_t)pool->layers * pool->pages_for((int64_t)prompt_tokens + *allowed_new - 1);
  return PA_OK;
}

PA_API int pa_kvpool_submit(pa_kvpool* pool, int64_t request_id, int32_t prompt_tokens,
                            int32_t max_new_tokens, int32_t* result) {
  if (!pool || !result) return PA_ERR_NULL;
  if (pool->requests.count(request_id)) return PA_ERR_VALUE;     // id in use
  int32_t allowed = 0;
  int64_t credit = 0;
  if (pa_kvpool_credit(pool, prompt_tokens, max_new_tokens, &allowed, &credit) != PA_OK ||
      credit > pool->num_pages) {
    *result = PA_KV_REJECT;
    return PA_OK;
  }
  pa_kvpool::Request r;
  r.prompt = prompt_tokens;
  r.allowed_new = allowed;
  r.credit = (int32_t)credit;
  pool->requests.emplace(request_id, std::move(r));
  pool->waiting.push_back(request_id);
  *result = PA_KV_WAIT;
  return PA_OK;
}

PA_API int pa_kvpool_admit(pa_kvpool* pool, int64_t* admitted, int32_t capacity, int32_t* count) {
  if (!pool || !count || (capacity > 0 && !admitted)) return PA_ERR_NULL;
  *count = 0;
  if (!(pool->static_batching && pool->active_count > 0)) {
    // how many fit, before anything changes: a too-small array leaves the pool untouched
    int64_t fit = 0, res = pool->reserved;
    for (int64_t id : pool->waiting) {
      const int32_t c = pool->requests.at(id).credit;
      if (res + c > pool->num_pages) break;
      res += c;
      ++fit;
    }
    if (fit > capacity) return PA_ERR_VALUE;
    while (!pool->waiting.empty()) {
      auto& r = pool->requests.at(pool->waiting.front());
      if (pool->reserved + r.credit > pool->num_pages) break;
      admitted[(*count)++] = pool->waiting.front();
      pool->waiting.pop_front();
      pool->reserved += r.credit;
      r.active = true;
      r.pages.assign(pool->layers, {});
      ++pool->active_count;
    }
  }
  for (int64_t id : pool->waiting) {
    auto& r = pool->requests.at(id);
    if (!r.waited) {
      r.waited = true;
      ++pool->stats.admission_waits;
    }
  }
  if (pool->active_count > pool->stats.peak_active) pool->stats.peak_active = pool->active_count;
  return PA_OK;
}

PA_API int pa_kvpool_grow(pa_kvpool* pool, int64_t request_id, int32_t length) {
  if (!pool) return PA_ERR_NULL;
  auto it = pool->requests.find(request_id);
  if (it == pool->requests.end() || !it->second.active) return PA_ERR_VALUE;
  auto& r = it->second;
  if (length < r.length || (int64_t)length > (int64_t)r.prompt + r.allowed_new - 1)
    return PA_ERR_VALUE;
  const int64_t need = pool->pages_for(length);
  for (auto& layer_pages : r.pages) {
    while ((int64_t)layer_pages.size() < need) {
      // credit was reserved at admission, so a free page always exists
      if (pool->free_pages.empty()) return PA_ERR_VALUE;
      layer_pages.push_back(pool->free_pages.top());
      pool->free_pages.pop();
    }
  }
  r.length = length;
  const int64_t used = pool->num_pages - (int64_t)pool->free_pages.size();
  if (used > pool->stats.peak_allocated) pool->stats.peak_allocated = used;
  pool->stats.free_pages = (int64_t)pool->free_pages.size();
  return PA_OK;
}

PA_API int pa_kvpool_step(pa_kvpool* pool) {
  if (!pool) return PA_ERR_NULL;
  if (pool->active_count > pool->stats.max_batch) pool->stats.max_batch = pool->active_count;
  return PA_OK;
}

PA_API int pa_kvpool_finish(pa_kvpool* pool, int64_t request_id) {
  if (!pool) return PA_ERR_NULL;
  auto it = pool->requests.find(request_id);
  if (it == pool->requests.end() || !it->second.active) return PA_ERR_VALUE;
  for (auto& layer_pages : it->second.pages)
    for (int32_t p : layer_pages) pool->free_pages.push(p);
  pool->reserved -= it->second.credit;
  --pool->active_count;
  pool->requests.erase(it);
  pool->stats.free_pages = (int64_t)pool->free_pages.size();
  return PA_OK;
}

PA_API int pa_kvpool_block_table(const pa_kvpool* pool, int64_t request_id, int32_t layer,
                                 int32_t* row, int32_t row_capacity, int32_t* num_pages) {
  if (!pool || !num_pages) return PA_ERR_NULL;
  auto it = pool->requests.find(request_id);
  if (it == pool->requests.end() || !it->second.active || layer < 0 || layer >= pool->layers)
    return PA_ERR_VALUE;
  const auto& pages = it->second.pages[layer];
  *num_pages = (int32_t)pages.size();
  if ((int64_t)pages.size() > row_capacity) return PA_ERR_VALUE;
  if (!pages.empty() && !row) return PA_ERR_NULL;
  for (size_t i = 0; i < pages.size(); ++i) row[i] = pages[i];
  for (int32_t i = (int32_t)pages.size(); i < row_capacity && row; ++i) row[i] = -1;
  return PA_OK;
}

PA_API int pa_kvpool_request_info(const pa_kvpool* pool, int64_t request_id, int32_t* allowed_new,
                                  int32_t* credit_pages, int32_t* length, int32_t* active) {
  if (!pool || !allowed_new || !credit_pages || !length || !active) return PA_ERR_NULL;
  auto it = pool->requests.find(request_id);
  if (it == pool->requests.end()) return PA_ERR_VALUE;
  *allowed_new = it->second.allowed_new;
  *credit_pages = it->second.credit;
  *length = it->second.length;
  *active = it->second.active ? 1 : 0;
  return PA_OK;
}

PA_API int pa_kvpool_get_stats(const pa_kvpool* pool, pa_kvpool_stats* out) {
  if (!pool || !out) return PA_ERR_NULL;
  *out = pool->stats;
  return PA_OK;
}
