// Host planner of the balanced launch (pa_balance_plan): whole (sequence,
// KV-head group) streams packed into work-groups, largest first, and laid
// out over each work-group's wavefronts.  Host code only; the kernel that
// follows the plan is in pa_decode_balanced.hip, the plan's layout in
// pa_balance_plan.h.  See include/pa_decode_balanced.h for the contract.
#include <algorithm>
#include <cstdint>
#include <utility>
#include <vector>

#include "pa_balance_plan.h"
#include "pa_decode.h"
#include "pa_decode_balanced.h"
#include "pa_host.h"

#define PA_API extern "C" __attribute__((visibility("default")))

namespace pa_host {

// A wavefront does not split a stream below this many pages unless the
// work-group's pages call for it (short pieces cost a merge each).
constexpr int kBalMinChunk = 4;

struct BalUnit {
  int b, g0, pages;          // heads g0 .. g0 + h - 1 of sequence b, ceil(L/16) pages
};
struct BalSeg {
  int b, g, p0, p1, L, kind, pieces, stride;
};

// A plan under construction: up to kBalMaxSeg segments per wavefront, in flat
// arrays reused from call to call (planning runs on every decode step of a
// serving loop, so it allocates nothing once warm).
struct BalPlan {
  int groups = 0;
  std::vector<BalSeg> seg;         // [wavefront][kBalMaxSeg]
  std::vector<uint8_t> nseg;       // segments per wavefront
  std::vector<int> bin_of, bin_start, bin_units, order, longs, shorts;   // packing scratch
  std::vector<uint64_t> tree;
  BalSeg* at(size_t w) { return seg.data() + w * pa::kBalMaxSeg; }
};

// One attempt at `groups` work-groups with units of h heads (h = 1, 2, 4 or
// 8): false when a wavefront would hold more segments or pages than a
// descriptor allows.  A work-group's 8 wavefronts form 8 / h lanes of h
// wavefronts; a lane streams its units' heads in lockstep (wavefront i of the
// lane takes head g0 + i), so the heads of a sequence that one lane holds are
// read together.  With h = 8 units are whole sequences and are never cut;
// otherwise a work-group's units are laid end to end and cut evenly over its
// lanes, and the pieces of a unit are merged in LDS (stride h).
static bool balance_attempt(const std::vector<BalUnit>& units, const std::vector<int>& idle,
                            const int32_t* lens, int groups, int h, BalPlan& bp) {
  const int lanes = pa::kBalWaves / h;
  const size_t nw = (size_t)groups * pa::kBalWaves;
  const int nunits = (int)units.size();
  bp.groups = groups;
  if (bp.seg.size() < nw * pa::kBalMaxSeg) bp.seg.resize(nw * pa::kBalMaxSeg);
  bp.nseg.assign(nw, 0);
  // largest unit first into the least-loaded work-group (ties: lowest index);
  // with h = 8 a work-group takes at most kBalMaxSeg sequences.  The
  // least-loaded group is the root of a tournament tree over the keys
  // load << 32 | index (a full group's key is all ones).
  bp.bin_of.assign(nunits, -1);
  bp.bin_start.assign((size_t)groups + 1, 0);
  {
    int leaves = 1;
    while (leaves < groups) leaves *= 2;
    constexpr uint64_t kFull = ~0ull;
    std::vector<uint64_t>& tree = bp.tree;
    tree.assign(2 * (size_t)leaves, kFull);
    for (int k = 0; k < groups; ++k) tree[(size_t)leaves + k] = (uint64_t)k;
    for (int n = leaves - 1; n >= 1; --n) tree[n] = std::min(tree[2 * n], tree[2 * n + 1]);
    for (int i = 0; i < nunits; ++i) {
      const uint64_t top = tree[1];
      if (top == kFull) return false;
      const int k = (int)(top & 0xFFFFFFFFu);
      bp.bin_of[i] = k;
      const int count = ++bp.bin_start[k + 1];
      size_t n = (size_t)leaves + k;
      uint64_t v = (h < pa::kBalWaves || count < pa::kBalMaxSeg)
                       ? (((top >> 32) + (uint64_t)units[i].pages) << 32) | (uint64_t)k
                       : kFull;
      tree[n] = v;
      for (; n > 1; n >>= 1) {                       // the path to the root
        v = std::min(v, tree[n ^ 1]);
        tree[n >> 1] = v;
      }
    }
  }
  // each work-group's units, in the order they were packed
  for (int k = 0; k < groups; ++k) bp.bin_start[k + 1] += bp.bin_start[k];
  bp.bin_units.resize(nunits);
  {
    std::vector<int> fill(bp.bin_start.begin(), bp.bin_start.end() - 1);
    for (int i = 0; i < nunits; ++i) bp.bin_units[fill[bp.bin_of[i]]++] = i;
  }
  auto add = [&](int k, int lane, const BalUnit& u, int p0, int p1) {
    for (int i = 0; i < h; ++i) {
      const size_t w = (size_t)k * pa::kBalWaves + lane * h + i;
      if (bp.nseg[w] >= pa::kBalMaxSeg) return false;
      bp.at(w)[bp.nseg[w]++] = {u.b, u.g0 + i, p0, p1, lens[u.b], 0, 0, 0};
    }
    return true;
  };
  for (int k = 0; k < groups; ++k) {
    const int* bin = bp.bin_units.data() + bp.bin_start[k];
    const int nb = bp.bin_start[k + 1] - bp.bin_start[k];
    int64_t load = 0;
    for (int j = 0; j < nb; ++j) load += units[bin[j]].pages;
    if (load == 0) continue;
    if (h == pa::kBalWaves) {
      if (load > pa::kBalMaxPages) return false;
      for (int j = 0; j < nb; ++j)
        if (!add(k, 0, units[bin[j]], 0, units[bin[j]].pages)) return false;
      continue;
    }
    const int per = (int)std::max<int64_t>((load + lanes - 1) / lanes, kBalMinChunk);
    if (per > pa::kBalMaxPages) return false;
    // long units (more than half a lane's share) first, each followed by a
    // turn of the short ones, so that the short ones spread over the lanes
    // instead of piling into the last: run r is the r-th long unit, then the
    // short units r, r + runs, r + 2 runs, ... (one run of short units alone
    // when no unit is long)
    bp.longs.clear();
    bp.shorts.clear();
    for (int j = 0; j < nb; ++j)
      (2 * units[bin[j]].pages > per ? bp.longs : bp.shorts).push_back(bin[j]);
    const int runs = std::max((int)bp.longs.size(), 1);
    bp.order.clear();
    for (int r = 0; r < runs; ++r) {
      if (r < (int)bp.longs.size()) bp.order.push_back(bp.longs[r]);
      for (size_t j = (size_t)r; j < bp.shorts.size(); j += (size_t)runs)
        bp.order.push_back(bp.shorts[j]);
    }
    // the units end to end, cut at every multiple of per (lane: the one
    // holding page `cursor`, lane_end: its end)
    int64_t cursor = 0, lane_end = per;
    int lane = 0;
    for (const int ui : bp.order) {
      const BalUnit& u = units[ui];
      int p = 0;
      if (cursor == lane_end) {
        ++lane;
        lane_end += per;
      }
      const int first_lane = lane;
      while (p < u.pages) {
        if (cursor == lane_end) {
          ++lane;
          lane_end += per;
        }
        const int take = (int)std::min<int64_t>(u.pages - p, lane_end - cursor);
        if (!add(k, lane, u, p, p + take)) return false;
        p += take;
        cursor += take;
      }
      const int last_lane = lane;
      if (last_lane > first_lane) {
        for (int i = 0; i < h; ++i) {
          const size_t w0 = (size_t)k * pa::kBalWaves + first_lane * h + i;
          BalSeg& f = bp.at(w0)[bp.nseg[w0] - 1];
          f.kind = 1;
          f.pieces = last_lane - first_lane + 1;
          f.stride = h;
          for (int l = first_lane + 1; l <= last_lane; ++l)
            bp.at((size_t)k * pa::kBalWaves + l * h + i)[0].kind = 2;
        }
      }
    }
  }
  // idle sequences: a zero-row segment each, on the wavefront with the fewest
  // segments, after a later piece and before a first piece
  for (int b : idle) {
    size_t best = 0;
    for (size_t w = 1; w < nw; ++w)
      if (bp.nseg[w] < bp.nseg[best]) best = w;
    const int n = bp.nseg[best];
    if (n >= pa::kBalMaxSeg) return false;
    BalSeg* v = bp.at(best);
    int at = n;
    if (n > 0 && v[n - 1].kind == 1) at = n - 1;
    if (at == 0 && n > 0 && v[0].kind == 2) at = 1;
    for (int j = n; j > at; --j) v[j] = v[j - 1];
    v[at] = {b, 8, 0, 0, 0, 0, 0, 0};
    ++bp.nseg[best];
  }
  for (size_t w = 0; w < nw; ++w) {
    int pages = 0;
    for (int j = 0; j < bp.nseg[w]; ++j) pages += bp.at(w)[j].p1 - bp.at(w)[j].p0;
    if (pages > pa::kBalMaxPages) return false;
  }
  return true;
}

int balance_plan(const pa_shape* shape, int batch, const int32_t* lens, int max_seq_len, int cus,
                 int h, BalPlan& bp) {
  if (h != 1 && h != 2 && h != 4 && h != 8) return PA_ERR_VALUE;
  std::vector<BalUnit> units;
  std::vector<int> idle;
  units.reserve((size_t)batch * (pa::kBalKvHeads / h));
  for (int b = 0; b < batch; ++b) {
    const int L = lens[b];
    if (L < 0 || L > max_seq_len) return PA_ERR_VALUE;
    const int np = ceil_div(L, pa::kBalPageTokens);
    if (np > shape->max_blocks_per_seq) return PA_ERR_VALUE;
    if (np == 0) {
      idle.push_back(b);
      continue;
    }
    for (int g = 0; g < pa::kBalKvHeads; g += h) units.push_back({b, g, np});
  }
  // longest first, in batch order among equals (a counting sort by pages)
  int maxp = 0;
  for (const BalUnit& u : units) maxp = std::max(maxp, u.pages);
  if (maxp > (1 << 16)) {
    std::stable_sort(units.begin(), units.end(),
                     [](const BalUnit& x, const BalUnit& y) { return x.pages > y.pages; });
  } else {
    std::vector<int> start((size_t)maxp + 2, 0);
    for (const BalUnit& u : units) ++start[(size_t)(maxp - u.pages) + 1];
    for (int p = 0; p <= maxp; ++p) start[(size_t)p + 1] += start[p];
    std::vector<BalUnit> sorted(units.size());
    for (const BalUnit& u : units) sorted[start[(size_t)(maxp - u.pages)]++] = u;
    units.swap(sorted);
  }
  int64_t total = 0;                                  // page-units over the lanes
  for (const BalUnit& u : units) total += u.pages;
  if (total >= ((int64_t)1 << 31)) return PA_ERR_VALUE;   // loads are 32-bit tree keys
  const int nunits = (int)units.size();
  const int lanes = pa::kBalWaves / h;
  int groups = std::max(1, std::min(cus, std::max(nunits, 1)));
  const int64_t need = (total + (int64_t)lanes * pa::kBalMaxPages - 1) /
                       ((int64_t)lanes * pa::kBalMaxPages);
  groups = (int)std::max<int64_t>(groups, need);
  const int limit = std::max(nunits, (int)((idle.size() + pa::kBalMaxSeg - 1) / pa::kBalMaxSeg) + 1);
  while (!balance_attempt(units, idle, lens, groups, h, bp)) {
    if (groups >= limit || groups > (1 << 20)) return PA_ERR_VALUE;
    groups = std::min<int64_t>((int64_t)groups * 2, limit);
  }
  return PA_OK;
}

int64_t plan_words(int groups) {
  return pa::kBalHeader + (int64_t)groups * pa::kBalWaves * pa::kBalDesc;
}

// The plan as the kernel reads it (every word written, unused ones zero).
void write_plan(const BalPlan& bp, const pa_shape* shape, int batch, int h, int32_t* plan) {
  std::fill(plan, plan + pa::kBalHeader, 0);
  plan[0] = pa::kBalMagic;
  plan[1] = bp.groups;
  plan[2] = batch;
  plan[3] = shape->max_blocks_per_seq;
  plan[4] = pa::kBalMaxSeg;
  plan[5] = h;
  const size_t nw = (size_t)bp.groups * pa::kBalWaves;
  for (size_t w = 0; w < nw; ++w) {
    int32_t* d = plan + pa::kBalHeader + w * pa::kBalDesc;
    const BalSeg* v = bp.seg.data() + w * pa::kBalMaxSeg;
    const int n = bp.nseg[w];
    int pages = 0;
    for (int j = 0; j < n; ++j) {
      int32_t* e = d + 8 + 8 * j;
      e[0] = v[j].b;
      e[1] = v[j].g;
      e[2] = v[j].p0;
      e[3] = v[j].p1;
      e[4] = v[j].L;
      e[5] = v[j].kind;
      e[6] = v[j].pieces;
      e[7] = v[j].stride;
      pages += v[j].p1 - v[j].p0;
    }
    d[0] = n;
    d[1] = pages;
    std::fill(d + 2, d + 8, 0);
    std::fill(d + 8 + 8 * n, d + pa::kBalDesc, 0);
  }
}

}  // namespace pa_host

using namespace pa_host;

PA_API int pa_balance_plan(const pa_shape* shape, int32_t batch, const int32_t* seq_lens_host,
                           int32_t max_seq_len, int32_t num_cus, int32_t heads_together,
                           int32_t* plan, int64_t capacity_words, int64_t* words_out,
                           int32_t* groups_out) {
  int rc = check_decode_sizes(shape, batch, max_seq_len);
  if (rc != PA_OK) return rc;
  if (!words_out || !groups_out || (batch > 0 && !seq_lens_host)) return PA_ERR_NULL;
  if (num_cus < 0 || capacity_words < 0) return PA_ERR_VALUE;
  int cu = num_cus;
  if (cu == 0 && (rc = current_cu_count(&cu)) != PA_OK) return rc;
  static thread_local BalPlan bp;
  rc = balance_plan(shape, batch, seq_lens_host, max_seq_len, cu, heads_together, bp);
  if (rc != PA_OK) return rc;
  const int64_t words = plan_words(bp.groups);
  *words_out = words;
  *groups_out = bp.groups;
  if (plan) {
    if (capacity_words < words) return PA_ERR_VALUE;
    write_plan(bp, shape, batch, heads_together, plan);
  }
  return PA_OK;
}
