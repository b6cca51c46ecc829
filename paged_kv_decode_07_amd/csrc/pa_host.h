// Host-side helpers shared by the library's entry points (argument checks,
// device queries, split planning).  Internal to the shared library: nothing
// here is exported.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "pa_decode.h"

namespace pa_host {

bool aligned(const void* p, size_t a);
int ceil_div(int a, int b);
// Compute units of the current device (queried once per device).
int current_cu_count(int* cu);
// Fixed geometry: 32 query heads, 8 KV heads, head_dim 64, 16-token pages.
int check_shape(const pa_shape* s);
int check_decode_sizes(const pa_shape* shape, int32_t batch, int32_t max_seq_len);
int check_rope(const pa_rope* rope, int64_t needed_positions);
// Split size without sequence lengths (fixed != 0: that size, validated).
int plan_split(const pa_shape* s, int batch, int max_seq_len, int fixed, int* pages, int* splits);

// Cost model of one decode launch, used to pick the split size from host
// sequence lengths: a work-group spends group_us on fixed costs, then
// streams its pages, all streaming work-groups sharing the HBM bandwidth
// equally but none faster than one CU alone (page_us per page of page_bytes
// bytes); empty grid slots cost empty_us; a multi-split plan adds the merge.
// The defaults were fitted to the BF16 kernel on MI355X over batch 8 .. 512
// and split sizes 8 .. 128.
// Up to `resident` work-groups may share a CU; a CU holding more than one
// streams shared_gain times the pages of one work-group alone (more waves
// per SIMD hide more of each page's latency).
struct PlanModel {
  double page_us = 0.6, group_us = 3.0, empty_us = 0.5, merge_us = 8.0;
  double hbm_bytes_per_us = 6.6e6;
  double page_bytes = 2.0 * 16 * 8 * 64 * 2;   // one K page and one V page, BF16
  int resident = 1;
  double shared_gain = 1.0;
  // a plan whose grid (batch x splits) fits the CUs at once, with splits of
  // at least kTwoWaveMinPages pages, streams two_wave_gain times faster per
  // work-group (INT4 pages: two wavefronts per KV head, for the grid and the
  // work-list launch alike)
  double two_wave_gain = 1.0;
};
// Shorter splits run one wavefront per KV head: their halves are too short to
// pay for the larger work-group and the merge of the two states (3- and
// 8-page splits measured 9% and 4% slower with two).
constexpr int kTwoWaveMinPages = 32;
// BF16 pages stream through one LDS slot per wavefront, except in a launch
// of fewer work-groups than CUs, or of one per CU with splits shorter than
// this: a two-slot ring then keeps enough pages in flight and hides the start
// of each short stream (measured: 4- and 32-page splits of 256 work-groups 4%
// faster with two slots, 64 balanced work-groups 13%; 128-page splits, and
// launches of more work-groups than CUs, 1-5% faster with one).
constexpr int kOneSlotMinPages = 64;
// worklist: the work-groups run in pa_decode_worklist's order (largest
// first, no empty slots) instead of the grid order.
double simulate_plan(const int32_t* lens, int batch, int max_seq_len, int ps, int cu, int xcds,
                     const PlanModel& m, bool worklist = false);
int plan_split_lengths(const pa_shape* s, int batch, const int32_t* lens, int max_seq_len,
                       int num_cus, const PlanModel& model, int* pages, int* splits,
                       bool worklist = false);
// The cost model fitted to the INT8-page kernel (defined with the INT8 entry points).
PlanModel plan_model_q8();
// The cost model for INT4 pages (defined with the quantised entry points).
PlanModel plan_model_q4();
// Bytes of split partials for `splits` splits per sequence (0 for one split).
size_t workspace_for(int batch, int splits);

// Work list for host lengths and a split size: one item (b, s) per split that
// holds pages, plus split 0 of every sequence without pages (its output row
// is still written), ordered by page count, largest first (ties: b, then s).
// work: host int32 [2 * capacity]; *count receives the number of items.
int build_worklist(int batch, const int32_t* lens, int max_seq_len, int ps, int32_t* work,
                   int capacity, int* count);

}  // namespace pa_host
