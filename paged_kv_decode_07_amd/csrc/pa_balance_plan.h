// Layout of a balanced-launch plan, shared by the host planner
// (pa_balance_plan.cpp) and the kernel that follows it
// (pa_decode_balanced.hip).
#pragma once

#include <stdint.h>

namespace pa {

// Plan layout (int32 words): a header of kBalHeader words, then one
// descriptor of kBalDesc words per wavefront, work-group by work-group.
// Descriptor: [0] segments, [1] pages, [2..7] unused; segment j (j <
// kBalMaxSeg) at 8 + 8 j: sequence b, KV head g (8: an idle sequence's zero
// rows), first page p0, end page p1, length L, kind (0 whole stream, 1 first
// piece of a split stream, 2 later piece), pieces (kind 1: how many), stride
// (kind 1: the later pieces are in wavefronts wave + stride, wave + 2 stride,
// ...).  A wavefront's first piece of a split stream is always its last
// segment, a later piece always its first.
constexpr int kBalHeader = 64;
constexpr int kBalDesc = 64;
constexpr int kBalMaxSeg = 7;
constexpr int kBalMaxPages = 256;
constexpr int32_t kBalMagic = 0x50414231;
// The geometry the planner counts in: tokens per page, KV heads, wavefronts
// per work-group (the kernel checks them against its own).
constexpr int kBalPageTokens = 16;
constexpr int kBalKvHeads = 8;
constexpr int kBalWaves = 8;

}  // namespace pa
