// Balanced launch of the paged GQA decode: one wavefront per (sequence, KV
// head) stream, whole streams packed into work-groups on the host, the
// pieces of a stream split over the wavefronts of its work-group merged in
// LDS.  The page arithmetic (scores on the matrix cores, the FP32 online
// softmax, P V) is that of pa_decode_kernel.h; only the spreading of the work
// differs.  See include/pa_decode_balanced.h for the contract.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <queue>
#include <utility>
#include <vector>

#include "pa_decode.h"
#include "pa_decode_balanced.h"
#include "pa_measure.h"
#include "pa_host.h"
#include "pa_balance_plan.h"
#include "pa_decode_kernel.h"

#define PA_API extern "C" __attribute__((visibility("default")))

namespace pa {

constexpr int kBalSegBlk = 1024;
static_assert(kBalPageTokens == kPage && kBalKvHeads == kHkv && kBalWaves == kWaves,
              "the planner's geometry is the kernel's");

struct BalancedArgs {
  const uint16_t* q;
  const void* k_pool;
  const void* v_pool;
  const float* kv_scales;
  const uint16_t* k_new;
  const uint16_t* v_new;
  void* k_pool_w;
  void* v_pool_w;
  float* kv_scales_w;
  const float* rope_cos;
  const float* rope_sin;
  int32_t rope_positions;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  void* out;
  const int32_t* plan;
  float xscale;
  int32_t num_pages;
  int32_t max_blocks;
  int32_t max_seq_len;
  int32_t batch;
};

// Timeline launch: per wavefront, the real-time counter at kStampTimes points
// of its work, then one word naming where it ran and how much it read.
constexpr int kStampWords = 8;
constexpr int kStampTimes = 7;

// LDS reads and writes that the compiler does not see as LDS accesses (it
// would wait for every direct-to-LDS page load in flight before one); a read
// waits for itself in the same instruction group.
__device__ __forceinline__ u32x4 lds_read16_now(uint32_t addr) {
  u32x4 v;
  asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
__device__ __forceinline__ uint32_t lds_read4_now(uint32_t addr) {
  uint32_t v;
  asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(addr) : "memory");
  return v;
}
__device__ __forceinline__ void lds_store8(uint32_t addr, u32x2 v) {
  asm volatile("ds_write_b64 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_store4u(uint32_t addr, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}

// The kernel body.  STAMPS: also read the real-time counter at the points of
// a wavefront's work that the timeline launch reports (the page arithmetic
// and every memory access are those of the plain launch).
template <int FMT, bool OUT_BF16, bool APPEND, bool ROPE, int RING, bool STAMPS>
__device__ __forceinline__ void balanced_body(const BalancedArgs& a, uint64_t* stamps) {
  static_assert(!ROPE || APPEND, "RoPE is fused with the append");
  constexpr bool Q8 = FMT == kFmtINT8;
  constexpr bool Q4 = FMT == kFmtINT4;
  constexpr bool QUANT = Q8 || Q4;
  using F = PageFormat<FMT>;
  using PageT = std::conditional_t<Q8, PageQ8, std::conditional_t<Q4, PageQ4, PageBF16>>;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int G = lane >> 4;
  const int n = lane & 15;
  uint64_t stamp[kStampTimes] = {};
  auto mark = [&stamp](int k) {
    if constexpr (STAMPS) stamp[k] = __builtin_amdgcn_s_memrealtime();
  };
  mark(0);                                       // start

  // RING: slots per wavefront for this launch (0: the format's default)
  constexpr int kDepth = RING > 0 ? RING : F::kRingDepth;
  constexpr bool kPairs = F::kPairs && kDepth >= 3;
  __shared__ __attribute__((aligned(16))) char ring[kDepth][kWaves][F::kSlot];
  // per segment: [q rows of its 4 heads (512 B) | new K row, new V row (256 B)
  // | RoPE cos, sin rows (256 B)]; after its pages, its staged output
  __shared__ __attribute__((aligned(16))) char segblk[kWaves][8][kBalSegBlk];
  // the new rows as the append stores them (RoPE applied; codes and scales)
  __shared__ __attribute__((aligned(16))) char newrows[kWaves][8][256];
  __shared__ float segml[kWaves][8][8];          // per segment: m, then l, of heads 0..3

  // ---- the wavefront's descriptor (one word per lane)
  const int32_t* desc = a.plan + kBalHeader + ((int64_t)blockIdx.x * kWaves + wave) * kBalDesc;
  const int dv = desc[lane];
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  mark(1);                                       // descriptor in
  auto dw = [&](int i) { return __builtin_amdgcn_readlane(dv, i); };
  int nseg = dw(0);
  int U = dw(1);
  {
    bool ok = nseg >= 0 && nseg <= kBalMaxSeg && U >= 0 && U <= kBalMaxPages;
    int cum = 0;
    for (int j = 0; ok && j < nseg; ++j) {
      const int b = dw(8 + 8 * j), g = dw(9 + 8 * j), p0 = dw(10 + 8 * j), p1 = dw(11 + 8 * j);
      const int L = dw(12 + 8 * j), kind = dw(13 + 8 * j), pieces = dw(14 + 8 * j);
      const int stride = dw(15 + 8 * j);
      ok = (unsigned)b < (unsigned)a.batch && (unsigned)g <= 8u && p0 >= 0 && p0 <= p1 &&
           p1 <= a.max_blocks && L >= 0 && (unsigned)kind <= 2u &&
           (g < 8 ? p0 < p1 : (p1 == 0 && kind == 0)) &&
           (kind != 1 || (pieces >= 2 && stride >= 1 && stride <= kWaves &&
                          wave + (pieces - 1) * stride < kWaves && j == nseg - 1)) &&
           (kind != 2 || j == 0);
      cum += p1 - p0;
    }
    if (!ok || cum != U) {             // a plan this kernel cannot follow: nothing is read
      nseg = 0;
      U = 0;
    }
  }

  // ---- everything that depends on the descriptor only, requested together
  // lengths: lane j holds segment j's device length
  const int my_b = __shfl(dv, 8 + 8 * min(lane, kBalMaxSeg - 1));
  const int lenv = a.seq_lens[(unsigned)my_b < (unsigned)a.batch ? my_b : 0];
  // page ids: lane t, word c holds page 64 c + t of the wavefront's stream
  int raw[kBalMaxPages / 64], segof[kBalMaxPages / 64], gof[kBalMaxPages / 64];
#pragma unroll
  for (int c = 0; c < kBalMaxPages / 64; ++c) {
    const int u = 64 * c + lane;
    int jj = 0, start = 0, st = 0;
    for (int j = 0; j < nseg; ++j) {
      const int len = dw(11 + 8 * j) - dw(10 + 8 * j);
      if (u >= st) { jj = j; start = st; }
      st += len;
    }
    int bb = nseg > 0 ? dw(8) : 0, p0 = 0, g = 0;
    for (int j = 0; j < nseg; ++j)
      if (jj == j) { bb = dw(8 + 8 * j); p0 = dw(10 + 8 * j); g = dw(9 + 8 * j); }
    const int page = p0 + (u - start);
    const bool valid = u < U && g < 8 && page < a.max_blocks;
    segof[c] = jj;
    gof[c] = g & 7;
    raw[c] = (c * 64 < U) ? a.block_tables[(int64_t)bb * a.max_blocks + (valid ? page : 0)] : 0;
    if (!valid) segof[c] = -1;
  }
  // q rows, new rows and RoPE rows of every segment, straight into LDS: one
  // 16-byte request per lane and segment (lanes 0..31 the 512 bytes of q,
  // 32..47 the K and V rows, 48..63 the cos and sin rows)
  for (int j = 0; j < nseg; ++j) {
    const int b = dw(8 + 8 * j), g = min(dw(9 + 8 * j), 7), L = dw(12 + 8 * j);
    const char* src = reinterpret_cast<const char*>(a.q) + ((int64_t)b * kHq + kGroup * g) * kD * 2 +
                      16 * (lane & 31);
    if (APPEND && lane >= 32 && lane < 48) {
      const uint16_t* row = (lane < 40 ? a.k_new : a.v_new) + ((int64_t)b * kHkv + g) * kD;
      src = reinterpret_cast<const char*>(row) + 16 * (lane & 7);
    }
    if (ROPE && lane >= 48) {
      const int pos = min(max(L - 1, 0), a.rope_positions - 1);
      const float* row = (lane < 56 ? a.rope_cos : a.rope_sin) + (int64_t)pos * (kD / 2);
      src = reinterpret_cast<const char*>(row) + 16 * (lane & 7);
    }
    __builtin_amdgcn_global_load_lds(src, &segblk[wave][j][0], 16, 0, 0);
  }
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  mark(2);                                       // lengths, page ids, q rows in

  // ---- segments a plan cannot hold: wrong device length, beyond the
  // declared bound or the table, or a used page id outside the pool
  // (page ids travel as id * 8 + KV head, bit 31 set for an id outside the pool)
  uint32_t lane_bad = 0;
  int ent[kBalMaxPages / 64];
#pragma unroll
  for (int c = 0; c < kBalMaxPages / 64; ++c) {
    const bool okp = (unsigned)raw[c] < (unsigned)a.num_pages;
    if (segof[c] >= 0 && !okp) lane_bad |= 1u << segof[c];
    ent[c] = (int)((uint32_t)((okp ? raw[c] : 0) << 3) | (uint32_t)gof[c] | (okp ? 0u : 0x80000000u));
  }
  // seg_bad: NaN rows (wrong device length, beyond the declared bound or the
  // table, a page outside the pool); len_bad: also no append (the plan's
  // slot is not the sequence's)
  uint32_t seg_bad = 0, len_bad = 0;
  for (int j = 0; j < nseg; ++j) {
    const int g = dw(9 + 8 * j), p1 = dw(11 + 8 * j), L = dw(12 + 8 * j);
    const int Ld = __builtin_amdgcn_readlane(lenv, j);
    const int nL = (L + kPage - 1) / kPage;
    const bool lb = Ld != L || nL > a.max_blocks || (g < 8 && p1 > nL);
    bool bad = lb || L > a.max_seq_len;
    bad |= __builtin_amdgcn_ballot_w64(((lane_bad >> j) & 1u) != 0) != 0;
    if (bad) seg_bad |= 1u << j;
    if (lb) len_bad |= 1u << j;
  }

  // ---- the page stream (all segments' pages back to back)
  const char* k_base = reinterpret_cast<const char*>(a.k_pool);
  const char* v_base = reinterpret_cast<const char*>(a.v_pool);
  const char* s_base = reinterpret_cast<const char*>(a.kv_scales);
  // the lane offsets of head 0; each stream entry names its head
  const PageDma dma = page_dma<FMT>(0, lane, k_base, v_base);
  // bytes between KV heads in a page: codes, scale lines
  constexpr uint32_t g_step = Q8 ? kHeadCodes : Q4 ? kHeadCodes4 : 2 * kD;
  constexpr uint32_t g_step_s = QUANT ? 2 * kPage * 4 : 0;
  auto packed = [&](int u) -> uint32_t {
    uint32_t v = (uint32_t)__builtin_amdgcn_readlane(ent[0], u & 63);
#pragma unroll
    for (int c = 1; c < kBalMaxPages / 64; ++c)
      if ((u >> 6) == c) v = (uint32_t)__builtin_amdgcn_readlane(ent[c], u & 63);
    return v;
  };
  auto fetch = [&](int u, int slot) {
    const uint32_t v = packed(u);
    const int64_t id = (v >> 3) & 0x0FFFFFFFu;
    const uint32_t gg = v & 7u;
    page_fetch<FMT>(dma, k_base, v_base, s_base, id, gg * g_step, gg * g_step_s,
                    &ring[slot][wave][0]);
  };
#pragma unroll
  for (int r = 0; r < kDepth; ++r)
    if (r < U) fetch(r, r);

  // LDS read addresses of this lane in slot 0 (as in the grid kernel)
  const uint32_t slot0 = lds_address(&ring[0][wave][0]);
  constexpr uint32_t kRingSlotBytes = kWaves * F::kSlot;
  const int jq = n >> 2, jr = n & 3;
  uint32_t ka = 0, va = 0, sa = 0;
  SlotAddrBF16 ad{};
  if constexpr (Q8) {
    ka = slot0 + 64 * n + 8 * G;
    va = slot0 + 1024 + 64 * (4 * G + jq) + 8 * jr;
    sa = slot0 + 2048 + 4 * (4 * G + (n & 3));
  } else if constexpr (Q4) {
    ka = slot0 + 32 * n + 8 * G;
    va = slot0 + 512 + 32 * (4 * G + jq) + 8 * jr;
    sa = slot0 + 1024 + 4 * (4 * G + (n & 3));
  } else {
    ad.k0 = slot0 + bf16_slot_offset(n, G);
    ad.k1 = slot0 + bf16_slot_offset(n, G + 4);
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
      ad.v[bb] = slot0 + 2048 + bf16_slot_offset(4 * G + jq, 2 * bb + (jr >> 1)) + 8 * (jr & 1);
  }
  auto lds_read = [&](PageT& pg, uint32_t off) {
    if constexpr (QUANT) lds_page_issue(pg, ka + off, va + off, sa + off);
    else lds_page_issue(pg, ad, off);
  };

  PageConsts pc;
  pc.xscale = a.xscale;
  pc.qbias = 0.f;
  pc.sel = (n & 1) ? 0x07060302u : 0x05040100u;
  if constexpr (Q4) pc.nib = nibble_consts();
  bf16x8_t qlo, qhi;
  LaneState st;

  auto of_head = [G](float v) {                  // v of head G (from lane 4G)
    const float v0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float v1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 4));
    const float v2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 8));
    const float v3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 12));
    return G == 0 ? v0 : (G == 1 ? v1 : (G == 2 ? v2 : v3));
  };
  auto head_sum = [](float v) {
    v += dpp_mov<0xB1>(v);
    v += dpp_mov<0x4E>(v);
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
  };

  int u = 0;                                      // pages consumed so far
  for (int j = 0; j < nseg; ++j) {
    const int g = dw(9 + 8 * j);
    if (g == 8) continue;                         // an idle sequence: rows written at the end
    const int p0 = dw(10 + 8 * j), p1 = dw(11 + 8 * j), L = dw(12 + 8 * j);
    const int kind = dw(13 + 8 * j);
    const bool bad = (seg_bad >> j) & 1u;
    const int npg = p1 - p0;
    const int nL = (L + kPage - 1) / kPage;
    const bool ends = p1 == nL;                   // holds the stream's last page
    const int tail_valid = L - (nL - 1) * kPage;
    // the append follows the separate append's rule: written when the target
    // page id lies in the pool (the length being the plan's)
    const bool app = APPEND && ends && !((len_bad >> j) & 1u) && !(packed(u + npg - 1) >> 31);
    const int app_slot = (L - 1) % kPage;
    const uint32_t blk = lds_address(&segblk[wave][j][0]);
    const uint32_t nrow = lds_address(&newrows[wave][j][0]);

    // the query operand of this stream's 4 heads (lane 16 G + n: head 4g +
    // n/4, dims {8G..} and {32+8G..})
    {
      const uint32_t qa = blk + (uint32_t)(n >> 2) * 128 + 16 * G;
      const u32x4 l4 = lds_read16_now(qa), h4 = lds_read16_now(qa + 64);
      uint4 lo = make_uint4(l4.x, l4.y, l4.z, l4.w), hi = make_uint4(h4.x, h4.y, h4.z, h4.w);
      if (ROPE) {
        const u32x4 c0 = lds_read16_now(blk + 768 + 32 * G), c1 = lds_read16_now(blk + 768 + 32 * G + 16);
        const u32x4 s0 = lds_read16_now(blk + 896 + 32 * G), s1 = lds_read16_now(blk + 896 + 32 * G + 16);
        const float cs[8] = {__uint_as_float(c0.x), __uint_as_float(c0.y), __uint_as_float(c0.z),
                             __uint_as_float(c0.w), __uint_as_float(c1.x), __uint_as_float(c1.y),
                             __uint_as_float(c1.z), __uint_as_float(c1.w)};
        const float sn[8] = {__uint_as_float(s0.x), __uint_as_float(s0.y), __uint_as_float(s0.z),
                             __uint_as_float(s0.w), __uint_as_float(s1.x), __uint_as_float(s1.y),
                             __uint_as_float(s1.z), __uint_as_float(s1.w)};
        rope_pairs8(lo, hi, cs, sn);
      }
      if constexpr (Q4) {
        q4_relayout(lo, hi, lane);
        float bias = q4_bias_part(lo, hi);
        bias += __shfl_xor(bias, 16);
        bias += __shfl_xor(bias, 32);
        pc.qbias = bias;
        lo = interleave_halves8(lo);
        hi = interleave_halves8(hi);
      }
      qlo = __builtin_bit_cast(bf16x8_t, lo);
      qhi = __builtin_bit_cast(bf16x8_t, hi);
    }
    // the new rows (lane c: K parts {8c..}, {32+8c..}; lane 4 + c: V), RoPE
    // on K, quantised for quantised pages, kept for the park and the append
    if (app && lane < 8) {
      const int c = lane & 3;
      const bool is_k = lane < 4;
      const uint32_t src = blk + 512 + (is_k ? 0 : 128) + 16 * c;
      const u32x4 l4 = lds_read16_now(src), h4 = lds_read16_now(src + 64);
      uint4 lo = make_uint4(l4.x, l4.y, l4.z, l4.w), hi = make_uint4(h4.x, h4.y, h4.z, h4.w);
      if (ROPE && is_k) {
        const u32x4 c0 = lds_read16_now(blk + 768 + 32 * c), c1 = lds_read16_now(blk + 768 + 32 * c + 16);
        const u32x4 s0 = lds_read16_now(blk + 896 + 32 * c), s1 = lds_read16_now(blk + 896 + 32 * c + 16);
        const float cs[8] = {__uint_as_float(c0.x), __uint_as_float(c0.y), __uint_as_float(c0.z),
                             __uint_as_float(c0.w), __uint_as_float(c1.x), __uint_as_float(c1.y),
                             __uint_as_float(c1.z), __uint_as_float(c1.w)};
        const float sn[8] = {__uint_as_float(s0.x), __uint_as_float(s0.y), __uint_as_float(s0.z),
                             __uint_as_float(s0.w), __uint_as_float(s1.x), __uint_as_float(s1.y),
                             __uint_as_float(s1.z), __uint_as_float(s1.w)};
        rope_pairs8(lo, hi, cs, sn);
      }
      if constexpr (QUANT) {
        u32x2 clo, chi;
        const float sc = quantize_quad_row<FMT>(lo, hi, clo, chi);
        lds_store16(nrow + 16 * lane, u32x4{clo.x, clo.y, chi.x, chi.y});
        if (c == 0) lds_store4(nrow + 128 + 4 * (is_k ? 0 : 1), sc);
      } else {
        // [K lo parts 0..3 | K hi parts | V lo | V hi] in 16-byte chunks
        lds_store16(nrow + 16 * ((is_k ? 0 : 8) + c), u32x4{lo.x, lo.y, lo.z, lo.w});
        lds_store16(nrow + 16 * ((is_k ? 0 : 8) + 4 + c), u32x4{hi.x, hi.y, hi.z, hi.w});
      }
    }

#pragma unroll
    for (int t = 0; t < 4; ++t) st.acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    st.m = -INFINITY;
    st.l = 0.f;
    st.wsum = 0.f;

    // overwrite the appended token's slot of the ring page with the new row
    auto park = [&](uint32_t slot_base) {
      if constexpr (QUANT) {
        using QL = QuantLayout<Q8 ? kFmtINT8 : kFmtINT4>;
        if (lane < 8) {
          const u32x4 w = lds_read16_now(nrow + 16 * lane);
          const int c = lane & 3;
          const uint32_t row = slot_base + (lane < 4 ? 0 : QL::kHead) + QL::kRow * app_slot;
          if constexpr (Q8) {
            lds_store8(row + 8 * c, u32x2{w.x, w.y});
            lds_store8(row + 32 + 8 * c, u32x2{w.z, w.w});
          } else {
            lds_store4u(row + 4 * c, w.x);
            lds_store4u(row + 16 + 4 * c, w.z);
          }
        }
        if (lane < 2)
          lds_store4u(slot_base + 2 * QL::kHead + 4 * (lane * 16 + app_slot),
                      lds_read4_now(nrow + 128 + 4 * lane));
      } else {
        if (lane < 16) {
          const u32x4 w = lds_read16_now(nrow + 16 * lane);
          const int row = lane >> 2;             // 0 K lo, 1 K hi, 2 V lo, 3 V hi
          lds_store16(slot_base + 2048 * (row >> 1) + bf16_slot_offset(app_slot, 4 * (row & 1) + (lane & 3)),
                      w);
        }
      }
    };
    auto step = [&](int i, auto masked) {
      constexpr bool MASK = decltype(masked)::value;
      const int slot = u % kDepth;
      const uint32_t off = slot * kRingSlotBytes;
      wait_page<F::kLoads, kDepth>(min(U - 1 - u, kDepth - 1));
      if (u == 0) mark(3);                         // first page in LDS
      if (MASK && app) park(slot0 + off);
      PageT cur;
      lds_read(cur, off);
      lds_page_ready(cur);
      if (u + kDepth < U) fetch(u + kDepth, slot);
      consume_page<FMT, MASK>(st, cur, qlo, qhi, pc, lane, MASK ? tail_valid : kPage);
      ++u;
      (void)i;
    };
    auto step2 = [&]() {
      const int slot_a = u % kDepth;
      const int slot_b = (u + 1) % kDepth;
      wait_page<F::kLoads, kDepth>(min(U - 2 - u, kDepth - 2));
      if (u == 0) mark(3);
      PageT pa_, pb_;
      lds_read(pa_, slot_a * kRingSlotBytes);
      lds_read(pb_, slot_b * kRingSlotBytes);
      lds_page_ready(pa_);
      lds_page_ready(pb_);
      if (u + kDepth < U) fetch(u + kDepth, slot_a);
      if (u + 1 + kDepth < U) fetch(u + 1 + kDepth, slot_b);
      consume_pages2<FMT>(st, pa_, pb_, qlo, qhi, pc, lane);
      u += 2;
    };
    {
      int i = 0;
      const int full = ends ? npg - 1 : npg;     // pages before a masked last one
      if constexpr (kPairs)
        for (; i + 1 < full; i += 2) step2();
      for (; i < full; ++i) step(i, std::false_type{});
      if (ends) step(i, std::true_type{});
    }

    // this segment's result: the normaliser of head n/4 over its 16 lanes;
    // lane 16 G + n takes head G's values from lane 4G
    st.l = head_sum(st.l);
    float o[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) o[t] = st.acc[t][0] + st.acc[t][1];
    if constexpr (Q4) {
      const float ws = of_head(head_sum(st.wsum));
#pragma unroll
      for (int t = 0; t < 4; ++t) o[t] -= q4_value_bias(t) * ws;
    }
    float m_out = of_head(st.m), l_out = of_head(st.l);
    if (bad) {
      m_out = __builtin_nanf("");
      l_out = __builtin_nanf("");
#pragma unroll
      for (int t = 0; t < 4; ++t) o[t] = __builtin_nanf("");
    }
    if (kind == 0) {
      const float inv = 1.f / l_out;
#pragma unroll
      for (int t = 0; t < 4; ++t) o[t] *= inv;
    } else if (lane < 16 && (lane & 3) == 0) {
      // head n/4's running maximum and normaliser (lanes 0, 4, 8, 12)
      lds_store4(lds_address(&segml[wave][j][n >> 2]), st.m);
      lds_store4(lds_address(&segml[wave][j][4 + (n >> 2)]), bad ? __builtin_nanf("") : st.l);
    }
    lds_store16(blk + 16 * lane, u32x4{__float_as_uint(o[0]), __float_as_uint(o[1]),
                                        __float_as_uint(o[2]), __float_as_uint(o[3])});
  }
  mark(4);                                       // last page consumed
  wait_vmem<0>();
  __builtin_amdgcn_s_waitcnt(0xC07F);           // lgkmcnt(0): the staged rows are in LDS

  // ---- outputs of whole streams, idle rows and the appended rows
  auto store_out = [&](int b, int g, const float* o) {
    const int64_t orow = ((int64_t)b * kHq + kGroup * g + G) * kD;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int d = out_dim<FMT>(t, n);
      if (OUT_BF16)
        reinterpret_cast<uint16_t*>(a.out)[orow + d] = (uint16_t)f32_to_bf16_rne(o[t]);
      else
        reinterpret_cast<float*>(a.out)[orow + d] = o[t];
    }
  };
  u = 0;
  for (int j = 0; j < nseg; ++j) {
    const int b = dw(8 + 8 * j), g = dw(9 + 8 * j), p0 = dw(10 + 8 * j), p1 = dw(11 + 8 * j);
    const int L = dw(12 + 8 * j), kind = dw(13 + 8 * j);
    const bool bad = (seg_bad >> j) & 1u;
    const bool lbad = (len_bad >> j) & 1u;
    if (g == 8) {
      // an idle sequence (no pages): every row of it is zero (NaN if the
      // device holds another length)
      const float fill = bad ? __builtin_nanf("") : 0.f;
      if (OUT_BF16) {
        uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + (int64_t)b * kHq * kD;
        const uint32_t f2 = f32_to_bf16_rne(fill) * 0x10001u;
        for (int k = lane; k < kHq * kD / 8; k += 64)
          reinterpret_cast<uint4*>(o)[k] = make_uint4(f2, f2, f2, f2);
      } else {
        float* o = reinterpret_cast<float*>(a.out) + (int64_t)b * kHq * kD;
        for (int k = lane; k < kHq * kD / 4; k += 64)
          reinterpret_cast<float4*>(o)[k] = make_float4(fill, fill, fill, fill);
      }
      continue;
    }
    const int npg = p1 - p0;
    const int nL = (L + kPage - 1) / kPage;
    if (kind == 0) {
      const float4 v = *reinterpret_cast<const float4*>(&segblk[wave][j][16 * lane]);
      const float o[4] = {v.x, v.y, v.z, v.w};
      store_out(b, g, o);
    }
    const uint32_t last_v = npg > 0 ? packed(u + npg - 1) : 0x80000000u;
    if (APPEND && p1 == nL && !lbad && !(last_v >> 31)) {
      const int id = (int)((last_v >> 3) & 0x0FFFFFFFu);
      const int app_slot = (L - 1) % kPage;
      const int c = lane & 3;
      const bool is_k = lane < 4;
      if constexpr (QUANT) {
        using QL = QuantLayout<Q8 ? kFmtINT8 : kFmtINT4>;
        if (lane < 8) {
          const u32x4 w = *reinterpret_cast<const u32x4*>(&newrows[wave][j][16 * lane]);
          uint8_t* row = reinterpret_cast<uint8_t*>(is_k ? a.k_pool_w : a.v_pool_w) +
                         (int64_t)id * QL::kPageBytes + g * QL::kHead + app_slot * QL::kRow;
          store_quad_codes<FMT>(row, c, u32x2{w.x, w.y}, u32x2{w.z, w.w});
          if (c == 0)
            a.kv_scales_w[(int64_t)id * kScalePageFloats + (g * 2 + (is_k ? 0 : 1)) * kPage + app_slot] =
                *reinterpret_cast<const float*>(&newrows[wave][j][128 + 4 * (is_k ? 0 : 1)]);
        }
      } else if (lane < 16) {
        const u32x4 w = *reinterpret_cast<const u32x4*>(&newrows[wave][j][16 * lane]);
        const int row = lane >> 2;               // 0 K lo, 1 K hi, 2 V lo, 3 V hi
        uint16_t* dst = reinterpret_cast<uint16_t*>(row < 2 ? a.k_pool_w : a.v_pool_w) +
                        (int64_t)id * kPageElems + app_slot * kRowElems + g * kD +
                        32 * (row & 1) + 8 * (lane & 3);
        *reinterpret_cast<u32x4*>(dst) = w;
      }
    }
    u += npg;
  }

  // ---- streams split over wavefronts: the wavefront holding the first
  // piece (its last segment) merges the pieces in wavefront order
  __syncthreads();
  if (nseg > 0) {
    const int j = nseg - 1;
    if (dw(13 + 8 * j) == 1) {
      const int b = dw(8 + 8 * j), g = dw(9 + 8 * j), pieces = dw(14 + 8 * j);
      const int stride = dw(15 + 8 * j);
      float M = -INFINITY;
      for (int i = 0; i < pieces; ++i) {
        const int w = wave + i * stride, s = i == 0 ? j : 0;
        M = fmaxf(M, segml[w][s][G]);
      }
      float num[4] = {0.f, 0.f, 0.f, 0.f}, den = 0.f;
      for (int i = 0; i < pieces; ++i) {
        const int w = wave + i * stride, s = i == 0 ? j : 0;
        const float wgt = __builtin_amdgcn_exp2f(segml[w][s][G] - M);
        den += wgt * segml[w][s][4 + G];
        const float4 v = *reinterpret_cast<const float4*>(&segblk[w][s][16 * lane]);
        num[0] += wgt * v.x;
        num[1] += wgt * v.y;
        num[2] += wgt * v.z;
        num[3] += wgt * v.w;
      }
      const float inv = 1.f / den;
      const float o[4] = {num[0] * inv, num[1] * inv, num[2] * inv, num[3] * inv};
      store_out(b, g, o);
    }
  }
  if constexpr (STAMPS) {
    mark(5);                                     // every output store issued
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    mark(6);                                     // every store acknowledged
    if (lane == 0) {
      // hardware ids: HW_ID (CU, shader array, engine) and XCC_ID (die)
      const uint32_t hw = __builtin_amdgcn_s_getreg((31 << 11) | 4);
      const uint32_t xcc = __builtin_amdgcn_s_getreg((15 << 11) | 20) & 0xFFFFu;
      uint64_t* d = stamps + ((int64_t)blockIdx.x * kWaves + wave) * kStampWords;
#pragma unroll
      for (int k = 0; k < kStampTimes; ++k) d[k] = stamp[k];
      d[kStampTimes] = (uint64_t)hw | ((uint64_t)xcc << 32) | ((uint64_t)(U & 0xFFFF) << 48);
    }
  }
}

template <int FMT, bool OUT_BF16, bool APPEND, bool ROPE, int RING = 0>
__global__ __launch_bounds__(kThreads, 2) void decode_balanced_kernel(BalancedArgs a) {
  balanced_body<FMT, OUT_BF16, APPEND, ROPE, RING, false>(a, nullptr);
}

// The same work with the timeline stamps (FP32 output, no RoPE): kStampWords
// words per wavefront.
template <int FMT, bool APPEND, int RING = 0>
__global__ __launch_bounds__(kThreads, 2) void decode_balanced_timeline_kernel(BalancedArgs a,
                                                                               uint64_t* stamps) {
  balanced_body<FMT, false, APPEND, false, RING, true>(a, stamps);
}

template <int FMT, int RING>
void launch_balanced_ring(const BalancedArgs& a, dim3 grid, bool out_bf16, bool fused, bool rope,
                          hipStream_t st) {
  const dim3 block(kThreads);
  if (out_bf16) {
    if (rope) hipLaunchKernelGGL((decode_balanced_kernel<FMT, true, true, true, RING>), grid, block, 0, st, a);
    else if (fused) hipLaunchKernelGGL((decode_balanced_kernel<FMT, true, true, false, RING>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((decode_balanced_kernel<FMT, true, false, false, RING>), grid, block, 0, st, a);
  } else {
    if (rope) hipLaunchKernelGGL((decode_balanced_kernel<FMT, false, true, true, RING>), grid, block, 0, st, a);
    else if (fused) hipLaunchKernelGGL((decode_balanced_kernel<FMT, false, true, false, RING>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((decode_balanced_kernel<FMT, false, false, false, RING>), grid, block, 0, st, a);
  }
}

template <int FMT, int RING>
void launch_timeline_ring(const BalancedArgs& a, uint64_t* stamps, dim3 grid, bool fused,
                          hipStream_t st) {
  const dim3 block(kThreads);
  if (fused) hipLaunchKernelGGL((decode_balanced_timeline_kernel<FMT, true, RING>), grid, block, 0, st, a, stamps);
  else hipLaunchKernelGGL((decode_balanced_timeline_kernel<FMT, false, RING>), grid, block, 0, st, a, stamps);
}

// two_slots (BF16 pages only): a two-slot ring instead of the default one slot;
// stamps: the kernel that also writes the timeline there (FP32 output, no
// RoPE), or NULL.
template <int FMT>
hipError_t launch_balanced(const BalancedArgs& a, int groups, bool out_bf16, bool fused, bool rope,
                           bool two_slots, uint64_t* stamps, hipStream_t st) {
  const dim3 grid(groups);
  if constexpr (FMT == kFmtBF16) {
    if (stamps) {
      if (two_slots) launch_timeline_ring<FMT, 2>(a, stamps, grid, fused, st);
      else launch_timeline_ring<FMT, 0>(a, stamps, grid, fused, st);
    } else if (two_slots) {
      launch_balanced_ring<FMT, 2>(a, grid, out_bf16, fused, rope, st);
    } else {
      launch_balanced_ring<FMT, 0>(a, grid, out_bf16, fused, rope, st);
    }
  } else {
    if (stamps) launch_timeline_ring<FMT, 0>(a, stamps, grid, fused, st);
    else launch_balanced_ring<FMT, 0>(a, grid, out_bf16, fused, rope, st);
  }
  return hipGetLastError();
}

}  // namespace pa


using namespace pa_host;


// Both balanced entry points; stamps (the timeline launch) or NULL.
static int decode_balanced_impl(const pa_shape* shape, int32_t batch, const void* q,
                                const void* k_new, const void* v_new, const pa_rope* rope,
                                void* k_pool, void* v_pool, void* kv_scales, int32_t page_format,
                                const int32_t* block_tables, const int32_t* seq_lens,
                                int32_t max_seq_len, float scale, void* out, int32_t out_dtype,
                                const int32_t* plan, int64_t plan_words, int32_t groups,
                                uint64_t* stamps, void* stream) {
  int rc = check_decode_sizes(shape, batch, max_seq_len);
  if (rc != PA_OK) return rc;
  if (out_dtype != PA_OUT_F32 && out_dtype != PA_OUT_BF16) return PA_ERR_VALUE;
  if (page_format < 0 || page_format > 2 || !std::isfinite(scale)) return PA_ERR_VALUE;
  if (batch == 0) return PA_OK;
  if (!q || !k_pool || !v_pool || !block_tables || !seq_lens || !out || !plan) return PA_ERR_NULL;
  if (page_format != 0 && !kv_scales) return PA_ERR_NULL;
  const bool fused = k_new != nullptr || v_new != nullptr;
  if (fused && (!k_new || !v_new)) return PA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k_pool, 16) || !aligned(v_pool, 16) || !aligned(out, 16) ||
      !aligned(block_tables, 4) || !aligned(seq_lens, 4) || !aligned(plan, 4) ||
      (kv_scales && !aligned(kv_scales, 16)) ||
      (fused && (!aligned(k_new, 16) || !aligned(v_new, 16))))
    return PA_ERR_ALIGN;
  if (rope) {
    if (!fused) return PA_ERR_VALUE;
    rc = check_rope(rope, max_seq_len);
    if (rc != PA_OK) return rc;
  }
  if (shape->num_pages < 1 && max_seq_len > 0) return PA_ERR_VALUE;
  // page ids travel with their KV head in one word (id * 8 + head)
  if (shape->num_pages > (1 << 28)) return PA_ERR_VALUE;
  if (groups < 1 || plan_words < pa::kBalHeader + (int64_t)groups * pa::kWaves * pa::kBalDesc)
    return PA_ERR_VALUE;
  pa::BalancedArgs a = {};
  a.q = (const uint16_t*)q;
  a.k_pool = k_pool;
  a.v_pool = v_pool;
  a.kv_scales = (const float*)kv_scales;
  a.k_new = (const uint16_t*)k_new;
  a.v_new = (const uint16_t*)v_new;
  a.k_pool_w = k_pool;
  a.v_pool_w = v_pool;
  a.kv_scales_w = (float*)kv_scales;
  a.rope_cos = rope ? rope->cos : nullptr;
  a.rope_sin = rope ? rope->sin : nullptr;
  a.rope_positions = rope ? rope->positions : 1;
  a.block_tables = block_tables;
  a.seq_lens = seq_lens;
  a.out = out;
  a.plan = plan;
  a.xscale = scale * pa::kLog2e;
  a.num_pages = shape->num_pages;
  a.max_blocks = shape->max_blocks_per_seq;
  a.max_seq_len = max_seq_len;
  a.batch = batch;
  const bool bf = out_dtype == PA_OUT_BF16;
  hipError_t e;
  // BF16 pages: two slots per wavefront when the plan leaves CUs idle (each
  // busy CU then needs more pages in flight), else one
  int cu = 0;
  const bool two_slots = current_cu_count(&cu) == PA_OK && groups < cu;
  if (page_format == 1) e = pa::launch_balanced<pa::kFmtINT8>(a, groups, bf, fused, rope != nullptr, false, stamps, (hipStream_t)stream);
  else if (page_format == 2) e = pa::launch_balanced<pa::kFmtINT4>(a, groups, bf, fused, rope != nullptr, false, stamps, (hipStream_t)stream);
  else e = pa::launch_balanced<pa::kFmtBF16>(a, groups, bf, fused, rope != nullptr, two_slots, stamps, (hipStream_t)stream);
  return e == hipSuccess ? PA_OK : PA_ERR_LAUNCH;
}

PA_API int pa_decode_balanced(const pa_shape* shape, int32_t batch, const void* q,
                              const void* k_new, const void* v_new, const pa_rope* rope,
                              void* k_pool, void* v_pool, void* kv_scales, int32_t page_format,
                              const int32_t* block_tables, const int32_t* seq_lens,
                              int32_t max_seq_len, float scale, void* out, int32_t out_dtype,
                              const int32_t* plan, int64_t plan_words, int32_t groups,
                              void* stream) {
  return decode_balanced_impl(shape, batch, q, k_new, v_new, rope, k_pool, v_pool, kv_scales,
                              page_format, block_tables, seq_lens, max_seq_len, scale, out,
                              out_dtype, plan, plan_words, groups, nullptr, stream);
}

PA_API int pa_decode_balanced_timeline(const pa_shape* shape, int32_t batch, const void* q,
                                       const void* k_new, const void* v_new, void* k_pool,
                                       void* v_pool, void* kv_scales, int32_t page_format,
                                       const int32_t* block_tables, const int32_t* seq_lens,
                                       int32_t max_seq_len, float scale, float* out,
                                       const int32_t* plan, int64_t plan_words, int32_t groups,
                                       uint64_t* stamps, int64_t stamp_words, void* stream) {
  if (!stamps) return PA_ERR_NULL;
  if (!aligned(stamps, 8)) return PA_ERR_ALIGN;
  if (groups < 1 || stamp_words < (int64_t)groups * pa::kWaves * pa::kStampWords)
    return PA_ERR_VALUE;
  return decode_balanced_impl(shape, batch, q, k_new, v_new, nullptr, k_pool, v_pool, kv_scales,
                              page_format, block_tables, seq_lens, max_seq_len, scale, out,
                              PA_OUT_F32, plan, plan_words, groups, stamps, stream);
}

PA_API int pa_wall_clock_khz(int32_t* khz) {
  if (!khz) return PA_ERR_NULL;
  int dev = 0, rate = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&rate, hipDeviceAttributeWallClockRate, dev) != hipSuccess)
    return PA_ERR_DEVICE;
  *khz = rate;
  return PA_OK;
}
