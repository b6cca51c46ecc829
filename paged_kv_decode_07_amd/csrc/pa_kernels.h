// Shared device code of the paged GQA decode library for gfx950 (CDNA4,
// wave64): geometry constants, BF16 and RoPE helpers, LDS and wait helpers,
// the output-row store and the split merge kernel.  The decode kernel is in
// pa_decode_kernel.h, the INT8 and INT4 page formats in pa_kernels_q8.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace pa {

constexpr int kHq = 32;
constexpr int kHkv = 8;
constexpr int kGroup = kHq / kHkv;              // 4 query heads per KV head
constexpr int kD = 64;
constexpr int kPage = 16;
constexpr int kRowElems = kHkv * kD;            // 512 BF16 = 1 KiB per token row
constexpr int kPageElems = kPage * kRowElems;   // 8192 BF16 = 16 KiB per page
constexpr int kWaves = kHkv;                    // one wavefront per KV head
constexpr int kThreads = kWaves * 64;
constexpr float kTau = 8.0f;                    // lazy-rescale threshold, log2 units
constexpr float kLog2e = 1.4426950408889634f;
// LDS page slots per wavefront, BF16 pages (build-time; the measured best).
// One slot: a page is read into registers before its slot is refilled, so the
// next page's load still overlaps this page's arithmetic, and the CU keeps
// 32 KiB in flight, where its BF16 page stream runs fastest (two slots measured
// about 1% slower on the 256 x 2048 batch, three slots 2-3% slower).
#ifndef PA_RING_DEPTH
#define PA_RING_DEPTH 1
#endif
constexpr int kRing = PA_RING_DEPTH;
constexpr int kMaxSplitPages = 256;             // longest split (4096 tokens)
static_assert(kRing >= 1 && kRing * kWaves * 4 * 1024 <= 160 * 1024, "LDS ring too large");

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two FP32 values -> a packed BF16 pair (a in the low half), rounded to
// nearest even by gfx950's v_cvt_pk_bf16_f32: one instruction, no branch.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16_rne(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}

// Round-to-nearest-even FP32 -> BF16 bits (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;   // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Rotary embedding of rotate-half pairs (x[i], x[i+32]).  Each product and
// the sum are rounded to FP32 on their own: contraction into a fused
// multiply-add is switched off here (only here), because the result is then
// rounded to BF16 and a one-ulp FP32 difference flips ties of that rounding.
// rope_pairs8: lo holds x[8c .. 8c+7], hi holds x[32+8c .. 32+8c+7] (BF16),
// cs/sn the cos/sin of their angles; the result is rounded to BF16 (RNE).
__device__ __forceinline__ float rope_first(float x1, float x2, float c, float s) {
#pragma clang fp contract(off)
  return x1 * c - x2 * s;                 // two rounded products, one rounded difference
}
__device__ __forceinline__ float rope_second(float x1, float x2, float c, float s) {
#pragma clang fp contract(off)
  return x2 * c + x1 * s;
}

__device__ __forceinline__ void rope_pairs8(uint4& lo, uint4& hi, const float* cs,
                                            const float* sn) {
  uint32_t l[4] = {lo.x, lo.y, lo.z, lo.w}, h[4] = {hi.x, hi.y, hi.z, hi.w};
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    uint32_t ol = 0, oh = 0;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      const int e = 2 * w + k;
      const float x1 = k ? bf16_hi(l[w]) : bf16_lo(l[w]);
      const float x2 = k ? bf16_hi(h[w]) : bf16_lo(h[w]);
      const float y1 = rope_first(x1, x2, cs[e], sn[e]);
      const float y2 = rope_second(x1, x2, cs[e], sn[e]);
      ol |= f32_to_bf16_rne(y1) << (16 * k);
      oh |= f32_to_bf16_rne(y2) << (16 * k);
    }
    l[w] = ol;
    h[w] = oh;
  }
  lo = make_uint4(l[0], l[1], l[2], l[3]);
  hi = make_uint4(h[0], h[1], h[2], h[3]);
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Byte address of an LDS object (what ds_read and M0 expect).
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Wait until at most N vector-memory operations of this wavefront are still
// outstanding (loads complete in issue order).
template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// s_waitcnt immediate for vmcnt(0) alone (expcnt and lgkmcnt at their
// maxima), in the gfx9 encoding: vmcnt in bits 3:0 and 15:14.
constexpr int kWaitVmcnt0 = 0x0F70;

// Wait until the oldest page of a ring has landed while the `later` pages
// requested after it (each LOADS instructions) may still be in flight;
// `later` is wave-uniform and below DEPTH (a one-slot ring waits for all).
template <int LOADS, int DEPTH, int K = DEPTH - 1>
__device__ __forceinline__ void wait_page(int later) {
  static_assert(DEPTH >= 1 && LOADS * (DEPTH - 1) <= 63, "ring depth beyond the vmcnt range");
  if constexpr (K == 0) {
    wait_vmem<0>();
  } else {
    if (later >= K) return wait_vmem<LOADS * K>();
    wait_page<LOADS, DEPTH, K - 1>(later);
  }
}

// LDS stores the compiler does not see as LDS accesses: it would otherwise
// wait for every outstanding direct-to-LDS load before them.
__device__ __forceinline__ void lds_store16(uint32_t addr, u32x4 v) {
  asm volatile("ds_write_b128 %0, %1" ::"v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ void lds_store4(uint32_t addr, float v) {
  asm volatile("ds_write_b32 %0, %1" ::"v"(addr), "v"(v) : "memory");
}

template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               CTRL, 0xF, 0xF, false));
}
template <bool OUT_BF16>
__device__ __forceinline__ void store_row16(void* out, int64_t row, int part, const float (&vals)[16]) {
  // row = b * kHq + h ; writes the 16 dims owned by `part`
  if (OUT_BF16) {
    uint16_t* o = reinterpret_cast<uint16_t*>(out) + row * kD;
    uint4 a, c;
    a.x = f32_to_bf16_rne(vals[0]) | (f32_to_bf16_rne(vals[1]) << 16);
    a.y = f32_to_bf16_rne(vals[2]) | (f32_to_bf16_rne(vals[3]) << 16);
    a.z = f32_to_bf16_rne(vals[4]) | (f32_to_bf16_rne(vals[5]) << 16);
    a.w = f32_to_bf16_rne(vals[6]) | (f32_to_bf16_rne(vals[7]) << 16);
    c.x = f32_to_bf16_rne(vals[8]) | (f32_to_bf16_rne(vals[9]) << 16);
    c.y = f32_to_bf16_rne(vals[10]) | (f32_to_bf16_rne(vals[11]) << 16);
    c.z = f32_to_bf16_rne(vals[12]) | (f32_to_bf16_rne(vals[13]) << 16);
    c.w = f32_to_bf16_rne(vals[14]) | (f32_to_bf16_rne(vals[15]) << 16);
    *reinterpret_cast<uint4*>(o + 8 * part) = a;
    *reinterpret_cast<uint4*>(o + 32 + 8 * part) = c;
  } else {
    float* o = reinterpret_cast<float*>(out) + row * kD;
    float4* p0 = reinterpret_cast<float4*>(o + 8 * part);
    float4* p1 = reinterpret_cast<float4*>(o + 32 + 8 * part);
    p0[0] = make_float4(vals[0], vals[1], vals[2], vals[3]);
    p0[1] = make_float4(vals[4], vals[5], vals[6], vals[7]);
    p1[0] = make_float4(vals[8], vals[9], vals[10], vals[11]);
    p1[1] = make_float4(vals[12], vals[13], vals[14], vals[15]);
  }
}

// What the split merge reads: lengths, the plan, the partials and the output.
struct MergeArgs {
  const int32_t* seq_lens;
  void* out;
  const float* part_acc;   // [B][S][Hq][D]
  const float* part_ml;    // [B][S][Hq][2]: running maximum (log2 units) and sum
  int32_t max_blocks;
  int32_t max_seq_len;     // host-declared bound; longer sequences are flagged
  int32_t pages_per_split;
  int32_t num_splits;      // S: splits per sequence in the grid
  int32_t preload;         // request partials before the length (small batches)
};

// Log-sum-exp merge of the splits of each multi-split sequence, in split
// order.  One work-group of 256 threads per sequence: thread = (head, 8 dims).
// Splits are read 8 at a time with all loads issued before any use, and each
// batch is absorbed once: the running maximum rises with the batch maximum
// (rescaling what was summed), then the batch's weights 2^(m_s - M) are
// added in split order.  The first 16 splits' partials (rows that exist in
// the workspace whatever the sequence's length) are requested together with
// the length when the batch is small (`preload`), so a sequence of up to 16
// splits costs one memory latency; a large batch, whose short sequences need
// no merge, requests only the splits a sequence has, after its length.
constexpr int kMergeBatch = 8;

struct MergeBatch {
  float m[kMergeBatch], l[kMergeBatch];
  float4 x0[kMergeBatch], x1[kMergeBatch];
};

// Partials of splits s0 .. s0+7 (those below `avail`; the others read split 0).
__device__ __forceinline__ void merge_load(MergeBatch& t, const MergeArgs& a, int64_t row0,
                                           int d0, int s0, int avail) {
#pragma unroll
  for (int k = 0; k < kMergeBatch; ++k) {
    const int64_t row = row0 + (int64_t)(s0 + k < avail ? s0 + k : 0) * kHq;
    const float4* src = reinterpret_cast<const float4*>(a.part_acc + row * kD + d0);
    t.m[k] = a.part_ml[row * 2];
    t.l[k] = a.part_ml[row * 2 + 1];
    t.x0[k] = src[0];
    t.x1[k] = src[1];
  }
}

// Keeps a batch's loads ahead of the code that follows: without this the
// compiler moves them after the length test's early exits, one memory
// latency later.
__device__ __forceinline__ void merge_pin(const MergeBatch& t) {
#pragma unroll
  for (int k = 0; k < kMergeBatch; ++k)
    asm volatile("" ::"v"(t.m[k]), "v"(t.l[k]), "v"(__builtin_bit_cast(f32x4_t, t.x0[k])),
                 "v"(__builtin_bit_cast(f32x4_t, t.x1[k]))
                 : "memory");
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const int b = blockIdx.x;
  const int h = threadIdx.x >> 3;
  const int d0 = (threadIdx.x & 7) * 8;
  const int64_t row0 = (int64_t)b * a.num_splits * kHq + h;   // split s at row0 + s*kHq
  MergeBatch first, second;
  const bool two = a.num_splits > kMergeBatch;   // uniform: a plan of more than 8 splits
  if (a.preload) {
    merge_load(first, a, row0, d0, 0, a.num_splits);
    if (two) merge_load(second, a, row0, d0, kMergeBatch, a.num_splits);
  }
  const int L = a.seq_lens[b];
  if (a.preload) {
    merge_pin(first);
    if (two) merge_pin(second);
  }
  const int n_pages = (L + kPage - 1) / kPage;
  if (L <= 0 || L > a.max_seq_len || n_pages > a.max_blocks ||
      n_pages > a.pages_per_split * a.num_splits)
    return;
  const int ns = (n_pages + a.pages_per_split - 1) / a.pages_per_split;
  if (ns <= 1) return;
  if (!a.preload) {
    merge_load(first, a, row0, d0, 0, ns);
    if (ns > kMergeBatch) merge_load(second, a, row0, d0, kMergeBatch, ns);
  }
  float M = -INFINITY;                           // running maximum (log2 units)
  float num[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  auto absorb = [&](const MergeBatch& t, int s0) {
    float bm = -INFINITY;
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k)
      if (s0 + k < ns) bm = fmaxf(bm, t.m[k]);
    if (bm > M) {                                // 2^(-inf) = 0 clears the empty start
      const float r = __builtin_amdgcn_exp2f(M - bm);
      den *= r;
#pragma unroll
      for (int e = 0; e < 8; ++e) num[e] *= r;
      M = bm;
    }
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      if (s0 + k >= ns) break;
      const float w = __builtin_amdgcn_exp2f(t.m[k] - M);
      den += w * t.l[k];
      num[0] += w * t.x0[k].x; num[1] += w * t.x0[k].y; num[2] += w * t.x0[k].z; num[3] += w * t.x0[k].w;
      num[4] += w * t.x1[k].x; num[5] += w * t.x1[k].y; num[6] += w * t.x1[k].z; num[7] += w * t.x1[k].w;
    }
  };
  absorb(first, 0);
  if (ns > kMergeBatch) absorb(second, kMergeBatch);    // ns > 8 implies `two`
  for (int s0 = 2 * kMergeBatch; s0 < ns; s0 += kMergeBatch) {
    MergeBatch t;
    merge_load(t, a, row0, d0, s0, ns);
    absorb(t, s0);
  }
  const float inv = 1.f / den;
  const int64_t orow = (int64_t)b * kHq + h;
  if (OUT_BF16) {
    uint16_t* o = reinterpret_cast<uint16_t*>(a.out) + orow * kD + d0;
    uint4 v;
    v.x = f32_to_bf16_rne(num[0] * inv) | (f32_to_bf16_rne(num[1] * inv) << 16);
    v.y = f32_to_bf16_rne(num[2] * inv) | (f32_to_bf16_rne(num[3] * inv) << 16);
    v.z = f32_to_bf16_rne(num[4] * inv) | (f32_to_bf16_rne(num[5] * inv) << 16);
    v.w = f32_to_bf16_rne(num[6] * inv) | (f32_to_bf16_rne(num[7] * inv) << 16);
    *reinterpret_cast<uint4*>(o) = v;
  } else {
    float4* o = reinterpret_cast<float4*>(reinterpret_cast<float*>(a.out) + orow * kD + d0);
    o[0] = make_float4(num[0] * inv, num[1] * inv, num[2] * inv, num[3] * inv);
    o[1] = make_float4(num[4] * inv, num[5] * inv, num[6] * inv, num[7] * inv);
  }
}

}  // namespace pa
