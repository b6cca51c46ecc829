// Device code for INT8 K/V pages (gfx950, wave64).
//
// Format: K and V codes are int8 in the BF16 pool's layout
// [num_pages][16 slots][8 KV heads][64 dims]; each (token, KV head) row of
// 64 values has its own FP32 scale, kept in a scale pool
// [num_pages][8 KV heads][2 (K, V)][16 slots] (1 KiB per page, 128 bytes per
// head).  A row is quantised symmetrically: scale = max|x| / 127 (FP32,
// correctly rounded), code = the FP32 quotient x / scale rounded to nearest
// even and clamped to [-128, 127]; an all-zero row has scale 0 and codes 0.
// The value a code stands for is code * scale.  (INT8 KV cache dequantised
// before attention and the symmetric quantiser: "Building an LLM inference
// engine from scratch: KV cache, operator fusion and quantisation practice",
// sections 5.1 and 3.4.)
//
// The decode kernel keeps the BF16 kernel's decomposition (one work-group per
// (sequence, split), wavefront g = KV head g, lane = 16 * part + token) and
// its arithmetic, with three changes:
//   * a page costs 17 KiB instead of 32 KiB; each wavefront's LDS ring slot
//     takes its 1 KiB of K codes, 1 KiB of V codes (16 token rows of 64
//     bytes each) and its 128-byte line of scales, in three direct-to-LDS
//     loads, and the ring is twice as deep for the same bytes in flight;
//   * K codes are widened to BF16 (exact: |code| <= 128 needs 8 significant
//     bits) for the same two matrix-core products per page; the K scale of
//     the lane's token joins the score multiplier: x = (q.code) * (scale *
//     log2 e * k_scale), i.e. the score of the dequantised key;
//   * V codes are widened to FP32 and the V scale joins the weight: acc +=
//     (p * v_scale) * code, while the normaliser sums p alone.
#pragma once

#include "pa_kernels.h"

namespace pa {

constexpr int kRowCodes = kHkv * kD;             // 512 bytes per token row
constexpr int kPageCodes = kPage * kRowCodes;    // 8 KiB per page (K or V)
constexpr int kScalePageFloats = kHkv * 2 * kPage;   // 256 floats = 1 KiB per page
#ifndef PA_Q8_RING_DEPTH
#define PA_Q8_RING_DEPTH 4
#endif
constexpr int kRingQ8 = PA_Q8_RING_DEPTH;
constexpr int kSlotQ8 = 1024 + 1024 + 256;       // K codes, V codes, scales (2 x 128 B used)
static_assert(kRingQ8 >= 2 && kRingQ8 * kWaves * kSlotQ8 <= 160 * 1024, "INT8 LDS ring too large");

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Upper halves of two FP32 words as one BF16 pair (a in the low half):
// exact for values with at most 8 significant bits.
__device__ __forceinline__ uint32_t bf16_pair_trunc(float a, float b) {
  return __builtin_amdgcn_perm(__float_as_uint(b), __float_as_uint(a), 0x07060302u);
}
// Byte k (0..3) of w as a signed integer, in FP32.
template <int K>
__device__ __forceinline__ float code_f32(uint32_t w) {
  return (float)(((int32_t)w << (24 - 8 * K)) >> 24);
}
// 8 int8 codes -> 8 BF16 values (the matrix-core operand).
__device__ __forceinline__ bf16x8_t codes_to_bf16x8(u32x2 c) {
  u32x4 o;
  o.x = bf16_pair_trunc(code_f32<0>(c.x), code_f32<1>(c.x));
  o.y = bf16_pair_trunc(code_f32<2>(c.x), code_f32<3>(c.x));
  o.z = bf16_pair_trunc(code_f32<0>(c.y), code_f32<1>(c.y));
  o.w = bf16_pair_trunc(code_f32<2>(c.y), code_f32<3>(c.y));
  return __builtin_bit_cast(bf16x8_t, o);
}

// One quantised row of 64 values is held by a quad of lanes: lane c (0..3)
// of the quad has dims {8c .. 8c+7} (lo) and {32+8c .. 32+8c+7} (hi) as
// BF16.  Returns this lane's 16 codes (lo, hi: 8 bytes each, in dim order)
// and the row's scale.  All four lanes of the quad must be active.
__device__ __forceinline__ float quad_max(float x) {
  x = fmaxf(x, dpp_mov<0xB1>(x));    // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_mov<0x4E>(x));    // quad_perm [2,3,0,1]
  return x;
}
__device__ __forceinline__ uint32_t pack_codes4(const float* r) {
  uint32_t w = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) w |= ((uint32_t)(int32_t)r[k] & 0xffu) << (8 * k);
  return w;
}
__device__ __forceinline__ float quantize_quad_row(uint4 lo, uint4 hi, u32x2& c_lo, u32x2& c_hi) {
  const uint32_t wl[4] = {lo.x, lo.y, lo.z, lo.w}, wh[4] = {hi.x, hi.y, hi.z, hi.w};
  float x[16];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    x[2 * w] = bf16_lo(wl[w]);
    x[2 * w + 1] = bf16_hi(wl[w]);
    x[8 + 2 * w] = bf16_lo(wh[w]);
    x[8 + 2 * w + 1] = bf16_hi(wh[w]);
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) amax = fmaxf(amax, fabsf(x[e]));
  amax = quad_max(amax);
  const float scale = amax / 127.f;                 // correctly rounded FP32 division
  float r[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float q = scale == 0.f ? 0.f : __builtin_rintf(x[e] / scale);   // ties to even
    r[e] = fminf(fmaxf(q, -128.f), 127.f);
  }
  c_lo = u32x2{pack_codes4(r), pack_codes4(r + 4)};
  c_hi = u32x2{pack_codes4(r + 8), pack_codes4(r + 12)};
  return scale;
}

struct DecodeArgsQ8 {
  const uint16_t* q;
  const int8_t* k_codes;
  const int8_t* v_codes;
  const float* kv_scales;
  const uint16_t* k_new;   // fused append: [B][Hkv][D] new-token rows, BF16
  const uint16_t* v_new;
  int8_t* k_codes_w;       // fused append: the same pools, written at slot L-1
  int8_t* v_codes_w;
  float* kv_scales_w;
  const float* rope_cos;
  const float* rope_sin;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  void* out;
  float* part_acc;
  float* part_ml;
  float xscale;
  int32_t num_pages;
  int32_t max_blocks;
  int32_t max_seq_len;
  int32_t pages_per_split;
  int32_t num_splits;
};

// One page slot of one lane: K and V codes of its token and dims, and the
// token's K and V scales (as FP32 bit patterns).
struct PageRegsQ8 {
  u32x2 klo, khi, vlo, vhi, sc;
};

// kaddr: slot + 64 token + 8 part (code rows); saddr: slot + 2048 + 4 token.
__device__ __forceinline__ void lds_page_issue_q8(PageRegsQ8& r, uint32_t kaddr, uint32_t saddr) {
  asm volatile(
      "ds_read_b64 %0, %5\n\t"
      "ds_read_b64 %1, %5 offset:32\n\t"
      "ds_read_b64 %2, %5 offset:1024\n\t"
      "ds_read_b64 %3, %5 offset:1056\n\t"
      "ds_read2_b32 %4, %6 offset1:16"
      : "=&v"(r.klo), "=&v"(r.khi), "=&v"(r.vlo), "=&v"(r.vhi), "=&v"(r.sc)
      : "v"(kaddr), "v"(saddr)
      : "memory");
}
__device__ __forceinline__ void lds_page_ready_q8(PageRegsQ8& r) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(r.klo), "+v"(r.khi), "+v"(r.vlo), "+v"(r.vhi), "+v"(r.sc)::"memory");
}

template <bool MASK>
__device__ __forceinline__ void consume_page_q8(LaneState& st, const PageRegsQ8& r, bf16x8_t qlo,
                                                bf16x8_t qhi, float xscale, int token, int valid) {
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  f32x4_t sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qlo, codes_to_bf16x8(r.klo), zero, 0, 0, 0);
  sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qhi, codes_to_bf16x8(r.khi), sc, 0, 0, 0);
  const float xs = xscale * __uint_as_float(r.sc.x);
  const float vscale = __uint_as_float(r.sc.y);
  float x[kGroup];
#pragma unroll
  for (int j = 0; j < kGroup; ++j) x[j] = sc[j] * xs;
  const bool live = !MASK || token < valid;
  bool raise = false;
#pragma unroll
  for (int j = 0; j < kGroup; ++j) raise |= live && (x[j] > st.m[j] + kTau);
  if (raise) {
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      const bool up = live && (x[j] > st.m[j] + kTau);
      const float mn = up ? x[j] : st.m[j];
      const float a = up ? __builtin_amdgcn_exp2f(st.m[j] - mn) : 1.f;  // m = -inf -> 0
      st.m[j] = mn;
      st.l[j] *= a;
#pragma unroll
      for (int e = 0; e < 16; ++e) st.acc[j][e] *= a;
    }
  }
  const uint32_t vw[4] = {r.vlo.x, r.vlo.y, r.vhi.x, r.vhi.y};
  float v[16];
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    v[4 * w + 0] = code_f32<0>(vw[w]);
    v[4 * w + 1] = code_f32<1>(vw[w]);
    v[4 * w + 2] = code_f32<2>(vw[w]);
    v[4 * w + 3] = code_f32<3>(vw[w]);
  }
#pragma unroll
  for (int j = 0; j < kGroup; ++j) {
    float p = __builtin_amdgcn_exp2f(x[j] - st.m[j]);
    // a slot past the sequence may hold any scale bits: select, never multiply
    float pv = p * vscale;
    if (MASK) {
      p = live ? p : 0.f;
      pv = live ? pv : 0.f;
    }
    st.l[j] += p;
#pragma unroll
    for (int e = 0; e < 16; ++e) st.acc[j][e] = __builtin_fmaf(pv, v[e], st.acc[j][e]);
  }
}

// Decode over INT8 pages; APPEND / ROPE as in decode_kernel (the new K/V row
// is quantised here, written to its slot with its scales, and its codes are
// used in place of what the page stream read for that slot).
template <bool OUT_BF16, bool APPEND, bool ROPE = false>
__global__ __launch_bounds__(kThreads, 2) void decode_q8_kernel(DecodeArgsQ8 a) {
  static_assert(!ROPE || APPEND, "RoPE is fused with the append");
  const int s = blockIdx.x;
  const int b = blockIdx.y;
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int token = lane & 15;
  const int part = lane >> 4;

  const int L = a.seq_lens[b];
  const int n_pages = (L + kPage - 1) / kPage;
  const bool bad_len = L < 0 || L > a.max_seq_len || n_pages > a.max_blocks ||
                       n_pages > a.pages_per_split * a.num_splits;
  const int n_splits_b = bad_len ? 1 : (n_pages + a.pages_per_split - 1) / a.pages_per_split;
  if (s >= (n_splits_b > 0 ? n_splits_b : 1)) return;

  float res[16];
  if (L == 0 || bad_len) {
    const float fill = bad_len ? __builtin_nanf("") : 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) res[e] = fill;
    if (token < kGroup) store_row16<OUT_BF16>(a.out, (int64_t)b * kHq + kGroup * g + token, part, res);
    return;
  }

  const int p0 = s * a.pages_per_split;
  const int p1 = min(p0 + a.pages_per_split, n_pages);
  const int last = p1 - 1;
  const int tail_valid = L - last * kPage;
  const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks;

  bf16x8_t qlo, qhi;
  {
    const uint16_t* qr = a.q + ((int64_t)b * kHq + kGroup * g + (token & 3)) * kD + 8 * part;
    uint4 lo = *reinterpret_cast<const uint4*>(qr);
    uint4 hi = *reinterpret_cast<const uint4*>(qr + 32);
    if (ROPE) {
      const int64_t row = (int64_t)(L - 1) * (kD / 2) + 8 * part;
      rope_pairs8(lo, hi, a.rope_cos + row, a.rope_sin + row);
    }
    qlo = __builtin_bit_cast(bf16x8_t, lo);
    qhi = __builtin_bit_cast(bf16x8_t, hi);
  }

  // fused append: lanes 0..3 quantise the new K row of head g (lane c: dims
  // {8c..} and {32+8c..}, rotated first with RoPE), lanes 4..7 the V row.
  // The codes are parked in LDS as [K, V][part][lo 8 B, hi 8 B], the two
  // scales after them.
  const bool app_here = APPEND && p1 == n_pages;
  const int app_slot = (L - 1) % kPage;
  __shared__ u32x4 new_codes[APPEND ? kWaves : 1][8];
  __shared__ float new_scales[APPEND ? kWaves : 1][2];
  if (app_here && lane < 8) {
    const int c = lane & 3;
    const bool is_k = lane < 4;
    const uint16_t* src = (is_k ? a.k_new : a.v_new) + ((int64_t)b * kHkv + g) * kD + 8 * c;
    uint4 lo = *reinterpret_cast<const uint4*>(src);
    uint4 hi = *reinterpret_cast<const uint4*>(src + 32);
    if (ROPE && is_k) {
      const int64_t row = (int64_t)(L - 1) * (kD / 2) + 8 * c;
      rope_pairs8(lo, hi, a.rope_cos + row, a.rope_sin + row);
    }
    u32x2 clo, chi;
    const float sc = quantize_quad_row(lo, hi, clo, chi);
    new_codes[APPEND ? g : 0][(is_k ? 0 : 4) + c] = u32x4{clo.x, clo.y, chi.x, chi.y};
    if (c == 0) new_scales[APPEND ? g : 0][is_k ? 0 : 1] = sc;
  }

  LaneState st;
#pragma unroll
  for (int j = 0; j < kGroup; ++j) {
    st.m[j] = -INFINITY;
    st.l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) st.acc[j][e] = 0.f;
  }

  int ent[kMaxSplitPages / 64];
#pragma unroll
  for (int c = 0; c < kMaxSplitPages / 64; ++c) {
    const int j = p0 + c * 64 + lane;
    ent[c] = (c * 64 < p1 - p0 && j <= last) ? bt[j] : 0;
  }
  bool bad_page = false;
  auto raw_page_id = [&](int i) -> int {
    const int j = i - p0;
    int id = __builtin_amdgcn_readlane(ent[0], j & 63);
#pragma unroll
    for (int c = 1; c < kMaxSplitPages / 64; ++c)
      if ((j >> 6) == c) id = __builtin_amdgcn_readlane(ent[c], j & 63);
    return id;
  };
  auto page_id = [&](int i) -> int64_t {
    const int id = raw_page_id(i);
    const bool ok = (unsigned)id < (unsigned)a.num_pages;
    bad_page |= !ok;
    return ok ? id : 0;
  };

  // ring slot r of wavefront g: [K codes 1 KiB | V codes 1 KiB | scales 256 B]
  __shared__ __attribute__((aligned(16))) char ring[kRingQ8][kWaves][kSlotQ8];
  // DMA lanes: codes, lane l -> token l/4, 16-byte chunk l%4 of the head's
  // 64-byte row; scales, lane l -> float l%32 of the head's 128-byte line
  const uint32_t code_lane = (uint32_t)((lane >> 2) * kRowCodes + g * kD + 16 * (lane & 3));
  const uint32_t scale_lane = (uint32_t)((g * 2 * kPage + (lane & 31)) * 4);
  const char* k_base = reinterpret_cast<const char*>(a.k_codes);
  const char* v_base = reinterpret_cast<const char*>(a.v_codes);
  const char* s_base = reinterpret_cast<const char*>(a.kv_scales);
  auto fetch = [&](int page, int slot) {            // 3 direct-to-LDS loads
    const int64_t id = page_id(page);
    const int64_t off = id * (int64_t)kPageCodes;
    const int64_t soff = id * (int64_t)(kScalePageFloats * 4);
    __builtin_amdgcn_global_load_lds(k_base + off + code_lane, &ring[slot][g][0], 16, 0, 0);
    __builtin_amdgcn_global_load_lds(v_base + off + code_lane, &ring[slot][g][1024], 16, 0, 0);
    __builtin_amdgcn_global_load_lds(s_base + soff + scale_lane, &ring[slot][g][2048], 4, 0, 0);
  };
  const uint32_t my_codes = lds_address(&ring[0][g][0]) + 64 * token + 8 * part;
  const uint32_t my_scales = lds_address(&ring[0][g][2048]) + 4 * token;
  constexpr uint32_t kRingSlotBytes = kWaves * kSlotQ8;

  auto step = [&](int i, auto masked) {
    constexpr bool MASK = decltype(masked)::value;
    const int slot = (i - p0) % kRingQ8;
    wait_vmem<3 * (kRingQ8 - 1)>();                 // page i has landed
    PageRegsQ8 cur;
    lds_page_issue_q8(cur, my_codes + slot * kRingSlotBytes, my_scales + slot * kRingSlotBytes);
    lds_page_ready_q8(cur);
    fetch(min(i + kRingQ8, last), slot);
    if (MASK && app_here && token == app_slot) {
      const u32x4 kc = new_codes[APPEND ? g : 0][part];
      const u32x4 vc = new_codes[APPEND ? g : 0][4 + part];
      cur.klo = u32x2{kc.x, kc.y};
      cur.khi = u32x2{kc.z, kc.w};
      cur.vlo = u32x2{vc.x, vc.y};
      cur.vhi = u32x2{vc.z, vc.w};
      cur.sc = u32x2{__float_as_uint(new_scales[APPEND ? g : 0][0]),
                     __float_as_uint(new_scales[APPEND ? g : 0][1])};
    }
    consume_page_q8<MASK>(st, cur, qlo, qhi, a.xscale, token, MASK ? tail_valid : kPage);
  };

#pragma unroll
  for (int r = 0; r < kRingQ8; ++r) fetch(min(p0 + r, last), r);
  for (int i = p0; i < last; ++i) step(i, std::false_type{});
  step(last, std::true_type{});
  wait_vmem<0>();
  if (app_here && lane < 8) {
    const int id = raw_page_id(last);
    if ((unsigned)id < (unsigned)a.num_pages) {
      const int c = lane & 3;
      const bool is_k = lane < 4;
      const u32x4 w = new_codes[APPEND ? g : 0][(is_k ? 0 : 4) + c];
      int8_t* dst = (is_k ? a.k_codes_w : a.v_codes_w) + (int64_t)id * kPageCodes +
                    app_slot * kRowCodes + g * kD + 8 * c;
      *reinterpret_cast<u32x2*>(dst) = u32x2{w.x, w.y};
      *reinterpret_cast<u32x2*>(dst + 32) = u32x2{w.z, w.w};
      if (c == 0)
        a.kv_scales_w[(int64_t)id * kScalePageFloats + (g * 2 + (is_k ? 0 : 1)) * kPage + app_slot] =
            new_scales[APPEND ? g : 0][is_k ? 0 : 1];
    }
  }

  merge_token_slots(st);

  if (bad_page) {
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      st.m[j] = __builtin_nanf("");
      st.l[j] = __builtin_nanf("");
#pragma unroll
      for (int e = 0; e < 16; ++e) st.acc[j][e] = __builtin_nanf("");
    }
  }

  if (n_splits_b == 1) {
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      if (token == j) {
        const float inv = 1.f / st.l[j];
#pragma unroll
        for (int e = 0; e < 16; ++e) res[e] = st.acc[j][e] * inv;
        store_row16<OUT_BF16>(a.out, (int64_t)b * kHq + kGroup * g + j, part, res);
      }
    }
  } else {
    const int64_t prow = ((int64_t)b * a.num_splits + s) * kHq + kGroup * g;
#pragma unroll
    for (int j = 0; j < kGroup; ++j) {
      if (token == j) {
#pragma unroll
        for (int e = 0; e < 16; ++e) res[e] = st.acc[j][e];
        store_row16<false>(a.part_acc, prow + j, part, res);
        if (part == 0) {
          a.part_ml[(prow + j) * 2 + 0] = st.m[j];
          a.part_ml[(prow + j) * 2 + 1] = st.l[j];
        }
      }
    }
  }
}

}  // namespace pa
