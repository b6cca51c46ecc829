// Device code of the paged GQA decode library for gfx950 (CDNA4, wave64).
//
// Work decomposition of pa_decode_attention:
//   * one work-group per (sequence b, split s); a split is a run of at most
//     `pages_per_split` consecutive logical pages of sequence b;
//   * 8 wavefronts per work-group, wavefront g serves KV head g and its 4
//     query heads 4g .. 4g+3 (grouped-query attention: 32 query heads share
//     8 KV heads);
//   * inside a wavefront, lane = 4 * token + part: `token` (0..15) is the
//     page slot the lane owns, `part` (0..3) selects 16 of the 64 head dims,
//     {8 part .. 8 part + 7} and {32 + 8 part .. 32 + 8 part + 7}.  One load
//     instruction of a wavefront therefore reads, for 16 tokens, 64
//     contiguous bytes of the 128-byte row of its KV head, and the 8
//     wavefronts of a work-group together read every byte of each 16 KiB K
//     page and 16 KiB V page.
//
// Arithmetic (the FP32 online softmax of the samir-vllm README's paged
// decode attention, written here for this lane layout):
//   * scores: q.k over the lane's 16 dims with v_dot2_f32_bf16 (BF16 products
//     are exact in FP32), summed over the 4 parts of a token with two DPP
//     quad permutes; x = score * scale * log2(e) so that exp2 is the
//     hardware v_exp_f32;
//   * each lane keeps its own running maximum m, sum l and unnormalised
//     output acc[4 heads][16 dims] for the tokens of its slot (the online
//     normaliser of Milakov and Gimelshein, 2018).  The running maximum is
//     only raised when a new score exceeds it by more than kTau (in log2
//     units); weights are then at most 2^kTau and the rescale of acc is
//     almost never executed after the first page;
//   * at the end of the split the 16 token slots are merged with the same
//     rule (max, rescale, add) across lanes; a single-split sequence writes
//     acc / l, a longer one writes (m, l, acc) for the merge kernel.
//
// Masking: slots past the sequence length in its last page (and anything a
// block table points at beyond the used pages) may hold any bits, NaN
// included.  Those tokens get weight 0 by selection and their V words are
// replaced by zeros, never multiplied.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Sum over the 4 lanes of a quad (the 4 dim-parts of one token), result in all 4.
__device__ __forceinline__ float quad_allsum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x),
                                                          0xB1, 0xF, 0xF, true));  // [1,0,3,2]
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x),
                                                          0x4E, 0xF, 0xF, true));  // [2,3,0,1]
  return x;
}

// Round-to-nearest-even FP32 -> BF16 bits (finite inputs; NaN stays NaN).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;   // quiet NaN
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

struct PageRegs {
  uint4 k0, k1, v0, v1;
};

// Running state of one lane: 4 query heads x 16 dims.
struct LaneState {
  float m[kGroup];
  float l[kGroup];
  float acc[kGroup][16];
};

__device__ __forceinline__ PageRegs load_page(const uint16_t* __restrict__ k_pool,
                                              const uint16_t* __restrict__ v_pool,
                                              int64_t phys, int lane_off) {
  const int64_t base = phys * kPageElems + lane_off;
  PageRegs r;
  r.k0 = *reinterpret_cast<const uint4*>(k_pool + base);
  r.k1 = *reinterpret_cast<const uint4*>(k_pool + base + 32);
  r.v0 = *reinterpret_cast<const uint4*>(v_pool + base);
  r.v1 = *reinterpret_cast<const uint4*>(v_pool + base + 32);
  return r;
}

// One page for one lane.  MASK: tokens at slot >= `valid` are not part of
// the sequence.
template <bool MASK>
__device__ __forceinline__ void consume_page(LaneState& st, const PageRegs& r,
                                             const uint32_t (&q)[kGroup][8], float xscale,
                                             int token, int valid) {
  const uint32_t kw[8] = {r.k0.x, r.k0.y, r.k0.z, r.k0.w, r.k1.x, r.k1.y, r.k1.z, r.k1.w};
  float x[kGroup];
#pragma unroll
  for (int j = 0; j < kGroup; ++j) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < 8; ++w) s = dot2_bf16(q[j][w], kw[w], s);
    x[j] = quad_allsum(s) * xscale;
  }
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
  uint32_t vw[8] = {r.v0.x, r.v0.y, r.v0.z, r.v0.w, r.v1.x, r.v1.y, r.v1.z, r.v1.w};
  if (MASK) {
#pragma unroll
    for (int w = 0; w < 8; ++w) vw[w] = live ? vw[w] : 0u;
  }
  float v[16];
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    v[2 * w] = bf16_lo(vw[w]);
    v[2 * w + 1] = bf16_hi(vw[w]);
  }
#pragma unroll
  for (int j = 0; j < kGroup; ++j) {
    float p = __builtin_amdgcn_exp2f(x[j] - st.m[j]);
    if (MASK) p = live ? p : 0.f;
    st.l[j] += p;
#pragma unroll
    for (int e = 0; e < 16; ++e) st.acc[j][e] = __builtin_fmaf(p, v[e], st.acc[j][e]);
  }
}

// Merge lane state with the lane `mask` away (xor); symmetric, so both lanes
// of a pair end with the same sums.
__device__ __forceinline__ void merge_lanes(LaneState& st, int mask) {
#pragma unroll
  for (int j = 0; j < kGroup; ++j) {
    const float mo = __shfl_xor(st.m[j], mask);
    const float lo = __shfl_xor(st.l[j], mask);
    const float mn = fmaxf(st.m[j], mo);
    const float fa = (st.m[j] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(st.m[j] - mn);
    const float fb = (mo == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mo - mn);
    st.l[j] = fa * st.l[j] + fb * lo;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float ao = __shfl_xor(st.acc[j][e], mask);
      st.acc[j][e] = fa * st.acc[j][e] + fb * ao;
    }
    st.m[j] = mn;
  }
}

// Dim index (0..63) of element e (0..15) owned by dim-part `part`.
__device__ __forceinline__ int dim_of(int part, int e) {
  return (e < 8) ? (8 * part + e) : (32 + 8 * part + (e - 8));
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

struct DecodeArgs {
  const uint16_t* q;
  const uint16_t* k_pool;
  const uint16_t* v_pool;
  const int32_t* block_tables;
  const int32_t* seq_lens;
  void* out;
  float* part_acc;     // [B][S][Hq][D]
  float* part_ml;      // [B][S][Hq][2]
  float xscale;        // scale * log2(e)
  int32_t num_pages;
  int32_t max_blocks;
  int32_t max_seq_len;     // host-declared bound; longer sequences are flagged
  int32_t pages_per_split;
  int32_t num_splits;  // S: splits per sequence in the grid
};

template <bool OUT_BF16>
__global__ __launch_bounds__(kThreads) void decode_kernel(DecodeArgs a) {
  const int s = blockIdx.x;
  const int b = blockIdx.y;
  const int g = threadIdx.x >> 6;      // KV head of this wavefront
  const int lane = threadIdx.x & 63;
  const int token = lane >> 2;
  const int part = lane & 3;

  const int L = a.seq_lens[b];
  const int n_pages = (L + kPage - 1) / kPage;
  const bool bad_len = L < 0 || L > a.max_seq_len || n_pages > a.max_blocks ||
                       n_pages > a.pages_per_split * a.num_splits;
  const int n_splits_b = bad_len ? 1 : (n_pages + a.pages_per_split - 1) / a.pages_per_split;
  if (s >= (n_splits_b > 0 ? n_splits_b : 1)) return;

  float res[16];
  if (L == 0 || bad_len) {
    // idle slot: zeros; impossible length: NaN (explicit, nothing read)
    const float fill = bad_len ? __builtin_nanf("") : 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) res[e] = fill;
    if (token < kGroup) store_row16<OUT_BF16>(a.out, (int64_t)b * kHq + kGroup * g + token, part, res);
    return;
  }

  const int p0 = s * a.pages_per_split;
  const int p1 = min(p0 + a.pages_per_split, n_pages);
  const int last = p1 - 1;
  const int tail_valid = L - last * kPage;           // 1..16 tokens valid in page `last`
  const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks;

  // query rows of the 4 heads of this group, this lane's 16 dims, as BF16 pairs
  uint32_t q[kGroup][8];
#pragma unroll
  for (int j = 0; j < kGroup; ++j) {
    const uint16_t* qr = a.q + ((int64_t)b * kHq + kGroup * g + j) * kD + 8 * part;
    const uint4 lo = *reinterpret_cast<const uint4*>(qr);
    const uint4 hi = *reinterpret_cast<const uint4*>(qr + 32);
    q[j][0] = lo.x; q[j][1] = lo.y; q[j][2] = lo.z; q[j][3] = lo.w;
    q[j][4] = hi.x; q[j][5] = hi.y; q[j][6] = hi.z; q[j][7] = hi.w;
  }

  LaneState st;
#pragma unroll
  for (int j = 0; j < kGroup; ++j) {
    st.m[j] = -INFINITY;
    st.l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) st.acc[j][e] = 0.f;
  }

  const int lane_off = token * kRowElems + g * kD + 8 * part;
  bool bad_page = false;
  auto page_id = [&](int i) -> int64_t {
    const int id = bt[i];
    const bool ok = (unsigned)id < (unsigned)a.num_pages;
    bad_page |= !ok;
    return ok ? id : 0;
  };

  // double-buffered page stream: page i+1 is in flight while page i is used
  PageRegs A = load_page(a.k_pool, a.v_pool, page_id(p0), lane_off);
  for (int i = p0;; i += 2) {
    PageRegs B = load_page(a.k_pool, a.v_pool, page_id(min(i + 1, last)), lane_off);
    if (i == last && tail_valid < kPage)
      consume_page<true>(st, A, q, a.xscale, token, tail_valid);
    else
      consume_page<false>(st, A, q, a.xscale, token, kPage);
    if (i + 1 > last) break;
    A = load_page(a.k_pool, a.v_pool, page_id(min(i + 2, last)), lane_off);
    if (i + 1 == last && tail_valid < kPage)
      consume_page<true>(st, B, q, a.xscale, token, tail_valid);
    else
      consume_page<false>(st, B, q, a.xscale, token, kPage);
    if (i + 2 > last) break;
  }

  // merge the 16 token slots (lane bits 2..5)
  merge_lanes(st, 4);
  merge_lanes(st, 8);
  merge_lanes(st, 16);
  merge_lanes(st, 32);

  if (bad_page) {
    // a block-table entry outside the pool: nothing was read from it; the
    // sequence's outputs (directly, or through a NaN partial) become NaN
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

// Log-sum-exp merge of the splits of each multi-split sequence, in split
// order.  One work-group of 256 threads per sequence: thread = (head, 8 dims).
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void merge_kernel(DecodeArgs a) {
  const int b = blockIdx.x;
  const int L = a.seq_lens[b];
  const int n_pages = (L + kPage - 1) / kPage;
  if (L <= 0 || L > a.max_seq_len || n_pages > a.max_blocks ||
      n_pages > a.pages_per_split * a.num_splits)
    return;
  const int ns = (n_pages + a.pages_per_split - 1) / a.pages_per_split;
  if (ns <= 1) return;
  const int h = threadIdx.x >> 3;
  const int d0 = (threadIdx.x & 7) * 8;
  const int64_t row0 = (int64_t)b * a.num_splits * kHq + h;   // split s at row0 + s*kHq
  float M = -INFINITY;
  for (int s = 0; s < ns; ++s) M = fmaxf(M, a.part_ml[(row0 + (int64_t)s * kHq) * 2]);
  float num[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  for (int s = 0; s < ns; ++s) {
    const int64_t row = row0 + (int64_t)s * kHq;
    const float w = __builtin_amdgcn_exp2f(a.part_ml[row * 2] - M);
    den += w * a.part_ml[row * 2 + 1];
    const float4* src = reinterpret_cast<const float4*>(a.part_acc + row * kD + d0);
    const float4 x0 = src[0], x1 = src[1];
    num[0] += w * x0.x; num[1] += w * x0.y; num[2] += w * x0.z; num[3] += w * x0.w;
    num[4] += w * x1.x; num[5] += w * x1.y; num[6] += w * x1.z; num[7] += w * x1.w;
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

}  // namespace pa
