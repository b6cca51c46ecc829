// Device code of the paged GQA decode library for gfx950 (CDNA4, wave64).
//
// Work decomposition of pa_decode_attention:
//   * one work-group per (sequence b, split s); a split is a run of at most
//     `pages_per_split` consecutive logical pages of sequence b;
//   * 8 wavefronts per work-group, wavefront g serves KV head g and its 4
//     query heads 4g .. 4g+3 (grouped-query attention: 32 query heads share
//     8 KV heads);
//   * inside a wavefront, lane = 16 * part + token: `token` (0..15) is the
//     page slot the lane owns, `part` (0..3) selects 16 of the 64 head dims,
//     {8 part .. 8 part + 7} and {32 + 8 part .. 32 + 8 part + 7}.  One load
//     instruction of a wavefront reads, for 16 tokens, 64 contiguous bytes
//     of the 128-byte row of its KV head, and the 8 wavefronts of a
//     work-group together read every byte of each 16 KiB K page and 16 KiB
//     V page.
//
// Page stream: each wavefront keeps a ring of kRing page slots in LDS (4 KiB
// each: its 2 KiB slice of the K page and of the V page).  Pages are fetched
// with gfx950's direct-to-LDS loads (global_load_lds_dwordx4: every lane's
// 16 bytes land at lane*16 of a 1 KiB LDS row, without passing through
// VGPRs); a slot is refilled as soon as its page has been copied to
// registers, so while a page is being used the next kRing pages are in
// flight: kRing x 32 KiB of HBM reads per work-group at a register cost of
// one page.  A wavefront only ever reads its own ring, so no barrier is needed:
// explicit vmcnt waits mark a slot as landed and the LDS reads are issued one
// page ahead of their use.
//
// Arithmetic (the FP32 online softmax of the samir-vllm README's paged
// decode attention, written here for this lane layout):
//   * scores: two v_mfma_f32_16x16x32_bf16 per page compute Q' K^T, where
//     the 16 rows of Q' are the 4 query heads of the group repeated 4 times
//     and K^T is the page (16 tokens x 64 dims).  With the matrix-core lane
//     layout (lane l holds row l%16 of the A operand's 8-wide k slice
//     8*(l/16), column l%16 of B, and rows 4*(l/16)..+3 of column l%16 of
//     the result) every lane receives the 4 heads' scores of its own token,
//     which is exactly what its part of P.V needs: no cross-lane reduction.
//     3/4 of the matrix work is the repetition; the matrix core has the room
//     and the VALU does not.  BF16 products are exact in FP32.
//     x = score * scale * log2(e) so that exp2 is the hardware v_exp_f32;
//   * each lane keeps its own running maximum m, sum l and unnormalised
//     output acc[4 heads][16 dims] for the tokens of its slot (the online
//     normaliser of Milakov and Gimelshein, 2018).  The running maximum is
//     only raised when a new score exceeds it by more than kTau (in log2
//     units); weights are then at most 2^kTau and the rescale of acc is
//     almost never executed after the first page;
//   * at the end of the split the 16 token slots are merged with the same
//     rule (common maximum, rescale, add) by DPP row reductions; a
//     single-split sequence writes acc / l, a longer one writes (m, l, acc)
//     for the merge kernel.
//
// Masking: slots past the sequence length in its last page (and anything a
// block table points at beyond the used pages) may hold any bits, NaN
// included.  Those tokens get weight 0 by selection and their V words are
// replaced by zeros, never multiplied.
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
#ifndef PA_RING_DEPTH
#define PA_RING_DEPTH 2
#endif
#ifndef PA_WG_PER_CU
#define PA_WG_PER_CU 1
#endif
constexpr int kRing = PA_RING_DEPTH;            // LDS page slots per wavefront
constexpr int kWgPerCu = PA_WG_PER_CU;          // work-groups resident per compute unit
constexpr int kMaxSplitPages = 256;             // longest split (4096 tokens)
static_assert(kRing >= 2 && kWgPerCu * kRing * kWaves * 4 * 1024 <= 160 * 1024,
              "LDS ring too large for the resident work-groups");

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

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

struct PageRegs {
  u32x4 k0, k1, v0, v1;
};

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

// The four 16-byte LDS rows of one page slot (K lo/hi, V lo/hi) of this lane.
// Issued without waiting; the registers are valid after lds_page_ready().
__device__ __forceinline__ void lds_page_issue(PageRegs& r, uint32_t addr) {
  asm volatile(
      "ds_read_b128 %0, %4\n\t"
      "ds_read_b128 %1, %4 offset:1024\n\t"
      "ds_read_b128 %2, %4 offset:2048\n\t"
      "ds_read_b128 %3, %4 offset:3072"
      : "=&v"(r.k0), "=&v"(r.k1), "=&v"(r.v0), "=&v"(r.v1)
      : "v"(addr)
      : "memory");
}
// Wait for the LDS reads (and scalar loads) of this wavefront; ties the
// registers to the wait so no use is scheduled before it.
__device__ __forceinline__ void lds_page_ready(PageRegs& r) {
  asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(r.k0), "+v"(r.k1), "+v"(r.v0), "+v"(r.v1)::"memory");
}

// Running state of one lane: 4 query heads x 16 dims.
struct LaneState {
  float m[kGroup];
  float l[kGroup];
  float acc[kGroup][16];
};

// One page for one lane.  MASK: tokens at slot >= `valid` are not part of
// the sequence.  qlo/qhi: this lane's rows of Q' (head token%4, dims of part).
template <bool MASK>
__device__ __forceinline__ void consume_page(LaneState& st, const PageRegs& r, bf16x8_t qlo,
                                             bf16x8_t qhi, float xscale, int token, int valid) {
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  f32x4_t sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qlo, __builtin_bit_cast(bf16x8_t, r.k0),
                                                       zero, 0, 0, 0);
  sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qhi, __builtin_bit_cast(bf16x8_t, r.k1), sc, 0, 0, 0);
  float x[kGroup];
#pragma unroll
  for (int j = 0; j < kGroup; ++j) x[j] = sc[j] * xscale;
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

// All-reduce over the 16 lanes of a row (the 16 token slots of one dim
// part) with DPP: quad permutes, then rotations by 4 and 8 within the row.
// Pure VALU; every lane of the row ends with the same value.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x),
                                                               CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float row_allsum(float x) {
  x += dpp_mov<0xB1>(x);    // quad_perm [1,0,3,2]
  x += dpp_mov<0x4E>(x);    // quad_perm [2,3,0,1]
  x += dpp_mov<0x124>(x);   // row_ror:4
  x += dpp_mov<0x128>(x);   // row_ror:8
  return x;
}
__device__ __forceinline__ float row_allmax(float x) {
  x = fmaxf(x, dpp_mov<0xB1>(x));
  x = fmaxf(x, dpp_mov<0x4E>(x));
  x = fmaxf(x, dpp_mov<0x124>(x));
  x = fmaxf(x, dpp_mov<0x128>(x));
  return x;
}

// Combine the 16 token slots of a row: rescale every slot to the row's
// largest running maximum, then sum l and acc over the row (the same merge
// rule as for split partials, applied 16 ways at once).
__device__ __forceinline__ void merge_token_slots(LaneState& st) {
#pragma unroll
  for (int j = 0; j < kGroup; ++j) {
    const float M = row_allmax(st.m[j]);
    const float f = (st.m[j] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(st.m[j] - M);
    st.l[j] = row_allsum(st.l[j] * f);
#pragma unroll
    for (int e = 0; e < 16; ++e) st.acc[j][e] = row_allsum(st.acc[j][e] * f);
    st.m[j] = M;
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
  const uint16_t* k_new;   // fused append: [B][Hkv][D] new-token rows (else unused)
  const uint16_t* v_new;
  uint16_t* k_pool_w;      // fused append: the same pools, written at slot L-1
  uint16_t* v_pool_w;
  const float* rope_cos;   // fused RoPE: [positions][32] cos / sin of the rotation angles
  const float* rope_sin;
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

// APPEND: the one-token append is fused in.  The work-group whose split
// holds the sequence's last page writes the new K/V row (token L-1) into its
// page slot and uses the same values, from registers, in place of what the
// page stream read for that slot; no other work-group reads that page.
// ROPE (with APPEND): the new query and key are rotated at their absolute
// position L-1 first; every work-group of the sequence rotates its own q
// rows (lane-local: a lane holds both halves of each rotate-half pair).
template <bool OUT_BF16, bool APPEND, bool ROPE = false>
// second bound: minimum waves per SIMD (a work-group puts 2 on each SIMD)
__global__ __launch_bounds__(kThreads, 2 * kWgPerCu) void decode_kernel(DecodeArgs a) {
  static_assert(!ROPE || APPEND, "RoPE is fused with the append");
  const int s = blockIdx.x;
  const int b = blockIdx.y;
  const int g = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // KV head of this wavefront
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

  // this lane's rows of Q': head 4g + token%4, dims {8 part..+7} and {32 + 8 part..+7}
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

  // fused append: the new K and V row of head g (128 + 128 bytes) is parked
  // in LDS for the page stream's last page (keeps 16 VGPRs free in the loop):
  // slots 0..7 hold K dims 8j..8j+7, slots 8..15 the V ones.  Lane c < 4
  // takes K dims {8c..} and {32+8c..} (one set of rotate-half pairs, rotated
  // here with RoPE), lane 4 + c the same V dims.
  const bool app_here = APPEND && p1 == n_pages;     // this split holds token L-1
  const int app_slot = (L - 1) % kPage;
  __shared__ uint4 new_rows[APPEND ? kWaves : 1][16];
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
    new_rows[g][(is_k ? 0 : 8) + c] = lo;
    new_rows[g][(is_k ? 0 : 8) + 4 + c] = hi;
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
  // The split's block-table entries (at most kMaxSplitPages) are loaded once
  // into VGPRs, entry j of the split in lane j%64 of ent[j/64], and picked
  // with v_readlane: no memory access for page ids inside the page stream.
  int ent[kMaxSplitPages / 64];
#pragma unroll
  for (int c = 0; c < kMaxSplitPages / 64; ++c) {
    const int j = p0 + c * 64 + lane;
    ent[c] = (c * 64 < p1 - p0 && j <= last) ? bt[j] : 0;
  }
  bool bad_page = false;
  auto raw_page_id = [&](int i) -> int {          // i: logical page, p0 <= i <= last
    const int j = i - p0;
    int id = __builtin_amdgcn_readlane(ent[0], j & 63);
#pragma unroll
    for (int c = 1; c < kMaxSplitPages / 64; ++c)
      if ((j >> 6) == c) id = __builtin_amdgcn_readlane(ent[c], j & 63);
    return id;
  };
  auto page_id = [&](int i) -> int64_t {          // validated; out-of-range -> flagged, 0
    const int id = raw_page_id(i);
    const bool ok = (unsigned)id < (unsigned)a.num_pages;
    bad_page |= !ok;
    return ok ? id : 0;
  };

  // LDS ring: slot r of wavefront g holds rows [K lo, K hi, V lo, V hi] x 64 lanes x 16 B
  __shared__ uint4 ring[kRing][kWaves][4][64];
  const uint32_t lane_bytes = 2u * lane_off;         // byte offset of this lane in a page
  const char* k_base = reinterpret_cast<const char*>(a.k_pool);
  const char* v_base = reinterpret_cast<const char*>(a.v_pool);
  auto fetch = [&](int page, int slot) {            // 4 direct-to-LDS loads
    const int64_t off = page_id(page) * (int64_t)(kPageElems * 2);   // uniform
    const char* kp = k_base + off;
    const char* vp = v_base + off;
    __builtin_amdgcn_global_load_lds(kp + lane_bytes, &ring[slot][g][0][0], 16, 0, 0);
    __builtin_amdgcn_global_load_lds(kp + lane_bytes + 64, &ring[slot][g][1][0], 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vp + lane_bytes, &ring[slot][g][2][0], 16, 0, 0);
    __builtin_amdgcn_global_load_lds(vp + lane_bytes + 64, &ring[slot][g][3][0], 16, 0, 0);
  };
  const uint32_t my_row = lds_address(&ring[0][g][0][lane]);
  constexpr uint32_t kSlotBytes = kWaves * 4 * 64 * 16;

  // One page of the stream: wait for page i, copy it from its slot to
  // registers, refill that slot with page i+kRing right away (so kRing pages
  // stay in flight while page i is used), then use it.
  auto step = [&](int i, auto masked) {
    constexpr bool MASK = decltype(masked)::value;
    const int slot = (i - p0) % kRing;
    wait_vmem<4 * (kRing - 1)>();                   // page i has landed
    PageRegs cur;
    lds_page_issue(cur, my_row + slot * kSlotBytes);
    lds_page_ready(cur);
    fetch(min(i + kRing, last), slot);
    if (MASK && app_here && token == app_slot) {           // the appended token
      const u32x4* nr = reinterpret_cast<const u32x4*>(&new_rows[APPEND ? g : 0][0]);
      cur.k0 = nr[part];
      cur.k1 = nr[4 + part];
      cur.v0 = nr[8 + part];
      cur.v1 = nr[12 + part];
    }
    consume_page<MASK>(st, cur, qlo, qhi, a.xscale, token, MASK ? tail_valid : kPage);
  };

  // prologue: pages p0 .. p0+kRing-1 in flight (clamped to the split's last
  // page, so the count of outstanding loads is the same on every path)
#pragma unroll
  for (int r = 0; r < kRing; ++r) fetch(min(p0 + r, last), r);
  // pages p0 .. last-1 in the loop; the split's last page is peeled off
  // after it (masked when partial, and the place of the appended token), so
  // the loop body has a single path and its accumulators stay in place
  for (int i = p0; i < last; ++i) step(i, std::false_type{});
  step(last, std::true_type{});
  wait_vmem<0>();                                   // drain the clamped extra fetches
  if (app_here && lane < 16) {
    // write the new row into its slot: lanes 0..15 each store 16 bytes
    const int id = raw_page_id(last);
    if ((unsigned)id < (unsigned)a.num_pages) {
      const int64_t off = (int64_t)id * kPageElems + app_slot * kRowElems + g * kD + 8 * (lane & 7);
      uint16_t* dst = (lane < 8 ? a.k_pool_w : a.v_pool_w) + off;
      *reinterpret_cast<uint4*>(dst) = new_rows[APPEND ? g : 0][lane];
    }
  }

  // merge the 16 token slots (lane bits 0..3: one DPP row)
  merge_token_slots(st);

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
// Splits are read 8 at a time with all loads issued before any use, so the
// loop costs one memory latency per 8 splits rather than one per split.
constexpr int kMergeBatch = 8;

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
  // pass 1: the largest running maximum over the splits
  float M = -INFINITY;
  for (int s0 = 0; s0 < ns; s0 += kMergeBatch) {
    float m[kMergeBatch];
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k)
      m[k] = (s0 + k < ns) ? a.part_ml[(row0 + (int64_t)(s0 + k) * kHq) * 2] : -INFINITY;
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) M = fmaxf(M, m[k]);
  }
  // pass 2: weights 2^(m_s - M), sums in split order
  float num[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  for (int s0 = 0; s0 < ns; s0 += kMergeBatch) {
    float m[kMergeBatch], l[kMergeBatch];
    float4 x0[kMergeBatch], x1[kMergeBatch];
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      const bool in = s0 + k < ns;
      const int64_t row = row0 + (int64_t)(in ? s0 + k : 0) * kHq;
      const float4* src = reinterpret_cast<const float4*>(a.part_acc + row * kD + d0);
      m[k] = in ? a.part_ml[row * 2] : -INFINITY;
      l[k] = a.part_ml[row * 2 + 1];
      x0[k] = src[0];
      x1[k] = src[1];
    }
#pragma unroll
    for (int k = 0; k < kMergeBatch; ++k) {
      if (s0 + k >= ns) break;
      const float w = __builtin_amdgcn_exp2f(m[k] - M);
      den += w * l[k];
      num[0] += w * x0[k].x; num[1] += w * x0[k].y; num[2] += w * x0[k].z; num[3] += w * x0[k].w;
      num[4] += w * x1[k].x; num[5] += w * x1[k].y; num[6] += w * x1[k].z; num[7] += w * x1[k].w;
    }
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
