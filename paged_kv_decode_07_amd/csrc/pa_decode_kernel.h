// Decode kernel of the paged GQA decode library for gfx950 (CDNA4, wave64),
// for BF16, INT8 and INT4 pages.
//
// Work decomposition: one work-group per (sequence b, split s); a split is a
// run of at most `pages_per_split` consecutive logical pages of sequence b.
// The 8 wavefronts of a work-group serve the 8 KV heads: wavefront g streams
// its head's slice of every page of the split (grouped-query attention: 32
// query heads share 8 KV heads; query heads 4g .. 4g+3 read KV head g).  With
// WPH = 2 (INT4 plans whose grid fits the CUs) a work-group has 16
// wavefronts, two per KV head, each streaming half of the split's pages.
//
// Page stream: each wavefront keeps a ring of page slots in LDS, filled with
// gfx950's direct-to-LDS loads (every lane's 4 or 16 bytes land at lane*size
// of the destination, without passing through VGPRs).  A slot is refilled as
// soon as its page has been read into registers, so while a page is used the
// next ring-depth pages are in flight (BF16 pages: one slot, INT8: two,
// INT4: three).  A wavefront only ever reads its own
// slots, so explicit vmcnt waits are the only synchronisation.  The split's
// block-table entries are preloaded into VGPRs and picked with v_readlane.
// Every load instruction requests whole 128-byte lines (BF16: 8 token rows
// of the head; INT8: the head's 1 KiB code block; INT4: the head's K and V
// blocks of 512 bytes, one per half-wave), with the non-temporal
// policy: on this part that pair streams 10-12% faster than half-line
// requests or the default policy.
//
// Arithmetic (the FP32 online softmax of the samir-vllm README's paged
// decode attention, on the matrix cores):
//
//   * scores are computed transposed, S^T = K Q^T, with one
//     v_mfma_f32_16x16x32_bf16 per 32 dims: the A operand is the page's K
//     (row = token, 8 dims per lane), the B operand is Q^T with column n
//     holding query head 4g + n / 4, so each head fills the 4 columns of one
//     quad of lanes.  Lane l = 16 G + n receives the scores of tokens
//     4G .. 4G+3 for column n; of these it keeps one, token 4G + n % 4, so
//     the 16 lanes of a head's quads in the four token groups hold its 16
//     scores once each.  The softmax then costs one exp2 per lane and page
//     (scores scaled by scale * log2(e) so that exp2 is the hardware
//     v_exp_f32);
//   * the P V product is v_mfma_f32_16x16x16_bf16 with k = tokens, whose A
//     operand lane 16 G + n supplies row n, tokens 4G .. 4G+3.  Each lane
//     packs its weight rounded to BF16 and the remainder (weight - its BF16
//     value, rounded again) into one word; a quad broadcast (DPP quad_perm)
//     gives every lane of the quad the words of its head's four tokens, and
//     v_perm keeps the BF16 halves for rows 4h, 4h+2 and the remainders for
//     rows 4h+1, 4h+3 (h = n / 4).  Each weight is carried to about 2^-16
//     relative.  Output rows 4G and 4G+1 of lane 16 G + n add up to head G's
//     unnormalised output in column n; rows 4G+2, 4G+3 repeat them and are
//     never read;
//   * V reaches the B operand (column = dim, k = 4 tokens per lane) through
//     gfx950's transposing LDS read ds_read_b64_tr_b16: within each group of
//     16 lanes, output lane i takes element i % 4 of the 4-element chunks
//     addressed by lanes 4c + i/4, c = 0..3; pointing lane 4c + q at dims
//     4q .. 4q+3 of token 4G + c gives lane i the 4 tokens of dim i.  For
//     INT8 codes the 16-bit unit is a pair of dims, so one read gives a lane
//     4 tokens of an even and an odd dim (two products per 32 dims);
//   * the online softmax keeps one running maximum per head, equal in every
//     lane of that head (the product sums over tokens, so a page's weights
//     share it); it is raised only when a score exceeds it by more than
//     kTau (a wave-wide vote; the page maximum is then reduced over the
//     head's 16 lanes).  Weights are then at most 2^kTau and the rescale
//     of the accumulators is almost never executed after the first page.  The
//     normaliser is a per-lane partial sum, reduced over the head's lanes at
//     the end;
//   * the accumulator is 4 products x 4 floats per lane (16 VGPRs), and the
//     VALU carries no multiply-add of P V.
//
// INT8 pages: K codes are widened to BF16 exactly for the score product and
// the K scale of each token joins the score multiplier; V codes are widened
// to BF16 exactly and the V scale joins the weight (p * v_scale), while the
// normaliser sums p alone.
//
// INT4 pages: a nibble u = code + 8 becomes a BF16 value without a
// conversion instruction: 128 + u = code + 136 for the first nibble of a
// 16-bit unit (masked in place), 16 + u = code + 24 for the others (a shift
// and one mask-and-or per pair).  The offsets are removed around each
// product.  Scores: minus the offsets times the query row is the accumulator
// input of the score product.  Values: each lane also sums the weights its
// products carry (the BF16 weight plus its BF16 remainder), rescaled with the
// accumulators, and each tile's offset times that sum is subtracted from the
// output.  A lane reads dims 16G .. 16G+15 of a token's K codes in one 64-bit
// LDS read; each word gives its dims in the order 0 4 1 5 2 6 3 7, and the
// query operand is exchanged between lanes and permuted to match.  One
// transposed read gives a lane 4 tokens x 4 dims (the 16-bit unit is 4
// codes), so tile e of the value product is dims 4n + e.  The 3-deep ring
// lets full pages be consumed two at a time (one vote and rescale for both,
// one 16x16x32 value product per tile over their 32 tokens); with its small
// pages this format is bound by its page stream's per-page requests.
//
// Masking: slots past the sequence in its last page may hold any bits.  Their
// scores are selected to -inf, their weights to 0, and for BF16 pages their V
// values are replaced by zeros before the product (0 * NaN would be NaN).
// A sequence whose block-table entry falls outside the pool reads nothing
// from it and gets NaN outputs; so does a length beyond the declared bound.
#pragma once

#include "pa_kernels_q8.h"

namespace pa {

typedef short bf16x4_t __attribute__((ext_vector_type(4)));

// Arguments of the decode kernel (either page format).
struct DecodeArgs {
  const uint16_t* q;
  const void* k_pool;          // BF16 [pages][16][8][64], int8 codes [pages][8][16][64]
  const void* v_pool;          // or INT4 code bytes [pages][8][16][32]
  const float* kv_scales;      // INT8 and INT4: [pages][8][2][16]
  const uint16_t* k_new;       // fused append: [B][8][64] BF16 rows
  const uint16_t* v_new;
  void* k_pool_w;              // fused append: the same pools, written at slot L-1
  void* v_pool_w;
  float* kv_scales_w;
  const float* rope_cos;
  const float* rope_sin;
  int32_t rope_positions;      // rows of rope_cos / rope_sin
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
  // optional work list: work item k (block k) is sequence work[2k], split
  // work[2k+1]; NULL: block k is split k % num_splits of sequence
  // k / num_splits
  const int32_t* work;
  int32_t num_work;
  int32_t batch;
};

// Page-format constants of the LDS ring (per wavefront slot).
template <int FMT>
struct PageFormat;
// kPairs: full pages are consumed two at a time (needs a ring of 3 or more).
#ifndef PA_PAIR_STEPS
#define PA_PAIR_STEPS 1
#endif
template <>
struct PageFormat<kFmtBF16> {
  static constexpr int kRingDepth = kRing;      // slots of 4 KiB (one)
  static constexpr int kSlot = 4096;            // [K | V] x 16 token rows x 128 B (swizzled pieces)
  static constexpr int kLoads = 4;              // direct-to-LDS loads per page
  static constexpr bool kPairs = PA_PAIR_STEPS && kRingDepth >= 3;
};

// BF16 slot layout: the head's K rows (2 KiB) then its V rows.  Each
// direct-to-LDS load carries 8 whole 128-byte token rows, so that every HBM
// line is requested in full by one instruction.  The 16-byte piece p (dims
// 8p .. 8p+7) of token t sits at piece position p ^ (t / 2) of the token's
// LDS row: the 16 lanes of a score-operand read (16 tokens, one piece) and of
// a transposed V read then fall on distinct or paired bank groups instead of
// one.  Byte offset of (t, p) within the K or V half:
__device__ __forceinline__ constexpr uint32_t bf16_slot_offset(int t, int p) {
  return (uint32_t)(16 * (8 * t + (p ^ (t >> 1))));
}
template <>
struct PageFormat<kFmtINT8> {
  static constexpr int kRingDepth = kRingQ8;    // slots of 2304 B
  static constexpr int kSlot = kSlotQ8;         // [K codes 16 x 64 B | V codes 16 x 64 B | scales]
  static constexpr int kLoads = 3;
  static constexpr bool kPairs = PA_PAIR_STEPS && kRingDepth >= 3;
};
template <>
struct PageFormat<kFmtINT4> {
  static constexpr int kRingDepth = kRingQ4;    // slots of 1280 B
  static constexpr int kSlot = kSlotQ4;         // [K codes 16 x 32 B | V codes 16 x 32 B | scales]
  static constexpr int kLoads = 2;              // K and V codes in one load, the scales
  static constexpr bool kPairs = PA_PAIR_STEPS && kRingDepth >= 3;
};

// Cache-policy bits of the page-stream loads: every page is read once, so
// every page format stream with the non-temporal policy (nt = 2).
#ifndef PA_STREAM_CPOL
#define PA_STREAM_CPOL 2
#endif
constexpr int kStreamCpol = PA_STREAM_CPOL;

// This lane's part of a page's direct-to-LDS loads for page format FMT and
// KV head g: the byte offsets within a page of its code loads (BF16: two per
// pool) and of its scale float, and its code pool (INT4: K for lanes 0..31,
// V for 32..63).  BF16 load j (tokens 8j .. 8j+7) has lane l take token
// t = 8j + l/8 and the piece whose swizzled position is l%8, so that lane l
// lands at byte bf16_slot_offset(t, that piece) - 1024 j of its destination;
// INT8 lane l takes bytes 16 l of the head's code block (token l/4, dims
// 16 (l%4) ..) and float l%32 of its scale line; INT4 lane l takes bytes
// 16 (l%32) of the head's K (l < 32) or V block, and the same scale float.
// The decode kernels and the page-stream measurement share these maps.
struct PageDma {
  uint32_t k, k1, s;
  const char* kv;
};
template <int FMT>
__device__ __forceinline__ PageDma page_dma(int g, int lane, const char* k_base,
                                            const char* v_base) {
  PageDma d{0u, 0u, 0u, k_base};
  if constexpr (FMT == kFmtINT8) {
    d.k = (uint32_t)(g * kHeadCodes + 16 * lane);                   // the head's 1 KiB block
    d.s = (uint32_t)((g * 2 * kPage + (lane & 31)) * 4);
  } else if constexpr (FMT == kFmtINT4) {
    d.kv = lane < 32 ? k_base : v_base;
    d.k = (uint32_t)(g * kHeadCodes4 + 16 * (lane & 31));           // 512 B of K, 512 B of V
    d.s = (uint32_t)((g * 2 * kPage + (lane & 31)) * 4);
  } else {
    const int t0 = lane >> 3, t1 = 8 + (lane >> 3);
    d.k = 2u * (uint32_t)(t0 * kRowElems + g * kD) + 16u * (uint32_t)((lane & 7) ^ (t0 >> 1));
    d.k1 = 2u * (uint32_t)(t1 * kRowElems + g * kD) + 16u * (uint32_t)((lane & 7) ^ (t1 >> 1));
  }
  return d;
}

// Request page `id` into the LDS slot `dst` (format FMT's slot layout), its
// head's blocks head_off and scale_off bytes past the lane offsets of d, with
// the streaming cache policy.
template <int FMT>
__device__ __forceinline__ void page_fetch(const PageDma& d, const char* k_base,
                                           const char* v_base, const char* s_base, int64_t id,
                                           uint32_t head_off, uint32_t scale_off, char* dst) {
  if constexpr (FMT == kFmtINT8) {
    const int64_t off = id * (int64_t)kPageCodes + head_off;
    __builtin_amdgcn_global_load_lds(k_base + off + d.k, dst, 16, 0, kStreamCpol);
    __builtin_amdgcn_global_load_lds(v_base + off + d.k, dst + 1024, 16, 0, kStreamCpol);
    __builtin_amdgcn_global_load_lds(s_base + id * (int64_t)(kScalePageFloats * 4) + scale_off + d.s,
                                     dst + 2048, 4, 0, kStreamCpol);
  } else if constexpr (FMT == kFmtINT4) {
    __builtin_amdgcn_global_load_lds(d.kv + id * (int64_t)kPageCodes4 + head_off + d.k, dst, 16, 0,
                                     kStreamCpol);
    __builtin_amdgcn_global_load_lds(s_base + id * (int64_t)(kScalePageFloats * 4) + scale_off + d.s,
                                     dst + 1024, 4, 0, kStreamCpol);
  } else {
    const int64_t off = id * (int64_t)(kPageElems * 2) + head_off;
    __builtin_amdgcn_global_load_lds(k_base + off + d.k, dst, 16, 0, kStreamCpol);
    __builtin_amdgcn_global_load_lds(k_base + off + d.k1, dst + 1024, 16, 0, kStreamCpol);
    __builtin_amdgcn_global_load_lds(v_base + off + d.k, dst + 2048, 16, 0, kStreamCpol);
    __builtin_amdgcn_global_load_lds(v_base + off + d.k1, dst + 3072, 16, 0, kStreamCpol);
  }
}

// Registers of one page for one lane.
struct PageBF16 {
  u32x4 k0, k1;       // K[token][8G..8G+7], K[token][32+8G..32+8G+7]
  u32x2 v[4];         // V, 4 tokens x 16-dim block b (transposed read)
};
// LDS read addresses of one lane in slot 0 (the swizzle makes them independent)
struct SlotAddrBF16 {
  uint32_t k0, k1, v[4];
};
struct PageQ8 {
  u32x2 k0, k1;       // K codes, 8 dims each
  u32x2 v[2];         // V codes: 4 tokens x (even, odd) dim pairs, dims 0..31 and 32..63
  uint32_t ks, vs;    // K and V scales of this lane's token 4G + n % 4
};
struct PageQ4 {
  u32x2 k;            // K codes of token n, dims 16G .. 16G+7 and 16G+8 .. 16G+15
  u32x2 v;            // V codes: 4 tokens x dims 4n .. 4n+3 (transposed read)
  uint32_t ks, vs;    // K and V scales of this lane's token 4G + n % 4
};

// The slot's reads for one lane: its two K pieces and its transposed-read
// chunks of the 4 V blocks, at the addresses of `ad` plus `off` (the slot).
__device__ __forceinline__ void lds_page_issue(PageBF16& r, const SlotAddrBF16& ad, uint32_t off) {
  asm volatile(
      "ds_read_b128 %0, %6\n\t"
      "ds_read_b128 %1, %7\n\t"
      "ds_read_b64_tr_b16 %2, %8\n\t"
      "ds_read_b64_tr_b16 %3, %9\n\t"
      "ds_read_b64_tr_b16 %4, %10\n\t"
      "ds_read_b64_tr_b16 %5, %11"
      : "=&v"(r.k0), "=&v"(r.k1), "=&v"(r.v[0]), "=&v"(r.v[1]), "=&v"(r.v[2]), "=&v"(r.v[3])
      : "v"(ad.k0 + off), "v"(ad.k1 + off), "v"(ad.v[0] + off), "v"(ad.v[1] + off),
        "v"(ad.v[2] + off), "v"(ad.v[3] + off)
      : "memory");
}
__device__ __forceinline__ void lds_page_ready(PageBF16& r) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(r.k0), "+v"(r.k1), "+v"(r.v[0]), "+v"(r.v[1]), "+v"(r.v[2]), "+v"(r.v[3])::"memory");
}
// kaddr: K codes of (token, 8G); vaddr: V chunk of this lane; saddr: the K
// scale of token 4G + n % 4 (its V scale 64 bytes on).
__device__ __forceinline__ void lds_page_issue(PageQ8& r, uint32_t kaddr, uint32_t vaddr,
                                         uint32_t saddr) {
  asm volatile(
      "ds_read_b64 %0, %6\n\t"
      "ds_read_b64 %1, %6 offset:32\n\t"
      "ds_read_b64_tr_b16 %2, %7\n\t"
      "ds_read_b64_tr_b16 %3, %7 offset:32\n\t"
      "ds_read_b32 %4, %8\n\t"
      "ds_read_b32 %5, %8 offset:64"
      : "=&v"(r.k0), "=&v"(r.k1), "=&v"(r.v[0]), "=&v"(r.v[1]), "=&v"(r.ks), "=&v"(r.vs)
      : "v"(kaddr), "v"(vaddr), "v"(saddr)
      : "memory");
}
__device__ __forceinline__ void lds_page_ready(PageQ8& r) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(r.k0), "+v"(r.k1), "+v"(r.v[0]), "+v"(r.v[1]), "+v"(r.ks), "+v"(r.vs)::"memory");
}

// kaddr: K codes of (token n, dims 16G..); vaddr: V chunk of this lane;
// saddr: the K scale of token 4G + n % 4 (its V scale 64 bytes on); OFF: the
// slot's offset from these addresses, as the reads' immediate offset.
template <uint32_t OFF = 0>
__device__ __forceinline__ void lds_page_issue(PageQ4& r, uint32_t kaddr, uint32_t vaddr,
                                         uint32_t saddr) {
  static_assert(OFF + 64 <= 65535, "LDS read offsets are 16 bits");
  asm volatile(
      "ds_read_b64 %0, %4 offset:%7\n\t"
      "ds_read_b64_tr_b16 %1, %5 offset:%7\n\t"
      "ds_read_b32 %2, %6 offset:%7\n\t"
      "ds_read_b32 %3, %6 offset:%8"
      : "=&v"(r.k), "=&v"(r.v), "=&v"(r.ks), "=&v"(r.vs)
      : "v"(kaddr), "v"(vaddr), "v"(saddr), "i"(OFF), "i"(OFF + 64)
      : "memory");
}
__device__ __forceinline__ void lds_page_ready(PageQ4& r) {
  asm volatile("s_waitcnt lgkmcnt(0)"
               : "+v"(r.k), "+v"(r.v), "+v"(r.ks), "+v"(r.vs)::"memory");
}

// 4 INT8 codes (bytes b0..b3 of w) -> BF16 pairs (b0, b2) and (b1, b3): the
// even-dim and odd-dim values of two tokens when w holds (t, even), (t, odd),
// (t+1, even), (t+1, odd).
__device__ __forceinline__ void codes_even_odd(uint32_t w, uint32_t& even, uint32_t& odd) {
  even = bf16_pair_trunc(code_f32<0>(w), code_f32<2>(w));
  odd = bf16_pair_trunc(code_f32<1>(w), code_f32<3>(w));
}

// Running state of one lane: the accumulators of the P V products (4 tiles
// of 16 x 16, this lane's rows 4G .. 4G+3 of column n), the head's running
// maximum m (log2 units, same in all lanes of the head), this lane's
// partial normaliser l and, for INT4 pages, its partial sum of weights wsum.
struct LaneState {
  f32x4_t acc[4];
  float m;
  float l;
  float wsum;
};

// Per-lane constants of the page arithmetic.  qbias (INT4 pages): 24 x the
// sum of this lane's query row; nib: the widening constants.
struct PageConsts {
  float xscale;
  float qbias;
  uint32_t sel;        // v_perm selector of the weight operand (row parity)
  NibbleConsts nib;
};

// Raw scores of one page for this lane: tokens 4G .. 4G+3, column n (INT4:
// the code bias already removed, through the product's accumulator input).
template <int FMT, typename Page>
__device__ __forceinline__ f32x4_t page_scores(const Page& r, bf16x8_t qlo, bf16x8_t qhi,
                                               const PageConsts& pc) {
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  f32x4_t s;
  if constexpr (FMT == kFmtINT8) {
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes_to_bf16x8(r.k0), qlo, zero, 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(codes_to_bf16x8(r.k1), qhi, s, 0, 0, 0);
  } else if constexpr (FMT == kFmtINT4) {
    bf16x8_t k0, k1;
    nibbles_to_bf16x8x2(r.k, pc.nib, k0, k1);
    const f32x4_t nb = {-pc.qbias, -pc.qbias, -pc.qbias, -pc.qbias};
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qlo, nb, 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qhi, s, 0, 0, 0);
  } else {
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, r.k0), qlo, zero, 0, 0, 0);
    s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, r.k1), qhi, s, 0, 0, 0);
  }
  return s;
}

// This lane's own score: element q = n % 4 of its 4 (tokens 4G .. 4G+3 of
// column n), i.e. token 4G + q of query head n / 4.
__device__ __forceinline__ float own_score(f32x4_t s, int q) {
  float v = s[0];
  v = q == 1 ? s[1] : v;
  v = q == 2 ? s[2] : v;
  v = q == 3 ? s[3] : v;
  return v;
}

// The lane's score in log2 units (scale, log2(e) and the K scale applied).
template <int FMT, typename Page>
__device__ __forceinline__ float page_logit(const Page& r, f32x4_t s, float xscale, int q) {
  float xs = xscale;
  if constexpr (FMT != kFmtBF16) xs = xscale * __uint_as_float(r.ks);
  return own_score(s, q) * xs;
}

// Raise the running maximum when a score passed it by more than kTau (mx is
// this lane's score; the new maximum is reduced over the 16 lanes of the
// head: its quad and the four token groups) and rescale.  The normaliser and
// weight sum belong to the lane's head n / 4; the accumulator rows of lane
// 16 G + n belong to head G, whose factor is taken from lane 4G.
__device__ __forceinline__ void raise_max(LaneState& st, float mx, int G) {
  if (__builtin_amdgcn_ballot_w64(mx > st.m + kTau)) {
    float pm = mx;
    pm = fmaxf(pm, dpp_mov<0xB1>(pm));          // quad_perm [1,0,3,2]
    pm = fmaxf(pm, dpp_mov<0x4E>(pm));          // quad_perm [2,3,0,1]
    pm = fmaxf(pm, __shfl_xor(pm, 16));
    pm = fmaxf(pm, __shfl_xor(pm, 32));
    const float mn = (pm > st.m + kTau) ? pm : st.m;
    const float a = __builtin_amdgcn_exp2f(st.m - mn);    // m = -inf -> 0
    st.m = mn;
    st.l *= a;
    st.wsum *= a;
    const float a0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, a), 0));
    const float a1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, a), 4));
    const float a2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, a), 8));
    const float a3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, a), 12));
    const float ag = G == 0 ? a0 : (G == 1 ? a1 : (G == 2 ? a2 : a3));
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) st.acc[b][rr] *= ag;
  }
}

// A operand of the P V product, built from each lane's own weight w (token
// 4G + q of head h = n / 4, q = n % 4).  Row n = 4h + q carries, for tokens
// 4G .. 4G+3 of head h, the BF16 weights (q even) or their remainders (q
// odd: weight - its BF16 value, rounded again); rows 4h+2 and 4h+3 repeat
// rows 4h and 4h+1 and their products are never read.  Each lane packs its
// weight and remainder into one word; a quad broadcast gives every lane of
// the quad the four tokens' words, and v_perm keeps the halves of its row.
// sel: 0x05040100 (q even, low halves) or 0x07060302 (q odd, high halves).
// WSUM (INT4 pages): the two parts' sum, the weight the products actually
// carry, is added to `wsum` (the code offsets are taken out with it, so that
// the rounding of the remainder does not leave a multiple of the offset).
template <bool WSUM = false>
__device__ __forceinline__ bf16x4_t weight_operand(float w, uint32_t sel, float* wsum = nullptr) {
  const uint32_t h = pack_bf16_rne(w, 0.f);
  const float whi = bf16_lo(h);
  const uint32_t hr = pack_bf16_rne(w, w - whi);             // [BF16(w) | BF16(remainder)]
  if constexpr (WSUM) *wsum += whi + bf16_hi(hr);
  // quad_perm [c,c,c,c] (control 0x55 c): every lane of the quad gets lane c's word
  const uint32_t t0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)hr, 0x00, 0xF, 0xF, false);
  const uint32_t t1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)hr, 0x55, 0xF, 0xF, false);
  const uint32_t t2 = (uint32_t)__builtin_amdgcn_mov_dpp((int)hr, 0xAA, 0xF, 0xF, false);
  const uint32_t t3 = (uint32_t)__builtin_amdgcn_mov_dpp((int)hr, 0xFF, 0xF, 0xF, false);
  u32x2 a;
  a.x = __builtin_amdgcn_perm(t1, t0, sel);                  // tokens 4G, 4G+1
  a.y = __builtin_amdgcn_perm(t3, t2, sel);                  // tokens 4G+2, 4G+3
  return __builtin_bit_cast(bf16x4_t, a);
}

// B operands of the P V product for one page: tile t (16 output dims) as 4
// BF16 values, tokens 4G .. 4G+3 of this lane's column (BF16 pages: V of
// dead slots already zeroed; INT4: code + 24).
template <int FMT, typename Page>
__device__ __forceinline__ void page_v_operands(const Page& r, const PageConsts& pc, u32x2* bv) {
  if constexpr (FMT == kFmtINT4) {
    // tile e: dim 4n + e of tokens 4G .. 4G+3 (nibble e of each 16-bit unit);
    // dead slots hold finite widened codes and weight 0
    uint32_t x[4], y[4];
    nibble_pairs2<0>(r.v, pc.nib, x[0], y[0]);
    nibble_pairs2<1>(r.v, pc.nib, x[1], y[1]);
    nibble_pairs2<2>(r.v, pc.nib, x[2], y[2]);
    nibble_pairs2<3>(r.v, pc.nib, x[3], y[3]);
#pragma unroll
    for (int e = 0; e < 4; ++e) bv[e] = u32x2{x[e], y[e]};
  } else if constexpr (FMT == kFmtINT8) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      uint32_t e0, o0, e1, o1;
      codes_even_odd(r.v[h].x, e0, o0);                    // tokens 4G, 4G+1
      codes_even_odd(r.v[h].y, e1, o1);                    // tokens 4G+2, 4G+3
      bv[2 * h] = u32x2{e0, e1};
      bv[2 * h + 1] = u32x2{o0, o1};
    }
  } else {
#pragma unroll
    for (int b = 0; b < 4; ++b) bv[b] = r.v[b];
  }
}

// acc += A V for one page.
template <int FMT, typename Page>
__device__ __forceinline__ void page_pv(LaneState& st, const Page& r, bf16x4_t A,
                                        const PageConsts& pc) {
  u32x2 bv[4];
  page_v_operands<FMT>(r, pc, bv);
#pragma unroll
  for (int b = 0; b < 4; ++b)
    st.acc[b] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(A, __builtin_bit_cast(bf16x4_t, bv[b]),
                                                          st.acc[b], 0, 0, 0);
}

// The lane's weight (p: softmax numerator; w: the P V weight, p times the V
// scale for quantised pages), a dead slot (MASK, own token at or past
// `valid`) at 0.
template <int FMT, bool MASK, typename Page>
__device__ __forceinline__ float page_weight(LaneState& st, const Page& r, float x, bool dead) {
  const float p = __builtin_amdgcn_exp2f(x - st.m);         // masked: exp2(-inf) = 0
  float w = p;
  if constexpr (FMT != kFmtBF16) {
    w = p * __uint_as_float(r.vs);
    if (MASK) w = dead ? 0.f : w;                            // scale bits of a dead slot
  }
  st.l += p;
  return w;
}

// One page into the running state; MASK: only the first `valid` tokens exist.
template <int FMT, bool MASK, typename Page>
__device__ __forceinline__ void consume_page(LaneState& st, Page& r, bf16x8_t qlo, bf16x8_t qhi,
                                           const PageConsts& pc, int lane, int valid) {
  const int G = lane >> 4;            // token group: tokens 4G .. 4G+3
  const int q = lane & 3;             // own token 4G + q (head n / 4)
  float x = page_logit<FMT>(r, page_scores<FMT>(r, qlo, qhi, pc), pc.xscale, q);
  const bool dead = MASK && 4 * G + q >= valid;
  if (MASK) x = dead ? -INFINITY : x;
  raise_max(st, x, G);
  const float w = page_weight<FMT, MASK>(st, r, x, dead);
  const bf16x4_t A = weight_operand<FMT == kFmtINT4>(w, pc.sel, &st.wsum);
  if constexpr (FMT == kFmtBF16) {
    if (MASK) {
      // tokens 4G .. 4G+3 sit in (lo, hi) halves of the two words
      const uint32_t m0 = (4 * G < valid ? 0x0000ffffu : 0u) | (4 * G + 1 < valid ? 0xffff0000u : 0u);
      const uint32_t m1 = (4 * G + 2 < valid ? 0x0000ffffu : 0u) | (4 * G + 3 < valid ? 0xffff0000u : 0u);
#pragma unroll
      for (int b = 0; b < 4; ++b) r.v[b] = u32x2{r.v[b].x & m0, r.v[b].y & m1};
    }
  }
  page_pv<FMT>(st, r, A, pc);
}

// Two full pages at once: their score products are independent, one vote and
// at most one rescale covers both, and their P V products follow each other;
// the two dependency chains overlap instead of running one after the other.
template <int FMT, typename Page>
__device__ __forceinline__ void consume_pages2(LaneState& st, const Page& ra, const Page& rb,
                                               bf16x8_t qlo, bf16x8_t qhi, const PageConsts& pc,
                                               int lane) {
  const int G = lane >> 4;
  const int q = lane & 3;
  const f32x4_t sa = page_scores<FMT>(ra, qlo, qhi, pc);
  const f32x4_t sb = page_scores<FMT>(rb, qlo, qhi, pc);
  const float xa = page_logit<FMT>(ra, sa, pc.xscale, q);
  const float xb = page_logit<FMT>(rb, sb, pc.xscale, q);
  raise_max(st, fmaxf(xa, xb), G);
  const float wa = page_weight<FMT, false>(st, ra, xa, false);
  const float wb = page_weight<FMT, false>(st, rb, xb, false);
  // one product over 32 tokens per tile: k = 8G .. 8G+7 of this lane are
  // tokens 4G .. 4G+3 of page a, then of page b, in both operands
  const bf16x4_t Aa = weight_operand<FMT == kFmtINT4>(wa, pc.sel, &st.wsum);
  const bf16x4_t Ab = weight_operand<FMT == kFmtINT4>(wb, pc.sel, &st.wsum);
  const u32x4 A8 = {__builtin_bit_cast(u32x2, Aa).x, __builtin_bit_cast(u32x2, Aa).y,
                    __builtin_bit_cast(u32x2, Ab).x, __builtin_bit_cast(u32x2, Ab).y};
  u32x2 va[4], vb[4];
  page_v_operands<FMT>(ra, pc, va);
  page_v_operands<FMT>(rb, pc, vb);
#pragma unroll
  for (int b = 0; b < 4; ++b)
    st.acc[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
        __builtin_bit_cast(bf16x8_t, A8), __builtin_bit_cast(bf16x8_t, u32x4{va[b].x, va[b].y, vb[b].x, vb[b].y}),
        st.acc[b], 0, 0, 0);
}

// Output dim of column n of tile b: BF16 pages, tile b = dims 16b .. 16b+15;
// INT8 pages, tile 2h + e = dims 32h + 8(n/4) + 2(n%4) + e; INT4 pages, tile
// e = dims 4n + e.
template <int FMT>
__device__ __forceinline__ int out_dim(int b, int n) {
  if constexpr (FMT == kFmtINT8) return 32 * (b >> 1) + 8 * (n >> 2) + 2 * (n & 3) + (b & 1);
  if constexpr (FMT == kFmtINT4) return 4 * n + b;
  return 16 * b + n;
}

// The new K/V row of KV head g straight into the pool (no LDS parking): lane
// c (K) and 4 + c (V), c = 0..3, hold the row parts {8c..8c+7} (lo) and
// {32+8c..} (hi); K is rotated first with RoPE at position `pos`, quantised
// pages quantise each row over its quad of lanes.  Lanes 0..7 call it
// together (the quantiser's quad reductions need all four lanes of a row).
template <int FMT, bool ROPE>
__device__ __forceinline__ void append_row_direct(const DecodeArgs& a, uint4 lo, uint4 hi, int id,
                                                  int slot, int pos, int g, int lane) {
  const int c = lane & 3;
  const bool is_k = lane < 4;
  if (ROPE && is_k) {
    const int64_t row = (int64_t)pos * (kD / 2) + 8 * c;
    rope_pairs8(lo, hi, a.rope_cos + row, a.rope_sin + row);
  }
  if constexpr (FMT == kFmtBF16) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(is_k ? a.k_pool_w : a.v_pool_w) +
                    (int64_t)id * kPageElems + slot * kRowElems + g * kD + 8 * c;
    *reinterpret_cast<uint4*>(dst) = lo;
    *reinterpret_cast<uint4*>(dst + 32) = hi;
  } else {
    using QL = QuantLayout<FMT>;
    u32x2 clo, chi;
    const float sc = quantize_quad_row<FMT>(lo, hi, clo, chi);
    uint8_t* row = reinterpret_cast<uint8_t*>(is_k ? a.k_pool_w : a.v_pool_w) +
                   (int64_t)id * QL::kPageBytes + g * QL::kHead + slot * QL::kRow;
    store_quad_codes<FMT>(row, c, clo, chi);
    if (c == 0) a.kv_scales_w[(int64_t)id * kScalePageFloats + (g * 2 + (is_k ? 0 : 1)) * kPage + slot] = sc;
  }
}

// WPH: wavefronts per KV head (1 or 2).  With 2, the two wavefronts of a head
// stream the first and second half of the split's pages, each with its own
// ring, and merge their running states through LDS at the end: the
// occupancy of two work-groups per CU without split partials or a merge
// launch.
template <int FMT, bool OUT_BF16, bool APPEND, bool ROPE = false, int WPH = 1, int RING = 0>
__global__ __launch_bounds__(kThreads * WPH, 2 * WPH) void decode_kernel(DecodeArgs a) {
  static_assert(WPH == 1 || WPH == 2, "one or two wavefronts per KV head");
  static_assert(!ROPE || APPEND, "RoPE is fused with the append");
  constexpr bool Q8 = FMT == kFmtINT8;
  constexpr bool Q4 = FMT == kFmtINT4;
  constexpr bool QUANT = Q8 || Q4;
  using F = PageFormat<FMT>;
  // a one-dimensional grid: block k is split k % S of sequence k / S (the
  // same dispatch order as a (S, B) grid, without its limit on B)
  int b = (int)(blockIdx.x / (unsigned)a.num_splits);
  int s = (int)blockIdx.x - b * a.num_splits;
  if (a.work) {
    // entries outside the batch or the plan are skipped, never followed
    b = a.work[2 * blockIdx.x];
    s = a.work[2 * blockIdx.x + 1];
    if ((unsigned)b >= (unsigned)a.batch || (unsigned)s >= (unsigned)a.num_splits) return;
  }
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = wave % kWaves;                  // KV head
  const int wh = wave / kWaves;                 // which half of the split's pages (WPH = 2)
  const int lane = threadIdx.x & 63;
  const int G = lane >> 4;
  const int n = lane & 15;

  // Everything that does not depend on the sequence's length is requested
  // together with it: the query rows and the block-table entries of this
  // split's window of the row.  The first pages can then be requested one
  // memory round trip after the start instead of two.
  const int p0 = s * a.pages_per_split;
  const int32_t* bt = a.block_tables + (int64_t)b * a.max_blocks;
  const int win = min(a.pages_per_split, a.max_blocks - p0);   // entries of the row in the window
  int ent[kMaxSplitPages / 64];
#pragma unroll
  for (int c = 0; c < kMaxSplitPages / 64; ++c) {
    const int j = c * 64 + lane;
    ent[c] = (c * 64 < win && j < win) ? bt[p0 + j] : 0;
  }
  uint4 q_lo, q_hi;
  {
    const uint16_t* qr = a.q + ((int64_t)b * kHq + kGroup * g + (n >> 2)) * kD + 8 * G;
    q_lo = *reinterpret_cast<const uint4*>(qr);
    q_hi = *reinterpret_cast<const uint4*>(qr + 32);
  }
  // fused append: lanes 0..3 hold the new K row of head g (lane c: dims
  // {8c..} and {32+8c..}), lanes 4..7 the V row; every split loads them, the
  // one holding the sequence's last page uses them
  // (every lane loads, lane l the row part of lane l % 8: a load under a
  // lane mask would make the compiler wait for it at the end of the mask)
  uint4 new_lo{}, new_hi{};
  if constexpr (APPEND) {
    const uint16_t* src = ((lane & 7) < 4 ? a.k_new : a.v_new) + ((int64_t)b * kHkv + g) * kD +
                          8 * (lane & 3);
    new_lo = *reinterpret_cast<const uint4*>(src);
    new_hi = *reinterpret_cast<const uint4*>(src + 32);
  }
  const int L = a.seq_lens[b];
  const int n_pages = (L + kPage - 1) / kPage;
  const bool bad_len = L < 0 || L > a.max_seq_len || n_pages > a.max_blocks ||
                       n_pages > a.pages_per_split * a.num_splits;
  const int n_splits_b = bad_len ? 1 : (n_pages + a.pages_per_split - 1) / a.pages_per_split;
  if (s >= (n_splits_b > 0 ? n_splits_b : 1)) return;

  if (L == 0 || bad_len) {
    float res[16];
    const float fill = bad_len ? __builtin_nanf("") : 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) res[e] = fill;
    if (n < kGroup) store_row16<OUT_BF16>(a.out, (int64_t)b * kHq + kGroup * g + n, G, res);
    // A length the call cannot attend (above max_seq_len, or beyond what the
    // plan's splits cover) still gets its new row, under the rule of the
    // separate append: 1 <= L <= 16 max_blocks and a valid page id (and, with
    // RoPE, a table row for position L-1).  Split 0's first wavefront of each
    // head writes it straight to the pool.
    if (APPEND && bad_len && wh == 0 && L >= 1 && n_pages <= a.max_blocks &&
        (!ROPE || L <= a.rope_positions)) {
      const int id = bt[n_pages - 1];
      if ((unsigned)id < (unsigned)a.num_pages && lane < 8)
        append_row_direct<FMT, ROPE>(a, new_lo, new_hi, id, (L - 1) % kPage, L - 1, g, lane);
    }
    return;
  }

  const int p1 = min(p0 + a.pages_per_split, n_pages);
  // this wavefront streams pages q0 .. last of the split (all of them for
  // WPH = 1; with WPH = 2 the second half may be empty)
  const int per = (p1 - p0 + WPH - 1) / WPH;
  const int q0 = p0 + wh * per;
  const int last = min(q0 + per, p1) - 1;
  const bool has_pages = q0 <= last;
  const int tail_valid = L - last * kPage;


  // B operand of the score product (set after the first page requests)
  bf16x8_t qlo, qhi;

  PageConsts pc;                 // xscale; INT4: the query bias and the widening constants
  pc.xscale = a.xscale;
  pc.qbias = 0.f;
  pc.sel = (n & 1) ? 0x07060302u : 0x05040100u;
  if constexpr (Q4) pc.nib = nibble_consts();

  // fused append: the new rows (K rotated first with RoPE) are parked in LDS,
  // as BF16 rows or as codes and scales, after the first page requests
  const bool app_here = APPEND && has_pages && last == n_pages - 1;
  const int app_slot = (L - 1) % kPage;
  __shared__ u32x4 new_rows[APPEND ? kWaves : 1][QUANT ? 8 : 16];   // 16-byte chunks
  __shared__ float new_scales[APPEND && QUANT ? kWaves : 1][2];

  LaneState st;
#pragma unroll
  for (int t = 0; t < 4; ++t) st.acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  st.m = -INFINITY;
  st.l = 0.f;
  st.wsum = 0.f;

  // ent[] (loaded above) holds the window's entries; only those up to
  // `last` are ever picked
  // a used entry of the split outside the pool (one vote over the window:
  // entry j of the row's window sits in lane j % 64 of ent[j / 64])
  int bad_page = 0;
  {
    bool mine = false;
#pragma unroll
    for (int c = 0; c < kMaxSplitPages / 64; ++c)
      mine |= p0 + c * 64 + lane < p1 && (unsigned)ent[c] >= (unsigned)a.num_pages;
    bad_page = __builtin_amdgcn_ballot_w64(mine) != 0;
  }
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
    return (unsigned)id < (unsigned)a.num_pages ? id : 0;   // a bad entry reads page 0 (outputs NaN)
  };

  // RING: slots per wavefront for this launch (0: the format's default).  A
  // one-slot ring still holds two slots of LDS, so that no more work-groups
  // share a CU than with two (more would put more pages in flight per CU than
  // its page stream runs fastest with).
  constexpr int kDepth = RING > 0 ? RING : F::kRingDepth;
  constexpr bool kPairs = PA_PAIR_STEPS && kDepth >= 3 && F::kPairs;
  __shared__ __attribute__((aligned(16))) char ring[kDepth < 2 ? 2 : kDepth][kWaves * WPH][F::kSlot];
  const char* k_base = reinterpret_cast<const char*>(a.k_pool);
  const char* v_base = reinterpret_cast<const char*>(a.v_pool);
  const char* s_base = reinterpret_cast<const char*>(a.kv_scales);
  const PageDma dma = page_dma<FMT>(g, lane, k_base, v_base);
  auto fetch = [&](int page, int slot) {
    page_fetch<FMT>(dma, k_base, v_base, s_base, page_id(page), 0u, 0u, &ring[slot][wave][0]);
  };
  // LDS read addresses of this lane in slot 0 of its wavefront
  const uint32_t slot0 = lds_address(&ring[0][wave][0]);
  constexpr uint32_t kRingSlotBytes = kWaves * WPH * F::kSlot;
  const int jq = n >> 2, jr = n & 3;              // transposed-read chunk: token 4G + jq
  uint32_t ka = 0, va = 0, sa = 0;
  SlotAddrBF16 ad{};
  if constexpr (Q8) {
    ka = slot0 + 64 * n + 8 * G;
    va = slot0 + 1024 + 64 * (4 * G + jq) + 8 * jr;
    sa = slot0 + 2048 + 4 * (4 * G + (n & 3));
  } else if constexpr (Q4) {
    // K: token n, bytes 8G .. 8G+7 (dims 16G .. 16G+15); V: dims 16 jr .. 16 jr
    // + 15 of token 4G + jq, so that lane n receives dims 4n .. 4n+3 of 4 tokens
    ka = slot0 + 32 * n + 8 * G;
    va = slot0 + 512 + 32 * (4 * G + jq) + 8 * jr;
    sa = slot0 + 1024 + 4 * (4 * G + (n & 3));
  } else {
    // K: token n, pieces G and G + 4; V block b (dims 16b .. 16b+15): dims
    // 4 jr .. 4 jr + 3 of token 4G + jq are bytes 8 (jr % 2) of piece 2b + jr/2
    ad.k0 = slot0 + bf16_slot_offset(n, G);
    ad.k1 = slot0 + bf16_slot_offset(n, G + 4);
#pragma unroll
    for (int bb = 0; bb < 4; ++bb)
      ad.v[bb] = slot0 + 2048 + bf16_slot_offset(4 * G + jq, 2 * bb + (jr >> 1)) + 8 * (jr & 1);
  }

  auto park_new_row = [&](uint32_t slot_base) {
    // overwrite the appended token's slot in the ring with the new row
    const int sl = APPEND ? g : 0;
    if constexpr (QUANT) {
      using QL = QuantLayout<Q8 ? kFmtINT8 : kFmtINT4>;
      if (lane < 8) {
        const u32x4 w = new_rows[sl][lane];
        uint8_t* row = reinterpret_cast<uint8_t*>(&ring[0][wave][0]) + (slot_base - slot0) +
                       (lane < 4 ? 0 : QL::kHead) + QL::kRow * app_slot;
        store_quad_codes<FMT>(row, lane & 3, u32x2{w.x, w.y}, u32x2{w.z, w.w});
      }
      if (lane < 2) {
        float* sp = reinterpret_cast<float*>(&ring[0][wave][0] + (slot_base - slot0) + 2 * QL::kHead);
        sp[lane * 16 + app_slot] = new_scales[APPEND && QUANT ? g : 0][lane];
      }
    } else {
      if (lane < 16) {
        // chunk lane: row lane/4 (K lo, K hi, V lo, V hi), part lane%4, i.e.
        // piece 4 (row % 2) + part of K (rows 0, 1) or V (rows 2, 3)
        const u32x4 w = reinterpret_cast<const u32x4*>(&new_rows[sl][0])[lane];
        const int row = lane >> 2;
        char* base = &ring[0][wave][0] + (slot_base - slot0) + 2048 * (row >> 1) +
                     bf16_slot_offset(app_slot, 4 * (row & 1) + (lane & 3));
        *reinterpret_cast<u32x4*>(base) = w;
      }
    }
  };

  using PageT = std::conditional_t<Q8, PageQ8, std::conditional_t<Q4, PageQ4, PageBF16>>;
  auto lds_read = [&](PageT& pg, uint32_t off) {
    if constexpr (QUANT) lds_page_issue(pg, ka + off, va + off, sa + off);
    else lds_page_issue(pg, ad, off);
  };
  auto step = [&](int i, auto masked) {
    constexpr bool MASK = decltype(masked)::value;
    const int slot = (i - q0) % kDepth;
    const uint32_t off = slot * kRingSlotBytes;
    wait_page<F::kLoads, kDepth>(min(last - i, kDepth - 1));   // page i landed
    if (MASK && app_here) park_new_row(slot0 + off);
    PageT cur;
    lds_read(cur, off);
    lds_page_ready(cur);
    if (i + kDepth <= last) fetch(i + kDepth, slot);
    consume_page<FMT, MASK>(st, cur, qlo, qhi, pc, lane, MASK ? tail_valid : kPage);
  };
  // pages i and i+1, both before the last page, in one pass, from ring slots
  // SA and SB (compile-time, so that the LDS reads take the slot offsets as
  // immediates); the ring keeps depth - 2 pages in flight while they are used
  auto step2 = [&](int i, auto slot_a, auto slot_b) {
    constexpr int SA = decltype(slot_a)::value, SB = decltype(slot_b)::value;
    wait_page<F::kLoads, kDepth>(min(last - i - 1, kDepth - 2));   // page i+1 landed
    PageT pa_, pb_;
    lds_page_issue<SA * kRingSlotBytes>(pa_, ka, va, sa);
    lds_page_issue<SB * kRingSlotBytes>(pb_, ka, va, sa);
    lds_page_ready(pa_);
    lds_page_ready(pb_);
    if (i + kDepth <= last) fetch(i + kDepth, SA);
    if (i + 1 + kDepth <= last) fetch(i + 1 + kDepth, SB);
    consume_pages2<FMT>(st, pa_, pb_, qlo, qhi, pc, lane);
  };

  // The prologue's loads (block-table window, query rows, new rows) were
  // requested together with the length and have arrived with it.  One
  // explicit wait for all of them, visible to the compiler's wait tracking,
  // keeps it from waiting on the page stream at their later uses.
  __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
#pragma unroll
  for (int r = 0; r < kDepth; ++r)
    if (q0 + r <= last) fetch(q0 + r, r);

  // while the first pages are in flight: the query operand and the new rows
  // B operand of the score product: column n = query head 4g + n/4, this
  // lane's 8 dims {8G..} (qlo) and {32+8G..} (qhi)
  {
    uint4 lo = q_lo, hi = q_hi;
    if (ROPE) {
      const int64_t row = (int64_t)(L - 1) * (kD / 2) + 8 * G;
      rope_pairs8(lo, hi, a.rope_cos + row, a.rope_sin + row);
    }
    if constexpr (Q4) {
      // lane G takes dims 16G .. 16G+15 (one 64-bit read of the K codes);
      // the offset of the widened codes over the row's 64 dims: this lane's
      // 16, then the 4 token groups
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
  if (app_here && lane < 8) {
    const int c = lane & 3;
    const bool is_k = lane < 4;
    uint4 lo = new_lo, hi = new_hi;
    if (ROPE && is_k) {
      const int64_t row = (int64_t)(L - 1) * (kD / 2) + 8 * c;
      rope_pairs8(lo, hi, a.rope_cos + row, a.rope_sin + row);
    }
    const int slot = APPEND ? g : 0;
    const uint32_t rows = lds_address(&new_rows[slot][0]);
    if constexpr (QUANT) {
      u32x2 clo, chi;
      const float sc = quantize_quad_row<FMT>(lo, hi, clo, chi);
      lds_store16(rows + 16 * lane, u32x4{clo.x, clo.y, chi.x, chi.y});
      if (c == 0) lds_store4(lds_address(&new_scales[APPEND && QUANT ? g : 0][is_k ? 0 : 1]), sc);
    } else {
      // [K lo parts 0..3 | K hi parts | V lo | V hi] in 16 chunks: 2 per lane
      lds_store16(rows + 16 * ((is_k ? 0 : 8) + c), u32x4{lo.x, lo.y, lo.z, lo.w});
      lds_store16(rows + 16 * ((is_k ? 0 : 8) + 4 + c), u32x4{hi.x, hi.y, hi.z, hi.w});
    }
  }
  if (has_pages) {
    int i = q0;
    if constexpr (kPairs) {
      // page i sits in slot (i - q0) % 3: the pairs cycle through slots
      // (0, 1), (2, 0), (1, 2)
      static_assert(kDepth == 3, "the pair loop is unrolled for a ring of three slots");
      using S0 = std::integral_constant<int, 0>;
      using S1 = std::integral_constant<int, 1>;
      using S2 = std::integral_constant<int, 2>;
      while (i + 1 < last) {
        step2(i, S0{}, S1{});
        i += 2;
        if (i + 1 >= last) break;
        step2(i, S2{}, S0{});
        i += 2;
        if (i + 1 >= last) break;
        step2(i, S1{}, S2{});
        i += 2;
      }
    }
    for (; i < last; ++i) step(i, std::false_type{});
    step(last, std::true_type{});
  }
  wait_vmem<0>();

  if (app_here && lane < (QUANT ? 8 : 16)) {
    const int id = raw_page_id(last);
    if ((unsigned)id < (unsigned)a.num_pages) {
      const int sl = APPEND ? g : 0;
      if constexpr (QUANT) {
        using QL = QuantLayout<Q8 ? kFmtINT8 : kFmtINT4>;
        const int c = lane & 3;
        const bool is_k = lane < 4;
        const u32x4 w = new_rows[sl][lane];
        uint8_t* row = reinterpret_cast<uint8_t*>(is_k ? a.k_pool_w : a.v_pool_w) +
                       (int64_t)id * QL::kPageBytes + g * QL::kHead + app_slot * QL::kRow;
        store_quad_codes<FMT>(row, c, u32x2{w.x, w.y}, u32x2{w.z, w.w});
        if (c == 0)
          a.kv_scales_w[(int64_t)id * kScalePageFloats + (g * 2 + (is_k ? 0 : 1)) * kPage + app_slot] =
              new_scales[APPEND && QUANT ? g : 0][is_k ? 0 : 1];
      } else {
        // chunk lane: K (lanes 0..7) or V (8..15); dims 8 (lane%4) (+32 for the hi parts)
        const u32x4 w = reinterpret_cast<const u32x4*>(&new_rows[sl][0])[lane];
        const int row = lane >> 2;                 // 0 K lo, 1 K hi, 2 V lo, 3 V hi
        uint16_t* dst = reinterpret_cast<uint16_t*>(row < 2 ? a.k_pool_w : a.v_pool_w) +
                        (int64_t)id * kPageElems + app_slot * kRowElems + g * kD +
                        32 * (row & 1) + 8 * (lane & 3);
        *reinterpret_cast<u32x4*>(dst) = w;
      }
    }
  }

  auto of_head = [G](float v) {                  // v of head G (from lane 4G)
    const float v0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const float v1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 4));
    const float v2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 8));
    const float v3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 12));
    return G == 0 ? v0 : (G == 1 ? v1 : (G == 2 ? v2 : v3));
  };

  if constexpr (WPH == 2) {
    // the second half's state joins the first through LDS, lane by lane (the
    // two wavefronts of a head have the same lane layout): the larger running
    // maximum is kept and each side is scaled by 2^(its maximum - the kept
    // one); the normaliser and weight sum belong to head n / 4, the
    // accumulator rows to head G, whose factors come from lane 4G
    constexpr int kXfer = 20;                    // 16 accumulators, m, l, wsum, bad-page flag
    __shared__ float xfer[kWaves][kXfer][64];
    if (wh == 1) {
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int rr = 0; rr < 4; ++rr) xfer[g][4 * t + rr][lane] = st.acc[t][rr];
      xfer[g][16][lane] = st.m;
      xfer[g][17][lane] = st.l;
      xfer[g][18][lane] = st.wsum;
      xfer[g][19][lane] = bad_page ? 1.f : 0.f;
    }
    __syncthreads();
    if (wh == 1) return;
    const float m1 = xfer[g][16][lane];
    const float mx = fmaxf(st.m, m1);            // the first half always holds a page
    const float a0 = __builtin_amdgcn_exp2f(st.m - mx);
    const float a1 = __builtin_amdgcn_exp2f(m1 - mx);   // an empty second half: m1 = -inf -> 0
    const float a0g = of_head(a0), a1g = of_head(a1);
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
        st.acc[t][rr] = st.acc[t][rr] * a0g + xfer[g][4 * t + rr][lane] * a1g;
    st.m = mx;
    st.l = st.l * a0 + xfer[g][17][lane] * a1;
    st.wsum = st.wsum * a0 + xfer[g][18][lane] * a1;
    bad_page |= xfer[g][19][lane] != 0.f;
  }

  // finish: the normaliser and weight sum of head n / 4 over its 16 lanes
  // (the quad and the four token groups); lane 16 G + n then takes head G's
  // values from lane 4G, and its tiles' rows 4G (BF16 weights) and 4G + 1
  // (remainders) add up to head G's unnormalised output at column n
  auto head_sum = [](float v) {
    v += dpp_mov<0xB1>(v);                       // quad_perm [1,0,3,2]
    v += dpp_mov<0x4E>(v);                       // quad_perm [2,3,0,1]
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
  };
  st.l = head_sum(st.l);
  float o[4];                                    // [tile]: head G, column n
#pragma unroll
  for (int t = 0; t < 4; ++t) o[t] = st.acc[t][0] + st.acc[t][1];
  if constexpr (Q4) {
    // the values were code + 136 (tile 0) or code + 24: take that times the
    // head's weight sum back out
    const float ws = of_head(head_sum(st.wsum));
#pragma unroll
    for (int t = 0; t < 4; ++t) o[t] -= q4_value_bias(t) * ws;
  }
  float m_out = of_head(st.m), l_out = of_head(st.l);
  if (bad_page) {
    m_out = __builtin_nanf("");
    l_out = __builtin_nanf("");
#pragma unroll
    for (int t = 0; t < 4; ++t) o[t] = __builtin_nanf("");
  }
  if (n_splits_b == 1) {
    const float inv = 1.f / l_out;
    const int64_t orow = ((int64_t)b * kHq + kGroup * g + G) * kD;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int d = out_dim<FMT>(t, n);
      if (OUT_BF16)
        reinterpret_cast<uint16_t*>(a.out)[orow + d] = (uint16_t)f32_to_bf16_rne(o[t] * inv);
      else
        reinterpret_cast<float*>(a.out)[orow + d] = o[t] * inv;
    }
  } else {
    const int64_t prow = ((int64_t)b * a.num_splits + s) * kHq + kGroup * g + G;
#pragma unroll
    for (int t = 0; t < 4; ++t) a.part_acc[prow * kD + out_dim<FMT>(t, n)] = o[t];
    if (n == 0) {
      a.part_ml[prow * 2 + 0] = m_out;
      a.part_ml[prow * 2 + 1] = l_out;
    }
  }
}

}  // namespace pa

namespace pa {

template <int FMT, int WPH, int RING = 0>
inline void launch_decode_kernel(const DecodeArgs& a, dim3 grid, bool out_bf16, bool fused,
                                 bool rope, hipStream_t st) {
  const dim3 block(kThreads * WPH);
  if (out_bf16) {
    if (rope) hipLaunchKernelGGL((decode_kernel<FMT, true, true, true, WPH, RING>), grid, block, 0, st, a);
    else if (fused) hipLaunchKernelGGL((decode_kernel<FMT, true, true, false, WPH, RING>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((decode_kernel<FMT, true, false, false, WPH, RING>), grid, block, 0, st, a);
  } else {
    if (rope) hipLaunchKernelGGL((decode_kernel<FMT, false, true, true, WPH, RING>), grid, block, 0, st, a);
    else if (fused) hipLaunchKernelGGL((decode_kernel<FMT, false, true, false, WPH, RING>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((decode_kernel<FMT, false, false, false, WPH, RING>), grid, block, 0, st, a);
  }
}

// Host: enqueue the decode kernel for page format FMT (plus the split merge
// when the plan has more than one split).  two_waves (INT4 pages only): two
// wavefronts per KV head, for plans whose grid fits the CUs at once (and
// whose splits are long; the caller decides).  two_slots (BF16 pages only):
// a two-slot ring instead of the default one slot (the caller decides).
// event_before/after (may be NULL) are recorded right around the decode
// kernel.  Returns a hipError_t.
template <int FMT>
inline hipError_t launch_decode(const DecodeArgs& a, int batch, bool out_bf16, bool fused,
                                bool rope, bool merge_preload, bool two_waves, bool two_slots,
                                hipStream_t st, hipEvent_t event_before, hipEvent_t event_after) {
  const dim3 grid = a.work ? dim3(a.num_work) : dim3(a.num_splits * batch);
  hipError_t e = hipSuccess;
  if (event_before && (e = hipEventRecord(event_before, st)) != hipSuccess) return e;
  if constexpr (FMT == kFmtINT4) {
    if (two_waves) launch_decode_kernel<FMT, 2>(a, grid, out_bf16, fused, rope, st);
    else launch_decode_kernel<FMT, 1>(a, grid, out_bf16, fused, rope, st);
  } else if constexpr (FMT == kFmtBF16) {
    if (two_slots) launch_decode_kernel<FMT, 1, 2>(a, grid, out_bf16, fused, rope, st);
    else launch_decode_kernel<FMT, 1>(a, grid, out_bf16, fused, rope, st);
  } else {
    launch_decode_kernel<FMT, 1>(a, grid, out_bf16, fused, rope, st);
  }
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (event_after && (e = hipEventRecord(event_after, st)) != hipSuccess) return e;
  if (a.num_splits > 1) {
    MergeArgs m;
    m.seq_lens = a.seq_lens;
    m.out = a.out;
    m.part_acc = a.part_acc;
    m.part_ml = a.part_ml;
    m.max_blocks = a.max_blocks;
    m.max_seq_len = a.max_seq_len;
    m.pages_per_split = a.pages_per_split;
    m.num_splits = a.num_splits;
    m.preload = merge_preload ? 1 : 0;
    if (out_bf16) hipLaunchKernelGGL(merge_kernel<true>, dim3(batch), dim3(256), 0, st, m);
    else hipLaunchKernelGGL(merge_kernel<false>, dim3(batch), dim3(256), 0, st, m);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pa
