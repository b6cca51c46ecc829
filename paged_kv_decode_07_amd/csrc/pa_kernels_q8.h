// Quantised K/V page formats for gfx950 (INT8 and INT4): constants, the
// quantiser and the code widening used by the decode kernel.
//
// INT8 format: K and V codes are int8 [num_pages][8 KV heads][16 slots][64
// dims]: within a page, each KV head's 16 token rows of codes are one
// contiguous 1 KiB block (a wavefront streams whole 128-byte lines of its own
// head).  Each (token, KV head) row of 64 values has its own FP32 scale, kept
// in a scale pool [num_pages][8 KV heads][2 (K, V)][16 slots] (1 KiB per
// page, one 128-byte line per head).  A row is quantised symmetrically: scale
// = max|x| / 127 (FP32, correctly rounded), code = the FP32 quotient x /
// scale rounded to nearest even and clamped to [-128, 127]; an all-zero row
// has scale 0 and codes 0.  The value a code stands for is code * scale.
//
// INT4 format: the same quantiser with 4 bits (scale = max|x| / 7, codes
// clamped to [-8, 7]) and the same scale pool; two codes per byte, each
// stored as code + 8, dim 2j in the low nibble of byte j of the row.  K and V
// are uint8 [num_pages][8][16][32]: one head's 16 rows are a 512-byte block.
//
// (The KV cache stored in INT8 or INT4 and dequantised for attention, and the
// symmetric quantiser: "Building an LLM inference engine from scratch: KV
// cache, operator fusion and quantisation practice", sections 5.1 and 3.4.)
#pragma once

#include "pa_kernels.h"

namespace pa {

// Page formats of the decode kernel.
constexpr int kFmtBF16 = 0;
constexpr int kFmtINT8 = 1;
constexpr int kFmtINT4 = 2;

constexpr int kHeadCodes = kPage * kD;           // 1 KiB: one head's 16 rows in a page
constexpr int kPageCodes = kHkv * kHeadCodes;    // 8 KiB per page (K or V)
constexpr int kScalePageFloats = kHkv * 2 * kPage;   // 256 floats = 1 KiB per page
// Ring depths (build-time; the measured best).  INT8 pages: 2 (a deeper ring
// would turn on the two-page pass, which the grid kernel only has for INT4
// pages).  INT4 pages: 3, the depth its two-page pass is unrolled for, or 2.
#ifndef PA_Q8_RING_DEPTH
#define PA_Q8_RING_DEPTH 2
#endif
constexpr int kRingQ8 = PA_Q8_RING_DEPTH;
constexpr int kSlotQ8 = 1024 + 1024 + 256;       // K codes, V codes, scales (2 x 128 B used)
static_assert(kRingQ8 >= 2 && kRingQ8 * kWaves * kSlotQ8 <= 160 * 1024, "INT8 LDS ring too large");

constexpr int kRowBytes4 = kD / 2;               // 32 bytes: one row of INT4 codes
constexpr int kHeadCodes4 = kPage * kRowBytes4;  // 512 bytes: one head's 16 rows in a page
constexpr int kPageCodes4 = kHkv * kHeadCodes4;  // 4 KiB per page (K or V)
#ifndef PA_Q4_RING_DEPTH
#define PA_Q4_RING_DEPTH 3
#endif
constexpr int kRingQ4 = PA_Q4_RING_DEPTH;
constexpr int kSlotQ4 = 512 + 512 + 256;         // K codes, V codes, scales (2 x 128 B used)
static_assert(kRingQ4 >= 2 && kRingQ4 * kWaves * kSlotQ4 <= 160 * 1024, "INT4 LDS ring too large");

// Code bytes of one row, one head's block and one page, per quantised format.
template <int FMT>
struct QuantLayout {
  static_assert(FMT == kFmtINT8 || FMT == kFmtINT4, "quantised format");
  static constexpr int kRow = FMT == kFmtINT8 ? kD : kRowBytes4;
  static constexpr int kHead = kPage * kRow;
  static constexpr int kPageBytes = kHkv * kHead;
  static constexpr float kQmax = FMT == kFmtINT8 ? 127.f : 7.f;
};

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

// INT4 widening without a conversion.  A nibble u at bits 3..6 of a 16-bit
// unit becomes the BF16 word 0x4180 | (u << 3), exactly 16 + u = code + 24;
// the first nibble of the unit (bits 0..3) becomes 0x4300 | u, exactly
// 128 + u = code + 136, which needs no shift.  The products of such values
// with BF16 operands are exact, and the offsets are taken out afterwards
// (each times the sum of the other operand over the dims it applies to).
constexpr float kNibbleBias4 = 24.f;        // nibbles 1, 2, 3 of a 16-bit unit
constexpr float kNibbleBias4First = 136.f;  // nibble 0
// The constants of the widening, held in registers the compiler cannot see
// through (an empty asm statement hides their values; the compiler itself
// materialises them), so that mask-and-bias is one v_and_or_b32 (a VALU
// instruction here takes one scalar operand and no literal besides it).
struct NibbleConsts {
  uint32_t mask;    // 0x00780078: bits 3..6 of each half
  uint32_t bias;    // 0x41804180: BF16 16.0 in each half
  uint32_t mask0;   // 0x000F000F: bits 0..3 of each half
  uint32_t bias0;   // 0x43004300: BF16 128.0 in each half
};
__device__ __forceinline__ NibbleConsts nibble_consts() {
  NibbleConsts c{0x00780078u, 0x41804180u, 0x000f000fu, 0x43004300u};
  asm volatile("" : "+s"(c.mask), "+v"(c.bias), "+s"(c.mask0), "+v"(c.bias0));
  return c;
}
// A right shift of a register pair as one 64-bit value (the compiler makes
// it a funnel shift and a shift; an instruction written in inline asm would
// escape its hazard tracking, e.g. against the accumulators of a matrix
// product still in flight).
template <int S>
__device__ __forceinline__ u32x2 shr64(u32x2 w) {
  const uint64_t v = (((uint64_t)w.y << 32) | w.x) >> S;
  return u32x2{(uint32_t)v, (uint32_t)(v >> 32)};
}
// Nibble pair E (bits 4E .. 4E+3 and 16+4E .. 16+4E+3) of w.x and of w.y ->
// a BF16 pair for each (the first in the low half).  Nibble 0 is masked in
// place; nibbles 1..3 take one 64-bit shift for both words (the bits it
// carries from w.y into w.x fall outside the mask).
template <int E>
__device__ __forceinline__ void nibble_pairs2(u32x2 w, const NibbleConsts& k, uint32_t& o0,
                                              uint32_t& o1) {
  if constexpr (E == 0) {
    o0 = (w.x & k.mask0) | k.bias0;
    o1 = (w.y & k.mask0) | k.bias0;
  } else {
    const u32x2 f = shr64<4 * E - 3>(w);
    o0 = (f.x & k.mask) | k.bias;
    o1 = (f.y & k.mask) | k.bias;
  }
}
// Two words of 8 INT4 codes each (16 consecutive dims of a row) -> 8 BF16
// values per word in the dim order 0 4 1 5 2 6 3 7 (dims 0 and 4 of each
// word code + 136, the others code + 24).
__device__ __forceinline__ void nibbles_to_bf16x8x2(u32x2 w, const NibbleConsts& k,
                                                    bf16x8_t& b0, bf16x8_t& b1) {
  uint32_t a[4], b[4];
  nibble_pairs2<0>(w, k, a[0], b[0]);
  nibble_pairs2<1>(w, k, a[1], b[1]);
  nibble_pairs2<2>(w, k, a[2], b[2]);
  nibble_pairs2<3>(w, k, a[3], b[3]);
  b0 = __builtin_bit_cast(bf16x8_t, u32x4{a[0], a[1], a[2], a[3]});
  b1 = __builtin_bit_cast(bf16x8_t, u32x4{b[0], b[1], b[2], b[3]});
}
// The matching reorder of 8 BF16 values (dims 0..7 -> 0 4 1 5 2 6 3 7), for
// the operand the INT4 codes are multiplied with.
__device__ __forceinline__ uint4 interleave_halves8(uint4 q) {
  return make_uint4(__builtin_amdgcn_perm(q.z, q.x, 0x05040100u),
                    __builtin_amdgcn_perm(q.z, q.x, 0x07060302u),
                    __builtin_amdgcn_perm(q.w, q.y, 0x05040100u),
                    __builtin_amdgcn_perm(q.w, q.y, 0x07060302u));
}

// INT4 pages: lane 16 G + n of the score product holds dims 16G .. 16G+15 of
// its query row (lo: 16G .., hi: 16G+8 ..), one 64-bit LDS read of the
// token's codes.  From the standard layout (lo: dims 8G .., hi: 32+8G ..)
// the lanes of column n exchange their parts: dims 16G.. are the lo (G < 2)
// or hi (G >= 2) part of lane G' = 2G mod 4, dims 16G+8.. that of lane
// G' + 1.  All 64 lanes must be active.
__device__ __forceinline__ void q4_relayout(uint4& lo, uint4& hi, int lane) {
  const int G = lane >> 4, n = lane & 15;
  const int src0 = 16 * ((2 * G) & 3) + n, src1 = src0 + 16;
  const bool upper = G >= 2;
  const uint32_t l[4] = {lo.x, lo.y, lo.z, lo.w}, h[4] = {hi.x, hi.y, hi.z, hi.w};
  uint32_t o0[4], o1[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const uint32_t a0 = (uint32_t)__shfl((int)l[k], src0), b0 = (uint32_t)__shfl((int)h[k], src0);
    const uint32_t a1 = (uint32_t)__shfl((int)l[k], src1), b1 = (uint32_t)__shfl((int)h[k], src1);
    o0[k] = upper ? b0 : a0;
    o1[k] = upper ? b1 : a1;
  }
  lo = make_uint4(o0[0], o0[1], o0[2], o0[3]);
  hi = make_uint4(o1[0], o1[1], o1[2], o1[3]);
}
// INT4 pages: this lane's part of the offset of the score product, in the
// layout of q4_relayout: 24 x the sum of its 16 query values plus (136 - 24)
// x those at dims 0, 4, 8, 12 of them (the first nibbles of the 16-bit
// code units).  The column's offset is the sum over the 4 lanes G.
__device__ __forceinline__ float q4_bias_part(uint4 lo, uint4 hi) {
  const uint32_t w[8] = {lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
  float sum = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) sum += bf16_lo(w[k]) + bf16_hi(w[k]);
  const float first = (bf16_lo(lo.x) + bf16_lo(lo.z)) + (bf16_lo(hi.x) + bf16_lo(hi.z));
  return kNibbleBias4 * sum + (kNibbleBias4First - kNibbleBias4) * first;
}
// INT4 pages: the value offset of output tile e (dims 4n + e: tile 0 holds
// the first nibbles)
__device__ __forceinline__ constexpr float q4_value_bias(int e) {
  return e == 0 ? kNibbleBias4First : kNibbleBias4;
}

// One quantised row of 64 values is held by a quad of lanes: lane c (0..3)
// of the quad has dims {8c .. 8c+7} (lo) and {32+8c .. 32+8c+7} (hi) as
// BF16.  All four lanes of the quad must be active.
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
// 8 codes in [-8, 7] -> one word, code + 8 per nibble, r[0] lowest.
__device__ __forceinline__ uint32_t pack_nibbles8(const float* r) {
  uint32_t w = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) w |= (uint32_t)((int32_t)r[k] + 8) << (4 * k);
  return w;
}
// The quad's row quantised to the format's codes.  Returns the row's scale
// and this lane's codes: INT8 c_lo, c_hi hold 8 bytes each (dims in order);
// INT4 c_lo.x, c_hi.x hold 8 nibbles each (c_lo.y, c_hi.y are 0).
template <int FMT>
__device__ __forceinline__ float quantize_quad_row(uint4 lo, uint4 hi, u32x2& c_lo, u32x2& c_hi) {
  constexpr float qmax = QuantLayout<FMT>::kQmax;
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
  const float scale = amax / qmax;                  // correctly rounded FP32 division
  float r[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const float q = scale == 0.f ? 0.f : __builtin_rintf(x[e] / scale);   // ties to even
    r[e] = fminf(fmaxf(q, -qmax - 1.f), qmax);
  }
  if constexpr (FMT == kFmtINT8) {
    c_lo = u32x2{pack_codes4(r), pack_codes4(r + 4)};
    c_hi = u32x2{pack_codes4(r + 8), pack_codes4(r + 12)};
  } else {
    c_lo = u32x2{pack_nibbles8(r), 0u};
    c_hi = u32x2{pack_nibbles8(r + 8), 0u};
  }
  return scale;
}
// Store a quad lane's codes into its row (row = the row's first code byte).
template <int FMT>
__device__ __forceinline__ void store_quad_codes(uint8_t* row, int c, u32x2 c_lo, u32x2 c_hi) {
  if constexpr (FMT == kFmtINT8) {
    *reinterpret_cast<u32x2*>(row + 8 * c) = c_lo;
    *reinterpret_cast<u32x2*>(row + 32 + 8 * c) = c_hi;
  } else {
    *reinterpret_cast<uint32_t*>(row + 4 * c) = c_lo.x;
    *reinterpret_cast<uint32_t*>(row + 16 + 4 * c) = c_hi.x;
  }
}

}  // namespace pa
