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

// INT4 widening without a conversion: the BF16 word 0x4180 | (u << 3) is
// exactly 16 + u for a nibble u, i.e. code + 24.  The products of such values
// with BF16 operands are exact, and the bias is taken out afterwards (24 x
// the sum of the other operand).  kNibbleBias4 is that offset.
constexpr float kNibbleBias4 = 24.f;
// The two constants of the widening, held in registers the compiler cannot
// see through, so that mask-and-bias is one v_and_or_b32 (a VALU instruction
// here takes one scalar operand and no literal besides it).
struct NibbleConsts {
  uint32_t mask;   // 0x00780078: bits 3..6 of each half
  uint32_t bias;   // 0x41804180: BF16 16.0 in each half
};
__device__ __forceinline__ NibbleConsts nibble_consts() {
  NibbleConsts c;
  asm volatile("s_mov_b32 %0, 0x00780078" : "=s"(c.mask));
  asm volatile("v_mov_b32 %0, 0x41804180" : "=v"(c.bias));
  return c;
}
// Nibble pair at bits 4E .. 4E+3 and 16+4E .. 16+4E+3 of w0 and of w1 -> a
// BF16 pair for each (code + 24 each; the first in the low half).  One 64-bit
// shift serves both words: the bits it carries across them fall outside the
// mask.
template <int E>
__device__ __forceinline__ void nibble_pairs2(uint32_t w0, uint32_t w1, const NibbleConsts& k,
                                              uint32_t& o0, uint32_t& o1) {
  const uint64_t w = ((uint64_t)w1 << 32) | w0;
  uint64_t f;
  if constexpr (E == 0) f = w << 3;
  else f = w >> (4 * E - 3);
  o0 = ((uint32_t)f & k.mask) | k.bias;
  o1 = ((uint32_t)(f >> 32) & k.mask) | k.bias;
}
// Two words of 8 INT4 codes each (dims 0..7 of a row piece) -> 8 BF16 values
// code + 24 per word, in the dim order 0 4 1 5 2 6 3 7.
__device__ __forceinline__ void nibbles_to_bf16x8x2(uint32_t w0, uint32_t w1, const NibbleConsts& k,
                                                    bf16x8_t& b0, bf16x8_t& b1) {
  uint32_t a[4], b[4];
  nibble_pairs2<0>(w0, w1, k, a[0], b[0]);
  nibble_pairs2<1>(w0, w1, k, a[1], b[1]);
  nibble_pairs2<2>(w0, w1, k, a[2], b[2]);
  nibble_pairs2<3>(w0, w1, k, a[3], b[3]);
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
