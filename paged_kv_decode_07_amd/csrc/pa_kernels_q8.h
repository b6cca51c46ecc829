// INT8 K/V page format for gfx950: constants, the quantiser and the code
// widening used by the decode kernel.
//
// Format: K and V codes are int8 [num_pages][8 KV heads][16 slots][64 dims]:
// within a page, each KV head's 16 token rows of codes are one contiguous
// 1 KiB block (a wavefront streams whole 128-byte lines of its own head).
// Each (token, KV head) row of 64 values has its own FP32 scale, kept in a
// scale pool [num_pages][8 KV heads][2 (K, V)][16 slots] (1 KiB per page, one
// 128-byte line per head).  A row is quantised symmetrically: scale =
// max|x| / 127 (FP32, correctly rounded), code = the FP32 quotient x / scale
// rounded to nearest even and clamped to [-128, 127]; an all-zero row has
// scale 0 and codes 0.  The value a code stands for is code * scale.  (INT8
// KV cache dequantised before attention and the symmetric quantiser:
// "Building an LLM inference engine from scratch: KV cache, operator fusion
// and quantisation practice", sections 5.1 and 3.4.)
#pragma once

#include "pa_kernels.h"

namespace pa {

constexpr int kHeadCodes = kPage * kD;           // 1 KiB: one head's 16 rows in a page
constexpr int kPageCodes = kHkv * kHeadCodes;    // 8 KiB per page (K or V)
constexpr int kScalePageFloats = kHkv * 2 * kPage;   // 256 floats = 1 KiB per page
#ifndef PA_Q8_RING_DEPTH
#define PA_Q8_RING_DEPTH 2
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

}  // namespace pa
