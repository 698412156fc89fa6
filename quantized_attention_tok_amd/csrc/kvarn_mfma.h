// kvarn_mfma.h -- helpers shared by the head_dim-128 matrix-core kernels
// (decode and chunked prefill) on gfx950.
//
// Operand encoding used by both kernels (v_mfma_f32_16x16x32_f16):
//   - a 4-bit key code z enters as the fp16 bit pattern 16 z (a subnormal,
//     value 16 z 2^-24), a 2-bit value code as z 2^4 or z 2^6 in the same
//     way: the code sits in bits 4-7 of the half.  Measured on gfx950,
//     products with subnormals whose only set bits are 0-3 lose precision
//     (about 5e-7 of the summed term magnitudes), while bits 4-7 are as exact
//     as normal fp16 operands.
//   - an fp32 operand x is scaled by a power of two 2^k that puts the largest
//     magnitude of its row into [2^9, 2^10) and split into fp16 hi + lo
//     parts; two MFMAs (hi, lo) give each product to about 2^-22 relative,
//     accumulated in fp32.
#pragma once

#include "kvarn_device.h"

namespace kvarn {
namespace mfma {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ half8 as_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  u4 v = {a, b, c, d};
  return __builtin_bit_cast(half8, v);
}

__device__ __forceinline__ uint32_t pack_h2(_Float16 lo, _Float16 hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

// hi and lo fp16 parts of x (x = hi + lo to about 2^-22 relative)
__device__ __forceinline__ void split_h(float x, _Float16& hi, _Float16& lo) {
  hi = (_Float16)x;
  lo = (_Float16)(x - (float)hi);
}

// 2^k as a float for k in [-126, 127].
__device__ __forceinline__ float pow2i(int k) { return __uint_as_float((uint32_t)(k + 127) << 23); }

// Exponent k of the power of two 2^k that brings max|x| into [2^13, 2^14);
// 0 when the maximum is zero or tiny.
__device__ __forceinline__ int fp16_scale_exp(float amax) {
  const int eb = (int)((__float_as_uint(amax) >> 23) & 0xff);   // amax in [2^(eb-127), 2^(eb-126))
  int k = 140 - eb;
  if (eb == 0 || k > 100) k = 0;
  return k;
}

// Reductions over the four 16-lane rows of a wave (lanes n, n+16, n+32, n+48).
__device__ __forceinline__ float wave_max16(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  return fmaxf(v, __shfl_xor(v, 32, 64));
}
__device__ __forceinline__ float wave_sum16(float v) {
  v += __shfl_xor(v, 16, 64);
  return v + __shfl_xor(v, 32, 64);
}

// Two code bytes -> two fp16 halves with the byte's low / high nibble in bits
// 4-7: `x` holds the bytes in bits 0-7 and 16-23 (v_perm_b32 output).
__device__ __forceinline__ uint32_t nib_lo(uint32_t x) { return (x << 4) & 0x00F000F0u; }
__device__ __forceinline__ uint32_t nib_hi(uint32_t x) { return x & 0x00F000F0u; }

}  // namespace mfma
}  // namespace kvarn
