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


typedef __fp16 half2v __attribute__((ext_vector_type(2)));

// Bytes p[0] and p[off] in bits 0-7 and 16-23 (built as two 16-bit lanes, so
// the compiler joins the two LDS byte loads with one v_perm_b32).
typedef unsigned short ushort2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t byte_pair(const uint8_t* p, int off) {
  ushort2v t;
  t.x = p[0];
  t.y = p[off];
  return __builtin_bit_cast(uint32_t, t);
}

// fp16 hi + lo parts of (a, b): hi rounds toward zero, lo holds the rest.
__device__ __forceinline__ void split_pair(float a, float b, uint32_t& hi, uint32_t& lo) {
  const half2v h = __builtin_amdgcn_cvt_pkrtz(a, b);
  const half2v l = __builtin_amdgcn_cvt_pkrtz(a - (float)h.x, b - (float)h.y);
  hi = __builtin_bit_cast(uint32_t, h);
  lo = __builtin_bit_cast(uint32_t, l);
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// value of lane (lane ^ M), M < 16, on the DPP paths (no LDS round trip):
// lane ^ 4 is the half-row mirror (lane ^ 7) followed by quad_perm [3,2,1,0]
template <int M>
__device__ __forceinline__ float xshfl(float v) {
  if constexpr (M == 1) return dpp_f<0xB1>(v);        // quad_perm [1,0,3,2]
  else if constexpr (M == 2) return dpp_f<0x4E>(v);   // quad_perm [2,3,0,1]
  else if constexpr (M == 8) return dpp_f<0x128>(v);  // row_ror:8
  else return dpp_f<0x1B>(dpp_f<0x141>(v));           // M == 4: row_half_mirror, quad_perm [3,2,1,0]
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}
// Reductions over the 16 lanes of a DPP row (every lane of the row gets it).
// The max runs on an integer key with the order of the floats (negative
// values have their magnitude bits flipped), which needs no NaN handling.
__device__ __forceinline__ float row_max16(float v) {
  int k = __float_as_int(v);
  k ^= (k >> 31) & 0x7FFFFFFF;
  k = max(k, dpp_i<0x128>(k));   // row_ror:8
  k = max(k, dpp_i<0x124>(k));   // row_ror:4
  k = max(k, dpp_i<0x122>(k));   // row_ror:2
  k = max(k, dpp_i<0x121>(k));   // row_ror:1
  return __int_as_float(k ^ ((k >> 31) & 0x7FFFFFFF));
}
__device__ __forceinline__ float row_sum16(float v) {
  v += dpp_f<0x128>(v);
  v += dpp_f<0x124>(v);
  v += dpp_f<0x122>(v);
  return v + dpp_f<0x121>(v);
}
__device__ __forceinline__ float lane_f(float v, int l) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), l));
}
// whole-wave reductions (every lane gets the result): within the 16-lane rows
// by DPP, across the rows by permlane swaps
__device__ __forceinline__ float wmax(float v) {
  v = row_max16(v);
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float wsum(float v) {
  v = row_sum16(v);
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Walsh-Hadamard butterfly on lane bit M: lower lane a + b, upper lane a - b.
// Bits 16 and 32 use the gfx950 permlane swaps: a swap of x with itself gives
// the lower lane (own, partner) and the upper lane (partner, own).
template <int M>
__device__ __forceinline__ float bfly(float x, int lane) {
  const float sg = __int_as_float(0x3F800000 | ((lane & M) ? 0x80000000 : 0));
  if constexpr (M >= 16) {
    const auto r = (M == 32) ? __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false)
                             : __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaf(sg, __uint_as_float(r[1]), __uint_as_float(r[0]));
  } else {
    return xshfl<M>(x) + x * sg;
  }
}

}  // namespace mfma
}  // namespace kvarn
