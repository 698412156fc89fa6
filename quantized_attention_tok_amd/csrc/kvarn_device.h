// kvarn_device.h -- small device helpers shared by the KVarN HIP kernels
// (gfx950, wave64).  Record layout constants follow the tile record described
// in include/kvarn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvarn {

constexpr int kTile = 128;   // tokens per tile
constexpr int kWave = 64;    // CDNA wavefront width

// Byte offsets of the record sections for head_dim D: codes, then the six
// scale vectors as fp32 (H = false, 116 D + 512 bytes) or as f16 rounded to
// nearest-even (H = true, 106 D + 256 bytes; SharpInference issue #433
// item 3, "f16 scales").
template <int D, bool H = false>
struct Rec {
  static constexpr int sb = H ? 2 : 4;   // bytes per stored scale
  static constexpr int kcode = 0;
  static constexpr int vcode = 64 * D;
  static constexpr int ktok = 96 * D;
  static constexpr int kscale = ktok + 128 * sb;
  static constexpr int kmin = kscale + D * sb;
  static constexpr int vchan = kmin + D * sb;
  static constexpr int vscale = vchan + D * sb;
  static constexpr int vmin = vscale + D * sb;
  static constexpr int bytes = vmin + D * sb;
  static constexpr int groups = D / 128;
};
static_assert(Rec<128>::bytes == 116 * 128 + 512 && Rec<128, true>::bytes == 106 * 128 + 256, "layout");

__host__ __device__ inline int64_t tile_bytes_rt(int d, bool h = false) {
  return h ? 106LL * d + 256 : 116LL * d + 512;
}

// Record layout for kb-bit keys and vb-bit values (gmlx PR #116 commit list:
// key and value widths chosen on their own, 1..8 bits).  The codes are LSB-
// first bit streams: key channel c's stream is 16 kb bytes with token t at bit
// kb t; value token t's stream is d vb / 8 bytes with channel c at bit vb c.
// For kb = 4, vb = 2 this is Rec<D, H> (nibbles and crumbs).
struct RecRT {
  int kcode, vcode, ktok, kscale, kmin, vchan, vscale, vmin, bytes;
};
__host__ __device__ inline RecRT rec_rt(int d, bool h, int kb, int vb) {
  const int sb = h ? 2 : 4;
  RecRT r;
  r.kcode = 0;
  r.vcode = 16 * kb * d;
  r.ktok = r.vcode + 16 * vb * d;
  r.kscale = r.ktok + 128 * sb;
  r.kmin = r.kscale + d * sb;
  r.vchan = r.kmin + d * sb;
  r.vscale = r.vchan + d * sb;
  r.vmin = r.vscale + d * sb;
  r.bytes = r.vmin + d * sb;
  return r;
}

// Scale element i of a section at p (fp32 or f16 storage), as fp32.
template <bool H>
__device__ __forceinline__ float sc_ld(const uint8_t* p, int i) {
  if constexpr (H) return (float)reinterpret_cast<const _Float16*>(p)[i];
  else return reinterpret_cast<const float*>(p)[i];
}
// elements i, i + 1 (i even)
template <bool H>
__device__ __forceinline__ float2 sc_ld2(const uint8_t* p, int i) {
  if constexpr (H) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 x = *reinterpret_cast<const h2*>(p + 2 * i);
    return make_float2((float)x[0], (float)x[1]);
  } else {
    return *reinterpret_cast<const float2*>(p + 4 * i);
  }
}
// elements i .. i + 3 (i a multiple of 4)
template <bool H>
__device__ __forceinline__ float4 sc_ld4(const uint8_t* p, int i) {
  if constexpr (H) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    const h4 x = *reinterpret_cast<const h4*>(p + 2 * i);
    return make_float4((float)x[0], (float)x[1], (float)x[2], (float)x[3]);
  } else {
    return *reinterpret_cast<const float4*>(p + 4 * i);
  }
}
// Raw buffer loads from one record.  The resource holds the record's base
// address and size (a load past the size returns zeros); a load's offset is
// a lane-dependent byte offset in a VGPR plus a uniform byte offset, so a
// group of loads that differ by constants shares one address register.
typedef __amdgpu_buffer_rsrc_t brsrc;
__device__ __forceinline__ brsrc make_rsrc(const uint8_t* p, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p), (short)0, bytes, 0x00020000);
}
// scale element i_lane + i_const of the section at byte `sec` (fp32 or f16 storage)
template <bool H>
__device__ __forceinline__ float sc_bl(brsrc r, int sec, int i_lane, int i_const) {
  if constexpr (H) {
    const auto x = __builtin_amdgcn_raw_buffer_load_b16(r, 2 * i_lane, sec + 2 * i_const, 0);
    return (float)__builtin_bit_cast(_Float16, x);
  } else {
    return __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r, 4 * i_lane, sec + 4 * i_const, 0));
  }
}
// elements i, i + 1 (i even)
template <bool H>
__device__ __forceinline__ float2 sc_bl2(brsrc r, int sec, int i_lane, int i_const) {
  if constexpr (H) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    const h2 x = __builtin_bit_cast(h2, __builtin_amdgcn_raw_buffer_load_b32(r, 2 * i_lane, sec + 2 * i_const, 0));
    return make_float2((float)x[0], (float)x[1]);
  } else {
    typedef float f2 __attribute__((ext_vector_type(2)));
    const f2 x = __builtin_bit_cast(f2, __builtin_amdgcn_raw_buffer_load_b64(r, 4 * i_lane, sec + 4 * i_const, 0));
    return make_float2(x[0], x[1]);
  }
}
// elements i .. i + 3 (i a multiple of 4)
template <bool H>
__device__ __forceinline__ float4 sc_bl4(brsrc r, int sec, int i_lane, int i_const) {
  if constexpr (H) {
    typedef _Float16 h4 __attribute__((ext_vector_type(4)));
    const h4 x = __builtin_bit_cast(h4, __builtin_amdgcn_raw_buffer_load_b64(r, 2 * i_lane, sec + 2 * i_const, 0));
    return make_float4((float)x[0], (float)x[1], (float)x[2], (float)x[3]);
  } else {
    typedef float f4 __attribute__((ext_vector_type(4)));
    const f4 x = __builtin_bit_cast(f4, __builtin_amdgcn_raw_buffer_load_b128(r, 4 * i_lane, sec + 4 * i_const, 0));
    return make_float4(x[0], x[1], x[2], x[3]);
  }
}
// 16 code bytes at byte voff + soff
typedef uint32_t u32x4b __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4b code_bl(brsrc r, int voff, int soff) {
  return __builtin_bit_cast(u32x4b, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}

// store element i.  f16: the fp32 value v is rounded to nearest-even half.
// The empty asm pins v as an fp32 register value: without it the compiler
// folds a producing multiply into v_fma_mixlo_f16, which rounds the exact
// product to half once instead of rounding the fp32 scale.
template <bool H>
__device__ __forceinline__ void sc_st(uint8_t* p, int i, float v) {
  if constexpr (H) {
    asm("" : "+v"(v));
    reinterpret_cast<_Float16*>(p)[i] = (_Float16)v;
  } else {
    reinterpret_cast<float*>(p)[i] = v;
  }
}

// fp32(1/sqrt(D)): 2^-k/2 for even log2(D); otherwise the rounded sqrt(2)
// scaled by a power of two (exact scaling, so still correctly rounded).
template <int D>
__device__ __forceinline__ float wht_scale() {
  if constexpr (D == 128) return 0x1.6a09e6p-4f;
  else if constexpr (D == 256) return 0x1p-4f;
  else return 0x1.6a09e6p-5f;  // 512
}

__device__ __forceinline__ float shfl_xor(float v, int m) { return __shfl_xor(v, m, kWave); }

// Wave-level butterfly reductions (every lane ends with the result).
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, shfl_xor(v, m));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += shfl_xor(v, m);
  return v;
}

}  // namespace kvarn
