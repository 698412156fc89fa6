// kvarn_device.h -- small device helpers shared by the KVarN HIP kernels
// (gfx950, wave64).  Record layout constants follow the tile record described
// in include/kvarn.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvarn {

constexpr int kTile = 128;   // tokens per tile
constexpr int kWave = 64;    // CDNA wavefront width

// Byte offsets of the record sections for head_dim D.
template <int D>
struct Rec {
  static constexpr int kcode = 0;
  static constexpr int vcode = 64 * D;
  static constexpr int ktok = 96 * D;
  static constexpr int kscale = 96 * D + 512;
  static constexpr int kmin = 100 * D + 512;
  static constexpr int vchan = 104 * D + 512;
  static constexpr int vscale = 108 * D + 512;
  static constexpr int vmin = 112 * D + 512;
  static constexpr int bytes = 116 * D + 512;
  static constexpr int groups = D / 128;
};

__host__ __device__ inline int64_t tile_bytes_rt(int d) { return 116LL * d + 512; }

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
