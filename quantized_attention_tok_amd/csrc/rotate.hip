// rotate.hip -- query rotation q_rot = H q along head_dim (orthonormal
// Walsh-Hadamard), SharpInference PR #434 commit list (llm_kvarn_rotate_query);
// issue #180 Algorithm step 1 (an orthonormal rotation preserves scores).
//
// One wave per row; lane l holds channels l + 64k.  Butterfly strides 1..32
// cross lanes, strides 64.. stay in the lane; ascending stride order and one
// final scale, the same arithmetic as the tile compressor's row transform.
#include "kvarn_launch.h"

namespace kvarn {
namespace {

template <int D>
__device__ __forceinline__ void wht_row_lanes(float (&x)[D / 64], int lane) {
  constexpr int K = D / 64;
#pragma unroll
  for (int h = 1; h < 64; h <<= 1) {
    const bool up = (lane & h) != 0;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      float p = shfl_xor(x[k], h);
      x[k] = up ? (p - x[k]) : (x[k] + p);
    }
  }
#pragma unroll
  for (int hk = 1; hk < K; hk <<= 1) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if ((k & hk) == 0) {
        float a = x[k], b = x[k + hk];
        x[k] = a + b;
        x[k + hk] = a - b;
      }
    }
  }
  const float c = wht_scale<D>();
#pragma unroll
  for (int k = 0; k < K; ++k) x[k] = x[k] * c;
}

template <int D>
__global__ void __launch_bounds__(256) rotate_kernel(const float* q, float* out, int64_t n_rows) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (row >= n_rows) return;
  float x[D / 64];
#pragma unroll
  for (int k = 0; k < D / 64; ++k) x[k] = q[row * D + lane + 64 * k];
  wht_row_lanes<D>(x, lane);
#pragma unroll
  for (int k = 0; k < D / 64; ++k) out[row * D + lane + 64 * k] = x[k];
}

}  // namespace

hipError_t launch_rotate(int d, int64_t n_rows, const float* q, float* q_rot, hipStream_t stream) {
  if (n_rows == 0) return hipSuccess;
  dim3 grid((unsigned)((n_rows + 3) / 4));
  switch (d) {
    case 128: hipLaunchKernelGGL(rotate_kernel<128>, grid, dim3(256), 0, stream, q, q_rot, n_rows); break;
    case 256: hipLaunchKernelGGL(rotate_kernel<256>, grid, dim3(256), 0, stream, q, q_rot, n_rows); break;
    case 512: hipLaunchKernelGGL(rotate_kernel<512>, grid, dim3(256), 0, stream, q, q_rot, n_rows); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace kvarn
