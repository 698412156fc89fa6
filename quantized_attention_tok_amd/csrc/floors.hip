// floors.hip -- measured floors of the part, for the benchmark's roofline
// denominators (libkvarn_floors.so; not part of the KVarN path).
//
//   kvarn_floor_read   plain coalesced read of a device buffer (16-byte loads,
//                      four in flight per lane): the achievable HBM read rate
//                      at a given size;
//   kvarn_floor_mfma   independent chains of one matrix op per wave (fp16
//                      16x16x32 or int8 16x16x64): the achievable matrix rate;
//   kvarn_floor_empty  an empty kernel: the launch floor inside a graph.
//
// Every launch checks its sizes on the host; the kernels touch nothing
// outside the buffers they are given.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int intx4 __attribute__((ext_vector_type(4)));

constexpr int kReadThreads = 256;
constexpr int kUnroll = 4;

__global__ void __launch_bounds__(kReadThreads) read_kernel(const uint4* __restrict__ src, size_t n16,
                                                           uint32_t* __restrict__ sink) {
  const size_t tid = (size_t)blockIdx.x * kReadThreads + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * kReadThreads;
  uint32_t acc = 0;
  size_t i = tid;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    uint4 v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = src[i + u * stride];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = src[i];
    acc ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[tid] = acc;   // one word per thread: keeps every load live
}

template <int KIND>
__global__ void __launch_bounds__(256) mfma_kernel(float* __restrict__ out, int iters) {
  const int lane = threadIdx.x & 63;
  if constexpr (KIND == 0) {
    half8 a, b;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      a[i] = (_Float16)(0.001f * (lane + i));
      b[i] = (_Float16)(0.002f * (lane - i));
    }
    floatx4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0;
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c3, 0, 0, 0);
    }
    const floatx4 s = c0 + c1 + c2 + c3;
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = s[0] + s[1] + s[2] + s[3];
  } else {
    intx4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = 0x01010101 * ((lane + i) & 7);
      b[i] = 0x01010101 * ((lane ^ i) & 7);
    }
    intx4 c0 = {0, 0, 0, 0}, c1 = c0, c2 = c0, c3 = c0;
    for (int it = 0; it < iters; ++it) {
      c0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c3, 0, 0, 0);
    }
    const intx4 s = c0 + c1 + c2 + c3;
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = (float)(s[0] + s[1] + s[2] + s[3]);
  }
}

__global__ void empty_kernel() {}

}  // namespace

extern "C" {

// Read `bytes` (a multiple of 16) from `buf` with `n_groups` workgroups of 256
// threads; `sink` must hold n_groups * 256 words.  Returns 0 on success, 1 on
// bad arguments, 5 when HIP reports a launch error.
int kvarn_floor_read(const void* buf, size_t bytes, uint32_t* sink, int n_groups, void* stream) {
  if (!buf || !sink || n_groups < 1 || (bytes % 16) != 0 || (reinterpret_cast<uintptr_t>(buf) & 15))
    return 1;
  hipLaunchKernelGGL(read_kernel, dim3(n_groups), dim3(kReadThreads), 0, (hipStream_t)stream,
                     static_cast<const uint4*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

// n_groups workgroups of 4 waves, each wave `iters` x 4 matrix ops on four
// independent accumulators; kind 0: v_mfma_f32_16x16x32_f16 (16384 flops
// each), kind 1: v_mfma_i32_16x16x64_i8 (32768 ops each).  `out` holds
// n_groups * 256 floats.
int kvarn_floor_mfma(float* out, int n_groups, int iters, int kind, void* stream) {
  if (!out || n_groups < 1 || iters < 1 || (kind != 0 && kind != 1)) return 1;
  if (kind == 0)
    hipLaunchKernelGGL(mfma_kernel<0>, dim3(n_groups), dim3(256), 0, (hipStream_t)stream, out, iters);
  else
    hipLaunchKernelGGL(mfma_kernel<1>, dim3(n_groups), dim3(256), 0, (hipStream_t)stream, out, iters);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

int kvarn_floor_empty(void* stream) {
  hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, (hipStream_t)stream);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"
