// window_mfma.hip -- the raw-window part of chunked prefill at head_dim 256
// and 512, on the fp32 matrix cores (v_mfma_f32_16x16x4_f32: exact fp32
// products, fp32 accumulation).
//
// Query position p of a chunk attends its compressed tiles [0, T(p)) and its
// raw tokens [128 T(p), p] with one softmax (PR #434 commit list: chunked
// prefill, a single streaming softmax over compressed tiles + FP32 window).
// The tile part runs as split partials on the wide tile kernels; this kernel
// computes the raw part of 16 consecutive positions of one or two query
// heads at a time, reading each raw key and value row once for the 16 rows
// (the per-row vector kernels read it once per row).  The block's raw tokens
// are cut into parts (grid z, in 16-token steps) so that several workgroups
// share a CU; each part writes one raw-domain partial (o unnormalised, running
// maximum in natural-log units, sum; -inf and 0 for a row the part does not
// reach) per row and head, in the slot of the decode combine's window split of
// that part.
//
// Workgroup = (16-row block, HG query heads of one KV head), 4 waves (HG = 2
// at head_dim 256, so each staged row serves two heads; 1 at 512, where the
// registers hold one head's query and output).  Per 16-token step the
// waves stage the tokens' key and value rows in LDS (rows padded by 4 floats,
// so the per-lane reads spread over the banks), then
//   scores  S[t][r] = sum_c k[t][c] q[r][c]: wave w contracts its quarter of
//           the channels (lane (g, r) supplies channels w D/4 + g D/16 ..
//           + D/16 of key row t = r and of query row r); the four partial
//           score blocks are summed in wave order through LDS, so every wave
//           holds the same scores;
//   softmax per row (lane (g, r): tokens 4g .. 4g + 3 of row r), online across
//           the steps, in log2 units;
//   values  O^T[c][r] += sum_t v[t][c] p[r][t] for the wave's quarter of the
//           channels (16-channel blocks).
#include <float.h>

#include "kvarn_launch.h"
#include "kvarn_mfma.h"

namespace kvarn {
namespace {

typedef float floatx4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int64_t tiles_at_pos(int64_t p, int window) {
  const int64_t ahead = p + 1 - window;
  return ahead > 0 ? ahead / kTile : 0;
}

// max / sum over the four 16-lane rows (lanes n, n + 16, n + 32, n + 48)
__device__ __forceinline__ float rows4_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows4_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

template <int D, int HG>
__global__ void __launch_bounds__(256) window_mfma_kernel(DecodeParams P, int chunk) {
  constexpr int CW = D / 4;            // channels per wave
  constexpr int KQ = D / 16;           // contraction steps per wave (one channel per lane group each)
  constexpr int NB = CW / 16;          // 16-channel output blocks per wave
  constexpr int RS = D + 4;            // padded LDS row, floats
  constexpr int F4 = 16 * D / 4;       // float4 of one 16-token block of keys (or values)
  constexpr int PT = 2 * F4 / 256;     // staged float4 per thread (keys, then values)
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int g = lane >> 4, n = lane & 15;
  const int rb = blockIdx.x, h0 = blockIdx.y * HG;   // heads h0 .. h0 + HG - 1
  const int kvh = h0 / P.G;
  const int r0 = 16 * rb;
  const int r = r0 + n;                                   // this lane's query row (column n)
  const bool row_ok = r < chunk;
  const int64_t prow = P.pos0 + r;
  const int64_t row_lo = row_ok ? (int64_t)kTile * tiles_at_pos(prow, P.window) : 0;
  const int64_t p_first = P.pos0 + r0;
  const int64_t p_last = P.pos0 + min(r0 + 15, chunk - 1);
  // raw tokens [t_lo, t_hi) of the block's part blockIdx.z of P.n_wsplit (16-token steps)
  const int64_t b_lo = (int64_t)kTile * tiles_at_pos(p_first, P.window);
  const int64_t steps = (p_last + 1 - b_lo + 15) / 16;
  const int part = blockIdx.z, n_parts = P.n_wsplit;
  const int64_t t_lo = b_lo + 16 * (steps * part / n_parts);
  const int64_t t_hi = min(p_last + 1, b_lo + 16 * (steps * (part + 1) / n_parts));
  const float scale_log2 = P.scale * mfma::kLog2e;

  __shared__ __attribute__((aligned(16))) float s_k[16 * RS];
  __shared__ __attribute__((aligned(16))) float s_v[16 * RS];
  __shared__ __attribute__((aligned(16))) floatx4 s_sp[HG][4][64];

  // query row r of each head, channels w CW + g KQ .. + KQ (B operand of the scores)
  float qv[HG][KQ];
#pragma unroll
  for (int hh = 0; hh < HG; ++hh) {
    const float* qs = P.q + ((int64_t)(row_ok ? r : 0) * P.n_q + h0 + hh) * D + w * CW + g * KQ;
#pragma unroll
    for (int j = 0; j < KQ / 4; ++j) {
      float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
      if (row_ok) x = reinterpret_cast<const float4*>(qs)[j];
      qv[hh][4 * j] = x.x; qv[hh][4 * j + 1] = x.y; qv[hh][4 * j + 2] = x.z; qv[hh][4 * j + 3] = x.w;
    }
  }
  const float* kbase = P.k_win + (int64_t)kvh * P.win_head_stride;
  const float* vbase = P.v_win + (int64_t)kvh * P.win_head_stride;
  const int64_t ts = P.win_tok_stride;

  // this thread's staging share of a 16-token step: float4 e = tid + 256 j of
  // the keys (e < F4) or values; tokens past t_hi read row t_hi - 1 and are
  // zeroed, so no load waits on a branch
  float4 st[PT];
  auto fetch = [&](int64_t tb) {
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const int e = tid + 256 * j;
      const int kv = e / F4, f = e % F4;
      const int tok = f / (D / 4), c4 = f % (D / 4);
      const int64_t t = tb + tok;
      const bool ok = t < t_hi;
      const int64_t tc = ok ? t : t_hi - 1;
      const float4 x = reinterpret_cast<const float4*>((kv ? vbase : kbase) + (tc - P.raw_base) * ts)[c4];
      st[j] = ok ? x : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };

  float m_run[HG], l_run[HG];   // softmax state of row r per head (log2 units)
  floatx4 O[HG][NB];            // channels w CW + 16 b + 4 g + i of row r
#pragma unroll
  for (int hh = 0; hh < HG; ++hh) {
    m_run[hh] = -INFINITY;
    l_run[hh] = 0.0f;
#pragma unroll
    for (int b = 0; b < NB; ++b) O[hh][b] = (floatx4){0.f, 0.f, 0.f, 0.f};
  }

  if (t_lo < t_hi) fetch(t_lo);
  for (int64_t tb = t_lo; tb < t_hi; tb += 16) {
    __syncthreads();   // every wave is done with the previous step's rows and score partials
#pragma unroll
    for (int j = 0; j < PT; ++j) {
      const int e = tid + 256 * j;
      const int kv = e / F4, f = e % F4;
      const int tok = f / (D / 4), c4 = f % (D / 4);
      *reinterpret_cast<float4*>((kv ? s_v : s_k) + tok * RS + 4 * c4) = st[j];
    }
    if (tb + 16 < t_hi) fetch(tb + 16);   // the next step's rows, while this one is computed
    __syncthreads();
    // scores, this wave's channel quarter: A = key rows (row n = token tb + n), B = query rows
    floatx4 sacc[HG];
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) sacc[hh] = (floatx4){0.f, 0.f, 0.f, 0.f};
    {
      const float* kr = s_k + n * RS + w * CW + g * KQ;
#pragma unroll
      for (int j = 0; j < KQ / 4; ++j) {
        const float4 a = reinterpret_cast<const float4*>(kr)[j];
#pragma unroll
        for (int hh = 0; hh < HG; ++hh) {
          sacc[hh] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.x, qv[hh][4 * j], sacc[hh], 0, 0, 0);
          sacc[hh] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.y, qv[hh][4 * j + 1], sacc[hh], 0, 0, 0);
          sacc[hh] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.z, qv[hh][4 * j + 2], sacc[hh], 0, 0, 0);
          sacc[hh] = __builtin_amdgcn_mfma_f32_16x16x4f32(a.w, qv[hh][4 * j + 3], sacc[hh], 0, 0, 0);
        }
      }
    }
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) s_sp[hh][w][lane] = sacc[hh];
    __syncthreads();
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      floatx4 s4 = s_sp[hh][0][lane];
#pragma unroll
      for (int ww = 1; ww < 4; ++ww) s4 += s_sp[hh][ww][lane];
      // lane (g, n): tokens tb + 4 g + i of row r
      float sv[4], tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t t = tb + 4 * g + i;
        const bool vis = row_ok && t >= row_lo && t <= prow && t < t_hi;
        sv[i] = vis ? s4[i] * scale_log2 : -INFINITY;
        tmax = fmaxf(tmax, sv[i]);
      }
      tmax = rows4_max(tmax);
      const float m_new = fmaxf(m_run[hh], tmax);
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run[hh] - m_use);   // 0 from -inf
      float pv[4], psum = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[i] = __builtin_amdgcn_exp2f(sv[i] - m_use);
        psum += pv[i];
      }
      l_run[hh] = l_run[hh] * alpha + rows4_sum(psum);
      m_run[hh] = m_new;
#pragma unroll
      for (int b = 0; b < NB; ++b) O[hh][b] *= alpha;
      // values: step i contracts tokens 4 g + i (K slot g); A row n = channel w CW + 16 b + n
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float* vr = s_v + (4 * g + i) * RS + w * CW + n;
#pragma unroll
        for (int b = 0; b < NB; ++b) O[hh][b] = __builtin_amdgcn_mfma_f32_16x16x4f32(vr[16 * b], pv[i], O[hh][b], 0, 0, 0);
      }
    }
  }

  if (!row_ok) return;
  const int nsp = P.n_tsplit + P.n_wsplit;
#pragma unroll
  for (int hh = 0; hh < HG; ++hh) {
    float* o = P.part + (((int64_t)r * P.n_q + h0 + hh) * nsp + P.n_tsplit + part) * (D + 4);
#pragma unroll
    for (int b = 0; b < NB; ++b)
      *reinterpret_cast<float4*>(o + w * CW + 16 * b + 4 * g) =
          make_float4(O[hh][b][0], O[hh][b][1], O[hh][b][2], O[hh][b][3]);
    if (w == 0 && g == 0) {   // natural-log units, as the decode combine reads them (-inf: nothing seen)
      o[D] = m_run[hh] == -INFINITY ? -INFINITY : m_run[hh] * 0.69314718055994531f;
      o[D + 1] = l_run[hh];
    }
  }
}

}  // namespace

hipError_t launch_window_mfma(int d, const DecodeParams& P, int chunk, hipStream_t stream) {
  const int blocks = (chunk + 15) / 16;
  const int parts = P.n_wsplit;
  if (d == 256 && P.G % 2 == 0)   // two heads of a KV head per workgroup
    hipLaunchKernelGGL((window_mfma_kernel<256, 2>), dim3(blocks, P.n_q / 2, parts), dim3(256), 0, stream, P, chunk);
  else if (d == 256)
    hipLaunchKernelGGL((window_mfma_kernel<256, 1>), dim3(blocks, P.n_q, parts), dim3(256), 0, stream, P, chunk);
  else if (d == 512)
    hipLaunchKernelGGL((window_mfma_kernel<512, 1>), dim3(blocks, P.n_q, parts), dim3(256), 0, stream, P, chunk);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kvarn
