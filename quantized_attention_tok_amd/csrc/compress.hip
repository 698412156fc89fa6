// compress.hip -- KVarN tile compressor for gfx950.
//
// One workgroup compresses the K tile or the V tile of one (tile, KV head):
// Walsh-Hadamard rotation of every token row, dual-axis Sinkhorn
// normalisation, asymmetric RTN and packing into the tile record
// (SharpInference issue #180, "Algorithm (per 128-token tile)" steps 1-4;
// SharpInference PR #434 commit list: channel-major K / token-major V packing,
// 2-bit bit packing, codes byte-identical to the CPU compressor).
//
// Every value that decides a code is computed with the same fp32 operations in
// the same order as the CPU oracle, so records are byte-identical:
//   - WHT butterflies in ascending stride, then one multiply by fp32(1/sqrt(D));
//   - every sum is a pairwise sum over contiguous halves;
//   - Sinkhorn is Sinkhorn-Knopp scaling of X*X (channel step, then token step,
//     8 iterations), means below FLT_MIN replaced by 1;
//   - IEEE division and square root (HIP's default correctly rounded forms),
//     round-half-even rint, no fused multiply-add (contraction off below).
//
// Thread layout (D = 32*W, W waves, 64*W threads): lane l holds tokens 2l and
// 2l+1, wave w holds channels [32w, 32w+32); each thread keeps its 2x32 tile
// values in registers.  Token sums are in-thread trees plus a W-way tree across
// waves through LDS.  Channel sums, minima and maxima over the 128 tokens take
// one in-lane step over the lane's two tokens, then a transpose through the
// wave's own LDS area, after which lanes 2c, 2c+1 each reduce 32 lane values
// of channel c in-thread and join the halves.
#include <float.h>

#include "kvarn_launch.h"

#pragma clang fp contract(off)

namespace kvarn {
namespace {

// Pairwise sum over contiguous halves of p[OFF .. OFF+N).
template <int N, int OFF, int LEN>
__device__ __forceinline__ float psum(const float (&p)[LEN]) {
  if constexpr (N == 1) {
    return p[OFF];
  } else {
    float left = psum<N / 2, OFF, LEN>(p);
    float right = psum<N / 2, OFF + N / 2, LEN>(p);
    return left + right;
  }
}

// Minimum and maximum on the vector min / max instructions: for finite
// operands the value that a compare-and-keep scan finds, except that a tie of
// -0 and +0 may keep either zero; every extreme is taken through + 0.0f before
// use, which makes a zero +0 either way.
struct OpAdd { __device__ float operator()(float a, float b) const { return a + b; } };
struct OpMin { __device__ float operator()(float a, float b) const { return fminf(a, b); } };
struct OpMax { __device__ float operator()(float a, float b) const { return fmaxf(a, b); } };

// Pairwise reduction over contiguous halves of p[OFF .. OFF+N).
template <int N, int OFF, int LEN, typename Op>
__device__ __forceinline__ float preduce(const float (&p)[LEN], Op op) {
  if constexpr (N == 1) {
    return p[OFF];
  } else {
    return op(preduce<N / 2, OFF, LEN>(p, op), preduce<N / 2, OFF + N / 2, LEN>(p, op));
  }
}

// Value of lane l ^ 1, by a data-parallel move (quad_perm [1,0,3,2]).
__device__ __forceinline__ float lane_xor1(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
}

constexpr int cmax(int a, int b) { return a > b ? a : b; }

// Orders this wave's LDS writes before its later LDS reads of other lanes'
// values: LDS operations of one wave complete in issue order, so only the
// compiler has to be kept from moving them (no workgroup barrier).
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// One wave's channel-transpose area in LDS: 32 channel rows of ROW floats,
// lanes 0-31 at columns 0-31 and lanes 32-63 at columns 36-67.  ROW = 72 up
// to D = 256, so that the 16-byte reads of lanes 2c, 2c+1 (rows c, columns 0
// or 36) fall in distinct banks across a quarter-wave; 68 at D = 512, where
// the sixteen areas must fit beside the other LDS (two of the 16-byte reads of
// a quarter-wave then share a bank group).
template <int D> constexpr int tx_row() { return D <= 256 ? 72 : 68; }

// Reduction over the wave's 128 tokens for each of its 32 channels, from f(j)
// = the lane's two-token value of channel j (lane l holds tokens 2l, 2l+1),
// through LDS: the lanes write f(j) into channel row j, lanes 2c and 2c+1 read
// lanes [0, 32) and [32, 64) of channel c, reduce them pairwise over contiguous
// halves and join the two halves, i.e. the pairwise tree over contiguous
// token blocks.  Returns the value for channel lane >> 1 of the wave's 32, in
// both lanes of the pair.  The area is the wave's own.
template <int ROW, typename F, typename Op>
__device__ __forceinline__ float chan_reduce_lds(F f, float* tx, int lane, Op op) {
  float* col = tx + lane + ((lane >> 5) << 2);
#pragma unroll
  for (int j = 0; j < 32; ++j) col[j * ROW] = f(j);
  wave_sync();
  // the 32-value tree as the join of its four 8-value subtrees, so that only
  // one quarter of the values is live at a time
  const float4* rd = reinterpret_cast<const float4*>(tx + (lane >> 1) * ROW + (lane & 1) * 36);
  float sub[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float4 v0 = rd[2 * q], v1 = rd[2 * q + 1];
    const float a[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
    sub[q] = preduce<8, 0, 8>(a, op);
  }
  const float half = op(op(sub[0], sub[1]), op(sub[2], sub[3]));
  return op(half, lane_xor1(half));
}

// RTN code of xn: rint((xn - lo) * inv) clamped to [0, levels]; fmaxf takes a
// NaN quotient to 0, as the test !(z >= 0) does.
__device__ __forceinline__ float code_of(float xn, float lo, float inv, float levels) {
  const float z = __builtin_rintf((xn - lo) * inv);
  return fminf(fmaxf(z, 0.0f), levels);
}

// GEN: kb-bit keys and vb-bit values (runtime widths, LSB-first bit streams);
// otherwise the K4V2 record (kb, vb ignored).
// Three waves per SIMD at D = 128 (registers capped at 168 per lane, the LDS
// area small enough): three workgroups share a CU.
template <int D, bool H, bool GEN>
__global__ void __launch_bounds__(2 * D, D == 128 ? 3 : 1)
compress_kernel(const float* __restrict__ kin, const float* __restrict__ vin,
                int64_t tok_stride, int64_t head_stride, int n_kv,
                uint8_t* __restrict__ records, int kb, int vb) {
  constexpr int W = D / 32;        // waves
  // channel offsets per LDS exchange round: two rounds of 16 at D = 128, so
  // that the exchange area (and the workgroup's LDS) allows four workgroups per CU
  constexpr int J = D == 128 ? 16 : kTile / W;
  using R = Rec<D, H>;
  if constexpr (!GEN) { kb = 4; vb = 2; }
  const RecRT o = rec_rt(D, H, kb, vb);

  // Reused by every phase: the padded WHT exchange (W x 128 rows of J + 1
  // floats); the two per-channel broadcast vectors followed by the per-wave
  // token partials (W x 128 x 2 floats) or the key code bytes (D x 64, or one
  // byte per code for the generic packing: D x 128).
  // Channel reductions through each wave's LDS transpose area, placed after
  // the two token-partial buffers, which are live at the same time.
  constexpr int kXS = J + 1;   // exchange row stride: odd, so rows start in distinct banks
  constexpr int kTxRow = tx_row<D>();
  constexpr int kTxWave = 32 * kTxRow;
  constexpr int kTxOff = 2 * D + 2 * W * kTile;
  constexpr int kSmem = cmax(cmax(W * kTile * kXS, kTxOff + W * kTxWave),
                             cmax(2 * D + 2 * W * kTile, GEN ? 34 * D : 18 * D));
  __shared__ __align__(16) float smem[kSmem];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int job = blockIdx.x;
  const int head = blockIdx.y;
  const bool is_key = blockIdx.z == 0;

  const float* src = (is_key ? kin : vin) + (int64_t)job * kTile * tok_stride +
                     (int64_t)head * head_stride;
  uint8_t* rec = records + ((int64_t)job * n_kv + head) * o.bytes;

  // ---- load rows 2l, 2l+1, channels [32w, 32w+32) ----
  float x[2][32];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float4* row = reinterpret_cast<const float4*>(src + (int64_t)(2 * lane + i) * tok_stride + 32 * w);
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      float4 f = row[q];
      x[i][4 * q + 0] = f.x; x[i][4 * q + 1] = f.y; x[i][4 * q + 2] = f.z; x[i][4 * q + 3] = f.w;
    }
  }

  // ---- WHT: strides 1..16 inside the thread ----
#pragma unroll
  for (int i = 0; i < 2; ++i) {
#pragma unroll
    for (int h = 1; h < 32; h <<= 1) {
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        if ((j & h) == 0) {
          float a = x[i][j], b = x[i][j + h];
          x[i][j] = a + b;
          x[i][j + h] = a - b;
        }
      }
    }
  }
  // ---- WHT: strides 32..D/2 across waves, J channel offsets per round ----
  if constexpr (W > 1) {
    float* xch = smem;  // [W][128][kXS]
    constexpr int kPer = 2 * J / W;  // (token, offset) columns per thread
#pragma unroll
    for (int r = 0; r < 32 / J; ++r) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < J; ++jj)
          xch[(w * kTile + 2 * lane + i) * kXS + jj] = x[i][r * J + jj];
      __syncthreads();
#pragma unroll
      for (int k = 0; k < kPer; ++k) {
        const int idx = tid * kPer + k;
        const int t = idx / J, jj = idx % J;
        float y[W];
#pragma unroll
        for (int u = 0; u < W; ++u) y[u] = xch[(u * kTile + t) * kXS + jj];
#pragma unroll
        for (int hs = 1; hs < W; hs <<= 1) {
#pragma unroll
          for (int u = 0; u < W; ++u) {
            if ((u & hs) == 0) {
              float a = y[u], b = y[u + hs];
              y[u] = a + b;
              y[u + hs] = a - b;
            }
          }
        }
#pragma unroll
        for (int u = 0; u < W; ++u) xch[(u * kTile + t) * kXS + jj] = y[u];
      }
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jj = 0; jj < J; ++jj)
          x[i][r * J + jj] = xch[(w * kTile + 2 * lane + i) * kXS + jj];
      __syncthreads();
    }
  }
  {
    const float c = wht_scale<D>();
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 32; ++j) x[i][j] = x[i][j] * c;
  }

  // ---- Sinkhorn-Knopp on Q = X*X: the squares are written as recomputed at
  // each use (the same rounded products; the compiler keeps them in registers
  // across the iterations) ----
  auto Qv = [&](int i, int j) -> float { return x[i][j] * x[i][j]; };

  // bc_v / bc_x: per-channel values, channel c written by the owner lane of
  // wave c / 32 and read by that wave only; tp: per-wave token partials, two
  // buffers taken by iteration parity, so that one barrier per iteration
  // separates both the writes from the reads of other waves and an
  // iteration's reads from the writes two iterations later.
  float* bc_v = smem;               // [D] per-channel broadcast
  float* bc_x = smem + D;           // [D] second per-channel broadcast
  float* tp2 = smem + 2 * D;        // [2][W][128] per-wave token partials

  float u[2] = {1.0f, 1.0f};        // 1 / r^2 for tokens 2l, 2l+1
  float mt[2] = {1.0f, 1.0f};
  float mc_own = 1.0f;              // channel mean square owned by this lane
  // reduction over the wave's 128 tokens per channel; this lane's result is
  // for channel ch_own, and one lane per channel (owner) stores it
  float* tx = smem + kTxOff + w * kTxWave;
  auto chan_reduce = [&](auto f, auto op) -> float { return chan_reduce_lds<kTxRow>(f, tx, lane, op); };
  const int ch_own = 32 * w + (lane >> 1);
  const bool owner = (lane & 1) == 0;
  constexpr float kInvT = 1.0f / 128.0f;
  constexpr float kInvD = 1.0f / (float)D;

  for (int it = 0; it < 8; ++it) {
    // channel step: mean over tokens of Q * u
    {
      const float sum = chan_reduce([&](int j) { return Qv(0, j) * u[0] + Qv(1, j) * u[1]; }, OpAdd{});
      float m = sum * kInvT;
      if (!(m >= FLT_MIN)) m = 1.0f;
      mc_own = m;
      if (owner) bc_v[ch_own] = 1.0f / m;
    }
    wave_sync();
    float* tp = tp2 + (it & 1) * (W * kTile);
    // token step: mean over channels of Q * v; the pairwise tree over the 32
    // products taken as eight 4-product sums, then the tree over those
    {
      float t[2][8];
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const float4 f = reinterpret_cast<const float4*>(bc_v + 32 * w)[q];
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const float p0 = Qv(i, 4 * q) * f.x, p1 = Qv(i, 4 * q + 1) * f.y;
          const float p2 = Qv(i, 4 * q + 2) * f.z, p3 = Qv(i, 4 * q + 3) * f.w;
          t[i][q] = (p0 + p1) + (p2 + p3);
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) tp[w * kTile + 2 * lane + i] = psum<8, 0, 8>(t[i]);
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float pw[W];
#pragma unroll
      for (int ww = 0; ww < W; ++ww) pw[ww] = tp[ww * kTile + 2 * lane + i];
      float m = psum<W, 0, W>(pw) * kInvD;
      if (!(m >= FLT_MIN)) m = 1.0f;
      mt[i] = m;
      u[i] = 1.0f / m;
    }
  }

  // ---- final spreads and normalised tile ----
  const float s_own = __builtin_sqrtf(mc_own);
  if (owner) bc_v[ch_own] = 1.0f / s_own;
  wave_sync();
  float r[2], ir[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    r[i] = __builtin_sqrtf(mt[i]);
    ir[i] = 1.0f / r[i];
  }
  {
    float is[32];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      float4 f = reinterpret_cast<const float4*>(bc_v + 32 * w)[q];
      is[4 * q + 0] = f.x; is[4 * q + 1] = f.y; is[4 * q + 2] = f.z; is[4 * q + 3] = f.w;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 32; ++j) x[i][j] = (x[i][j] * ir[i]) * is[j];
  }
  // every wave has read the last iteration's token partials before the code
  // and extreme staging below overwrites them
  __syncthreads();

  if (is_key) {
    // ---- keys: per channel over the 128 tokens, 4 bits ----
    const float lo = chan_reduce([&](int j) { return OpMin{}(x[0][j], x[1][j]); }, OpMin{}) + 0.0f;
    const float hi = chan_reduce([&](int j) { return OpMax{}(x[0][j], x[1][j]); }, OpMax{}) + 0.0f;
    const float klev = GEN ? (float)((1 << kb) - 1) : 15.0f;
    float delta = (hi - lo) / klev;
    float inv = (delta >= FLT_MIN) ? 1.0f / delta : 0.0f;
    if (owner) {
      bc_v[ch_own] = lo;
      bc_x[ch_own] = inv;
      sc_st<H>(rec + o.kscale, ch_own, delta * s_own);
      sc_st<H>(rec + o.kmin, ch_own, lo * s_own);
    }
    if (w == 0) {
      sc_st<H>(rec + o.ktok, 2 * lane, r[0]);
      sc_st<H>(rec + o.ktok, 2 * lane + 1, r[1]);
    }
    __syncthreads();  // the code staging below overlaps other waves' transpose areas
    if constexpr (GEN) {
      uint8_t* kst = reinterpret_cast<uint8_t*>(smem + 2 * D);  // [D][128] one byte per code
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const float lj = bc_v[32 * w + j], ij = bc_x[32 * w + j];
        const int z0 = (int)code_of(x[0][j], lj, ij, klev);
        const int z1 = (int)code_of(x[1][j], lj, ij, klev);
        *reinterpret_cast<uint16_t*>(kst + (32 * w + j) * kTile + 2 * lane) = (uint16_t)(z0 | (z1 << 8));
      }
      __syncthreads();
      // dword q of channel c's stream holds the codes whose bits meet [32 q, 32 q + 32)
      const int per = 4 * kb;   // dwords per channel
      uint32_t* dst = reinterpret_cast<uint32_t*>(rec + o.kcode);
      for (int i = tid; i < D * per; i += 2 * D) {
        const int c = i / per, q = i - c * per;
        const int t0 = (32 * q) / kb, t1 = (32 * q + 31) / kb;
        uint32_t acc = 0;
        for (int t = t0; t <= t1; ++t) {
          const int pos = kb * t - 32 * q;   // in (-kb, 32)
          const uint32_t z = kst[c * kTile + t];
          acc |= pos >= 0 ? (z << pos) : (z >> -pos);
        }
        dst[i] = acc;
      }
    } else {
      uint8_t* kst = reinterpret_cast<uint8_t*>(smem + 2 * D);  // [D][64] bytes
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        const float lj = bc_v[32 * w + j], ij = bc_x[32 * w + j];
        int z0 = (int)code_of(x[0][j], lj, ij, 15.0f);
        int z1 = (int)code_of(x[1][j], lj, ij, 15.0f);
        kst[(32 * w + j) * 64 + lane] = (uint8_t)(z0 | (z1 << 4));
      }
      __syncthreads();
      // coalesced copy of the D*64 code bytes: 32 bytes per thread
      const uint4* s4 = reinterpret_cast<const uint4*>(kst);
      uint4* d4 = reinterpret_cast<uint4*>(rec + R::kcode);
#pragma unroll
      for (int q = 0; q < 2; ++q) d4[tid * 2 + q] = s4[tid * 2 + q];
    }
  } else {
    // ---- values: per token over each 128-channel group, 2 bits ----
    float* mm = smem + 2 * D;  // [W][128][2]
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      float lo = x[i][0], hi = x[i][0];
#pragma unroll
      for (int j = 1; j < 32; ++j) { lo = OpMin{}(lo, x[i][j]); hi = OpMax{}(hi, x[i][j]); }
      mm[(w * kTile + 2 * lane + i) * 2 + 0] = lo;
      mm[(w * kTile + 2 * lane + i) * 2 + 1] = hi;
    }
    if (owner) sc_st<H>(rec + o.vchan, ch_own, s_own);
    __syncthreads();
    const int g = w / 4;  // channel group of this wave
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int t = 2 * lane + i;
      float lo = mm[((4 * g) * kTile + t) * 2 + 0];
      float hi = mm[((4 * g) * kTile + t) * 2 + 1];
#pragma unroll
      for (int ww = 1; ww < 4; ++ww) {
        lo = OpMin{}(lo, mm[((4 * g + ww) * kTile + t) * 2 + 0]);
        hi = OpMax{}(hi, mm[((4 * g + ww) * kTile + t) * 2 + 1]);
      }
      lo = lo + 0.0f;
      hi = hi + 0.0f;
      const float vlev = GEN ? (float)((1 << vb) - 1) : 3.0f;
      float delta = (hi - lo) / vlev;
      float inv = (delta >= FLT_MIN) ? 1.0f / delta : 0.0f;
      if constexpr (GEN) {
        // the wave's 32 channels fill dwords [w vb, w vb + vb) of token t's stream
        uint32_t* dst = reinterpret_cast<uint32_t*>(rec + o.vcode + t * (D * vb / 8)) + w * vb;
        uint64_t acc = 0;
        int nb = 0, q = 0;
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          const uint64_t z = (uint64_t)code_of(x[i][j], lo, inv, vlev);
          acc |= z << nb;
          nb += vb;
          if (nb >= 32) {
            dst[q++] = (uint32_t)acc;
            acc >>= 32;
            nb -= 32;
          }
        }
      } else {
        uint32_t packed[2] = {0u, 0u};
#pragma unroll
        for (int j = 0; j < 32; ++j) {
          uint32_t z = (uint32_t)code_of(x[i][j], lo, inv, 3.0f);
          packed[j / 16] |= z << (2 * (j % 16));
        }
        reinterpret_cast<uint2*>(rec + R::vcode + t * (D / 4) + 8 * w)[0] = make_uint2(packed[0], packed[1]);
      }
      if ((w & 3) == 0) {
        sc_st<H>(rec + o.vscale, t * R::groups + g, delta * r[i]);
        sc_st<H>(rec + o.vmin, t * R::groups + g, lo * r[i]);
      }
    }
  }
}

}  // namespace

// Launch the compressor for n_tiles x n_kv tile-heads (keys and values);
// h16: store the scales as f16; kb / vb: key / value code widths.
template <bool H, bool GEN>
hipError_t launch_compress_hg(int d, int n_tiles, int n_kv, const float* k, const float* v,
                              int64_t tok_stride, int64_t head_stride, uint8_t* rec, int kb,
                              int vb, hipStream_t stream) {
  dim3 grid(n_tiles, n_kv, 2);
  switch (d) {
    case 128:
      hipLaunchKernelGGL((compress_kernel<128, H, GEN>), grid, dim3(256), 0, stream, k, v,
                         tok_stride, head_stride, n_kv, rec, kb, vb);
      break;
    case 256:
      hipLaunchKernelGGL((compress_kernel<256, H, GEN>), grid, dim3(512), 0, stream, k, v,
                         tok_stride, head_stride, n_kv, rec, kb, vb);
      break;
    case 512:
      hipLaunchKernelGGL((compress_kernel<512, H, GEN>), grid, dim3(1024), 0, stream, k, v,
                         tok_stride, head_stride, n_kv, rec, kb, vb);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_compress(int d, bool h16, int kb, int vb, int n_tiles, int n_kv, const float* k,
                           const float* v, int64_t tok_stride, int64_t head_stride, void* records,
                           hipStream_t stream) {
  uint8_t* rec = static_cast<uint8_t*>(records);
  const bool gen = !(kb == 4 && vb == 2);
  if (h16)
    return gen ? launch_compress_hg<true, true>(d, n_tiles, n_kv, k, v, tok_stride, head_stride, rec, kb, vb, stream)
               : launch_compress_hg<true, false>(d, n_tiles, n_kv, k, v, tok_stride, head_stride, rec, kb, vb, stream);
  return gen ? launch_compress_hg<false, true>(d, n_tiles, n_kv, k, v, tok_stride, head_stride, rec, kb, vb, stream)
             : launch_compress_hg<false, false>(d, n_tiles, n_kv, k, v, tok_stride, head_stride, rec, kb, vb, stream);
}

}  // namespace kvarn
