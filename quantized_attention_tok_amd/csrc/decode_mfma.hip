// decode_mfma.hip -- fused split-tile decode attention for head_dim 128 on
// gfx950 matrix cores.
//
// One launch does the whole decode step for a batch (SharpInference issue #433
// item 2: fixed worst-case grid, early exit, LSE combine, inverse WHT after
// combining the rotated tile partials; PR #434 commit list: single streaming
// softmax over compressed tiles + FP32 window, deferred inverse WHT):
//   - tile workgroups: 4 waves share each 128-token tile (a quarter of its
//     tokens each, with one online-softmax stream per wave); records are
//     staged in LDS with 16-byte loads, double-buffered.  Scores and the value
//     aggregate of a tile are G x 128 x 128 contractions and run on
//     v_mfma_f32_16x16x32_f16 (rows padded to 16):
//        S^T[t][h] = sum_c zK[t][c] * q~[h][c],   q~ = q' * kscale (issue #180
//        Algorithm step 4: scales folded at read time; colibri PR #399 review
//        note: q . xhat = rotate(q) . code, never reconstruct the cache)
//        O[h][c]   = sum_t w[h][t] * zV[t][c],    w = p * vscale
//     Codes enter the MFMA exactly as fp16 subnormals with the code in bits
//     4-7 (16 z 2^-24 for nibbles; z 2^-20 or z 2^-18 for 2-bit codes), built
//     with a byte-permute, a shift and a mask.  Placing the code above bit 3
//     matters: measured on gfx950, products with subnormals whose only set
//     bits are 0-3 lose precision (about 5e-7 of the summed term magnitudes),
//     while bits 4-7 are as accurate as normal fp16 (3e-8).  The fp32 operands
//     (q~, w) are split into fp16 hi + lo parts, so products are exact to about
//     2^-22 and accumulate in fp32.
//   - window workgroups: 32 raw fp32 tokens each, K and V rows staged in LDS
//     together; scores and aggregate on the vector units.
//   - each workgroup writes one (m, l, o) partial per query head; a second
//     launch (one workgroup per query head) merges them with an online LSE,
//     applies the inverse WHT to the rotated tile part, adds the raw window
//     part and normalises.  A single-launch variant with a completion counter
//     was measured slower: device-scope fences on gfx950 write back and
//     invalidate the whole L2, and the last workgroup's merge of ~70 partials
//     through uncached loads was latency-bound.
// If q_rot is NULL the tile workgroups rotate the query themselves (the same
// Walsh-Hadamard butterflies as kvarn_rotate_query).
#include <float.h>

#include "kvarn_launch.h"

namespace kvarn {
namespace {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int D = 128;
constexpr int kRecBytes = 116 * D + 512;   // 15360
constexpr int kOffV = 64 * D;              // V codes
constexpr int kOffKtok = 96 * D;
constexpr int kOffKscale = 96 * D + 512;
constexpr int kOffKmin = 100 * D + 512;
constexpr int kOffVchan = 104 * D + 512;
constexpr int kOffVscale = 108 * D + 512;
constexpr int kOffVmin = 112 * D + 512;
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ half8 as_half8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  typedef uint32_t u4 __attribute__((ext_vector_type(4)));
  u4 v = {a, b, c, d};
  return __builtin_bit_cast(half8, v);
}

__device__ __forceinline__ uint32_t pack_h2(_Float16 lo, _Float16 hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
}

// 2^k as a float for k in [-126, 127].
__device__ __forceinline__ float pow2i(int k) { return __uint_as_float((uint32_t)(k + 127) << 23); }

// Scale 2^(14-E) that brings max|x| into [2^13, 2^14) (fp16 range with room
// for the hi/lo split); 1 when max is zero or tiny.
__device__ __forceinline__ int fp16_scale_exp(float amax) {
  const int eb = (int)((__float_as_uint(amax) >> 23) & 0xff);   // amax in [2^(eb-127), 2^(eb-126))
  int k = 140 - eb;
  if (eb == 0 || k > 100) k = 0;
  return k;
}

__device__ __forceinline__ void st_part(float* p, float v) { *p = v; }

__device__ __forceinline__ float wave_max16(float v) {
  v = fmaxf(v, __shfl_xor(v, 16, 64));
  return fmaxf(v, __shfl_xor(v, 32, 64));
}
__device__ __forceinline__ float wave_sum16(float v) {
  v += __shfl_xor(v, 16, 64);
  return v + __shfl_xor(v, 32, 64);
}

// Per-wave running state of the online softmax for the query heads this lane
// holds as a column (lane & 15) and the output accumulator for the rows
// (lane >> 4)*4 + i.
struct WaveState {
  float m;          // running max (log2 domain) of head (lane & 15)
  float l;          // running sum of head (lane & 15)
  floatx4 o[8];     // o'[head 4*(lane>>4)+i][channel of instance nb]
};

// Process one quarter of a tile held in LDS at `rec` (15360 bytes): wave w
// handles the 32 tokens {8r + 2w, 8r + 2w + 1 : r < 16}, i.e. QK token blocks
// 2w and 2w+1 and PV token step w, with its own online-softmax stream.  qrot
// holds the rotated query rows (LDS, [G][128]).
template <int G>
__device__ __forceinline__ void tile_quarter(const uint8_t* rec, const float* qrot, float scale_log2,
                                             WaveState& st, int lane, int w) {
  const int n = lane & 15;   // MFMA column: query head (QK) / channel slot (PV)
  const int g = lane >> 4;   // K group / output row group
  const bool real_head = n < G;

  // ---- q~ = q' * kscale for this lane's head n and channels 32 k4 + 8 g + e ----
  float qt[4][8];
  float bias_part = 0.0f;
  float amax = 0.0f;
  const float* ks = reinterpret_cast<const float*>(rec + kOffKscale);
  const float* km = reinterpret_cast<const float*>(rec + kOffKmin);
#pragma unroll
  for (int k4 = 0; k4 < 4; ++k4) {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const int c0 = 32 * k4 + 8 * g + 4 * h2;
      const float4 sc = *reinterpret_cast<const float4*>(ks + c0);
      const float4 mn = *reinterpret_cast<const float4*>(km + c0);
      const float4 q = real_head ? *reinterpret_cast<const float4*>(qrot + n * D + c0) : make_float4(0, 0, 0, 0);
      qt[k4][4 * h2 + 0] = q.x * sc.x; qt[k4][4 * h2 + 1] = q.y * sc.y;
      qt[k4][4 * h2 + 2] = q.z * sc.z; qt[k4][4 * h2 + 3] = q.w * sc.w;
      bias_part += q.x * mn.x + q.y * mn.y + q.z * mn.z + q.w * mn.w;
#pragma unroll
      for (int i = 0; i < 4; ++i) amax = fmaxf(amax, fabsf(qt[k4][4 * h2 + i]));
    }
  }
  amax = wave_max16(amax);
  const float bias = wave_sum16(bias_part);
  const int fexp = fp16_scale_exp(amax);
  const float f16inv = pow2i(fexp - 4);     // q~ * f / 16
  const float unscale = pow2i(24 - fexp);   // S = acc * 2^24 / f

  // ---- QK for token blocks 2w (low nibble of byte w) and 2w+1 (high nibble) ----
  floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  const uint32_t sel = (uint32_t)w | (12u << 8) | ((uint32_t)(4 + w) << 16) | (12u << 24);
#pragma unroll
  for (int k4 = 0; k4 < 4; ++k4) {
    uint32_t bh[4], bl[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const float x0 = qt[k4][2 * p] * f16inv, x1 = qt[k4][2 * p + 1] * f16inv;
      const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
      bh[p] = pack_h2(h0, h1);
      bl[p] = pack_h2((_Float16)(x0 - (float)h0), (_Float16)(x1 - (float)h1));
    }
    const half8 Bh = as_half8(bh[0], bh[1], bh[2], bh[3]);
    const half8 Bl = as_half8(bl[0], bl[1], bl[2], bl[3]);
    uint32_t ae[4], ao[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const uint32_t c0 = *reinterpret_cast<const uint32_t*>(rec + (32 * k4 + 8 * g + 2 * p) * 64 + 4 * n);
      const uint32_t c1 = *reinterpret_cast<const uint32_t*>(rec + (32 * k4 + 8 * g + 2 * p + 1) * 64 + 4 * n);
      ae[p] = __builtin_amdgcn_perm(c1 << 4, c0 << 4, sel) & 0x00F000F0u;   // 16 z, token 8n + 2w
      ao[p] = __builtin_amdgcn_perm(c1, c0, sel) & 0x00F000F0u;             // 16 z, token 8n + 2w + 1
    }
    const half8 Ae = as_half8(ae[0], ae[1], ae[2], ae[3]);
    const half8 Ao = as_half8(ao[0], ao[1], ao[2], ao[3]);
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ae, Bh, acc0, 0, 0, 0);
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ae, Bl, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ao, Bh, acc1, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ao, Bl, acc1, 0, 0, 0);
  }

  // ---- scores (log2 domain): s[j][i] is token 8(4g + i) + 2w + j, head n ----
  const float* ktok = reinterpret_cast<const float*>(rec + kOffKtok);
  const float* vsc = reinterpret_cast<const float*>(rec + kOffVscale);
  const float* vmn = reinterpret_cast<const float*>(rec + kOffVmin);
  float s[2][4], vs[2][4], vm[2][4];
  float tmax = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t0 = 8 * (4 * g + i) + 2 * w;
    const float2 kt = *reinterpret_cast<const float2*>(ktok + t0);
    const float2 va = *reinterpret_cast<const float2*>(vsc + t0);
    const float2 ma = *reinterpret_cast<const float2*>(vmn + t0);
    s[0][i] = scale_log2 * kt.x * (acc0[i] * unscale + bias);
    s[1][i] = scale_log2 * kt.y * (acc1[i] * unscale + bias);
    vs[0][i] = va.x; vs[1][i] = va.y; vm[0][i] = ma.x; vm[1][i] = ma.y;
    tmax = fmaxf(tmax, fmaxf(s[0][i], s[1][i]));
  }
  tmax = wave_max16(tmax);
  const float m_new = fmaxf(st.m, tmax);
  const float alpha = __builtin_amdgcn_exp2f(st.m - m_new);   // 0 on the first tile
  float psum = 0.0f, upart = 0.0f, wmax = 0.0f;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float pj = __builtin_amdgcn_exp2f(s[j][i] - m_new);
      psum += pj;
      upart += pj * vm[j][i];
      wmax = fmaxf(wmax, vs[j][i]);
      s[j][i] = pj * vs[j][i];          // w = p * vscale
    }
  psum = wave_sum16(psum);
  const float u = wave_sum16(upart);
  st.l = st.l * alpha + psum;
  st.m = m_new;
  wmax = wave_max16(wmax);
  const int vexp = fp16_scale_exp(wmax);
  const float fv = pow2i(vexp);

  // ---- PV over token step w: O = W * ZV, 8 channel blocks x (hi, lo) ----
  uint32_t wh[4], wl[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const float x0 = s[0][q] * fv, x1 = s[1][q] * fv;
    const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
    wh[q] = pack_h2(h0, h1);
    wl[q] = pack_h2((_Float16)(x0 - (float)h0), (_Float16)(x1 - (float)h1));
  }
  const half8 Wh = as_half8(wh[0], wh[1], wh[2], wh[3]);
  const half8 Wl = as_half8(wl[0], wl[1], wl[2], wl[3]);
  floatx4 po[8];
  const uint8_t* vcode = rec + kOffV;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int dw = 4 * qb + (n >> 2);
    const uint32_t bsel = (uint32_t)(n & 3);
    const uint32_t vsel = bsel | (12u << 8) | ((4u + bsel) << 16) | (12u << 24);
    uint32_t pr[4], prs[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int ta = 8 * (4 * g + q) + 2 * w;
      const uint32_t da = *reinterpret_cast<const uint32_t*>(vcode + ta * (D / 4) + 4 * dw);
      const uint32_t db = *reinterpret_cast<const uint32_t*>(vcode + (ta + 1) * (D / 4) + 4 * dw);
      pr[q] = __builtin_amdgcn_perm(db, da, vsel);
      prs[q] = pr[q] << 4;
    }
    // crumb kk lands in bits 4-5 (kk even) or 6-7 (kk odd) of each half
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const uint32_t mask = (kk & 1) ? 0x00C000C0u : 0x00300030u;
      const half8 Bv = (kk < 2) ? as_half8(prs[0] & mask, prs[1] & mask, prs[2] & mask, prs[3] & mask)
                                : as_half8(pr[0] & mask, pr[1] & mask, pr[2] & mask, pr[3] & mask);
      floatx4 z = {0.f, 0.f, 0.f, 0.f};
      z = __builtin_amdgcn_mfma_f32_16x16x32_f16(Wh, Bv, z, 0, 0, 0);
      po[4 * qb + kk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Wl, Bv, z, 0, 0, 0);
    }
  }

  // ---- fold: o' = o' * alpha_h + vchan_c * (O * 2^24 / (fv 2^shift) + u_h) ----
  const float* vch = reinterpret_cast<const float*>(rec + kOffVchan);
  float alpha_r[4], u_r[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    alpha_r[i] = __shfl(alpha, 4 * g + i, 64);
    u_r[i] = __shfl(u, 4 * g + i, 64);
  }
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const float4 vc = *reinterpret_cast<const float4*>(vch + 4 * (16 * qb + n));
    const float vcv[4] = {vc.x, vc.y, vc.z, vc.w};
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      const int nb = 4 * qb + kk;
      const float un = pow2i(24 - vexp - ((kk & 1) ? 6 : 4));
#pragma unroll
      for (int i = 0; i < 4; ++i)
        st.o[nb][i] = st.o[nb][i] * alpha_r[i] + vcv[kk] * (po[nb][i] * un + u_r[i]);
    }
  }
}

// Channel held by output instance nb of lane column n.
__device__ __forceinline__ int out_channel(int nb, int n) { return 4 * (16 * (nb >> 2) + n) + (nb & 3); }

constexpr int kRow = D + 4;                 // padded window row (528 bytes)
constexpr int kWinRowsLds = kWinChunkFused; // window rows staged per workgroup
constexpr int kMax3(int a, int b, int c) { return a > b ? (a > c ? a : c) : (b > c ? b : c); }
// double-buffered records | window K and V rows | combine reduction [4][2][8][D]
constexpr int kLdsBytes = kMax3(2 * kRecBytes, 2 * kWinRowsLds * kRow * 4, 4 * 2 * 8 * D * 4);

template <int G>
__global__ void __launch_bounds__(256) decode_fused_kernel(DecodeParams P) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int n_split = P.n_tsplit + P.n_wsplit;

  __shared__ __attribute__((aligned(16))) uint8_t s_buf[kLdsBytes];   // records / window rows / scratch
  __shared__ __attribute__((aligned(16))) float s_q[G][D];
  __shared__ float s_ml[4][G][2];

  const SeqView sv = seq_view(P, b);
  const bool is_tile = split < P.n_tsplit;
  int t_begin = 0, t_end = 0, w_begin = 0, w_end = 0;
  if (is_tile) {
    t_begin = split * P.tps;
    t_end = min(sv.nt, t_begin + P.tps);
  } else {
    w_begin = (split - P.n_tsplit) * kWinChunkFused;
    w_end = min(sv.nw, w_begin + kWinChunkFused);
  }
  float* part = P.part + (((int64_t)b * P.n_q + (int64_t)kvh * G) * n_split + split) * (D + 4);
  const int64_t hs = (int64_t)n_split * (D + 4);   // partial of head h at part + h * hs
  const bool empty = is_tile ? (t_begin >= t_end) : (w_begin >= w_end);

  if (empty) {
    for (int i = tid; i < G * (D + 4); i += 256) {
      const int h = i / (D + 4), c = i % (D + 4);
      st_part(&part[h * hs + c], (c == D) ? -INFINITY : 0.0f);
    }
  } else if (is_tile) {
    // first record's loads go out before the query rotation
    const uint8_t* recs = P.records + (sv.rec_row0 * (int64_t)P.n_kv + kvh) * kRecBytes;
    const int64_t rstride = (int64_t)P.n_kv * kRecBytes;
    constexpr int kU4 = kRecBytes / 16;             // 960 uint4 per record
    uint4 t0v, t1v, t2v, t3v;                       // this thread's share of one record
#define KVARN_LOAD_REC(tile_)                                                              \
    do {                                                                                   \
      const uint4* src_ = reinterpret_cast<const uint4*>(recs + (int64_t)(tile_) * rstride); \
      t0v = src_[tid];                                                                     \
      t1v = src_[tid + 256];                                                               \
      t2v = src_[tid + 512];                                                               \
      if (tid + 768 < kU4) t3v = src_[tid + 768];                                          \
    } while (0)
#define KVARN_STORE_REC(buf_)                                                              \
    do {                                                                                   \
      uint4* dst_ = reinterpret_cast<uint4*>(s_buf + (buf_) * kRecBytes);                  \
      dst_[tid] = t0v;                                                                     \
      dst_[tid + 256] = t1v;                                                               \
      dst_[tid + 512] = t2v;                                                               \
      if (tid + 768 < kU4) dst_[tid + 768] = t3v;                                          \
    } while (0)
    KVARN_LOAD_REC(t_begin);
    // rotated query rows for the G heads
    const float* qsrc = (P.q_rot ? P.q_rot : P.q) + ((int64_t)b * P.n_q + (int64_t)kvh * G) * D;
    if (P.q_rot) {
      for (int i = tid; i < G * D; i += 256) s_q[i / D][i % D] = qsrc[i];
    } else {
      for (int h = wv; h < G; h += 4) {
        float x0 = qsrc[h * D + lane], x1 = qsrc[h * D + lane + 64];
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
          const bool up = (lane & m) != 0;
          const float p0 = __shfl_xor(x0, m, 64), p1 = __shfl_xor(x1, m, 64);
          x0 = up ? (p0 - x0) : (x0 + p0);
          x1 = up ? (p1 - x1) : (x1 + p1);
        }
        const float a = x0, c = x1;
        s_q[h][lane] = (a + c) * wht_scale<D>();
        s_q[h][lane + 64] = (a - c) * wht_scale<D>();
      }
    }
    KVARN_STORE_REC(0);
    __syncthreads();
    WaveState st;
    st.m = -INFINITY;
    st.l = 0.0f;
#pragma unroll
    for (int nb = 0; nb < 8; ++nb) st.o[nb] = (floatx4){0.f, 0.f, 0.f, 0.f};
    const float scale_log2 = P.scale * kLog2e;
    int cur = 0;
    for (int tile = t_begin; tile < t_end; ++tile) {
      const bool more = tile + 1 < t_end;
      if (more) KVARN_LOAD_REC(tile + 1);            // in flight during the compute
      tile_quarter<G>(s_buf + cur * kRecBytes, &s_q[0][0], scale_log2, st, lane, wv);
      if (more) KVARN_STORE_REC(cur ^ 1);
      __syncthreads();
      cur ^= 1;
    }
#undef KVARN_LOAD_REC
#undef KVARN_STORE_REC
    // ---- merge the 4 waves' streams into one partial ----
    float* s_o = reinterpret_cast<float*>(s_buf);   // [4][G][D]
    const int n = lane & 15, g = lane >> 4;
    if (n < G && g == 0) {
      s_ml[wv][n][0] = st.m;
      s_ml[wv][n][1] = st.l;
    }
#pragma unroll
    for (int nb = 0; nb < 8; ++nb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int h = 4 * g + i;
        if (h < G) s_o[(wv * G + h) * D + out_channel(nb, n)] = st.o[nb][i];
      }
    __syncthreads();
    for (int i = tid; i < G * D; i += 256) {
      const int h = i / D, c = i % D;
      float M = -INFINITY;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, s_ml[w][h][0]);
      float L = 0.0f, o = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float mw = s_ml[w][h][0];
        const float wt = (mw == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mw - M);
        L += wt * s_ml[w][h][1];
        o += wt * s_o[(w * G + h) * D + c];
      }
      st_part(&part[h * hs + c], o);
      if (c == 0) {
        st_part(&part[h * hs + D], M);        // log2 domain
        st_part(&part[h * hs + D + 1], L);
      }
    }
  } else {
    // ---- raw window chunk [w_begin, w_end): K and V rows staged together ----
    float* s_k = reinterpret_cast<float*>(s_buf);                 // [32][kRow]
    float* s_v = s_k + kWinRowsLds * kRow;                        // [32][kRow]
    float* s_sc = s_q[0];                                         // reused after scores: [G][32]
    const float* kb = P.k_win + sv.win_off + (int64_t)kvh * P.win_head_stride;
    const float* vb = P.v_win + sv.win_off + (int64_t)kvh * P.win_head_stride;
    const int nw = w_end - w_begin;
    {
      // thread: row tid/8, float4 columns 4*(tid%8) .. +3, for K and for V
      const int r = tid >> 3, c4 = (tid & 7) * 4;
      float4 tk[4], tv[4];
      if (r < nw) {
        const float4* rk = reinterpret_cast<const float4*>(kb + (int64_t)(w_begin + r) * P.win_tok_stride);
        const float4* rv = reinterpret_cast<const float4*>(vb + (int64_t)(w_begin + r) * P.win_tok_stride);
#pragma unroll
        for (int j = 0; j < 4; ++j) { tk[j] = rk[c4 + j]; tv[j] = rv[c4 + j]; }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) { tk[j] = make_float4(0.f, 0.f, 0.f, 0.f); tv[j] = tk[j]; }
      }
      const float* qsrc = P.q + ((int64_t)b * P.n_q + (int64_t)kvh * G) * D;
      for (int i = tid; i < G * D; i += 256) s_q[i / D][i % D] = qsrc[i];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        *reinterpret_cast<float4*>(s_k + r * kRow + 4 * (c4 + j)) = tk[j];
        *reinterpret_cast<float4*>(s_v + r * kRow + 4 * (c4 + j)) = tv[j];
      }
    }
    __syncthreads();
    const float scale_log2 = P.scale * kLog2e;
    // scores: thread = (token tid/8, channel eighth tid%8), reduced over 8 lanes
    float sc_mine = 0.0f;   // score of (token tid/8) for head (tid%8) when tid%8 < G
    {
      const int t = tid >> 3, e8 = tid & 7;
      float a[G];
#pragma unroll
      for (int h = 0; h < G; ++h) a[h] = 0.0f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float4 kk = *reinterpret_cast<const float4*>(s_k + t * kRow + 16 * e8 + 4 * j);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          const float4 qq = *reinterpret_cast<const float4*>(&s_q[h][16 * e8 + 4 * j]);
          a[h] += qq.x * kk.x + qq.y * kk.y + qq.z * kk.z + qq.w * kk.w;
        }
      }
#pragma unroll
      for (int h = 0; h < G; ++h) {
        float v = a[h];
        v += __shfl_xor(v, 1, 64);
        v += __shfl_xor(v, 2, 64);
        v += __shfl_xor(v, 4, 64);
        if (e8 == h) sc_mine = (t < nw) ? v * scale_log2 : -INFINITY;
      }
    }
    __syncthreads();   // s_q is reused for the probabilities below
    if ((tid & 7) < G) s_sc[(tid & 7) * kWinRowsLds + (tid >> 3)] = sc_mine;
    __syncthreads();
    for (int h = wv; h < G; h += 4) {
      const float sc = (lane < kWinRowsLds) ? s_sc[h * kWinRowsLds + lane] : -INFINITY;
      const float m = wave_max(sc);
      const float p = (lane < nw) ? __builtin_amdgcn_exp2f(sc - m) : 0.0f;
      const float l = wave_sum(p);
      if (lane < kWinRowsLds) s_sc[h * kWinRowsLds + lane] = p;
      if (lane == 0) { s_ml[0][h][0] = m; s_ml[0][h][1] = l; }
    }
    __syncthreads();
    for (int i = tid; i < G * D; i += 256) {
      const int h = i / D, c = i % D;
      float o = 0.0f;
#pragma unroll 8
      for (int t = 0; t < kWinRowsLds; ++t) o += s_sc[h * kWinRowsLds + t] * s_v[t * kRow + c];
      st_part(&part[h * hs + c], o);
      if (c == 0) {
        st_part(&part[h * hs + D], s_ml[0][h][0]);
        st_part(&part[h * hs + D + 1], s_ml[0][h][1]);
      }
    }
  }

}

// ---------------------------------------------------------------------------
// Combine: one workgroup per (query head, sequence).  Thread (quarter sq, channel
// pair c2) folds the splits s = sq, sq+4, ... with an online log-sum-exp; the
// four quarters are merged in LDS; the rotated tile part gets one inverse WHT,
// the raw window part is added, and the result is divided by L.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) decode_combine128_kernel(DecodeParams P) {
  const int hq = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int sq = tid >> 6, c2 = (tid & 63) * 2;
  const int n_split = P.n_tsplit + P.n_wsplit;
  const float* ph = P.part + ((int64_t)b * P.n_q + hq) * (int64_t)n_split * (D + 4);
  __shared__ float s_m[4][64], s_l[4][64];
  __shared__ __attribute__((aligned(16))) float s_o[4][2][D];
  __shared__ float s_rot[D];

  float M = -INFINITY, L = 0.0f;
  float t0 = 0.f, t1 = 0.f, w0 = 0.f, w1 = 0.f;
  auto fold = [&](int s, float m, float l, float2 v) {
    if (m == -INFINITY) return;
    if (m > M) {
      const float r = __builtin_amdgcn_exp2f(M - m);   // 0 when M = -inf
      L *= r; t0 *= r; t1 *= r; w0 *= r; w1 *= r;
      M = m;
    }
    const float wt = __builtin_amdgcn_exp2f(m - M);
    L += wt * l;
    if (s < P.n_tsplit) { t0 += wt * v.x; t1 += wt * v.y; }
    else { w0 += wt * v.x; w1 += wt * v.y; }
  };
  int s = sq;
  // batches of 4 splits per thread: all loads of a batch are issued first
  for (; s + 12 < n_split; s += 16) {
    float m[4], l[4];
    float2 v[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float* ps = ph + (int64_t)(s + 4 * j) * (D + 4);
      m[j] = ps[D];
      l[j] = ps[D + 1];
      v[j] = *reinterpret_cast<const float2*>(ps + c2);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) fold(s + 4 * j, m[j], l[j], v[j]);
  }
  for (; s < n_split; s += 4) {
    const float* ps = ph + (int64_t)s * (D + 4);
    fold(s, ps[D], ps[D + 1], *reinterpret_cast<const float2*>(ps + c2));
  }
  s_m[sq][tid & 63] = M;
  s_l[sq][tid & 63] = L;
  __syncthreads();
  // weight of this quarter in the merged result
  float Mall = -INFINITY;
#pragma unroll
  for (int k = 0; k < 4; ++k) Mall = fmaxf(Mall, s_m[k][tid & 63]);
  float Lall = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float mk = s_m[k][tid & 63];
    Lall += (mk == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mk - Mall) * s_l[k][tid & 63];
  }
  const float wq = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M - Mall);
  s_o[sq][0][c2] = wq * t0;
  s_o[sq][0][c2 + 1] = wq * t1;
  s_o[sq][1][c2] = wq * w0;
  s_o[sq][1][c2 + 1] = wq * w1;
  __syncthreads();
  if (tid < 64) {
    const int lane = tid;
    float r0 = 0.f, r1 = 0.f, a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      r0 += s_o[k][0][lane]; r1 += s_o[k][0][lane + 64];
      a0 += s_o[k][1][lane]; a1 += s_o[k][1][lane + 64];
    }
#pragma unroll
    for (int m = 1; m < 64; m <<= 1) {
      const bool up = (lane & m) != 0;
      const float p0 = __shfl_xor(r0, m, 64), p1 = __shfl_xor(r1, m, 64);
      r0 = up ? (p0 - r0) : (r0 + p0);
      r1 = up ? (p1 - r1) : (r1 + p1);
    }
    const float x = r0, y = r1;
    r0 = (x + y) * wht_scale<D>();
    r1 = (x - y) * wht_scale<D>();
    const float invL = 1.0f / Lall;   // every thread of a channel pair holds the same Lall
    float* o = P.out + ((int64_t)b * P.n_q + hq) * D;
    o[lane] = (r0 + a0) * invL;
    o[lane + 64] = (r1 + a1) * invL;
  }
  (void)s_rot;
}

}  // namespace

hipError_t launch_decode_fused(const DecodeParams& P, int batch, hipStream_t stream) {
  dim3 grid(P.n_tsplit + P.n_wsplit, P.n_kv, batch);
  hipError_t e = hipSuccess;
  switch (P.G) {
    case 1: hipLaunchKernelGGL(decode_fused_kernel<1>, grid, dim3(256), 0, stream, P); break;
    case 2: hipLaunchKernelGGL(decode_fused_kernel<2>, grid, dim3(256), 0, stream, P); break;
    case 4: hipLaunchKernelGGL(decode_fused_kernel<4>, grid, dim3(256), 0, stream, P); break;
    case 8: hipLaunchKernelGGL(decode_fused_kernel<8>, grid, dim3(256), 0, stream, P); break;
    default: return hipErrorInvalidValue;
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine128_kernel, dim3(P.n_q, batch), dim3(256), 0, stream, P);
  return hipGetLastError();
}

}  // namespace kvarn
