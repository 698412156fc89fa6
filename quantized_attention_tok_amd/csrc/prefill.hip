// prefill.hip -- chunked prefill attention for head_dim 128 on gfx950 matrix
// cores.
//
// Query position p of the chunk attends the tiles [0, T(p)) in compressed form
// and the raw tokens [128 T(p), p] (T(p) = max(0, floor((p + 1 - W) / 128)),
// the decode view at p), with one streaming softmax over both and the inverse
// WHT applied once, between the tile part (rotated domain) and the raw part
// (PR #434 commit list: chunked prefill with a single streaming softmax over
// compressed tiles + FP32 window and a deferred inverse WHT; issue #433 item 1:
// the Q.K score block of the compressed tiles belongs on the matrix units).
//
// Work split: one wave owns 16 query rows (16 consecutive positions of one
// query head: one MFMA column block) for the whole computation, so the online
// softmax never leaves the wave; a workgroup is 4 such waves of one KV head
// sharing the staged tile records (double-buffered in LDS) and raw K/V rows.
// Per compressed tile and wave:
//   S^T[t][r] = sum_c zK[t][c] q~[r][c],   q~ = q' kscale      (fp16 MFMA,
//               code nibbles and hi/lo q~, 8 row blocks of 16 tokens)
//   O'[r][c] += sum_t w[r][t] zV[t][c],    w = p vscale        (fp16 MFMA,
//               hi/lo w and 2-bit codes, 4 token steps x 8 channel blocks)
// The score layout of the first product (lane (g, r) holds tokens
// 32 s + 8 g .. + 7 of row r) is exactly the A-operand layout of the second,
// so the probabilities go from one to the other without data movement.
// After the last tile each row's O' is rotated back with the WHT butterflies
// (in-lane and across the 16 lanes of a row), then the raw tokens are added
// with fp32 MFMAs (v_mfma_f32_16x16x4_f32): scores from the raw query and raw
// keys, and the aggregate of raw values straight into the same accumulator.
#include <float.h>

#include "kvarn_launch.h"
#include "kvarn_mfma.h"

namespace kvarn {
namespace {

using namespace mfma;

constexpr int kRows = 16;                          // query rows per wave
constexpr int kQRow = D + 4;                       // padded LDS row of q' (floats)
constexpr int kRawTok = 32;                        // raw tokens staged per step
constexpr int kRawRow = D + 4;                     // padded LDS row of raw K / V (floats)
constexpr int kLdsRec = 2 * kRecBytes;             // double-buffered records
constexpr int kLdsQ = 4 * kRows * kQRow * 4;       // q' rows of the 4 waves
constexpr int kLdsRaw = 2 * kRawTok * kRawRow * 4; // raw K and V rows
constexpr int kLdsBytes = (kLdsRec + kLdsQ) > kLdsRaw ? (kLdsRec + kLdsQ) : kLdsRaw;

__device__ __forceinline__ int tiles_at(int64_t p, int window) {
  const int64_t ahead = p + 1 - window;
  return ahead > 0 ? (int)(ahead / kTile) : 0;
}

__global__ void __launch_bounds__(256) prefill_mfma_kernel(PrefillParams P) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int kvh = blockIdx.y;
  const int G = P.G;
  const int n_blk = ((P.chunk + kRows - 1) / kRows) * G;   // (position group, head) column blocks
  const int blk_first = blockIdx.x * 4;
  const int blk_last = min(blk_first + 3, n_blk - 1);
  const int blk = blk_first + wv;
  const bool active = blk < n_blk;
  const int pg = (active ? blk : blk_last) / G;
  const int hq = kvh * G + (active ? blk : blk_last) % G;
  const int r0 = kRows * pg;                                // chunk row of column 0
  const int64_t prow = P.pos0 + r0 + n;                     // position of this lane's column
  const bool row_ok = active && (r0 + n < P.chunk);
  const int T_row = row_ok ? tiles_at(prow, P.window) : 0;
  const int64_t p_wlast = P.pos0 + min(r0 + kRows - 1, P.chunk - 1);
  const int T_wave = active ? tiles_at(p_wlast, P.window) : 0;
  // positions spanned by the workgroup
  const int64_t p_first = P.pos0 + kRows * (blk_first / G);
  const int64_t p_last = P.pos0 + min(kRows * (blk_last / G) + kRows - 1, P.chunk - 1);
  const int T_wg = tiles_at(p_last, P.window);

  __shared__ __attribute__((aligned(16))) uint8_t s_lds[kLdsBytes];
  float* s_q = reinterpret_cast<float*>(s_lds + kLdsRec) + wv * kRows * kQRow;
  const float scale_log2 = P.scale * kLog2e;

  // ---- stage the first record and this wave's rotated query rows ----
  const uint8_t* recs = P.records + (int64_t)kvh * kRecBytes;
  const int64_t rstride = (int64_t)P.n_kv * kRecBytes;
  constexpr int kU4 = kRecBytes / 16;
  uint4 t0v, t1v, t2v, t3v;
#define KVARN_LOAD_REC(tile_)                                                              \
  do {                                                                                     \
    const uint4* src_ = reinterpret_cast<const uint4*>(recs + (int64_t)(tile_) * rstride); \
    t0v = src_[tid];                                                                       \
    t1v = src_[tid + 256];                                                                 \
    t2v = src_[tid + 512];                                                                 \
    if (tid + 768 < kU4) t3v = src_[tid + 768];                                            \
  } while (0)
#define KVARN_STORE_REC(buf_)                                                              \
  do {                                                                                     \
    uint4* dst_ = reinterpret_cast<uint4*>(s_lds + (buf_) * kRecBytes);                    \
    dst_[tid] = t0v;                                                                       \
    dst_[tid + 256] = t1v;                                                                 \
    dst_[tid + 512] = t2v;                                                                 \
    if (tid + 768 < kU4) dst_[tid + 768] = t3v;                                            \
  } while (0)
  if (T_wg > 0) KVARN_LOAD_REC(0);
  for (int i = lane; i < kRows * (D / 4); i += 64) {
    const int r = i >> 5, c4 = i & 31;
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (active && r0 + r < P.chunk)
      x = *reinterpret_cast<const float4*>(P.q_rot + ((int64_t)(r0 + r) * P.n_q + hq) * D + 4 * c4);
    *reinterpret_cast<float4*>(s_q + r * kQRow + 4 * c4) = x;
  }
  if (T_wg > 0) KVARN_STORE_REC(0);
  __syncthreads();
  // max |q'| of row n (bound for the fp16 scale of q~)
  float qmax = 0.0f;
#pragma unroll
  for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      const float4 x = *reinterpret_cast<const float4*>(s_q + n * kQRow + 32 * k4 + 8 * g + 4 * h2);
      qmax = fmaxf(qmax, fmaxf(fmaxf(fabsf(x.x), fabsf(x.y)), fmaxf(fabsf(x.z), fabsf(x.w))));
    }
  qmax = wave_max16(qmax);

  float m_run = -INFINITY, l_run = 0.0f;       // softmax state of row n (log2 domain)
  floatx4 O[2][4];                              // rows 4g + i, channel 64 qb + 4 n + kk
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) O[qb][kk] = (floatx4){0.f, 0.f, 0.f, 0.f};

  // byte (n & 3) of two code dwords into the low bytes of two halves
  const uint32_t nb = (uint32_t)(n & 3);
  const uint32_t sel = nb | (12u << 8) | ((4u + nb) << 16) | (12u << 24);

  // ---- compressed tiles ----
  int cur = 0;
  for (int j = 0; j < T_wg; ++j) {
    const bool more = j + 1 < T_wg;
    if (more) KVARN_LOAD_REC(j + 1);   // in flight during the compute
    if (j < T_wave) {
      const uint8_t* rec = s_lds + cur * kRecBytes;
      const float* ks = reinterpret_cast<const float*>(rec + kOffKscale);
      const float* km = reinterpret_cast<const float*>(rec + kOffKmin);
      const float2 kk2 = *reinterpret_cast<const float2*>(ks + 2 * lane);
      const float kmx = wave_max(fmaxf(kk2.x, kk2.y));   // tile max kscale (>= 0)
      const int fexp = fp16_scale_exp(kmx * qmax);
      const float f16inv = pow2i(fexp - 4);
      const float unscale = pow2i(24 - fexp);
      floatx4 acc[4][2];
#pragma unroll
      for (int bg = 0; bg < 4; ++bg) acc[bg][0] = acc[bg][1] = (floatx4){0.f, 0.f, 0.f, 0.f};
      float bias_part = 0.0f;
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        // B: q~ of row n, channels 32 k4 + 8 g .. + 7, hi and lo
        uint32_t bh[4], bl[4];
#pragma unroll
        for (int h2 = 0; h2 < 2; ++h2) {
          const int c0 = 32 * k4 + 8 * g + 4 * h2;
          const float4 q = *reinterpret_cast<const float4*>(s_q + n * kQRow + c0);
          const float4 sc = *reinterpret_cast<const float4*>(ks + c0);
          const float4 mn = *reinterpret_cast<const float4*>(km + c0);
          bias_part += q.x * mn.x + q.y * mn.y + q.z * mn.z + q.w * mn.w;
          _Float16 h0, h1, h2_, h3, l0, l1, l2, l3;
          split_h(q.x * sc.x * f16inv, h0, l0);
          split_h(q.y * sc.y * f16inv, h1, l1);
          split_h(q.z * sc.z * f16inv, h2_, l2);
          split_h(q.w * sc.w * f16inv, h3, l3);
          bh[2 * h2] = pack_h2(h0, h1);
          bh[2 * h2 + 1] = pack_h2(h2_, h3);
          bl[2 * h2] = pack_h2(l0, l1);
          bl[2 * h2 + 1] = pack_h2(l2, l3);
        }
        const half8 Bh = as_half8(bh[0], bh[1], bh[2], bh[3]);
        const half8 Bl = as_half8(bl[0], bl[1], bl[2], bl[3]);
#pragma unroll
        for (int bg = 0; bg < 4; ++bg) {
          // A: code byte 16 bg + n (tokens 32 bg + 2n, + 1) of channels 32 k4 + 8 g .. + 7
          uint32_t ae[4], ao[4];
#pragma unroll
          for (int p = 0; p < 4; ++p) {
            const int c = 32 * k4 + 8 * g + 2 * p;
            const uint32_t d0 = *reinterpret_cast<const uint32_t*>(rec + c * 64 + 16 * bg + 4 * (n >> 2));
            const uint32_t d1 = *reinterpret_cast<const uint32_t*>(rec + (c + 1) * 64 + 16 * bg + 4 * (n >> 2));
            const uint32_t x = __builtin_amdgcn_perm(d1, d0, sel);
            ae[p] = nib_lo(x);
            ao[p] = nib_hi(x);
          }
          const half8 Ae = as_half8(ae[0], ae[1], ae[2], ae[3]);
          const half8 Ao = as_half8(ao[0], ao[1], ao[2], ao[3]);
          acc[bg][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ae, Bh, acc[bg][0], 0, 0, 0);
          acc[bg][0] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ae, Bl, acc[bg][0], 0, 0, 0);
          acc[bg][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ao, Bh, acc[bg][1], 0, 0, 0);
          acc[bg][1] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ao, Bl, acc[bg][1], 0, 0, 0);
        }
      }
      const float bias = wave_sum16(bias_part);
      // scores (log2 domain): token 32 bg + 8 g + 2 i + nib of row n
      const bool vis = j < T_row;
      const float* ktok = reinterpret_cast<const float*>(rec + kOffKtok);
      float tmax = -INFINITY;
#pragma unroll
      for (int bg = 0; bg < 4; ++bg) {
        const float4 ka = *reinterpret_cast<const float4*>(ktok + 32 * bg + 8 * g);
        const float4 kb = *reinterpret_cast<const float4*>(ktok + 32 * bg + 8 * g + 4);
        const float kt[8] = {ka.x, ka.y, ka.z, ka.w, kb.x, kb.y, kb.z, kb.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int nib = 0; nib < 2; ++nib) {
            const float sv = vis ? scale_log2 * kt[2 * i + nib] * (acc[bg][nib][i] * unscale + bias) : -INFINITY;
            acc[bg][nib][i] = sv;
            tmax = fmaxf(tmax, sv);
          }
      }
      tmax = wave_max16(tmax);
      const float m_new = fmaxf(m_run, tmax);
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);   // 0 while nothing was seen
      const float* vsc = reinterpret_cast<const float*>(rec + kOffVscale);
      const float* vmn = reinterpret_cast<const float*>(rec + kOffVmin);
      const float2 vv = *reinterpret_cast<const float2*>(vsc + 2 * lane);
      const int vexp = fp16_scale_exp(wave_max(fmaxf(vv.x, vv.y)));   // p <= 1, w <= max vscale
      const float fv = pow2i(vexp);
      // PV: token step bg uses the probabilities this lane already holds
      float psum = 0.0f, upart = 0.0f;
      floatx4 z[2][4];
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) z[qb][kk] = (floatx4){0.f, 0.f, 0.f, 0.f};
      const uint8_t* vcode = rec + kOffV;
#pragma unroll
      for (int bg = 0; bg < 4; ++bg) {
        const float4 va = *reinterpret_cast<const float4*>(vsc + 32 * bg + 8 * g);
        const float4 vb = *reinterpret_cast<const float4*>(vsc + 32 * bg + 8 * g + 4);
        const float4 ma = *reinterpret_cast<const float4*>(vmn + 32 * bg + 8 * g);
        const float4 mb = *reinterpret_cast<const float4*>(vmn + 32 * bg + 8 * g + 4);
        const float vs8[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
        const float vm8[8] = {ma.x, ma.y, ma.z, ma.w, mb.x, mb.y, mb.z, mb.w};
        uint32_t wh[4], wl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          _Float16 hh[2], ll[2];
#pragma unroll
          for (int nib = 0; nib < 2; ++nib) {
            const float pj = __builtin_amdgcn_exp2f(acc[bg][nib][i] - m_use);
            psum += pj;
            upart += pj * vm8[2 * i + nib];
            split_h(pj * vs8[2 * i + nib] * fv, hh[nib], ll[nib]);
          }
          wh[i] = pack_h2(hh[0], hh[1]);
          wl[i] = pack_h2(ll[0], ll[1]);
        }
        const half8 Wh = as_half8(wh[0], wh[1], wh[2], wh[3]);
        const half8 Wl = as_half8(wl[0], wl[1], wl[2], wl[3]);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          // B: byte 16 qb + n of tokens 32 bg + 8 g .. + 7; crumb kk is channel 64 qb + 4 n + kk
          uint32_t pr[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            const int t = 32 * bg + 8 * g + 2 * q;
            const uint32_t da = *reinterpret_cast<const uint32_t*>(vcode + t * (D / 4) + 16 * qb + 4 * (n >> 2));
            const uint32_t db = *reinterpret_cast<const uint32_t*>(vcode + (t + 1) * (D / 4) + 16 * qb + 4 * (n >> 2));
            pr[q] = __builtin_amdgcn_perm(db, da, sel);
          }
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const uint32_t mask = (kk & 1) ? 0x00C000C0u : 0x00300030u;
            const int sh = (kk < 2) ? 4 : 0;   // crumbs 0, 1 move up into bits 4-7
            const half8 Bv = as_half8((pr[0] << sh) & mask, (pr[1] << sh) & mask, (pr[2] << sh) & mask,
                                      (pr[3] << sh) & mask);
            z[qb][kk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Wh, Bv, z[qb][kk], 0, 0, 0);
            z[qb][kk] = __builtin_amdgcn_mfma_f32_16x16x32_f16(Wl, Bv, z[qb][kk], 0, 0, 0);
          }
        }
      }
      l_run = l_run * alpha + wave_sum16(psum);
      const float u = wave_sum16(upart);
      m_run = m_new;
      // o' = o' alpha_r + vchan_c (Z 2^24 / (fv 2^shift) + u_r)
      const float* vch = reinterpret_cast<const float*>(rec + kOffVchan);
      float ar[4], ur[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ar[i] = __shfl(alpha, 4 * g + i, 64);
        ur[i] = __shfl(u, 4 * g + i, 64);
      }
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const float4 vc = *reinterpret_cast<const float4*>(vch + 64 * qb + 4 * n);
        const float vcv[4] = {vc.x, vc.y, vc.z, vc.w};
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          const float un = pow2i(24 - vexp - ((kk & 1) ? 6 : 4));
#pragma unroll
          for (int i = 0; i < 4; ++i) O[qb][kk][i] = O[qb][kk][i] * ar[i] + vcv[kk] * (z[qb][kk][i] * un + ur[i]);
        }
      }
    }
    if (more) KVARN_STORE_REC(cur ^ 1);
    __syncthreads();
    cur ^= 1;
  }
#undef KVARN_LOAD_REC
#undef KVARN_STORE_REC

  // ---- inverse WHT of the tile part: channel 64 qb + 4 n + kk of row 4 g + i ----
  if (T_wave > 0) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {   // channel bits 0, 1 (kk)
        const float a0 = O[qb][0][i], a1 = O[qb][1][i], a2 = O[qb][2][i], a3 = O[qb][3][i];
        const float b0 = a0 + a1, b1 = a0 - a1, b2 = a2 + a3, b3 = a2 - a3;
        O[qb][0][i] = b0 + b2;
        O[qb][1][i] = b1 + b3;
        O[qb][2][i] = b0 - b2;
        O[qb][3][i] = b1 - b3;
      }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {   // channel bit 6 (qb)
        const float a = O[0][kk][i], b = O[1][kk][i];
        O[0][kk][i] = a + b;
        O[1][kk][i] = a - b;
      }
#pragma unroll
    for (int m = 1; m < 16; m <<= 1) {   // channel bits 2-5 (lane n)
      const bool up = (n & m) != 0;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float x = O[qb][kk][i];
            const float y = __shfl_xor(x, m, 64);
            O[qb][kk][i] = up ? (y - x) : (x + y);
          }
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i) O[qb][kk][i] *= wht_scale<D>();
  }

  // ---- raw tokens [128 T(p), p] on fp32 MFMA ----
  float4 qr[8];   // raw query of row n, channels 16 jj + 4 g .. + 3
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    qr[jj] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row_ok)
      qr[jj] = *reinterpret_cast<const float4*>(P.q + ((int64_t)(r0 + n) * P.n_q + hq) * D + 16 * jj + 4 * g);
  }
  float* s_k = reinterpret_cast<float*>(s_lds);
  float* s_v = s_k + kRawTok * kRawRow;
  const int64_t raw_lo = (int64_t)kTile * tiles_at(p_first, P.window);
  const int64_t wave_lo = (int64_t)kTile * tiles_at(P.pos0 + r0, P.window);
  const int64_t row_lo = (int64_t)kTile * T_row;
  const float* kbase = P.k + (int64_t)kvh * P.head_stride;
  const float* vbase = P.v + (int64_t)kvh * P.head_stride;
  for (int64_t t0 = raw_lo; t0 <= p_last; t0 += kRawTok) {
    __syncthreads();   // previous readers of the staging rows are done
    {
      const int r = tid >> 3, c4 = tid & 7;
      const int64_t t = t0 + r;
      float4 kx[4], vx[4];
      if (t <= p_last) {
        const float4* rk = reinterpret_cast<const float4*>(kbase + (t - P.raw_base) * P.tok_stride);
        const float4* rv = reinterpret_cast<const float4*>(vbase + (t - P.raw_base) * P.tok_stride);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kx[e] = rk[c4 + 8 * e];
          vx[e] = rv[c4 + 8 * e];
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          kx[e] = make_float4(0.f, 0.f, 0.f, 0.f);
          vx[e] = kx[e];
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        *reinterpret_cast<float4*>(s_k + r * kRawRow + 4 * (c4 + 8 * e)) = kx[e];
        *reinterpret_cast<float4*>(s_v + r * kRawRow + 4 * (c4 + 8 * e)) = vx[e];
      }
    }
    __syncthreads();
#pragma unroll 1
    for (int sb = 0; sb < kRawTok / 16; ++sb) {
      const int64_t tb = t0 + 16 * sb;
      if (!active || tb > p_wlast || tb + 15 < wave_lo) continue;   // wave-uniform
      // S^T[t][r]: A = raw keys (row n = token tb + n), B = raw query of row n;
      // MFMA (jj, e) contracts channels 16 jj + 4 g' + e over K slots g'
      floatx4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) {
        const float4 ka = *reinterpret_cast<const float4*>(s_k + (16 * sb + n) * kRawRow + 16 * jj + 4 * g);
        sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(ka.x, qr[jj].x, sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(ka.y, qr[jj].y, sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(ka.z, qr[jj].z, sacc, 0, 0, 0);
        sacc = __builtin_amdgcn_mfma_f32_16x16x4f32(ka.w, qr[jj].w, sacc, 0, 0, 0);
      }
      // lane (g, n): tokens tb + 4 g + i of row n
      float sv[4];
      float tmax = -INFINITY;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t t = tb + 4 * g + i;
        const bool vis = row_ok && t >= row_lo && t <= prow;
        sv[i] = vis ? sacc[i] * scale_log2 : -INFINITY;
        tmax = fmaxf(tmax, sv[i]);
      }
      tmax = wave_max16(tmax);
      const float m_new = fmaxf(m_run, tmax);
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      float pv[4], psum = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[i] = __builtin_amdgcn_exp2f(sv[i] - m_use);
        psum += pv[i];
      }
      l_run = l_run * alpha + wave_sum16(psum);
      m_run = m_new;
      float ar[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) ar[i] = __shfl(alpha, 4 * g + i, 64);
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int i = 0; i < 4; ++i) O[qb][kk][i] *= ar[i];
      // O[r][c] += sum_t p[r][t] v[t][c]; step i: K slot g is token tb + 4 g + i
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const float4 vv = *reinterpret_cast<const float4*>(s_v + (16 * sb + 4 * g + i) * kRawRow + 64 * qb + 4 * n);
          O[qb][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(pv[i], vv.x, O[qb][0], 0, 0, 0);
          O[qb][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(pv[i], vv.y, O[qb][1], 0, 0, 0);
          O[qb][2] = __builtin_amdgcn_mfma_f32_16x16x4f32(pv[i], vv.z, O[qb][2], 0, 0, 0);
          O[qb][3] = __builtin_amdgcn_mfma_f32_16x16x4f32(pv[i], vv.w, O[qb][3], 0, 0, 0);
        }
      }
    }
  }

  // ---- normalise and store rows 4 g + i ----
  if (!active) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float li = __shfl(l_run, 4 * g + i, 64);
    const int r = r0 + 4 * g + i;
    if (r < P.chunk) {
      const float inv = 1.0f / li;
      float* o = P.out + ((int64_t)r * P.n_q + hq) * D;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
        *reinterpret_cast<float4*>(o + 64 * qb + 4 * n) =
            make_float4(O[qb][0][i] * inv, O[qb][1][i] * inv, O[qb][2][i] * inv, O[qb][3][i] * inv);
    }
  }
}

}  // namespace

hipError_t launch_prefill_mfma(const PrefillParams& P, hipStream_t stream) {
  const int n_blk = ((P.chunk + kRows - 1) / kRows) * P.G;
  dim3 grid((n_blk + 3) / 4, P.n_kv);
  hipLaunchKernelGGL(prefill_mfma_kernel, grid, dim3(256), 0, stream, P);
  return hipGetLastError();
}

}  // namespace kvarn
