// decode.hip -- KVarN split-tile decode attention for gfx950.
//
// Per sequence b and query head h (KV head h/G), one query attends the
// sequence's compressed tiles and its raw FP32 window:
//   tiles  (rotated domain): q~_c = q'_c kscale_c, bias = sum_c q'_c kmin_c,
//          score_t = tau * ktok_t * (sum_c q~_c zK_tc + bias);
//          w_t = p_t vscale_{t,g}, u_g = sum_t p_t vmin_{t,g},
//          o'_c += vchan_c (sum_t w_t zV_tc + u_g)
//   window (raw domain):     score_t = tau * q . k_t,  o_c += p_t v_tc
// (issue #180 Algorithm step 4: scales folded at read time; PR #434 commit
// list: single streaming softmax over compressed tiles + FP32 window with a
// deferred inverse WHT.)
//
// Split-tile schedule (issue #433 item 2): a fixed worst-case grid of
// (split, KV head, sequence) workgroups; splits beyond a sequence's tiles or
// window exit at once and write nothing (the combine reads only the splits
// that hold tiles or window tokens of the sequence).  Each workgroup keeps an online
// softmax (running max, sum, rescaled accumulator; state initialised to
// m = -inf, l = 0 before the first tile -- the hazard the PR #434 review
// points at) and writes (m, l, o) per query head.  The combine kernel merges
// the partials with log-sum-exp weights, applies the inverse WHT once to the
// merged rotated-domain tile part, adds the raw-domain window part and
// normalises.
#include <float.h>

#include "kvarn_launch.h"
#include "kvarn_mfma.h"

namespace kvarn {

namespace {

// ---------------------------------------------------------------------------
// partial kernel: one (split, kv head, sequence)
// ---------------------------------------------------------------------------
// GEN: records with P.kb-bit keys and P.vb-bit values (LSB-first bit
// streams); otherwise the K4V2 record.
template <int D, int G, bool H, bool GEN>
__global__ void __launch_bounds__(kDecThreads) decode_partial_kernel(DecodeParams P) {
  const int kb = GEN ? P.kb : 4, vb = GEN ? P.vb : 2;
  const RecRT R = rec_rt(D, H, kb, vb);
  const uint32_t kmask = (1u << kb) - 1u, vmask = (1u << vb) - 1u;
  constexpr int NG = D / 128;                 // value channel groups
  constexpr int HH = (G >= 2 && D == 128) ? 2 : 1;   // head halves (K: 128 tokens x HH)
  constexpr int GH = G / HH;                  // heads per thread in the K phase
  constexpr int CPT = (D >= kDecThreads) ? D / kDecThreads : 1;  // V channels per thread
  constexpr int VH = (D * HH >= kDecThreads) ? HH : 1;            // V head split
  constexpr int GV = G / VH;                  // heads per thread in the V phase
  static_assert(CPT * kDecThreads / VH >= D || D == 128, "layout");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int n_split = P.n_tsplit + P.n_wsplit;

  __shared__ __attribute__((aligned(16))) float s_q[G][D];   // rotated (tiles) or raw (window) query
  // q~ of the current tile [channel][head] in the key phase, then w = p * vscale
  // [group][token][head] (a token's heads contiguous) in the value phase: the
  // same D * G floats
  __shared__ __attribute__((aligned(16))) float s_qw[D * G];
  float(*s_qt)[G] = reinterpret_cast<float(*)[G]>(s_qw);
  float(*s_w)[kTile][G] = reinterpret_cast<float(*)[kTile][G]>(s_qw);
  // D = 512: the two halves of the workgroup sum a token's scores over the two
  // channel halves (otherwise only 128 threads would work on the keys); the
  // softmax waves add them (ktok kept apart from the value scales that
  // overwrite it).  The scores, then probabilities, of head h then sit on
  // the first half's sums of head h, which the same lanes read just before.
  // With both overlays the head_dim-512 workgroup fits twice in a CU's LDS.
  constexpr int KP = D >= 512 ? 2 : 1;
  __shared__ float s_kp[KP][G][kTile];
  __shared__ float s_ktok[kTile];
  __shared__ float s_sco[KP == 2 ? 1 : G * kTile];
  float(*s_sc)[kTile] = reinterpret_cast<float(*)[kTile]>(KP == 2 ? &s_kp[0][0][0] : s_sco);
  __shared__ float s_u[G][NG];                // sum p * vmin
  __shared__ float s_bias[G];
  __shared__ float s_m[G], s_l[G], s_alpha[G];
  // K codes, then V codes (+ 16 bytes: a code's second byte may be read past the end)
  __shared__ __attribute__((aligned(16))) uint8_t s_code[(GEN ? 128 : 64) * D + 16];
  __shared__ float s_scale[3 * D + 128];      // kscale, kmin, ktok  |  vchan, vscale, vmin

  const SeqView sv = seq_view(P, b);
  const int nt = sv.nt;
  const int nw = sv.nw;
  const bool is_tile = split < P.n_tsplit;
  int t_begin = 0, t_end = 0, w_begin = 0, w_end = 0;
  if (is_tile) {
    t_begin = split * P.tps;
    t_end = min(nt, t_begin + P.tps);
  } else {
    w_begin = (split - P.n_tsplit) * kWinChunk;
    w_end = min(nw, w_begin + kWinChunk);
  }

  float* part = P.part + (((int64_t)b * P.n_q + (int64_t)kvh * G) * n_split + split) * (D + 4);
  // a split with no tiles or tokens of this sequence writes nothing: the
  // combine reads only the splits that hold some
  const bool empty = is_tile ? (t_begin >= t_end) : (w_begin >= w_end);
  if (empty) return;

  // query rows for this KV head's G heads
  const float* qsrc = (is_tile ? P.q_rot : P.q) + ((int64_t)b * P.n_q + (int64_t)kvh * G) * D;
  for (int i = tid; i < G * D; i += kDecThreads) s_q[i / D][i % D] = qsrc[i];
  if (tid < G) { s_m[tid] = -INFINITY; s_l[tid] = 0.0f; s_alpha[tid] = 1.0f; }

  // V accumulators: thread owns channels c = (tid % (256/VH)) + k*(256/VH), heads hv*GV..
  constexpr int VSTRIDE = kDecThreads / VH;
  const int vc0 = tid % VSTRIDE;
  const int hv = tid / VSTRIDE;
  constexpr int VC = (D + VSTRIDE - 1) / VSTRIDE;   // channels per thread
  float acc[GV][VC];
#pragma unroll
  for (int h = 0; h < GV; ++h)
#pragma unroll
    for (int k = 0; k < VC; ++k) acc[h][k] = 0.0f;
  __syncthreads();

  if (is_tile) {
    const uint8_t* base = P.records + ((sv.rec_row0 + t_begin) * (int64_t)P.n_kv + kvh) * R.bytes;
    for (int tile = t_begin; tile < t_end; ++tile, base += (int64_t)P.n_kv * R.bytes) {
      // ---- stage K codes and key scales ----
      {
        const uint4* src = reinterpret_cast<const uint4*>(base + R.kcode);
        uint4* dst = reinterpret_cast<uint4*>(s_code);
        for (int i = tid; i < kb * D; i += kDecThreads) dst[i] = src[i];
        for (int i = tid; i < D; i += kDecThreads) {
          s_scale[i] = sc_ld<H>(base + R.kscale, i);
          s_scale[D + i] = sc_ld<H>(base + R.kmin, i);
        }
        if (tid < kTile) s_scale[2 * D + tid] = sc_ld<H>(base + R.ktok, tid);
      }
      __syncthreads();
      // q~ = q' * kscale and bias = q' . kmin
      for (int i = tid; i < G * D; i += kDecThreads) {
        const int h = i / D, c = i % D;
        s_qt[c][h] = s_q[h][c] * s_scale[c];
      }
      for (int h = wv; h < G; h += kDecThreads / 64) {
        float a = 0.0f;
        for (int c = lane; c < D; c += 64) a += s_q[h][c] * s_scale[D + c];
        a = wave_sum(a);
        if (lane == 0) s_bias[h] = a;
      }
      __syncthreads();
      // ---- K scores: thread = (token, head half), or (token, channel half) at D = 512 ----
      if constexpr (KP == 2) {
        const int t = tid % kTile;
        const int cp = tid / kTile;
        float sacc[G];
#pragma unroll
        for (int h = 0; h < G; ++h) sacc[h] = 0.0f;
        for (int c = cp * (D / 2); c < (cp + 1) * (D / 2); ++c) {
          float z;
          if constexpr (GEN) {
            const int bit = kb * t;
            const uint8_t* p = s_code + c * 16 * kb + (bit >> 3);
            z = (float)((((uint32_t)p[0] | ((uint32_t)p[1] << 8)) >> (bit & 7)) & kmask);
          } else {
            const uint32_t byte = s_code[c * 64 + (t >> 1)];
            z = (float)((byte >> ((t & 1) * 4)) & 15u);
          }
#pragma unroll
          for (int h = 0; h < G; ++h) sacc[h] += s_qt[c][h] * z;
        }
#pragma unroll
        for (int h = 0; h < G; ++h) s_kp[cp][h][t] = sacc[h];
        if (cp == 0) s_ktok[t] = s_scale[2 * D + t];
      } else {
        const int t = tid % kTile;
        const int hh = tid / kTile;
        if (hh < HH) {
          float sacc[GH];
#pragma unroll
          for (int h = 0; h < GH; ++h) sacc[h] = 0.0f;
          for (int c = 0; c < D; ++c) {
            float z;
            if constexpr (GEN) {   // token t of channel c's stream: bits [kb t, kb t + kb)
              const int bit = kb * t;
              const uint8_t* p = s_code + c * 16 * kb + (bit >> 3);
              z = (float)((((uint32_t)p[0] | ((uint32_t)p[1] << 8)) >> (bit & 7)) & kmask);
            } else {
              const uint32_t byte = s_code[c * 64 + (t >> 1)];
              z = (float)((byte >> ((t & 1) * 4)) & 15u);
            }
#pragma unroll
            for (int h = 0; h < GH; ++h) sacc[h] += s_qt[c][hh * GH + h] * z;
          }
          const float ktok = s_scale[2 * D + t];
#pragma unroll
          for (int h = 0; h < GH; ++h) {
            const int hg = hh * GH + h;
            s_sc[hg][t] = P.scale * ktok * (sacc[h] + s_bias[hg]);
          }
        }
      }
      __syncthreads();
      // ---- stage V codes and value scales (K buffers are free) ----
      {
        const uint4* src = reinterpret_cast<const uint4*>(base + R.vcode);
        uint4* dst = reinterpret_cast<uint4*>(s_code);
        for (int i = tid; i < vb * D; i += kDecThreads) dst[i] = src[i];
        for (int i = tid; i < D; i += kDecThreads) s_scale[i] = sc_ld<H>(base + R.vchan, i);
        for (int i = tid; i < kTile * NG; i += kDecThreads) {
          s_scale[D + i] = sc_ld<H>(base + R.vscale, i);
          s_scale[2 * D + i] = sc_ld<H>(base + R.vmin, i);
        }
      }
      // ---- online softmax over this tile: one wave per head ----
      for (int h = wv; h < G; h += kDecThreads / 64) {
        float s0, s1;
        if constexpr (KP == 2) {
          s0 = P.scale * s_ktok[lane] * ((s_kp[0][h][lane] + s_kp[1][h][lane]) + s_bias[h]);
          s1 = P.scale * s_ktok[lane + 64] * ((s_kp[0][h][lane + 64] + s_kp[1][h][lane + 64]) + s_bias[h]);
        } else {
          s0 = s_sc[h][lane];
          s1 = s_sc[h][lane + 64];
        }
        const float mt = wave_max(fmaxf(s0, s1));
        const float m_old = s_m[h];
        const float m_new = fmaxf(m_old, mt);
        const float p0 = __expf(s0 - m_new), p1 = __expf(s1 - m_new);
        const float psum = wave_sum(p0 + p1);
        s_sc[h][lane] = p0;
        s_sc[h][lane + 64] = p1;
        if (lane == 0) {
          const float alpha = __expf(m_old - m_new);   // 0 on the first tile (m_old = -inf)
          s_alpha[h] = alpha;
          s_l[h] = s_l[h] * alpha + psum;
          s_m[h] = m_new;
        }
      }
      __syncthreads();
      // w = p * vscale, u = sum p * vmin  (value scales are staged now)
      for (int i = tid; i < G * NG * kTile; i += kDecThreads) {
        const int g = i / (kTile * G), r = i % (kTile * G), t = r / G, h = r % G;
        s_w[g][t][h] = s_sc[h][t] * s_scale[D + t * NG + g];
      }
      for (int i = wv; i < G * NG; i += kDecThreads / 64) {
        const int h = i / NG, g = i % NG;
        float a = s_sc[h][lane] * s_scale[2 * D + lane * NG + g] +
                  s_sc[h][lane + 64] * s_scale[2 * D + (lane + 64) * NG + g];
        a = wave_sum(a);
        if (lane == 0) s_u[h][g] = a;
      }
      __syncthreads();
      // ---- V aggregate: thread = (channels, head part) ----
#pragma unroll
      for (int k = 0; k < VC; ++k) {
        const int c = vc0 + k * VSTRIDE;
        if (c < D) {
          const int g = c / 128;
          const int sh = 2 * (c & 3);
          float pacc[GV];
#pragma unroll
          for (int h = 0; h < GV; ++h) pacc[h] = 0.0f;
          for (int t = 0; t < kTile; ++t) {
            float z;
            if constexpr (GEN) {   // channel c of token t's stream: bits [vb c, vb c + vb)
              const int bit = vb * c;
              const uint8_t* p = s_code + t * (D * vb / 8) + (bit >> 3);
              z = (float)((((uint32_t)p[0] | ((uint32_t)p[1] << 8)) >> (bit & 7)) & vmask);
            } else {
              z = (float)((s_code[t * (D / 4) + (c >> 2)] >> sh) & 3u);
            }
#pragma unroll
            for (int h = 0; h < GV; ++h) pacc[h] += s_w[g][t][hv * GV + h] * z;
          }
          const float vch = s_scale[c];
#pragma unroll
          for (int h = 0; h < GV; ++h) {
            const int hg = hv * GV + h;
            acc[h][k] = acc[h][k] * s_alpha[hg] + vch * (pacc[h] + s_u[hg][g]);
          }
        }
      }
      __syncthreads();
    }
  } else {
    // ---- raw window chunk [w_begin, w_end) ----
    const float* kb = P.k_win + sv.win_off + (int64_t)kvh * P.win_head_stride;
    const float* vb = P.v_win + sv.win_off + (int64_t)kvh * P.win_head_stride;
    const int n = w_end - w_begin;
    // scores: each wave takes four tokens per step, 16 lanes per token; a lane
    // reads 16-byte pieces 64 channels apart of its token's key row (the 16
    // lanes of a token read whole 256-byte runs) and the 16 partial dot
    // products are summed across the lanes' DPP row
    {
      const int piece = lane & 15;
      for (int tb = 4 * wv; tb < kWinChunk; tb += 16) {   // wave-uniform
        // the query pieces are read from LDS in every step, not held in registers
        asm volatile("" ::: "memory");
        const int t = tb + (lane >> 4);
        const bool ok = t < n;
        const float* krow = kb + (int64_t)(w_begin + (ok ? t : 0)) * P.win_tok_stride + 4 * piece;
        float4 kk[D / 64];
#pragma unroll
        for (int i = 0; i < D / 64; ++i) kk[i] = *reinterpret_cast<const float4*>(krow + 64 * i);
#pragma unroll
        for (int h = 0; h < G; ++h) {
          float a = 0.0f;
#pragma unroll
          for (int i = 0; i < D / 64; ++i) {
            const float4 qq = *reinterpret_cast<const float4*>(&s_q[h][4 * piece + 64 * i]);
            a += qq.x * kk[i].x + qq.y * kk[i].y + qq.z * kk[i].z + qq.w * kk[i].w;
          }
          a = mfma::row_sum16(a);
          if (piece == 0) s_sc[h][t] = ok ? P.scale * a : -INFINITY;
        }
      }
    }
    __syncthreads();
    for (int h = wv; h < G; h += kDecThreads / 64) {
      const float s0 = s_sc[h][lane];
      const float m = wave_max(s0);
      const float p = (lane < n) ? __expf(s0 - m) : 0.0f;
      const float l = wave_sum(p);
      s_sc[h][lane] = p;
      if (lane == 0) { s_m[h] = m; s_l[h] = l; s_alpha[h] = 0.0f; }
    }
    __syncthreads();
    // all of the thread's channels at once, tokens eight at a time, so the
    // value loads are in flight together rather than one per token
    if (vc0 < D) {
      const float* vcol = vb + (int64_t)w_begin * P.win_tok_stride + vc0;
      int t = 0;
      for (; t + 8 <= n; t += 8) {
        float v[8][VC];
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int k = 0; k < VC; ++k) v[u][k] = vcol[(int64_t)(t + u) * P.win_tok_stride + k * VSTRIDE];
#pragma unroll
        for (int u = 0; u < 8; ++u)
#pragma unroll
          for (int h = 0; h < GV; ++h) {
            const float p = s_sc[hv * GV + h][t + u];
#pragma unroll
            for (int k = 0; k < VC; ++k) acc[h][k] += p * v[u][k];
          }
      }
      for (; t < n; ++t) {
#pragma unroll
        for (int h = 0; h < GV; ++h) {
          const float p = s_sc[hv * GV + h][t];
#pragma unroll
          for (int k = 0; k < VC; ++k) acc[h][k] += p * vcol[(int64_t)t * P.win_tok_stride + k * VSTRIDE];
        }
      }
    }
  }

  // ---- write the partial (m, l, o) per query head ----
#pragma unroll
  for (int k = 0; k < VC; ++k) {
    const int c = vc0 + k * VSTRIDE;
    if (c < D) {
#pragma unroll
      for (int h = 0; h < GV; ++h) {
        const int hg = hv * GV + h;
        part[(int64_t)hg * n_split * (D + 4) + c] = acc[h][k];
      }
    }
  }
  if (tid < G) {
    part[(int64_t)tid * n_split * (D + 4) + D] = s_m[tid];
    part[(int64_t)tid * n_split * (D + 4) + D + 1] = s_l[tid];
  }
}

// ---------------------------------------------------------------------------
// combine kernel: one workgroup of NWV waves per (query head, sequence); lane
// l owns channels l + 64 k.  Only the splits that hold tiles or window tokens
// of the row are read (the split kernels write nothing for the others):
// virtual split v < nvt is tile split v, the rest window split v - nvt.
// Every wave first takes the largest running max M and the weighted sum L
// over all of them; wave w then folds the splits v = w, w + NWV, ... with
// weights exp(m_v - M), U splits at a time with all their loads in flight,
// the tile partials (rotated domain) and the window partials (raw domain)
// apart.  The wave sums add up in LDS (one thread per channel and part);
// wave 0 applies the inverse WHT to the tile sum, adds the window sum and
// divides by L.
// ---------------------------------------------------------------------------
template <int D, int NWV>
__global__ void __launch_bounds__(64 * NWV) decode_combine_kernel(DecodeParams P) {
  constexpr int K = D / 64;
  constexpr int U = 4;
  const int hq = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int nts = P.n_tsplit;
  const int n_split = P.n_tsplit + P.n_wsplit;
  const float* part = P.part + ((int64_t)b * P.n_q + hq) * n_split * (D + 4);
  __shared__ float s_o[NWV][2 * D];
  const SeqView sv = seq_view(P, b);
  const int nvt = min(nts, (sv.nt + P.tps - 1) / P.tps);
  const int nvw = P.wparts ? P.wparts : min(P.n_wsplit, (sv.nw + P.wchunk - 1) / P.wchunk);
  const int nv = nvt + nvw;   // >= 1: every row sees a tile or a token
  auto split_of = [&](int v) { return v < nvt ? v : nts + (v - nvt); };

  // M, then L, over every split (the same in every wave)
  float M = -INFINITY;
  for (int j = lane; j < nv; j += 64) M = fmaxf(M, part[(int64_t)split_of(j) * (D + 4) + D]);
  M = wave_max(M);
  float L = 0.0f;
  for (int j = lane; j < nv; j += 64) {
    const float* ps = part + (int64_t)split_of(j) * (D + 4);
    L += __expf(ps[D] - M) * ps[D + 1];
  }
  const float Lall = wave_sum(L);

  float orot[K], oraw[K];
#pragma unroll
  for (int k = 0; k < K; ++k) { orot[k] = 0.0f; oraw[k] = 0.0f; }
  for (int v0 = w; v0 < nv; v0 += U * NWV) {   // wave-uniform
    float o[U][K], wt[U], wr[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int v = v0 + u * NWV;
      const bool ok = v < nv;   // past the end: split v0 again, weight 0
      const float* ps = part + (int64_t)split_of(ok ? v : v0) * (D + 4);
#pragma unroll
      for (int k = 0; k < K; ++k) o[u][k] = ps[lane + 64 * k];
      const float wgt = ok ? __expf(ps[D] - M) : 0.0f;
      wt[u] = v < nvt ? wgt : 0.0f;
      wr[u] = v < nvt ? 0.0f : wgt;
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int k = 0; k < K; ++k) {
        orot[k] = fmaf(wt[u], o[u][k], orot[k]);
        oraw[k] = fmaf(wr[u], o[u][k], oraw[k]);
      }
  }
  if constexpr (NWV > 1) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      s_o[w][lane + 64 * k] = orot[k];
      s_o[w][D + lane + 64 * k] = oraw[k];
    }
    __syncthreads();
    for (int i = tid; i < 2 * D; i += 64 * NWV) {   // each element read and written by one thread
      float a = 0.0f;
#pragma unroll
      for (int x = 0; x < NWV; ++x) a += s_o[x][i];
      s_o[0][i] = a;
    }
    __syncthreads();
    if (w != 0) return;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      orot[k] = s_o[0][lane + 64 * k];
      oraw[k] = s_o[0][D + lane + 64 * k];
    }
  }
  // inverse WHT (the WHT itself) of the merged rotated-domain part
#pragma unroll
  for (int h = 1; h < 64; h <<= 1) {
    const bool up = (lane & h) != 0;
#pragma unroll
    for (int k = 0; k < K; ++k) {
      float p = shfl_xor(orot[k], h);
      orot[k] = up ? (p - orot[k]) : (orot[k] + p);
    }
  }
#pragma unroll
  for (int hk = 1; hk < K; hk <<= 1) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
      if ((k & hk) == 0) {
        float a = orot[k], c = orot[k + hk];
        orot[k] = a + c;
        orot[k + hk] = a - c;
      }
    }
  }
  const float c = wht_scale<D>();
  const float invL = 1.0f / Lall;
  float* o = P.out + ((int64_t)b * P.n_q + hq) * D;
#pragma unroll
  for (int k = 0; k < K; ++k) o[lane + 64 * k] = (orot[k] * c + oraw[k]) * invL;
}

template <int D, int G>
hipError_t launch_decode_dg(const DecodeParams& P, int batch, hipStream_t stream) {
  const bool gen = !(P.kb == 4 && P.vb == 2);
  if (D >= 256 && !gen) {
    // K4V2 at head_dim 256 / 512: tile splits on the matrix cores; in decode
    // the window splits run in the same grid, in prefill the raw windows of
    // 16 consecutive rows at a time on the matrix cores (one partial per row)
    hipError_t e = hipSuccess;
    if (P.mode == 0) {
      if (P.n_tsplit + P.n_wsplit > 0) e = launch_decode_wide(D, P, batch, stream);
      if (e != hipSuccess) return e;
    } else {
      if (P.n_tsplit > 0)
        e = D == 256 ? launch_prefill_tiles256(P, batch, stream) : launch_decode_wide(D, P, batch, stream);
      if (e != hipSuccess) return e;
      if (P.n_wsplit > 0) e = launch_window_mfma(D, P, batch, stream);
      if (e != hipSuccess) return e;
    }
  } else {
  dim3 grid(P.n_tsplit + P.n_wsplit, P.n_kv, batch);
  if (P.h16) {
    if (gen)
      hipLaunchKernelGGL((decode_partial_kernel<D, G, true, true>), grid, dim3(kDecThreads), 0, stream, P);
    else
      hipLaunchKernelGGL((decode_partial_kernel<D, G, true, false>), grid, dim3(kDecThreads), 0, stream, P);
  } else {
    if (gen)
      hipLaunchKernelGGL((decode_partial_kernel<D, G, false, true>), grid, dim3(kDecThreads), 0, stream, P);
    else
      hipLaunchKernelGGL((decode_partial_kernel<D, G, false, false>), grid, dim3(kDecThreads), 0, stream, P);
  }
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // sixteen waves past 16 splits, four past 4, else one; in prefill (one
  // workgroup per chunk row and head) one wave up to 16 splits
  if (P.n_tsplit + P.n_wsplit > 16)
    hipLaunchKernelGGL((decode_combine_kernel<D, 16>), dim3(P.n_q, batch), dim3(1024), 0, stream, P);
  else if (P.n_tsplit + P.n_wsplit > 4 && P.mode == 0)
    hipLaunchKernelGGL((decode_combine_kernel<D, 4>), dim3(P.n_q, batch), dim3(256), 0, stream, P);
  else
    hipLaunchKernelGGL((decode_combine_kernel<D, 1>), dim3(P.n_q, batch), dim3(64), 0, stream, P);
  return hipGetLastError();
}

template <int D>
hipError_t launch_decode_d(const DecodeParams& P, int batch, hipStream_t stream) {
  switch (P.G) {
    case 1: return launch_decode_dg<D, 1>(P, batch, stream);
    case 2: return launch_decode_dg<D, 2>(P, batch, stream);
    case 4: return launch_decode_dg<D, 4>(P, batch, stream);
    case 8: return launch_decode_dg<D, 8>(P, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

// Sequence b (blockIdx.x), KV head h (blockIdx.y): the newest token's key and
// value rows to window token n_win[b] - 1.
__global__ void __launch_bounds__(128) append_window_kernel(DecodeParams P, float* k_win, float* v_win, int d) {
  const int b = blockIdx.x, h = blockIdx.y;
  const int64_t dst = (int64_t)b * P.win_seq_stride + (P.win_start[b] + P.n_win[b] - 1) * P.win_tok_stride +
                      (int64_t)h * P.win_head_stride;
  const int64_t src = ((int64_t)b * P.n_kv + h) * d;
  for (int c = 4 * threadIdx.x; c < d; c += 4 * blockDim.x) {
    *reinterpret_cast<float4*>(k_win + dst + c) = *reinterpret_cast<const float4*>(P.k_new + src + c);
    *reinterpret_cast<float4*>(v_win + dst + c) = *reinterpret_cast<const float4*>(P.v_new + src + c);
  }
}

hipError_t launch_append_window(int d, const DecodeParams& P, float* k_win, float* v_win, int batch,
                                hipStream_t stream) {
  hipLaunchKernelGGL(append_window_kernel, dim3(batch, P.n_kv), dim3(128), 0, stream, P, k_win, v_win, d);
  return hipGetLastError();
}

hipError_t launch_decode(int d, const DecodeParams& P, int batch, hipStream_t stream) {
  switch (d) {
    case 128: return launch_decode_d<128>(P, batch, stream);
    case 256: return launch_decode_d<256>(P, batch, stream);
    case 512: return launch_decode_d<512>(P, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvarn
