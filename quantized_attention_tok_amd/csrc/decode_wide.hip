// decode_wide.hip -- matrix-core tile splits of the split-tile decode for
// head_dim 256 and 512 over K4V2 records on gfx950.
//
// The same two contractions as the head_dim-128 decode (SharpInference issue
// #433 item 2: split tiles merged by a log-sum-exp combine; issue #180
// Algorithm step 4: scales folded in at read time, the cache never
// reconstructed):
//   S[(h,part)][t] = sum_c q~[(h,part)][c] zK[t][c]        q~ = q' kscale
//   O[(h,part)][c] = sum_t w_g[(h,part)][t] zV[t][c]       w_g = p vscale_{t,g}
// on v_mfma_f32_16x16x32_f16 with fp32 operands split into fp16 hi/lo rows and
// codes as fp16 subnormals (code in bits 4-7), over D / 32 channel steps for
// the scores and D / 128 value groups of eight 16-channel blocks for the
// aggregate; each value group has its own per-token scale, so its w operand
// rows are written afresh.
//
// Workgroup = (tile split, KV head, sequence), 4 waves.  The split's tiles
// run one after the other; wave w owns the 32-token quarter w of every tile
// and keeps its own online softmax state (running max, sum, rescaled output
// columns) across them, so the waves meet once per tile (the q~ operands of
// the tile, double-buffered) and once at the end, where their states merge
// into one partial per query head.  The partial holds the rotated-domain
// output sum, the running max in natural-log units and the sum of weights,
// as the vector-unit window splits and the combine kernel expect.
//
// Each wave stages its own codes in a private LDS area: the K codes (channel
// row c of 16 bytes at 16 c + 16 (c / 8)), then, once the scores are taken,
// the V codes over them (token row t of D / 4 bytes at (D / 4) t + 32 (t / 8)).
// The padding puts the rows one MFMA operand gathers in distinct banks.
//
// Lanes of one wave hand data to each other through LDS (codes, w rows)
// with no barrier: a wave's LDS accesses complete in program order, but the
// compiler reasons per lane and may keep a value loaded earlier when the lane
// itself stored nothing at that address (it did so for the w rows, which only
// the lanes of present heads write).  lds_sync() marks each hand-off.
#include <float.h>

#include "kvarn_launch.h"
#include "kvarn_mfma.h"

namespace kvarn {
namespace {

using mfma::as_half8;
using mfma::bfly;
using mfma::byte_pair;
using mfma::floatx4;
using mfma::fp16_scale_exp;
using mfma::half8;
using mfma::pow2i;
using mfma::row_max16;
using mfma::row_sum16;
using mfma::split_pair;
using mfma::wmax;
using mfma::wsum;

constexpr float kLog2eW = 1.4426950408889634f;
constexpr float kLn2W = 0.6931471805599453f;
constexpr int kWRowW = 20;   // dwords per w operand row (80 bytes)
constexpr int kRowsW = 16;   // MFMA operand rows; rows that hold no head part stay zero

constexpr int align16w(int x) { return (x + 15) / 16 * 16; }

// compiler memory barrier: LDS loads after it are issued afresh, and no LDS
// access moves across it
__device__ __forceinline__ void lds_sync() { asm volatile("" ::: "memory"); }

// native 16-byte vector (arrays of it stay in registers)
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// G here counts the operand heads of a workgroup: query heads x query rows
template <int D, int G>
struct WideLds {
  // head h's fp16 hi and lo parts sit in operand rows RPH h and RPH h + 1, so
  // lane group g of an MFMA result holds heads HPL g .. HPL g + HPL - 1
  static constexpr int HPL = G > 4 ? 2 : 1;
  static constexpr int RPH = 4 / HPL;
  static constexpr int code_wave = 18 * D;                   // K codes, then V codes
  static constexpr int code = 0;                             // [wave]
  static constexpr int wop = 4 * code_wave;                  // [wave][16 rows][kWRowW] dwords
  static constexpr int wop_wave = kRowsW * kWRowW * 4;
  static constexpr int qt = wop + 4 * wop_wave;              // [2][D/32][16 rows][4] uint4
  static constexpr int qt_tile = (D / 32) * kRowsW * 64;
  static constexpr int us = qt + 2 * qt_tile;                // [2][G] f32: score unscale
  static constexpr int bias = us + 2 * G * 4;                // [2][G] f32: sum_c q'_c kmin_c
  static constexpr int fv = bias + 2 * G * 4;                // [2] int: w fp16 scale exponent
  static constexpr int ml = align16w(fv + 8);                // [G][4] float2: m, l per wave
  static constexpr int bytes = ml + G * 4 * 8;
  static constexpr int mo = 0;                               // merge: [wave][G][D] f32
  static_assert(8 * D + 128 <= code_wave, "a wave's V codes fit its K-code area");
  static_assert(4 * G * D * 4 <= us, "the merge area lies below the per-tile scalars");
  static_assert((wop % 16) == 0 && (qt % 16) == 0, "aligned sections");
};

// Raw-window split ws of sequence b, KV head kvh (decode, launched after the
// tile splits in the same grid): window tokens [64 ws, min(nw, 64 ws + 64)),
// the G query heads' raw rows, one softmax per head over the split's tokens.
// Scores: each wave takes four tokens per step, 16 lanes per token; a lane
// reads 16-byte pieces 64 channels apart of its token's key row (the 16 lanes
// of a token read whole 256-byte runs), takes the query pieces from LDS, and
// the 16 partial products sum over the DPP row.  Values: thread t owns
// channels t + 256 k of every head, eight tokens' rows loaded at a time.
// Writes the raw-domain partial of each head: o, the running max in
// natural-log units and the sum of weights.
template <int D, int G>
__device__ __forceinline__ void wide_window_split(const DecodeParams& P, uint8_t* lds, const SeqView& sv, int b,
                                                  int kvh, int ws, int split, int n_split) {
  constexpr int WC = kWinChunk;
  constexpr int CPT = D / 256;           // value channels per thread
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int w0 = ws * WC;
  const int n = min(WC, sv.nw - w0);     // >= 1: the caller skips empty splits
  float* s_q = reinterpret_cast<float*>(lds);   // [G][D] raw query rows
  float* s_p = s_q + G * D;                     // [G][WC] scores, then weights
  float* s_ml = s_p + G * WC;                   // [G][2] max (natural log), sum
  const float* qsrc = P.q + ((int64_t)b * P.n_q + (int64_t)kvh * G) * D;
  for (int i = tid; i < G * D / 4; i += 256)
    reinterpret_cast<float4*>(s_q)[i] = reinterpret_cast<const float4*>(qsrc)[i];
  const int64_t ts = P.win_tok_stride;
  const float* kb = P.k_win + sv.win_off + (int64_t)kvh * P.win_head_stride + (int64_t)w0 * ts;
  const float* vb = P.v_win + sv.win_off + (int64_t)kvh * P.win_head_stride + (int64_t)w0 * ts;
  __syncthreads();

  const float c_log2 = P.scale * kLog2eW;
  const int piece = lane & 15;
  for (int tb = 4 * wv; tb < n; tb += 16) {   // wave-uniform
    const int t = tb + (lane >> 4);
    const float* krow = kb + (int64_t)(t < n ? t : 0) * ts + 4 * piece;
    float4 kk[D / 64];
#pragma unroll
    for (int i = 0; i < D / 64; ++i) kk[i] = *reinterpret_cast<const float4*>(krow + 64 * i);
#pragma unroll
    for (int h = 0; h < G; ++h) {
      float a = 0.0f;
#pragma unroll
      for (int i = 0; i < D / 64; ++i) {
        const float4 q4 = *reinterpret_cast<const float4*>(s_q + h * D + 4 * piece + 64 * i);
        a += q4.x * kk[i].x + q4.y * kk[i].y + q4.z * kk[i].z + q4.w * kk[i].w;
      }
      a = row_sum16(a);
      if (piece == 0 && t < n) s_p[h * WC + t] = a * c_log2;
    }
  }
  __syncthreads();
  for (int h = wv; h < G; h += 4) {
    const float sc = lane < n ? s_p[h * WC + lane] : -INFINITY;
    const float m = wmax(sc);   // finite: the split holds a token
    const float p = lane < n ? __builtin_amdgcn_exp2f(sc - m) : 0.0f;
    const float l = wsum(p);
    s_p[h * WC + lane] = p;
    if (lane == 0) {
      s_ml[2 * h] = m * kLn2W;
      s_ml[2 * h + 1] = l;
    }
  }
  __syncthreads();

  float acc[G][CPT];
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int k = 0; k < CPT; ++k) acc[h][k] = 0.0f;
  const float* vcol = vb + tid;
  int t = 0;
  for (; t + 8 <= n; t += 8) {
    float v[8][CPT];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int k = 0; k < CPT; ++k) v[u][k] = vcol[(int64_t)(t + u) * ts + 256 * k];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = s_p[h * WC + t + u];
#pragma unroll
        for (int k = 0; k < CPT; ++k) acc[h][k] = fmaf(p, v[u][k], acc[h][k]);
      }
  }
  for (; t < n; ++t) {
    float v[CPT];
#pragma unroll
    for (int k = 0; k < CPT; ++k) v[k] = vcol[(int64_t)t * ts + 256 * k];
#pragma unroll
    for (int h = 0; h < G; ++h) {
      const float p = s_p[h * WC + t];
#pragma unroll
      for (int k = 0; k < CPT; ++k) acc[h][k] = fmaf(p, v[k], acc[h][k]);
    }
  }
#pragma unroll
  for (int h = 0; h < G; ++h) {
    float* o = P.part + (((int64_t)b * P.n_q + (int64_t)kvh * G + h) * n_split + split) * (D + 4);
#pragma unroll
    for (int k = 0; k < CPT; ++k) o[tid + 256 * k] = acc[h][k];
    if (tid == 0) {
      o[D] = s_ml[2 * h];
      o[D + 1] = s_ml[2 * h + 1];
    }
  }
}

// Rotated query rows of the operand heads wv + 4 k that a wave prepares
// (clamped rows are read, never used); with q_rot NULL the wave rotates the
// raw rows itself: the Walsh-Hadamard butterflies on channel bits 0-5 across
// lanes (DPP and permlane swaps), bits 6 and up between a lane's registers
// (channel lane + 64 i), ascending, then the 1/sqrt(D) scale.  Operand head
// v stands for query row b0 + v / G, head kvh G + v % G.
template <int D, int G, int VH, int PPW>
__device__ __forceinline__ void wave_query_rows(const DecodeParams& P, int b0, int kvh, int wv, int lane,
                                                float (&qp)[PPW][D / 64]) {
  constexpr int CPL = D / 64;
  const bool rot = P.q_rot == nullptr;
#pragma unroll
  for (int k = 0; k < PPW; ++k) {
    const int v = wv + 4 * k;
    const int vc = v < VH ? v : 0;
    const float* qsrc = (rot ? P.q : P.q_rot) + ((int64_t)(b0 + vc / G) * P.n_q + (int64_t)kvh * G + vc % G) * D;
#pragma unroll
    for (int i = 0; i < CPL; ++i) qp[k][i] = qsrc[lane + 64 * i];
    if (rot) {   // uniform
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        float x = qp[k][i];
        x = bfly<1>(x, lane);
        x = bfly<2>(x, lane);
        x = bfly<4>(x, lane);
        x = bfly<8>(x, lane);
        x = bfly<16>(x, lane);
        qp[k][i] = bfly<32>(x, lane);
      }
#pragma unroll
      for (int s = 1; s < CPL; s <<= 1) {
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          if ((i & s) == 0) {
            const float a = qp[k][i], c = qp[k][i + s];
            qp[k][i] = a + c;
            qp[k][i + s] = a - c;
          }
        }
      }
#pragma unroll
      for (int i = 0; i < CPL; ++i) qp[k][i] *= wht_scale<D>();
    }
  }
}

// RP query rows per workgroup (2 only in prefill, where neighbouring rows see
// the same tiles and G <= 4 leaves half of the operand rows free): operand
// head v stands for query row r = v / G, head h = v % G.  A row whose visible
// tiles end earlier (a pair on both sides of a tile boundary) has its operand
// heads masked on the tiles it does not see.
template <int D, int G, bool H, int RP>
__global__ void __launch_bounds__(256) decode_wide_kernel(DecodeParams P) {
  constexpr int VH = RP * G;             // operand heads
  using L = WideLds<D, VH>;
  using R = Rec<D, H>;
  constexpr int NB = D / 128;            // value groups
  constexpr int HPL = L::HPL, RPH = L::RPH;
  constexpr int K4 = D / 32;             // channel steps of the score products
  constexpr int CPL = D / 64;            // channels per lane in the query prep / K-code slice
  constexpr int VPL = D / 128;           // 16-byte pieces of the wave's V codes per lane
  constexpr int PPW = (VH + 3) / 4;      // operand heads prepared per wave
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b0 = blockIdx.z * RP;        // first query row (sequence in decode)
  const SeqView sv = seq_view(P, b0);
  int nt_r[RP];
  nt_r[0] = sv.nt;
  if constexpr (RP == 2) nt_r[1] = seq_view(P, b0 + 1).nt;   // same record rows (prefill view)
  const int nt_max = RP == 2 ? max(nt_r[0], nt_r[RP - 1]) : nt_r[0];
  const int n_split = P.n_tsplit + P.n_wsplit;

  __shared__ __attribute__((aligned(16))) uint8_t lds[L::bytes];

  if constexpr (RP == 1) {
    static_assert((G * D + G * kWinChunk + 2 * G) * 4 <= L::bytes, "the window split fits the LDS area");
    if (split >= P.n_tsplit) {   // a raw-window split (decode)
      const int ws = split - P.n_tsplit;
      if (ws * kWinChunk < sv.nw) wide_window_split<D, G>(P, lds, sv, b0, kvh, ws, split, n_split);
      return;
    }
  }

  // partial of operand head v: row b0 + v / G, head kvh G + v % G
  auto part_of = [&](int v) {
    return P.part + (((int64_t)(b0 + v / G) * P.n_q + (int64_t)kvh * G + v % G) * n_split + split) * (D + 4);
  };
  const int t_begin = split * P.tps;
  const int t_end = min(nt_max, t_begin + P.tps);
  if (t_begin >= t_end) return;   // no tiles here: the combine does not read this split

  float qp[PPW][CPL];
  wave_query_rows<D, G, VH, PPW>(P, b0, kvh, wv, lane, qp);
  // operand rows that hold no head part stay zero (both q~ buffers, every w area)
  if constexpr (RPH > 2 || VH < 8) {
    for (int i = tid; i < 2 * K4 * kRowsW * 4; i += 256) {
      const int r = (i >> 2) & (kRowsW - 1);
      if ((r % RPH) >= 2 || r / RPH >= VH) reinterpret_cast<uint4*>(lds + L::qt)[i] = make_uint4(0, 0, 0, 0);
    }
    for (int i = tid; i < 4 * kRowsW * (kWRowW / 4); i += 256) {
      const int r = (i / (kWRowW / 4)) % kRowsW;
      if ((r % RPH) >= 2 || r / RPH >= VH) reinterpret_cast<uint4*>(lds + L::wop)[i] = make_uint4(0, 0, 0, 0);
    }
  }

  float m_w[HPL], l_w[HPL], o_w[HPL][8 * NB];
#pragma unroll
  for (int jj = 0; jj < HPL; ++jj) {
    m_w[jj] = -INFINITY;
    l_w[jj] = 0.0f;
#pragma unroll
    for (int q = 0; q < 8 * NB; ++q) o_w[jj][q] = 0.0f;
  }
  const float c_log2 = P.scale * kLog2eW;
  const int64_t rstride = (int64_t)P.n_kv * R::bytes;
  const uint8_t* rec = P.records + ((sv.rec_row0 + t_begin) * (int64_t)P.n_kv + kvh) * R::bytes;
  uint8_t* cs = lds + L::code + wv * L::code_wave;
  uint32_t* wrow = reinterpret_cast<uint32_t*>(lds + L::wop + wv * L::wop_wave);
  const int tok = 32 * wv + 2 * n;                      // the lane's two tokens of the quarter
  const int vci = 16 * (n & 7) + 8 * (n >> 3);          // its first output channel of a value group

  // The tile's registers.  With PF (head_dim 256 in decode, where the registers allow)
  // each group is loaded for the next tile right after its last use in this
  // one, so the loads of tile j + 1 are in flight while tile j is computed;
  // otherwise every group is loaded at the top of its own tile.
  constexpr bool PF = D == 256 && RP == 1;
  float ks[CPL], km[CPL];
  float4 vmx4[NB / 2];   // wave 0: value scales of tokens 2 lane, 2 lane + 1
  u32x4 kc[CPL], vc[VPL];
  float2 kt;
  float vs[2 * NB], vm[2 * NB];   // token tok + e, group cb at e NB + cb
  float vch[NB][8];               // channel scales of the lane's output channels
  auto ld_kscale = [&](const uint8_t* r) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      ks[i] = sc_ld<H>(r + R::kscale, lane + 64 * i);
      km[i] = sc_ld<H>(r + R::kmin, lane + 64 * i);
    }
  };
  auto ld_vmax = [&](const uint8_t* r) {
    if (wv == 0) {
#pragma unroll
      for (int i = 0; i < NB / 2; ++i) vmx4[i] = sc_ld4<H>(r + R::vscale, 2 * NB * lane + 4 * i);
    }
  };
  auto ld_kcode = [&](const uint8_t* r) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) kc[i] = *reinterpret_cast<const u32x4*>(r + (lane + 64 * i) * 64 + 16 * wv);
  };
  auto ld_ktok = [&](const uint8_t* r) { kt = sc_ld2<H>(r + R::ktok, tok); };
  auto ld_vcode = [&](const uint8_t* r) {
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      vc[i] = *reinterpret_cast<const u32x4*>(r + R::vcode + 8 * D * wv + 16 * (lane + 64 * i));
  };
  auto ld_vscale = [&](const uint8_t* r) {
#pragma unroll
    for (int i = 0; i < NB / 2; ++i) {
      const float4 x = sc_ld4<H>(r + R::vscale, tok * NB + 4 * i);
      const float4 y = sc_ld4<H>(r + R::vmin, tok * NB + 4 * i);
      vs[4 * i] = x.x; vs[4 * i + 1] = x.y; vs[4 * i + 2] = x.z; vs[4 * i + 3] = x.w;
      vm[4 * i] = y.x; vm[4 * i + 1] = y.y; vm[4 * i + 2] = y.z; vm[4 * i + 3] = y.w;
    }
    if constexpr (PF) {   // otherwise read per value group in the aggregate
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
        const float4 va = sc_ld4<H>(r + R::vchan, 128 * cb + vci);
        const float4 vb = sc_ld4<H>(r + R::vchan, 128 * cb + vci + 4);
        vch[cb][0] = va.x; vch[cb][1] = va.y; vch[cb][2] = va.z; vch[cb][3] = va.w;
        vch[cb][4] = vb.x; vch[cb][5] = vb.y; vch[cb][6] = vb.z; vch[cb][7] = vb.w;
      }
    }
  };
  auto ld_all = [&](const uint8_t* r) {
    ld_kscale(r); ld_vmax(r); ld_kcode(r); ld_vcode(r); ld_ktok(r); ld_vscale(r);
  };
  if constexpr (PF) ld_all(rec);

  for (int j = t_begin; j < t_end; ++j, rec += rstride) {
    const int buf = (j - t_begin) & 1;
    const uint8_t* nrec = j + 1 < t_end ? rec + rstride : rec;   // the last tile reloads itself
    if constexpr (!PF) ld_all(rec);

    // ---- prep: q~ hi/lo operand rows, score unscale, bias, w scale ----
#pragma unroll
    for (int k = 0; k < PPW; ++k) {
      const int h = wv + 4 * k;   // operand head
      if (h < VH) {   // wave-uniform
        float y[CPL];
        float am = 0.0f, bs = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          y[i] = qp[k][i] * ks[i];
          am = fmaxf(am, fabsf(y[i]));
          bs = fmaf(qp[k][i], km[i], bs);
        }
        const float amax = wmax(am);
        const float bias = wsum(bs);
        const int fe = fp16_scale_exp(amax);   // amax 2^fe in [2^13, 2^14)
        const float f = pow2i(fe - 4);
        // channel c -> uint4 [k4 = c / 32][row][(c / 8) % 4], half c % 8; channel
        // lane + 64 i has k4 = 2 i + lane / 32
        uint16_t* qt = reinterpret_cast<uint16_t*>(lds + L::qt + buf * L::qt_tile);
        const int i0 = (((lane >> 5) * kRowsW + RPH * h) * 4 + ((lane >> 3) & 3)) * 8 + (lane & 7);
#pragma unroll
        for (int i = 0; i < CPL; i += 2) {
          uint32_t hi, lo;
          split_pair(y[i] * f, y[i + 1] * f, hi, lo);
          const int ia = i0 + i * 2 * kRowsW * 32;
          const int ib = ia + 2 * kRowsW * 32;
          qt[ia] = (uint16_t)(hi & 0xFFFFu);
          qt[ia + 32] = (uint16_t)(lo & 0xFFFFu);   // row RPH h + 1
          qt[ib] = (uint16_t)(hi >> 16);
          qt[ib + 32] = (uint16_t)(lo >> 16);
        }
        if (lane == 0) {
          reinterpret_cast<float*>(lds + L::us)[buf * VH + h] = pow2i(24 - fe);
          reinterpret_cast<float*>(lds + L::bias)[buf * VH + h] = bias;
        }
      }
    }
    if constexpr (PF) ld_kscale(nrec);
    if (wv == 0) {
      float vmx = 0.0f;   // the tile's largest value scale
#pragma unroll
      for (int i = 0; i < NB / 2; ++i)
        vmx = fmaxf(vmx, fmaxf(fmaxf(vmx4[i].x, vmx4[i].y), fmaxf(vmx4[i].z, vmx4[i].w)));
      const float vmax = wmax(vmx);   // p <= 1, so w <= the largest value scale
      if (lane == 0) reinterpret_cast<int*>(lds + L::fv)[buf] = fp16_scale_exp(vmax);
    }
    if constexpr (PF) ld_vmax(nrec);
    // ---- the wave's K codes into its own area ----
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = lane + 64 * i;
      *reinterpret_cast<u32x4*>(cs + 16 * c + 16 * (c >> 3)) = kc[i];
    }
    if constexpr (PF) ld_kcode(nrec);
    __syncthreads();   // q~ operands and the tile's scalars are ready

    // ---- scores: A = q~ rows, B = code nibbles of tokens 2 n, 2 n + 1 of the quarter ----
    const uint4* qtu = reinterpret_cast<const uint4*>(lds + L::qt + buf * L::qt_tile);
    floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    const uint8_t* kg = cs + 144 * g + n;   // channel 32 k4 + 8 g + j at kg[576 k4 + 16 j]
#pragma unroll
    for (int k4 = 0; k4 < K4; ++k4) {
      const uint4 a = qtu[(k4 * kRowsW + n) * 4 + g];
      const half8 A = as_half8(a.x, a.y, a.z, a.w);
      uint32_t e[4], o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t x = byte_pair(kg + 576 * k4 + 32 * i, 16);
        e[i] = (x << 4) & 0x00F000F0u;   // token 2 n
        o[i] = x & 0x00F000F0u;          // token 2 n + 1
      }
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, as_half8(e[0], e[1], e[2], e[3]), acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, as_half8(o[0], o[1], o[2], o[3]), acc1, 0, 0, 0);
    }

    // ---- online softmax of the quarter (lane (g, n): rows 4 g + i = head HPL g + i / RPH, part i % RPH) ----
    const int vexp = reinterpret_cast<const int*>(lds + L::fv)[buf];
    const float fv = pow2i(vexp);
    const float k0 = kt.x * c_log2, k1 = kt.y * c_log2;
    if constexpr (PF) ld_ktok(nrec);
    float p0[HPL], p1[HPL];
#pragma unroll
    for (int jj = 0; jj < HPL; ++jj) {
      const int h = HPL * g + jj;   // operand head
      const int hc = h < VH ? h : VH - 1;
      const float us = reinterpret_cast<const float*>(lds + L::us)[buf * VH + hc];
      const float bi = reinterpret_cast<const float*>(lds + L::bias)[buf * VH + hc];
      // a row that does not see tile j (its visible tiles end earlier) is masked
      const bool seen = RP == 1 || j < nt_r[(hc / G) & (RP - 1)];
      const float s0 = seen ? k0 * fmaf(acc0[RPH * jj] + acc0[RPH * jj + 1], us, bi) : -INFINITY;
      const float s1 = seen ? k1 * fmaf(acc1[RPH * jj] + acc1[RPH * jj + 1], us, bi) : -INFINITY;
      const float m_new = fmaxf(m_w[jj], row_max16(fmaxf(s0, s1)));
      const bool none = m_new == -INFINITY;   // masked, and no earlier tile: state stays empty
      const float alpha = none ? 1.0f : __builtin_amdgcn_exp2f(m_w[jj] - m_new);   // 0 on the first tile
      p0[jj] = none ? 0.0f : __builtin_amdgcn_exp2f(s0 - m_new);
      p1[jj] = none ? 0.0f : __builtin_amdgcn_exp2f(s1 - m_new);
      m_w[jj] = m_new;
      l_w[jj] = fmaf(l_w[jj], alpha, p0[jj] + p1[jj]);   // summed over the row in the merge
#pragma unroll
      for (int q = 0; q < 8 * NB; ++q) o_w[jj][q] *= alpha;
    }

    // ---- the wave's V codes over its K codes ----
    lds_sync();
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const int off = 16 * (lane + 64 * i);
      const int t = off / (D / 4);
      *reinterpret_cast<u32x4*>(cs + (D / 4) * t + 32 * (t >> 3) + off % (D / 4)) = vc[i];
    }
    if constexpr (PF) ld_vcode(nrec);
    lds_sync();

    // ---- value aggregate per group: A = w rows, B = crumbs of tokens 8 g + j,
    //      channels 128 cb + 16 (n % 8) + 8 (n / 8) + qb ----
    const float un_lo = pow2i(24 - vexp - 4), un_hi = pow2i(24 - vexp - 6);
    const uint8_t* vg = cs + 8 * (D / 4) * g + 32 * g + 4 * (n & 7) + 2 * (n >> 3);
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      lds_sync();   // the previous group's w rows are read before they are overwritten
      float u[HPL];
#pragma unroll
      for (int jj = 0; jj < HPL; ++jj) {
        const int h = HPL * g + jj;
        uint32_t hi, lo;
        split_pair(p0[jj] * (vs[cb] * fv), p1[jj] * (vs[NB + cb] * fv), hi, lo);
        if (h < VH) {
          wrow[(RPH * h) * kWRowW + n] = hi;
          wrow[(RPH * h + 1) * kWRowW + n] = lo;
        }
        u[jj] = row_sum16(p0[jj] * vm[cb] + p1[jj] * vm[NB + cb]);   // sum_t p vmin over the quarter
      }
      lds_sync();   // every lane's w rows of this group are read afresh
      const uint4 wa = *reinterpret_cast<const uint4*>(wrow + n * kWRowW + 4 * g);
      const half8 A = as_half8(wa.x, wa.y, wa.z, wa.w);
      uint32_t x[2][4];
#pragma unroll
      for (int pq = 0; pq < 4; ++pq) {
#pragma unroll
        for (int e = 0; e < 2; ++e) x[e][pq] = byte_pair(vg + 32 * cb + (D / 2) * pq + e, D / 4);
      }
      float vcg[8];
      if constexpr (PF) {
#pragma unroll
        for (int qb = 0; qb < 8; ++qb) vcg[qb] = vch[cb][qb];
      } else {
        const float4 vca = sc_ld4<H>(rec + R::vchan, 128 * cb + vci);
        const float4 vcb = sc_ld4<H>(rec + R::vchan, 128 * cb + vci + 4);
        vcg[0] = vca.x; vcg[1] = vca.y; vcg[2] = vca.z; vcg[3] = vca.w;
        vcg[4] = vcb.x; vcg[5] = vcb.y; vcg[6] = vcb.z; vcg[7] = vcb.w;
      }
#pragma unroll
      for (int qb = 0; qb < 8; ++qb) {
        const int e = qb >> 2, cr = qb & 3;
        const uint32_t mask = (cr & 1) ? 0x00C000C0u : 0x00300030u;
        uint32_t bv[4];
#pragma unroll
        for (int pq = 0; pq < 4; ++pq) bv[pq] = ((cr < 2) ? (x[e][pq] << 4) : x[e][pq]) & mask;
        const floatx4 z = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, as_half8(bv[0], bv[1], bv[2], bv[3]),
                                                               (floatx4){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        const float un = (cr & 1) ? un_hi : un_lo;
#pragma unroll
        for (int jj = 0; jj < HPL; ++jj)
          o_w[jj][8 * cb + qb] = fmaf(vcg[qb], fmaf(z[RPH * jj] + z[RPH * jj + 1], un, u[jj]), o_w[jj][8 * cb + qb]);
      }
    }
    if constexpr (PF) ld_vscale(nrec);
  }

  // ---- merge the four wave states into one partial per query head ----
  __syncthreads();   // every wave is done with the areas the merge overwrites
  float* s_mo = reinterpret_cast<float*>(lds + L::mo);
  float2* s_ml = reinterpret_cast<float2*>(lds + L::ml);
#pragma unroll
  for (int jj = 0; jj < HPL; ++jj) {
    const int h = HPL * g + jj;   // operand head
    const float lsum = row_sum16(l_w[jj]);
    if (h < VH) {
#pragma unroll
      for (int cb = 0; cb < NB; ++cb) {
#pragma unroll
        for (int qb = 0; qb < 8; ++qb) s_mo[(wv * VH + h) * D + 128 * cb + vci + qb] = o_w[jj][8 * cb + qb];
      }
      if (n == 0) s_ml[h * 4 + wv] = make_float2(m_w[jj], lsum);
    }
  }
  __syncthreads();
  for (int i = tid; i < VH * D; i += 256) {
    const int h = i / D, c = i % D;   // operand head, channel
    float M = s_ml[h * 4].x;
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, s_ml[h * 4 + w].x);
    float o = 0.0f, l = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float2 ml = s_ml[h * 4 + w];
      const float sc = ml.x == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ml.x - M);   // also when M = -inf
      o = fmaf(sc, s_mo[(w * VH + h) * D + c], o);
      l = fmaf(sc, ml.y, l);
    }
    float* part = part_of(h);
    part[c] = o;
    if (c == 0) {
      part[D] = M * kLn2W;   // natural-log units, as the combine expects (-inf: empty)
      part[D + 1] = l;
    }
  }
}

// Head_dim 512, one query row per workgroup (decode, and prefill rows that
// are not paired): the same contractions with the value
// aggregate split by channels.  Wave w scores the 32-token quarter w of every
// tile (as decode_wide_kernel) but aggregates value group w (channels
// 128 w .. 128 w + 127) over all 128 tokens, so a lane keeps 16 output sums
// instead of 64.  The waves share one running max per head (the largest of
// the four quarter maxima, through LDS); each wave writes the w rows and the
// sums of p vmin of its quarter for all four value groups, and reads those of
// its own group from every quarter.  Three barriers per tile: q~ operands
// ready, quarter maxima ready, w rows ready.  The registers this frees hold
// the next tile's K codes, in flight while the current tile is computed.
// Loads go through a buffer resource of the tile's record (one address
// register per group of loads).  Output: one partial per query head, each
// wave writing its group's channels (no merge).
template <int G, bool H>
__global__ void __launch_bounds__(256) decode_wide_cs_kernel(DecodeParams P) {
  constexpr int D = 512;
  constexpr int VH = G;
  using R = Rec<D, H>;
  constexpr int NB = 4;                  // value groups, one per wave
  constexpr int HPL = G > 4 ? 2 : 1;
  constexpr int RPH = 4 / HPL;
  constexpr int K4 = D / 32;
  constexpr int CPL = D / 64;
  constexpr int PPW = (VH + 3) / 4;
  // LDS: per-wave code areas (K codes of the quarter: channel row c of 16
  // bytes at 16 c + 16 (c / 8); then the group's V codes: token row t of 32
  // bytes at 32 t + 32 (t / 8)), q~ operands, w rows [group][quarter], and the
  // per-tile scalars
  constexpr int code_wave = 18 * D;
  constexpr int o_qt = 4 * code_wave;                   // [D/32][16 rows][4] uint4
  constexpr int o_w = o_qt + K4 * kRowsW * 64;          // [group][quarter][16 rows][kWRowW] dwords
  constexpr int w_blk = kRowsW * kWRowW * 4;
  constexpr int o_qmax = o_w + NB * 4 * w_blk;          // [quarter][VH] f32
  constexpr int o_u = o_qmax + 4 * VH * 4;              // [group][quarter][VH] f32
  constexpr int o_us = o_u + NB * 4 * VH * 4;           // [VH] f32: score unscale
  constexpr int o_bias = o_us + VH * 4;                 // [VH] f32
  constexpr int o_l = o_bias + VH * 4;                  // [quarter][VH] f32: sums at the end
  constexpr int o_fv = o_l + 4 * VH * 4;                // int: w fp16 scale exponent
  constexpr int lds_bytes = o_fv + 16;
  static_assert(32 * 128 + 32 * 16 <= code_wave, "a wave's V codes fit its K-code area");
  static_assert((G * D + G * kWinChunk + 2 * G) * 4 <= lds_bytes, "the window split fits the LDS area");
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const SeqView sv = seq_view(P, b);   // decode: sequence b; prefill: chunk row b
  const int n_split = P.n_tsplit + P.n_wsplit;

  __shared__ __attribute__((aligned(16))) uint8_t lds[lds_bytes];

  if (split >= P.n_tsplit) {   // a raw-window split (decode; a prefill grid holds tile splits alone)
    const int ws = split - P.n_tsplit;
    if (ws * kWinChunk < sv.nw) wide_window_split<D, G>(P, lds, sv, b, kvh, ws, split, n_split);
    return;
  }
  const int t_begin = split * P.tps;
  const int t_end = min(sv.nt, t_begin + P.tps);
  if (t_begin >= t_end) return;   // no tiles here: the combine does not read this split

  float qp[PPW][CPL];
  wave_query_rows<D, G, VH, PPW>(P, b, kvh, wv, lane, qp);
  // operand rows that hold no head part stay zero (q~ and every w block)
  if constexpr (RPH > 2 || VH < 8) {
    for (int i = tid; i < K4 * kRowsW * 4; i += 256) {
      const int r = (i >> 2) & (kRowsW - 1);
      if ((r % RPH) >= 2 || r / RPH >= VH) reinterpret_cast<uint4*>(lds + o_qt)[i] = make_uint4(0, 0, 0, 0);
    }
    for (int i = tid; i < NB * 4 * kRowsW * (kWRowW / 4); i += 256) {
      const int r = (i / (kWRowW / 4)) % kRowsW;
      if ((r % RPH) >= 2 || r / RPH >= VH) reinterpret_cast<uint4*>(lds + o_w)[i] = make_uint4(0, 0, 0, 0);
    }
  }

  float m_run[HPL], l_q[HPL], o_c[HPL][8];
#pragma unroll
  for (int jj = 0; jj < HPL; ++jj) {
    m_run[jj] = -INFINITY;
    l_q[jj] = 0.0f;
#pragma unroll
    for (int q = 0; q < 8; ++q) o_c[jj][q] = 0.0f;
  }
  const float c_log2 = P.scale * kLog2eW;
  const int64_t rstride = (int64_t)P.n_kv * R::bytes;
  const uint8_t* rec = P.records + ((sv.rec_row0 + t_begin) * (int64_t)P.n_kv + kvh) * R::bytes;
  uint8_t* cs = lds + wv * code_wave;
  float* s_qmax = reinterpret_cast<float*>(lds + o_qmax);
  float* s_u = reinterpret_cast<float*>(lds + o_u);
  const int tok = 32 * wv + 2 * n;                      // the lane's two tokens of the quarter
  const int vci = 16 * (n & 7) + 8 * (n >> 3);          // its first output channel of the group

  // the tile's registers: the K codes (the largest group) are loaded for
  // tile j + 1 right after tile j's are stored, so they are in flight while
  // tile j is computed; the other groups are loaded at the top of their tile
  float ks[CPL], km[CPL];
  float4 vmx4[NB / 2];   // wave 0: value scales of tokens 2 lane, 2 lane + 1
  u32x4b kc[CPL], vc[4];
  float2 kt;
  float vs[2 * NB], vm[2 * NB];   // token tok + e, group cb at e NB + cb
  float vch[8];                   // channel scales of the lane's output channels 128 wv + vci + qb
  // loads through a buffer resource of the tile's record: one address
  // register per group of loads
  auto ld_kscale = [&](brsrc r) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      ks[i] = sc_bl<H>(r, R::kscale, lane, 64 * i);
      km[i] = sc_bl<H>(r, R::kmin, lane, 64 * i);
    }
  };
  auto ld_vmax = [&](brsrc r) {
    if (wv == 0) {
#pragma unroll
      for (int i = 0; i < NB / 2; ++i) vmx4[i] = sc_bl4<H>(r, R::vscale, 2 * NB * lane, 4 * i);
    }
  };
  auto ld_kcode = [&](brsrc r) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) kc[i] = code_bl(r, lane * 64 + 16 * wv, i * 64 * 64);
  };
  auto ld_ktok = [&](brsrc r) { kt = sc_bl2<H>(r, R::ktok, tok, 0); };
  // group wv's 32 bytes of every token row: piece e = lane + 64 i is token e / 2, half e % 2
  auto ld_vcode = [&](brsrc r) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      vc[i] = code_bl(r, (lane >> 1) * (D / 4) + 32 * wv + 16 * (lane & 1), R::vcode + 32 * i * (D / 4));
  };
  auto ld_vscale = [&](brsrc r) {
#pragma unroll
    for (int i = 0; i < NB / 2; ++i) {
      const float4 x = sc_bl4<H>(r, R::vscale, tok * NB, 4 * i);
      const float4 y = sc_bl4<H>(r, R::vmin, tok * NB, 4 * i);
      vs[4 * i] = x.x; vs[4 * i + 1] = x.y; vs[4 * i + 2] = x.z; vs[4 * i + 3] = x.w;
      vm[4 * i] = y.x; vm[4 * i + 1] = y.y; vm[4 * i + 2] = y.z; vm[4 * i + 3] = y.w;
    }
  };
  auto ld_vchan = [&](brsrc r) {
    const float4 va = sc_bl4<H>(r, R::vchan, 128 * wv + vci, 0);
    const float4 vb = sc_bl4<H>(r, R::vchan, 128 * wv + vci, 4);
    vch[0] = va.x; vch[1] = va.y; vch[2] = va.z; vch[3] = va.w;
    vch[4] = vb.x; vch[5] = vb.y; vch[6] = vb.z; vch[7] = vb.w;
  };
  ld_kcode(make_rsrc(rec, R::bytes));

  for (int j = t_begin; j < t_end; ++j, rec += rstride) {
    const uint8_t* nxt = j + 1 < t_end ? rec + rstride : rec;   // the last tile reloads its own K codes
    {
      const brsrc rc = make_rsrc(rec, R::bytes);
      ld_kscale(rc); ld_vmax(rc); ld_ktok(rc); ld_vcode(rc); ld_vscale(rc); ld_vchan(rc);
    }
    // ---- prep: q~ hi/lo operand rows, score unscale, bias ----
#pragma unroll
    for (int k = 0; k < PPW; ++k) {
      const int h = wv + 4 * k;   // operand head
      if (h < VH) {   // wave-uniform
        float y[CPL];
        float am = 0.0f, bs = 0.0f;
#pragma unroll
        for (int i = 0; i < CPL; ++i) {
          y[i] = qp[k][i] * ks[i];
          am = fmaxf(am, fabsf(y[i]));
          bs = fmaf(qp[k][i], km[i], bs);
        }
        const float amax = wmax(am);
        const float bias = wsum(bs);
        const int fe = fp16_scale_exp(amax);   // amax 2^fe in [2^13, 2^14)
        const float f = pow2i(fe - 4);
        // channel c -> uint4 [k4 = c / 32][row][(c / 8) % 4], half c % 8; channel
        // lane + 64 i has k4 = 2 i + lane / 32
        uint16_t* qt = reinterpret_cast<uint16_t*>(lds + o_qt);
        const int i0 = (((lane >> 5) * kRowsW + RPH * h) * 4 + ((lane >> 3) & 3)) * 8 + (lane & 7);
#pragma unroll
        for (int i = 0; i < CPL; i += 2) {
          uint32_t hi, lo;
          split_pair(y[i] * f, y[i + 1] * f, hi, lo);
          const int ia = i0 + i * 2 * kRowsW * 32;
          const int ib = ia + 2 * kRowsW * 32;
          qt[ia] = (uint16_t)(hi & 0xFFFFu);
          qt[ia + 32] = (uint16_t)(lo & 0xFFFFu);   // row RPH h + 1
          qt[ib] = (uint16_t)(hi >> 16);
          qt[ib + 32] = (uint16_t)(lo >> 16);
        }
        if (lane == 0) {
          reinterpret_cast<float*>(lds + o_us)[h] = pow2i(24 - fe);
          reinterpret_cast<float*>(lds + o_bias)[h] = bias;
        }
      }
    }
    if (wv == 0) {
      float vmx = 0.0f;   // the tile's largest value scale
#pragma unroll
      for (int i = 0; i < NB / 2; ++i)
        vmx = fmaxf(vmx, fmaxf(fmaxf(vmx4[i].x, vmx4[i].y), fmaxf(vmx4[i].z, vmx4[i].w)));
      const float vmax = wmax(vmx);   // p <= 1, so w <= the largest value scale
      if (lane == 0) reinterpret_cast<int*>(lds + o_fv)[0] = fp16_scale_exp(vmax);
    }
    // ---- the wave's K codes into its own area ----
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = lane + 64 * i;
      *reinterpret_cast<u32x4*>(cs + 16 * c + 16 * (c >> 3)) = kc[i];
    }
    lds_sync();   // the reload stays after the last use
    ld_kcode(make_rsrc(nxt, R::bytes));
    __syncthreads();   // (1) q~ operands and the tile's scalars are ready

    // ---- scores of the quarter: A = q~ rows, B = code nibbles of tokens 2 n, 2 n + 1 ----
    const uint4* qtu = reinterpret_cast<const uint4*>(lds + o_qt);
    floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    const uint8_t* kg = cs + 144 * g + n;   // channel 32 k4 + 8 g + j at kg[576 k4 + 16 j]
#pragma unroll
    for (int k4 = 0; k4 < K4; ++k4) {
      const uint4 a = qtu[(k4 * kRowsW + n) * 4 + g];
      const half8 A = as_half8(a.x, a.y, a.z, a.w);
      uint32_t e[4], o[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t x = byte_pair(kg + 576 * k4 + 32 * i, 16);
        e[i] = (x << 4) & 0x00F000F0u;   // token 2 n
        o[i] = x & 0x00F000F0u;          // token 2 n + 1
      }
      acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, as_half8(e[0], e[1], e[2], e[3]), acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, as_half8(o[0], o[1], o[2], o[3]), acc1, 0, 0, 0);
    }
    // lane (g, n): rows 4 g + i = head HPL g + i / RPH, part i % RPH
    const int vexp = reinterpret_cast<const int*>(lds + o_fv)[0];
    const float fv = pow2i(vexp);
    const float k0 = kt.x * c_log2, k1 = kt.y * c_log2;
    float s0[HPL], s1[HPL];
#pragma unroll
    for (int jj = 0; jj < HPL; ++jj) {
      const int h = HPL * g + jj;   // operand head
      const int hc = h < VH ? h : VH - 1;
      const float us = reinterpret_cast<const float*>(lds + o_us)[hc];
      const float bi = reinterpret_cast<const float*>(lds + o_bias)[hc];
      s0[jj] = k0 * fmaf(acc0[RPH * jj] + acc0[RPH * jj + 1], us, bi);
      s1[jj] = k1 * fmaf(acc1[RPH * jj] + acc1[RPH * jj + 1], us, bi);
      const float qm = row_max16(fmaxf(s0[jj], s1[jj]));
      if (n == 0 && h < VH) s_qmax[wv * VH + h] = qm;
    }
    __syncthreads();   // (2) the four quarter maxima are ready

    // ---- softmax with the tile maximum; w rows and p vmin sums of the quarter, every group ----
    float p0[HPL], p1[HPL];
#pragma unroll
    for (int jj = 0; jj < HPL; ++jj) {
      const int h = HPL * g + jj;
      const int hc = h < VH ? h : VH - 1;
      const float mt = fmaxf(fmaxf(s_qmax[hc], s_qmax[VH + hc]), fmaxf(s_qmax[2 * VH + hc], s_qmax[3 * VH + hc]));
      const float m_new = fmaxf(m_run[jj], mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run[jj] - m_new);   // 0 on the first tile
      p0[jj] = __builtin_amdgcn_exp2f(s0[jj] - m_new);
      p1[jj] = __builtin_amdgcn_exp2f(s1[jj] - m_new);
      m_run[jj] = m_new;
      l_q[jj] = fmaf(l_q[jj], alpha, p0[jj] + p1[jj]);   // summed over the row and the quarters at the end
#pragma unroll
      for (int q = 0; q < 8; ++q) o_c[jj][q] *= alpha;
    }
#pragma unroll
    for (int cb = 0; cb < NB; ++cb) {
      uint32_t* wrow = reinterpret_cast<uint32_t*>(lds + o_w + (cb * 4 + wv) * w_blk);
#pragma unroll
      for (int jj = 0; jj < HPL; ++jj) {
        const int h = HPL * g + jj;
        uint32_t hi, lo;
        split_pair(p0[jj] * (vs[cb] * fv), p1[jj] * (vs[NB + cb] * fv), hi, lo);
        const float u = row_sum16(p0[jj] * vm[cb] + p1[jj] * vm[NB + cb]);   // sum_t p vmin over the quarter
        if (h < VH) {
          wrow[(RPH * h) * kWRowW + n] = hi;
          wrow[(RPH * h + 1) * kWRowW + n] = lo;
          if (n == 0) s_u[(cb * 4 + wv) * VH + h] = u;
        }
      }
    }
    // ---- the group's V codes over the wave's K codes ----
    lds_sync();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int e = lane + 64 * i, t = e >> 1;
      *reinterpret_cast<u32x4*>(cs + 32 * t + 32 * (t >> 3) + 16 * (e & 1)) = vc[i];
    }
    __syncthreads();   // (3) every quarter's w rows and sums are ready

    // ---- value aggregate of group wv: A = w rows of quarter q, B = crumbs of
    //      tokens 32 q + 8 g + j, channels 128 wv + 16 (n % 8) + 8 (n / 8) + qb ----
    const float un_lo = pow2i(24 - vexp - 4), un_hi = pow2i(24 - vexp - 6);
    float u[HPL];
#pragma unroll
    for (int jj = 0; jj < HPL; ++jj) {
      const int hc = min(HPL * g + jj, VH - 1);
      u[jj] = (s_u[(wv * 4) * VH + hc] + s_u[(wv * 4 + 1) * VH + hc]) +
              (s_u[(wv * 4 + 2) * VH + hc] + s_u[(wv * 4 + 3) * VH + hc]);
    }
    half8 A[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4 wa =
          *reinterpret_cast<const uint4*>(lds + o_w + (wv * 4 + q) * w_blk + (n * kWRowW + 4 * g) * 4);
      A[q] = as_half8(wa.x, wa.y, wa.z, wa.w);
    }
    // token 32 q + 8 g + j at vg[q][.. j ..]; this lane's two bytes at + 0, + 1
    const uint8_t* vg = cs + 4 * (n & 7) + 2 * (n >> 3);
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      uint32_t x[4][4];   // [quarter][token pair]
#pragma unroll
      for (int q = 0; q < 4; ++q) {
#pragma unroll
        for (int pq = 0; pq < 4; ++pq) {
          const int t = 32 * q + 8 * g + 2 * pq;   // rows t, t + 1 lie in one padded block of 8
          x[q][pq] = byte_pair(vg + 32 * t + 32 * (t >> 3) + e, 32);
        }
      }
#pragma unroll
      for (int cr = 0; cr < 4; ++cr) {
        const uint32_t mask = (cr & 1) ? 0x00C000C0u : 0x00300030u;
        floatx4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          uint32_t bv[4];
#pragma unroll
          for (int pq = 0; pq < 4; ++pq) bv[pq] = ((cr < 2) ? (x[q][pq] << 4) : x[q][pq]) & mask;
          z = __builtin_amdgcn_mfma_f32_16x16x32_f16(A[q], as_half8(bv[0], bv[1], bv[2], bv[3]), z, 0, 0, 0);
        }
        const int qb = 4 * e + cr;
        const float un = (cr & 1) ? un_hi : un_lo;
#pragma unroll
        for (int jj = 0; jj < HPL; ++jj)
          o_c[jj][qb] = fmaf(vch[qb], fmaf(z[RPH * jj] + z[RPH * jj + 1], un, u[jj]), o_c[jj][qb]);
      }
    }
  }

  // ---- write the partials: each wave its group's channels; the sum of
  //      weights over the quarters through LDS ----
  float* s_l = reinterpret_cast<float*>(lds + o_l);
#pragma unroll
  for (int jj = 0; jj < HPL; ++jj) {
    const int h = HPL * g + jj;
    const float lq = row_sum16(l_q[jj]);
    if (h < VH) {
      float* part = P.part + (((int64_t)b * P.n_q + (int64_t)kvh * G + h) * n_split + split) * (D + 4);
      *reinterpret_cast<float4*>(part + 128 * wv + vci) = make_float4(o_c[jj][0], o_c[jj][1], o_c[jj][2], o_c[jj][3]);
      *reinterpret_cast<float4*>(part + 128 * wv + vci + 4) = make_float4(o_c[jj][4], o_c[jj][5], o_c[jj][6], o_c[jj][7]);
      if (n == 0) s_l[wv * VH + h] = lq;
    }
  }
  __syncthreads();
  if (wv == 0) {
#pragma unroll
    for (int jj = 0; jj < HPL; ++jj) {
      const int h = HPL * g + jj;
      if (n == 0 && h < VH) {
        float* part = P.part + (((int64_t)b * P.n_q + (int64_t)kvh * G + h) * n_split + split) * (D + 4);
        part[D] = m_run[jj] * kLn2W;   // natural-log units, as the combine expects
        part[D + 1] = (s_l[h] + s_l[VH + h]) + (s_l[2 * VH + h] + s_l[3 * VH + h]);
      }
    }
  }
}

// decode (mode 0): the tile splits, then the window splits, in one grid;
// prefill: the tile splits alone (the window kernel takes the raw rows)
template <int D, int G>
hipError_t launch_wide_dg(const DecodeParams& P, int batch, hipStream_t stream) {
  if (P.mode == 0 && P.n_wsplit > 0 && P.wchunk != kWinChunk) return hipErrorInvalidValue;
  const int nx = P.n_tsplit + (P.mode == 0 ? P.n_wsplit : 0);
  // prefill rows in pairs when G <= 4 and the chunk has an even number of rows
  if constexpr (G <= 4) {
    if (P.mode == 1 && batch % 2 == 0) {
      const dim3 grid(P.n_tsplit, P.n_kv, batch / 2);
      if (P.h16)
        hipLaunchKernelGGL((decode_wide_kernel<D, G, true, 2>), grid, dim3(256), 0, stream, P);
      else
        hipLaunchKernelGGL((decode_wide_kernel<D, G, false, 2>), grid, dim3(256), 0, stream, P);
      return hipGetLastError();
    }
  }
  const dim3 grid(nx, P.n_kv, batch);
  if constexpr (D == 512) {   // one row per workgroup: the channel-split kernel
    if (P.h16)
      hipLaunchKernelGGL((decode_wide_cs_kernel<G, true>), grid, dim3(256), 0, stream, P);
    else
      hipLaunchKernelGGL((decode_wide_cs_kernel<G, false>), grid, dim3(256), 0, stream, P);
    return hipGetLastError();
  }
  if (P.h16)
    hipLaunchKernelGGL((decode_wide_kernel<D, G, true, 1>), grid, dim3(256), 0, stream, P);
  else
    hipLaunchKernelGGL((decode_wide_kernel<D, G, false, 1>), grid, dim3(256), 0, stream, P);
  return hipGetLastError();
}

template <int D>
hipError_t launch_wide_d(const DecodeParams& P, int batch, hipStream_t stream) {
  switch (P.G) {
    case 1: return launch_wide_dg<D, 1>(P, batch, stream);
    case 2: return launch_wide_dg<D, 2>(P, batch, stream);
    case 4: return launch_wide_dg<D, 4>(P, batch, stream);
    case 8: return launch_wide_dg<D, 8>(P, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_wide(int d, const DecodeParams& P, int batch, hipStream_t stream) {
  switch (d) {
    case 256: return launch_wide_d<256>(P, batch, stream);
    case 512: return launch_wide_d<512>(P, batch, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace kvarn
