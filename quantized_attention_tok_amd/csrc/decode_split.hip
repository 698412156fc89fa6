// decode_split.hip -- split-tile decode attention for head_dim 128 on gfx950.
//
// One decode step is two launches (SharpInference issue #433 item 2: fixed
// worst-case grid with early exit, log-sum-exp combine, inverse WHT applied
// once to the combined rotated partials; PR #434 commit list: a single
// streaming softmax over the compressed tiles and the FP32 window):
//
//   decode_split_kernel<G, TPW, H, APP>: workgroup = (split, KV head,
//     sequence) with 4 TPW waves.  Split s owns the tiles [TPW s, TPW s + TPW)
//     and the raw window tokens [E s, E s + E) of its sequence (E <= 16 from
//     the split plan: the window spread over the tile splits).  H: f16 scales;
//     APP: the call appends the newest token, so window token n_win - 1 comes
//     from k_new / v_new and the wave that takes it also stores it into the
//     window (the FP32 window staging of the PR #434 commit list, in the same
//     launch).
//     Tiles: wave (tau, wq) owns the 32-token quarter wq of tile tau from
//     loads to value aggregate.  It loads only its own slice (the 16 code
//     bytes of its tokens in every channel row, its 32 V-code rows, its
//     per-token scales straight into registers), stages the codes in a
//     private LDS area and needs no barrier once the shared q~ operands are
//     written, so every wave computes as soon as its own bytes land.
//       S[(h,part)][t] = sum_c q~[(h,part)][c] zK[t][c]     q~ = q' kscale
//       O[(h,part)][c] = sum_t w[(h,part)][t] zV[t][c]      w  = p vscale
//     (issue #180 Algorithm step 4: scales folded in at read time; colibri PR
//     #399 review note: q . xhat = rotate(q) . code, the cache is never
//     reconstructed).  Both contractions run on v_mfma_f32_16x16x32_f16.  The
//     fp32 operand is split into fp16 hi and lo parts that occupy adjacent
//     MFMA rows, so one MFMA yields both halves of a product for two query
//     heads and a lane adds them in registers.  Codes enter as fp16
//     subnormals with the code in bits 4-7 (16 z 2^-24 for nibbles, z 2^-20 or
//     z 2^-18 for 2-bit codes): products of such subnormals are exact on
//     gfx950, while codes in bits 0-3 lose precision.
//     Window tokens: one wave per token scores the raw key with the raw
//     query (q . k needs no rotation) and rotates the value row (H v), so
//     every partial of the launch is in the rotated domain.
//     The waves merge their (m, l, o) states in LDS into one partial per
//     query head.
//   decode_combine_kernel: per (query head, sequence), 4 waves merge the
//     partials with an online log-sum-exp; the sum gets one inverse WHT and
//     is divided by L.
//
// LDS bank conflicts: a wave's K-code channel rows and V-code token rows are
// padded by one row every 8 rows, so the byte gathers of one MFMA operand hit
// distinct banks; the hi/lo operand rows of w use an 80-byte stride.
//
// If q_rot is NULL the workgroups rotate the query themselves (the same
// Walsh-Hadamard butterflies as kvarn_rotate_query).
#include <float.h>

#include "kvarn_launch.h"
#include "kvarn_mfma.h"

namespace kvarn {
namespace {

using namespace mfma;

constexpr int kWRow = 20;            // dwords per hi/lo operand row of w (80 bytes)
constexpr int kMRows = 16;           // MFMA operand rows; rows >= 2G stay zero
// A wave's codes in LDS: K-code channel row c (16 bytes, its 32 tokens) at
// 16 c + 16 (c / 8); V-code token row t (32 bytes) at 32 (t + t / 8).  The
// padding puts the rows one MFMA operand gathers in distinct banks while every
// gather address stays a per-lane base plus a constant offset.
constexpr int kKCodeWave = 16 * 144;          // 2304
constexpr int kVCodeWave = 4 * 9 * 32;        // 1152
constexpr int kCodeWave = kKCodeWave + kVCodeWave;

constexpr int align16(int x) { return (x + 15) / 16 * 16; }

// LDS layout of a split workgroup (G query heads per KV head, TPW tiles).
template <int G, int TPW>
struct Lds {
  static constexpr int kNW = 4 * TPW;                       // waves
  // MFMA operand rows: head h's fp16 hi and lo parts sit in rows RPH h and
  // RPH h + 1, so lane group g of an MFMA result holds heads HPL g .. + HPL - 1
  // (one head per lane group for G <= 4; the other rows stay zero)
  static constexpr int HPL = G > 4 ? 2 : 1;
  static constexpr int RPH = 4 / HPL;
  static constexpr int code = 0;                            // [wave] K and V codes of its tokens
  static constexpr int wop = kNW * kCodeWave;               // [wave][16 rows][kWRow] dwords: w hi/lo
  static constexpr int wop_wave = kMRows * kWRow * 4;
  static constexpr int qt = wop + kNW * wop_wave;           // [TPW][k4][16 rows][4] uint4: q~ hi/lo
  static constexpr int qt_tile = 4 * kMRows * 64;
  static constexpr int winw = qt + TPW * qt_tile;           // [G][16] f32: window weights
  static constexpr int winv = winw + G * kWinPerSplit * 4;  // [16][D] f32: rotated window values
  static constexpr int winp = winv + kWinPerSplit * D * 4;  // [G][16][4] f32: window q . k row sums
  static constexpr int us = winp + G * kWinPerSplit * 16;   // [TPW][G] f32: score unscale
  static constexpr int bias = us + TPW * G * 4;             // [TPW][G] f32: sum_c q'_c kmin_c
  static constexpr int fv = bias + TPW * G * 4;             // [TPW] int: w fp16 scale exponent
  static constexpr int ml = align16(fv + TPW * 4);          // [G][wave] float2: m, l
  static constexpr int bytes = ml + kNW * G * 8;
  static constexpr int mo = 0;                              // merge: [wave][G][D] f32 (over codes, w, q~)
  static_assert(kNW * G * D * 4 <= winw, "merge area fits below the window entries");
  static_assert(kNW <= 16, "the merge gives each wave's state one lane of a 16-lane row");
  static_assert((wop % 16) == 0 && (qt % 16) == 0 && (winv % 16) == 0, "aligned sections");
};

// x holds element lane, y element lane + 64 of a 128-vector: y <- H_128 x / sqrt(128)
__device__ __forceinline__ void wht128(float& x, float& y, int lane) {
  x = bfly<1>(x, lane); y = bfly<1>(y, lane);
  x = bfly<2>(x, lane); y = bfly<2>(y, lane);
  x = bfly<4>(x, lane); y = bfly<4>(y, lane);
  x = bfly<8>(x, lane); y = bfly<8>(y, lane);
  x = bfly<16>(x, lane); y = bfly<16>(y, lane);
  x = bfly<32>(x, lane); y = bfly<32>(y, lane);
  const float a = x, c = y;
  x = (a + c) * wht_scale<D>();
  y = (a - c) * wht_scale<D>();
}

// APP: the call appends the newest token (P.k_new, P.v_new): window token
// n_win - 1 is read from them and stored into the window.
template <int G, int TPW, bool H, bool APP>
__global__ void __launch_bounds__(256 * TPW) decode_split_kernel(DecodeParams P) {
  using L = Lds<G, TPW>;
  using R = Rec<D, H>;
  constexpr int NW = L::kNW;
  constexpr int NT = 64 * NW;
  constexpr int HPL = L::HPL, RPH = L::RPH;
  constexpr int PPW = (TPW * G + NW - 1) / NW;         // (tile, head) prep pairs per wave
  constexpr int KW = (kWinPerSplit + NW - 1) / NW;     // window tokens per wave
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  // Every kernel argument the workgroup needs, read before any branch and
  // pinned in registers together: one round of scalar loads, not a chain.
  const SeqView sv = seq_view_decode(P, b);
  const int n_split = P.n_tsplit, n_q = P.n_q, n_kv = P.n_kv;
  const float p_scale = P.scale;
  const float *p_q = P.q, *p_qrot = P.q_rot, *p_kwin = P.k_win, *p_vwin = P.v_win;
  const uint8_t* p_rec = P.records;
  float* p_part = P.part;
  const int64_t p_hst = P.win_head_stride, p_tok = P.win_tok_stride;
  asm volatile("" ::"s"(sv.nt), "s"(sv.nw), "s"(sv.rec_row0), "s"(sv.win_off), "s"(n_split),
               "s"(n_q), "s"(n_kv), "s"(p_scale), "s"(p_q), "s"(p_qrot), "s"(p_kwin), "s"(p_vwin),
               "s"(p_rec), "s"(p_part), "s"(p_hst), "s"(p_tok));

  __shared__ __attribute__((aligned(16))) uint8_t lds[L::bytes];
  float2* s_ml = reinterpret_cast<float2*>(lds + L::ml);
  float* s_mo = reinterpret_cast<float*>(lds + L::mo);
  float* s_winw = reinterpret_cast<float*>(lds + L::winw);
  float* s_winv = reinterpret_cast<float*>(lds + L::winv);
  float* s_winp = reinterpret_cast<float*>(lds + L::winp);

  float* part = p_part + (((int64_t)b * n_q + (int64_t)kvh * G) * n_split + split) * (D + 4);
  const int64_t hs = (int64_t)n_split * (D + 4);   // partial of head h at part + h * hs
  const int j0 = split * TPW;
  const int ntl = max(0, min(TPW, sv.nt - j0));                     // tiles of this split
  const int wps = P.wchunk;                                          // window tokens per split (<= 16)
  const int nwt = max(0, min(wps, sv.nw - wps * split));             // window tokens of this split
  if (ntl == 0 && nwt == 0) {
    for (int i = tid; i < G * (D + 2); i += NT) {
      const int h = i / (D + 2), c = i % (D + 2);
      part[h * hs + c] = (c == D) ? -INFINITY : 0.0f;
    }
    return;
  }
  const float c_log2 = p_scale * kLog2e;
  const int tau = wv >> 2, wq = wv & 3;
  const bool has_tile = tau < ntl;
  const int64_t rstride = (int64_t)n_kv * R::bytes;
  const uint8_t* recs = p_rec + ((sv.rec_row0 + j0) * (int64_t)n_kv + kvh) * R::bytes;
  const float* qsrc = (p_qrot ? p_qrot : p_q) + ((int64_t)b * n_q + (int64_t)kvh * G) * D;
  const float* qraw = p_q + ((int64_t)b * n_q + (int64_t)kvh * G) * D;

  // ---- 1. loads.  Window rows first: the waits for the tile loads below then
  //      never include them.  Inside a split with tiles every wave issues the
  //      same loads (missing tiles and pairs read tile 0), so the waits are exact.
  // (read only under the conditions they are loaded under)
  float wk0[KW], wk1[KW], wv0[KW], wv1[KW], qw0[G], qw1[G];
#pragma unroll
  for (int h = 0; h < G; ++h) {
    if (wv < nwt) {
      qw0[h] = qraw[h * D + lane];
      qw1[h] = qraw[h * D + lane + 64];
    }
  }
  const float* kwin = p_kwin + sv.win_off + (int64_t)kvh * p_hst;
  const float* vwin = p_vwin + sv.win_off + (int64_t)kvh * p_hst;
  // APP: the newest window token (n_win - 1) is read from k_new / v_new and
  // stored into the window by the wave that takes it (section 4)
  const int t_new = APP ? sv.nw - 1 : -1;
#pragma unroll
  for (int k = 0; k < KW; ++k) {
    const int tr = wv + NW * k;
    if (tr < nwt) {
      if (APP && wps * split + tr == t_new) {   // wave-uniform
        const float* ks = P.k_new + ((int64_t)b * n_kv + kvh) * D;
        const float* vs = P.v_new + ((int64_t)b * n_kv + kvh) * D;
        wk0[k] = ks[lane];
        wk1[k] = ks[lane + 64];
        wv0[k] = vs[lane];
        wv1[k] = vs[lane + 64];
      } else {
        const int64_t row = (int64_t)(wps * split + tr) * p_tok;
        wk0[k] = kwin[row + lane];
        wk1[k] = kwin[row + lane + 64];
        wv0[k] = vwin[row + lane];
        wv1[k] = vwin[row + lane + 64];
      }
    }
  }
  uint4 kc0, kc1, vcd;   // (read only by waves with a tile)
  float2 kt, vsc, vmn;
  float4 vca, vcb;
  if (ntl > 0) {   // workgroup-uniform
    // (a) prep pairs (tile tt, head h): query row, the tile's kscale / kmin / vscale
    float pq0[PPW], pq1[PPW], pks0[PPW], pks1[PPW], pkm0[PPW], pkm1[PPW];
    float2 pvs[PPW];
#pragma unroll
    for (int k = 0; k < PPW; ++k) {
      const int pr = wv + NW * k;
      const bool ok = pr < TPW * G && pr / G < ntl;
      const int tt = ok ? pr / G : 0, h = ok ? pr % G : 0;
      const uint8_t* rp = recs + tt * rstride;
      pq0[k] = qsrc[h * D + lane];
      pq1[k] = qsrc[h * D + lane + 64];
      pks0[k] = sc_ld<H>(rp + R::kscale, lane);
      pks1[k] = sc_ld<H>(rp + R::kscale, lane + 64);
      pkm0[k] = sc_ld<H>(rp + R::kmin, lane);
      pkm1[k] = sc_ld<H>(rp + R::kmin, lane + 64);
      pvs[k] = sc_ld2<H>(rp + R::vscale, 2 * lane);
    }
    // keep the prep loads ahead of the tile loads in the memory queue
    asm volatile("" ::: "memory");
    // (b) own tile slice: K codes of channels lane, lane + 64 (16 bytes each), V codes,
    //     per-token scales of tokens 32 wq + 2 n, +1, value channel scales
    {
      const uint8_t* rg = recs + (has_tile ? tau : 0) * rstride;
      kc0 = *reinterpret_cast<const uint4*>(rg + lane * 64 + 16 * wq);
      kc1 = *reinterpret_cast<const uint4*>(rg + (lane + 64) * 64 + 16 * wq);
      vcd = *reinterpret_cast<const uint4*>(rg + R::vcode + 32 * 32 * wq + 16 * lane);
      const int tok = 32 * wq + 2 * n;
      kt = sc_ld2<H>(rg + R::ktok, tok);
      vsc = sc_ld2<H>(rg + R::vscale, tok);
      vmn = sc_ld2<H>(rg + R::vmin, tok);
      const int vci = 16 * (n & 7) + 8 * (n >> 3);
      vca = sc_ld4<H>(rg + R::vchan, vci);
      vcb = sc_ld4<H>(rg + R::vchan, vci + 4);
    }

    // ---- 2. prep: rotated query, q~ hi/lo operand rows, unscale, bias, w scale ----
#pragma unroll
    for (int k = 0; k < PPW; ++k) {
      const int pr = wv + NW * k, tt = pr / G, h = pr % G;
      const bool ok = pr < TPW * G && tt < ntl;   // wave-uniform; the math runs either way
      {
        float x0 = pq0[k], x1 = pq1[k];
        if (!p_qrot) wht128(x0, x1, lane);
        const float y0 = x0 * pks0[k], y1 = x1 * pks1[k];
        const float amax = wmax(fmaxf(fabsf(y0), fabsf(y1)));
        const float bias = wsum(x0 * pkm0[k] + x1 * pkm1[k]);
        const int fe = fp16_scale_exp(amax);   // amax 2^fe in [2^13, 2^14)
        const float f = pow2i(fe - 4);
        uint32_t hi, lo;
        split_pair(y0 * f, y1 * f, hi, lo);   // halves: channel lane, channel lane + 64
        // channel c -> uint4 [k4 = c / 32][row][g' = (c / 8) % 4], half c % 8
        const float vmax = wmax(fmaxf(pvs[k].x, pvs[k].y));   // p <= 1, so w <= max vscale
        if (ok) {
          uint16_t* qt = reinterpret_cast<uint16_t*>(lds + L::qt + tt * L::qt_tile);
          const int i0 = (((lane >> 5) * kMRows + RPH * h) * 4 + ((lane >> 3) & 3)) * 8 + (lane & 7);
          const int i1 = i0 + 2 * kMRows * 32;   // channel + 64: k4 + 2
          qt[i0] = (uint16_t)(hi & 0xFFFFu);
          qt[i0 + 32] = (uint16_t)(lo & 0xFFFFu);   // row RPH h + 1
          qt[i1] = (uint16_t)(hi >> 16);
          qt[i1 + 32] = (uint16_t)(lo >> 16);
          if (lane == 0) {
            reinterpret_cast<float*>(lds + L::us)[tt * G + h] = pow2i(24 - fe);
            reinterpret_cast<float*>(lds + L::bias)[tt * G + h] = bias;
            if (h == 0) reinterpret_cast<int*>(lds + L::fv)[tt] = fp16_scale_exp(vmax);
          }
        }
      }
    }
  }
  // q~ operand rows that hold no head part stay zero
  if constexpr (RPH > 2 || G < 8) {
    for (int i = tid; i < TPW * 4 * kMRows * 4; i += NT) {
      const int r = (i >> 2) & (kMRows - 1);
      if ((r % RPH) >= 2 || r / RPH >= G) reinterpret_cast<uint4*>(lds + L::qt)[i] = make_uint4(0, 0, 0, 0);
    }
  }
  __syncthreads();   // q~ operands and per-tile scalars are ready; codes may still be in flight

  // ---- 3. the wave's tile quarter: tokens 32 wq .. 32 wq + 31 of tile tau ----
  float m_w[HPL], l_w[HPL], o_w[HPL][8];   // (set and read only by waves with a tile)
  if (has_tile) {
    uint8_t* kcs = lds + L::code + wv * kCodeWave;   // channel row c at 16 c + 16 (c / 8)
    uint8_t* vcs = kcs + kKCodeWave;                 // token row t at 32 (t + t / 8)
    {
      const int c0 = lane, c1 = lane + 64;
      *reinterpret_cast<uint4*>(kcs + 16 * c0 + 16 * (c0 >> 3)) = kc0;
      *reinterpret_cast<uint4*>(kcs + 16 * c1 + 16 * (c1 >> 3)) = kc1;
      const int t = lane >> 1;
      *reinterpret_cast<uint4*>(vcs + 32 * (t + (t >> 3)) + 16 * (lane & 1)) = vcd;
    }
    const uint4* qtu = reinterpret_cast<const uint4*>(lds + L::qt + tau * L::qt_tile);
    // scores: A = q~ rows, B = code nibbles of tokens 2 n, 2 n + 1 (of the quarter)
    floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    const uint8_t* kg = kcs + 144 * g + n;   // channel 32 k4 + 8 g + j at kg[576 k4 + 16 j]
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      const uint4 a = qtu[(k4 * kMRows + n) * 4 + g];
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
    // lane (g, n): rows 4 g + i = (head HPL g + i / RPH, part i % RPH)
    const int vexp = reinterpret_cast<const int*>(lds + L::fv)[tau];
    const float fv = pow2i(vexp);
    const float k0 = kt.x * c_log2, k1 = kt.y * c_log2;
    const float vs0 = vsc.x * fv, vs1 = vsc.y * fv;
    uint32_t* wrow = reinterpret_cast<uint32_t*>(lds + L::wop + wv * L::wop_wave);
    if constexpr (RPH > 2 || G < 8) {   // w rows that hold no head part stay zero
      for (int i = lane; i < kMRows * (kWRow / 4); i += 64) {
        const int r = i / (kWRow / 4);
        if ((r % RPH) >= 2 || r / RPH >= G) reinterpret_cast<uint4*>(wrow)[i] = make_uint4(0, 0, 0, 0);
      }
    }
    float u_w[HPL];
#pragma unroll
    for (int jj = 0; jj < HPL; ++jj) {
      const int h = HPL * g + jj;
      const int hc = h < G ? h : G - 1;
      const float us = reinterpret_cast<const float*>(lds + L::us)[tau * G + hc];
      const float bi = reinterpret_cast<const float*>(lds + L::bias)[tau * G + hc];
      const float s0 = k0 * fmaf(acc0[RPH * jj] + acc0[RPH * jj + 1], us, bi);
      const float s1 = k1 * fmaf(acc1[RPH * jj] + acc1[RPH * jj + 1], us, bi);
      const float mt = row_max16(fmaxf(s0, s1));
      const float p0 = __builtin_amdgcn_exp2f(s0 - mt), p1 = __builtin_amdgcn_exp2f(s1 - mt);
      m_w[jj] = mt;
      l_w[jj] = p0 + p1;                                  // summed over the row in the merge
      u_w[jj] = row_sum16(p0 * vmn.x + p1 * vmn.y);       // sum_t p vmin over the quarter
      uint32_t hi, lo;
      split_pair(p0 * vs0, p1 * vs1, hi, lo);
      if (h < G) {
        wrow[(RPH * h) * kWRow + n] = hi;
        wrow[(RPH * h + 1) * kWRow + n] = lo;
      }
    }
    // value aggregate: A = w rows of the quarter, B = crumbs of tokens 8 g + j,
    // channels 16 (n % 8) + 8 (n / 8) + qb
    const uint4 wa = *reinterpret_cast<const uint4*>(wrow + n * kWRow + 4 * g);
    const half8 A = as_half8(wa.x, wa.y, wa.z, wa.w);
    // token 8 g + j at vg[32 j]; this lane's two bytes at + 0, + 1
    const uint8_t* vg = vcs + 288 * g + 4 * (n & 7) + 2 * (n >> 3);
    uint32_t x[2][4];
#pragma unroll
    for (int pq = 0; pq < 4; ++pq) {
#pragma unroll
      for (int e = 0; e < 2; ++e) x[e][pq] = byte_pair(vg + 64 * pq + e, 32);
    }
    const float vch[8] = {vca.x, vca.y, vca.z, vca.w, vcb.x, vcb.y, vcb.z, vcb.w};
    const float un_lo = pow2i(24 - vexp - 4), un_hi = pow2i(24 - vexp - 6);
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
      for (int jj = 0; jj < HPL; ++jj) o_w[jj][qb] = vch[qb] * fmaf(z[RPH * jj] + z[RPH * jj + 1], un, u_w[jj]);
    }
  }

  // ---- 4. window tokens: raw scores, rotated values ----
#pragma unroll
  for (int k = 0; k < KW; ++k) {
    const int tr = wv + NW * k;
    if (tr < nwt) {   // wave-uniform
      if (APP && wps * split + tr == t_new) {   // the appended token: into the window (the API's window is writable)
        const int64_t row = (int64_t)t_new * p_tok;
        float* kw = const_cast<float*>(kwin);
        float* vw = const_cast<float*>(vwin);
        kw[row + lane] = wk0[k];
        kw[row + lane + 64] = wk1[k];
        vw[row + lane] = wv0[k];
        vw[row + lane + 64] = wv1[k];
      }
      float sc[G];
#pragma unroll
      for (int h = 0; h < G; ++h) sc[h] = row_sum16(qw0[h] * wk0[k] + qw1[h] * wk1[k]);
      float v0 = wv0[k], v1 = wv1[k];
      wht128(v0, v1, lane);
      s_winv[tr * D + lane] = v0;
      s_winv[tr * D + lane + 64] = v1;
      if (n == 0) {   // the four row sums of each head's q . k
#pragma unroll
        for (int h = 0; h < G; ++h) s_winp[(h * kWinPerSplit + tr) * 4 + g] = sc[h];
      }
    }
  }

  // ---- 5. merge the workgroup's states ----
  const int n_act = 4 * ntl;   // waves holding a tile state
  if (wv < n_act) {
#pragma unroll
    for (int jj = 0; jj < HPL; ++jj) {
      const int h = HPL * g + jj;
      const float lt = row_sum16(l_w[jj]);
      if (n == 0 && h < G) s_ml[h * NW + wv] = make_float2(m_w[jj], lt);
    }
  }
  __syncthreads();   // every wave is done with its codes and w rows: the merge area may be written
  // Head maxima and sums, lane-parallel in every wave: lane (g, n) of head
  // HPL g + jj takes wave n's state (n < n_act) and window token n (n < nwt).
  float Mh[HPL];
#pragma unroll
  for (int jj = 0; jj < HPL; ++jj) {
    const int hr = HPL * g + jj;
    const int h = hr < G ? hr : G - 1;
    const float2 ml = (n < n_act) ? s_ml[h * NW + n] : make_float2(-INFINITY, 0.0f);
    float sc = -INFINITY;
    if (n < nwt) {
      const float4 r = *reinterpret_cast<const float4*>(s_winp + 4 * (h * kWinPerSplit + n));
      sc = ((r.x + r.y) + (r.z + r.w)) * c_log2;
    }
    const float M = row_max16(fmaxf(ml.x, sc));
    const float ww = (n < nwt) ? __builtin_amdgcn_exp2f(sc - M) : 0.0f;
    const float ls = (n < n_act) ? __builtin_amdgcn_exp2f(ml.x - M) * ml.y : 0.0f;
    const float L = row_sum16(ls + ww);
    Mh[jj] = M;
    if (wv == 0 && hr < G) {
      if (n < nwt) s_winw[h * kWinPerSplit + n] = ww;
      if (n == 0) {
        part[h * hs + D] = M;   // log2 domain
        part[h * hs + D + 1] = L;
      }
    }
  }
  if (wv < n_act) {
#pragma unroll
    for (int jj = 0; jj < HPL; ++jj) {
      const int h = HPL * g + jj;
      if (h < G) {
        const float sc = __builtin_amdgcn_exp2f(m_w[jj] - Mh[jj]);
        float* dst = s_mo + (wv * G + h) * D + 16 * (n & 7) + 8 * (n >> 3);
        *reinterpret_cast<float4*>(dst) =
            make_float4(o_w[jj][0] * sc, o_w[jj][1] * sc, o_w[jj][2] * sc, o_w[jj][3] * sc);
        *reinterpret_cast<float4*>(dst + 4) =
            make_float4(o_w[jj][4] * sc, o_w[jj][5] * sc, o_w[jj][6] * sc, o_w[jj][7] * sc);
      }
    }
  }
  __syncthreads();
  for (int i = tid; i < G * D; i += NT) {
    const int h = i / D, c = i % D;
    float o = 0.0f;
    for (int w = 0; w < n_act; ++w) o += s_mo[(w * G + h) * D + c];
    for (int t = 0; t < nwt; ++t) o += s_winw[h * kWinPerSplit + t] * s_winv[t * D + c];
    part[h * hs + c] = o;
  }
}

// ---------------------------------------------------------------------------
// Combine: one workgroup of 4 waves per (query head, sequence); lane l owns
// channels 2l, 2l+1.  Wave w folds splits [PW w + 4 PW k, +PW) with an online
// log-sum-exp (all loads of a pass in flight, split j's weight read from lane
// j); the four wave states merge in LDS, wave 0 applies the inverse WHT and
// divides by L.
// ---------------------------------------------------------------------------
template <int PW>
__global__ void __launch_bounds__(256) decode_combine_kernel(DecodeParams P) {
  const int hq = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int ns = P.n_tsplit;
  const float* ph = P.part + ((int64_t)b * P.n_q + hq) * (int64_t)ns * (D + 4);
  __shared__ float s_st[4][2];
  __shared__ __attribute__((aligned(16))) float s_o[4][D];
  float M = -INFINITY, Lt = 0.0f, t0 = 0.f, t1 = 0.f;
  for (int base = PW * w; base < ns; base += 4 * PW) {
    float2 v[PW];
#pragma unroll
    for (int j = 0; j < PW; ++j)
      v[j] = (base + j < ns) ? *reinterpret_cast<const float2*>(ph + (int64_t)(base + j) * (D + 4) + 2 * lane)
                             : make_float2(0.f, 0.f);
    float m = -INFINITY, l = 0.0f;
    if (lane < PW && base + lane < ns) {
      const float2 ml = *reinterpret_cast<const float2*>(ph + (int64_t)(base + lane) * (D + 4) + D);
      m = ml.x;
      l = ml.y;
    }
    const float mc = wmax(m);
    if (mc > M) {
      const float r = __builtin_amdgcn_exp2f(M - mc);   // 0 while M = -inf
      Lt *= r; t0 *= r; t1 *= r;
      M = mc;
    }
    const float wgt = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - M);
    Lt += wsum(wgt * l);
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int j = 0; j < PW; j += 2) {   // split j's weight is lane j's
      const float w0 = lane_f(wgt, j), w1 = lane_f(wgt, j + 1);
      t0 += w0 * v[j].x;
      t1 += w0 * v[j].y;
      a0 += w1 * v[j + 1].x;
      a1 += w1 * v[j + 1].y;
    }
    t0 += a0;
    t1 += a1;
  }
  if (lane == 0) { s_st[w][0] = M; s_st[w][1] = Lt; }
  __syncthreads();
  float Mall = fmaxf(fmaxf(s_st[0][0], s_st[1][0]), fmaxf(s_st[2][0], s_st[3][0]));
  const float sc = (M == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(M - Mall);
  *reinterpret_cast<float2*>(&s_o[w][2 * lane]) = make_float2(t0 * sc, t1 * sc);
  __syncthreads();
  if (w == 0) {
    float Lall = 0.0f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float mk = s_st[k][0];
      Lall += (mk == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mk - Mall) * s_st[k][1];
    }
    float x = 0.f, y = 0.f;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float2 o = *reinterpret_cast<const float2*>(&s_o[k][2 * lane]);
      x += o.x;
      y += o.y;
    }
    // inverse WHT: channel bit 0 in-lane, bits 1-6 across lanes
    {
      const float a = x, c = y;
      x = a + c;
      y = a - c;
    }
    x = bfly<1>(x, lane); y = bfly<1>(y, lane);
    x = bfly<2>(x, lane); y = bfly<2>(y, lane);
    x = bfly<4>(x, lane); y = bfly<4>(y, lane);
    x = bfly<8>(x, lane); y = bfly<8>(y, lane);
    x = bfly<16>(x, lane); y = bfly<16>(y, lane);
    x = bfly<32>(x, lane); y = bfly<32>(y, lane);
    const float inv = 1.0f / Lall;
    float* o = P.out + ((int64_t)b * P.n_q + hq) * D + 2 * lane;
    *reinterpret_cast<float2*>(o) = make_float2(x * wht_scale<D>() * inv, y * wht_scale<D>() * inv);
  }
}

template <int G, bool H, bool APP>
hipError_t launch_split_gha(const DecodeParams& P, int batch, hipStream_t stream) {
  dim3 grid(P.n_tsplit, P.n_kv, batch);
  switch (P.tps) {
    case 1: hipLaunchKernelGGL((decode_split_kernel<G, 1, H, APP>), grid, dim3(256), 0, stream, P); break;
    case 2: hipLaunchKernelGGL((decode_split_kernel<G, 2, H, APP>), grid, dim3(512), 0, stream, P); break;
    case 4: hipLaunchKernelGGL((decode_split_kernel<G, 4, H, APP>), grid, dim3(1024), 0, stream, P); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int G, bool H>
hipError_t launch_split_gh(const DecodeParams& P, int batch, hipStream_t stream) {
  return P.k_new ? launch_split_gha<G, H, true>(P, batch, stream) : launch_split_gha<G, H, false>(P, batch, stream);
}

template <int G>
hipError_t launch_split_g(const DecodeParams& P, int batch, hipStream_t stream) {
  return P.h16 ? launch_split_gh<G, true>(P, batch, stream) : launch_split_gh<G, false>(P, batch, stream);
}

}  // namespace

hipError_t launch_decode_fused(const DecodeParams& P, int batch, hipStream_t stream) {
  hipError_t e;
  switch (P.G) {
    case 1: e = launch_split_g<1>(P, batch, stream); break;
    case 2: e = launch_split_g<2>(P, batch, stream); break;
    case 4: e = launch_split_g<4>(P, batch, stream); break;
    case 8: e = launch_split_g<8>(P, batch, stream); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess) return e;
  // passes of 16 splits per wave while one pass of the four waves covers every
  // split, else 32 (fewer, longer passes)
  if (P.n_tsplit <= 64)
    hipLaunchKernelGGL(decode_combine_kernel<16>, dim3(P.n_q, batch), dim3(256), 0, stream, P);
  else
    hipLaunchKernelGGL(decode_combine_kernel<32>, dim3(P.n_q, batch), dim3(256), 0, stream, P);
  return hipGetLastError();
}

}  // namespace kvarn
