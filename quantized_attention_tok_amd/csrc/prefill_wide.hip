// prefill_wide.hip -- the compressed-tile part of chunked prefill at head_dim
// 256 on gfx950 matrix cores.
//
// Query position p of the chunk attends the tiles [0, T(p)) in compressed
// form and the raw tokens [128 T(p), p] (T(p) = max(0, floor((p + 1 - W) /
// 128)), the decode view at p).  This kernel computes, for every chunk row and
// query head, the streaming-softmax partial (m, l, o') of one tile split s:
// the tiles [tps s, tps s + tps) among those the row sees, in the rotated
// domain.  The decode combine then merges the tile splits, applies the inverse
// WHT once and joins the raw-window partials of the window kernel (PR #434
// commit list: chunked prefill with a single streaming softmax over compressed
// tiles + FP32 window and a deferred inverse WHT; issue #433 items 1 and 3: the
// Q.K score block of the compressed tiles on the matrix units, head_dim 256
// chunked prefill).
//
// Work split: a row group is 16 consecutive positions of one query head (one
// MFMA column block); a workgroup of 8 waves serves 8 row groups of one KV
// head, one per wave, each wave over all 128 tokens of every tile of its
// split.  Per tile the 8 waves first unpack the tile together into LDS
// operand tiles in the fp16 layout the MFMAs read (one buffer: 64 KB of key
// operands, 64 KB of value operands and the per-tile constants, so the tile
// is unpacked between two barriers and one workgroup fits a CU), then each
// wave computes, for its 16 rows r and each 64-token half of the tile,
//   S^T[t][r] = sum_c zK[t][c] q~[c][r] + b[r]   (fp16 MFMA over eight
//               32-channel steps; q~ = q' kscale as hi + lo parts, b =
//               sum_c q'_c kmin_c by a small MFMA too)
//   O^T[c][r] += sum_t zV[t][c] w_g[r][t]        (fp16 MFMA; w_g = p vscale_g
//               as hi + lo parts, g = c / 128 the value group of channel c)
// with the operand encodings of the head_dim-128 kernels: a 4-bit key code in
// bits 4-7 of an fp16 half (the subnormal 16 z), a 2-bit value code in bits
// 4-5 or 6-7.  The score layout of the first product (lane (g, r) holds tokens
// 16 b + 4 g .. + 3 of row r) is the B-operand layout of the second, and the
// second leaves row r in lane r, so the softmax state of a row never moves
// between lanes.
#include <float.h>

#include "kvarn_launch.h"
#include "kvarn_mfma.h"

namespace kvarn {
namespace {

using mfma::as_half8;
using mfma::floatx4;
using mfma::half8;
using mfma::pack_h2;
using mfma::pow2i;

typedef _Float16 h2v __attribute__((ext_vector_type(2)));
typedef __fp16 fp16x2 __attribute__((ext_vector_type(2)));   // cvt_pkrtz result

constexpr int DW = 256;                   // head_dim
constexpr int KS = DW / 32;               // 32-channel steps of the score product
constexpr int QB = DW / 64;               // 64-channel output blocks
constexpr int kThr = 512;                 // 8 waves
constexpr int kOpW = 128 * DW * 2;        // one tile's K (or V) operands: 64 KB
// per-tile constants: f32 alpha[t], vsf[g][t], vmin[g][t], vcu[c];
// f16 kh[c], kl[c], mh[c], ml[c]; int ek, ev, em
constexpr int cAlpha = 0, cVsf = 512, cVmin = 1536, cVcu = 2560;
constexpr int cKh = 3584, cKl = 4096, cMh = 4608, cMl = 5120, cExp = 5632;
constexpr int cBytes = 5648;
constexpr int kLdsK = 0, kLdsV = kOpW, kLdsC = 2 * kOpW;
constexpr int kLdsW = kLdsC + cBytes;
// lazy running maximum: raised only when a tile's maximum exceeds it by more
// than kTau (log2 units), so probabilities stay below 2^kTau
constexpr float kTau = 8.0f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ int exp_floor(float x, int lo, int hi) {
  const int e = (int)((__float_as_uint(x) >> 23) & 0xff) - 127;
  return e < lo ? lo : (e > hi ? hi : e);
}
// sums and maxima over the four 16-lane rows of a wave (lanes n, n + 16,
// n + 32, n + 48); a permlane swap of a value with itself gives each lane its
// own and its partner's value
__device__ __forceinline__ float rows_sum(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float rows_max(float v) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// WHT butterfly across lanes M = 16 or 32 apart: the lower lane gets a + b,
// the upper a - b
template <int M>
__device__ __forceinline__ float bfly_rows(float x, int lane) {
  const auto r = (M == 32) ? __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false)
                           : __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float sg = (lane & M) ? -1.0f : 1.0f;
  return fmaf(sg, __uint_as_float(r[1]), __uint_as_float(r[0]));
}
// maximum of a non-negative value over the wave (bit order = float order)
__device__ __forceinline__ float wave_max_nn(float v) {
  int k = __float_as_int(v);
  k = max(k, __builtin_amdgcn_update_dpp(0, k, 0x128, 0xF, 0xF, false));   // row_ror:8
  k = max(k, __builtin_amdgcn_update_dpp(0, k, 0x124, 0xF, 0xF, false));   // row_ror:4
  k = max(k, __builtin_amdgcn_update_dpp(0, k, 0x122, 0xF, 0xF, false));   // row_ror:2
  k = max(k, __builtin_amdgcn_update_dpp(0, k, 0x121, 0xF, 0xF, false));   // row_ror:1
  k = max(max(__builtin_amdgcn_readlane(k, 0), __builtin_amdgcn_readlane(k, 16)),
          max(__builtin_amdgcn_readlane(k, 32), __builtin_amdgcn_readlane(k, 48)));
  return __int_as_float(k);
}
__device__ __forceinline__ float max4(float4 x) { return fmaxf(fmaxf(x.x, x.y), fmaxf(x.z, x.w)); }
__device__ __forceinline__ int tiles_at(int64_t p, int window) {
  const int64_t ahead = p + 1 - window;
  return ahead > 0 ? (int)(ahead / kTile) : 0;
}
__device__ __forceinline__ h2v as_h2(uint32_t x) { return __builtin_bit_cast(h2v, x); }
__device__ __forceinline__ uint32_t as_u(h2v x) { return __builtin_bit_cast(uint32_t, x); }

// Operand tiles in LDS, 16-byte chunks.  K (A operand of the scores): chunk
// (k4, b, g, n) holds token 16 b + n, channels 32 k4 + 8 g .. + 7, at 16-byte
// index (k4 * 8 + b) * 64 + 16 g + (n ^ swk(b, n)).  V (A operand of the
// aggregate): chunk (s, q, g, n) holds channel 64 (q / 4) + 4 n + q % 4 of
// tokens 32 s + 16 (j / 4) + 4 g + j % 4 (K slot j = 0..7), at
// (s * 16 + q) * 64 + 16 g + (n ^ swv(q, n)).  The XOR swizzles keep the
// cooperative writes and the per-lane MFMA reads free of bank conflicts.
__device__ __forceinline__ int swk(int b, int n) { return ((b & 3) << 1) | ((n >> 3) & 1) | (((b >> 2) & 1) << 3); }
__device__ __forceinline__ int swv(int q, int n) { return ((q >> 2) & 1) ^ ((n >> 3) & 1); }

// What one thread loads of a record for the unpack: one dword of 8 K channel
// rows (channel step = wave), two bytes of 8 V token rows (token step wave % 4,
// channel half wave / 4), the four scales of the section whose tile maximum its
// wave needs, and the inputs of its share of the constants.  Constant work by
// wave: 0, 1: alpha (ek); 2, 3: kh, kl (ek); 4, 5: vsf, vmin (ev);
// 6, 7: vcu (ev), mh, ml (em).
struct TileRegsW {
  uint32_t k[8];
  uint32_t v[8];
  float4 xa, xb;
  float2 c0, c1;
};

template <bool H>
__device__ __forceinline__ void load_tile(const uint8_t* rec, int lane, int wv, TileRegsW& r) {
  using R = Rec<DW, H>;
  const int hi4 = lane >> 4, lo4 = lane & 15;
  {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(rec + (8 * (4 * wv + hi4)) * 64) + lo4;
#pragma unroll
    for (int e = 0; e < 8; ++e) r.k[e] = src[16 * e];
  }
  {
    const uint8_t* vcode = rec + R::vcode + 32 * (wv >> 2) + 2 * lo4;
    const int s = wv & 3;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        r.v[4 * h + i] = *reinterpret_cast<const uint16_t*>(vcode + (32 * s + 16 * h + 4 * hi4 + i) * (DW / 4));
  }
  const int role = wv >> 1;
  const int i2 = 2 * (64 * (wv & 1) + lane);
  r.xa = sc_ld4<H>(rec + (role < 2 ? R::kscale : R::vscale), 4 * lane);
  r.xb = sc_ld4<H>(rec + R::kmin, 4 * lane);
  if (role == 0) r.c0 = make_float2(sc_ld<H>(rec + R::ktok, 64 * (wv & 1) + lane), 0.0f);
  else r.c0 = sc_ld2<H>(rec + (role == 1 ? R::kscale : role == 2 ? R::vscale : R::vchan), i2);
  r.c1 = sc_ld2<H>(rec + (role == 2 ? R::vmin : R::kmin), i2);
}

// Unpack one tile (from TileRegsW) into the K / V operand buffers and the
// constant area:
//   alpha[t]   = scale log2(e) ktok[t] 2^(7 + ek)        (score factor)
//   vsf[g][t]  = vscale[t][g] 2^(13 - tau - ev)          (w = p vsf < 2^14)
//   vmin[g][t] = vmin[t][g]
//   vcu[c]     = vchan[c] 2^(24 - shift(c)) / 2^(13 - tau - ev)
//   kh + kl    = kscale[c] 2^(13 - ek)                   (fp16 hi, lo)
//   mh + ml    = kmin[c] 2^(13 - em)                     (fp16 hi, lo)
// with ek, ev, em the floor(log2) of the tile's largest kscale, vscale, |kmin|
// (stored for the compute), shift 4 for even channels and 6 for odd ones (the
// crumb's bit position).
__device__ __forceinline__ void unpack_tile(const TileRegsW& r, uint8_t* kdst, uint8_t* vdst, uint8_t* buf, int lane,
                                            int wv, float scale_log2) {
  const int hi4 = lane >> 4, lo4 = lane & 15;
  {   // keys: channel step wv, channel group hi4, tokens 8 lo4 .. + 7
    const int b0 = lo4 >> 1, n3 = lo4 & 1;   // token 8 lo4 + tt: block lo4 / 2, n = 8 n3 + tt
    uint4* dst = reinterpret_cast<uint4*>(kdst) + (wv * 8 + b0) * 64 + 16 * hi4;
    const int sw = swk(b0, 8 * n3);
    uint32_t lo[8], hi[8];   // low / high nibbles of every byte, in bits 4-7
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      lo[e] = (r.k[e] << 4) & 0xF0F0F0F0u;
      hi[e] = r.k[e] & 0xF0F0F0F0u;
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t sel = (uint32_t)j | (0x0Cu << 8) | ((uint32_t)(4 + j) << 16) | (0x0Cu << 24);
      uint32_t ev4[4], od4[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        ev4[k] = __builtin_amdgcn_perm(lo[2 * k + 1], lo[2 * k], sel);
        od4[k] = __builtin_amdgcn_perm(hi[2 * k + 1], hi[2 * k], sel);
      }
      const int n0 = 8 * n3 + 2 * j;
      dst[n0 ^ sw] = make_uint4(ev4[0], ev4[1], ev4[2], ev4[3]);
      dst[(n0 + 1) ^ sw] = make_uint4(od4[0], od4[1], od4[2], od4[3]);
    }
  }
  {   // values: token step wv % 4, token group hi4, channels 128 (wv / 4) + 8 lo4 .. + 7
    uint4* dst = reinterpret_cast<uint4*>(vdst) + ((wv & 3) * 16) * 64 + 16 * hi4;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const uint32_t sel = (uint32_t)bb | (0x0Cu << 8) | ((uint32_t)(4 + bb) << 16) | (0x0Cu << 24);
      uint32_t x[4];   // pair p: tokens of K slots 2p, 2p + 1
#pragma unroll
      for (int pq = 0; pq < 4; ++pq) x[pq] = __builtin_amdgcn_perm(r.v[2 * pq + 1], r.v[2 * pq], sel);
      const int n = (2 * lo4 + bb) & 15;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const uint32_t mask = (kc & 1) ? 0x00C000C0u : 0x00300030u;
        uint32_t d[4];
#pragma unroll
        for (int pq = 0; pq < 4; ++pq) d[pq] = ((kc < 2) ? (x[pq] << 4) : x[pq]) & mask;
        const int q8 = 8 * (wv >> 2) + 4 * (lo4 >> 3) + kc;
        dst[q8 * 64 + (n ^ swv(q8, n))] = make_uint4(d[0], d[1], d[2], d[3]);
      }
    }
  }
  // constants: each wave needs one or two tile maxima
  const int role = wv >> 1;
  const int t = 64 * (wv & 1) + lane;      // token of role 0
  const int i2 = 2 * t;                    // element pair of roles 1-3
  const int ea = exp_floor(wave_max_nn(max4(r.xa)), role < 2 ? -114 : -100, role < 2 ? 120 : 100);
  int* ex = reinterpret_cast<int*>(buf + cExp);
  if (role == 0) {
    reinterpret_cast<float*>(buf + cAlpha)[t] = scale_log2 * r.c0.x * pow2i(7 + ea);
    if (wv == 0 && lane == 0) ex[0] = ea;
  } else if (role == 1) {
    const float x0 = r.c0.x * pow2i(13 - ea), x1 = r.c0.y * pow2i(13 - ea);
    const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
    reinterpret_cast<uint32_t*>(buf + cKh)[t] = pack_h2(h0, h1);
    reinterpret_cast<uint32_t*>(buf + cKl)[t] = pack_h2((_Float16)(x0 - (float)h0), (_Float16)(x1 - (float)h1));
  } else if (role == 2) {
    // elements i2, i2 + 1 are (token t', group 0) and (t', group 1), t' = i2 / 2
    const float f = pow2i(13 - (int)kTau - ea);
    float* vsf = reinterpret_cast<float*>(buf + cVsf);
    float* vmn = reinterpret_cast<float*>(buf + cVmin);
    vsf[t] = r.c0.x * f;
    vsf[128 + t] = r.c0.y * f;
    vmn[t] = r.c1.x;
    vmn[128 + t] = r.c1.y;
    if (wv == 4 && lane == 0) ex[1] = ea;
  } else {
    const int uexp = 13 - (int)kTau - ea;
    reinterpret_cast<float2*>(buf + cVcu)[t] = make_float2(r.c0.x * pow2i(24 - 4 - uexp), r.c0.y * pow2i(24 - 6 - uexp));
    const int em = exp_floor(wave_max_nn(fmaxf(fmaxf(fabsf(r.xb.x), fabsf(r.xb.y)), fmaxf(fabsf(r.xb.z), fabsf(r.xb.w)))),
                             -100, 100);
    const float x0 = r.c1.x * pow2i(13 - em), x1 = r.c1.y * pow2i(13 - em);
    const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
    reinterpret_cast<uint32_t*>(buf + cMh)[t] = pack_h2(h0, h1);
    reinterpret_cast<uint32_t*>(buf + cMl)[t] = pack_h2((_Float16)(x0 - (float)h0), (_Float16)(x1 - (float)h1));
    if (wv == 6 && lane == 0) ex[2] = em;
  }
}

// Grid: (ceil(row groups / 8), KV head, tile split).  Chunk row b, query head
// h, tile split s: partial at part + ((b n_q + h) (n_tsplit + n_wsplit) + s)
// (D + 4): o' (rotated domain, unnormalised), then m (natural-log units) and
// l.  A row writes the splits whose tiles it sees (the combine reads no other).
template <bool H>
__global__ void __launch_bounds__(kThr) prefill_tiles256_kernel(DecodeParams P, int chunk) {
  using R = Rec<DW, H>;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int n = lane & 15, g = lane >> 4;
  const int kvh = blockIdx.y;
  const int s = blockIdx.z;
  const int G = P.G;
  const int n_blk = ((chunk + 15) / 16) * G;   // (position group, head) column blocks
  const int blk_first = blockIdx.x * 8;
  const int blk_last = min(blk_first + 7, n_blk - 1);
  const int blk = blk_first + wv;
  const bool active = blk < n_blk;
  const int pg = (active ? blk : blk_last) / G;
  const int hq = kvh * G + (active ? blk : blk_last) % G;
  const int r0 = 16 * pg;                                   // chunk row of column 0
  const int64_t prow = P.pos0 + r0 + n;                     // position of this lane's row
  const bool row_ok = active && (r0 + n < chunk);
  const int T_row = row_ok ? tiles_at(prow, P.window) : 0;
  const int T_wave = active ? tiles_at(P.pos0 + min(r0 + 15, chunk - 1), P.window) : 0;
  const int ja = P.tps * s;
  const int jend = min(ja + P.tps, tiles_at(P.pos0 + min(16 * (blk_last / G) + 15, chunk - 1), P.window));
  if (ja >= jend) return;   // no row of the workgroup sees a tile of this split

  __shared__ __attribute__((aligned(16))) uint8_t s_lds[kLdsW];
  const float scale_log2 = P.scale * mfma::kLog2e;
  const uint8_t* recs = P.records + (int64_t)kvh * R::bytes;
  const int64_t rstride = (int64_t)P.n_kv * R::bytes;
  const uint8_t* cst = s_lds + kLdsC;
  const uint4* kop = reinterpret_cast<const uint4*>(s_lds + kLdsK);
  const uint4* vop = reinterpret_cast<const uint4*>(s_lds + kLdsV);

  TileRegsW tr;
  load_tile<H>(recs + (int64_t)ja * rstride, lane, wv, tr);

  // ---- this lane's rotated query: row n, channels 32 k4 + 8 g .. + 7 ----
  float qv[KS][8];
  {
    const bool rot = P.q_rot == nullptr;
    const float* qp = (rot ? P.q : P.q_rot) + ((int64_t)(row_ok ? r0 + n : 0) * P.n_q + hq) * DW + 8 * g;
#pragma unroll
    for (int k4 = 0; k4 < KS; ++k4) {
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
      if (row_ok) {
        a = *reinterpret_cast<const float4*>(qp + 32 * k4);
        b = *reinterpret_cast<const float4*>(qp + 32 * k4 + 4);
      }
      qv[k4][0] = a.x; qv[k4][1] = a.y; qv[k4][2] = a.z; qv[k4][3] = a.w;
      qv[k4][4] = b.x; qv[k4][5] = b.y; qv[k4][6] = b.z; qv[k4][7] = b.w;
    }
    if (rot) {   // q' = H q: butterfly strides in ascending order, then one scale (the
                 // rounding of the separate rotation and of the oracle's fp32 transform)
#pragma unroll
      for (int k4 = 0; k4 < KS; ++k4)
#pragma unroll
        for (int hb = 1; hb < 8; hb <<= 1)   // strides 1, 2, 4: channel bits 0-2
#pragma unroll
          for (int jj = 0; jj < 8; ++jj)
            if (!(jj & hb)) {
              const float a = qv[k4][jj], b = qv[k4][jj | hb];
              qv[k4][jj] = a + b;
              qv[k4][jj | hb] = a - b;
            }
#pragma unroll
      for (int k4 = 0; k4 < KS; ++k4)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj)       // strides 8, 16: channel bits 3, 4 across the 16-lane rows
          qv[k4][jj] = bfly_rows<32>(bfly_rows<16>(qv[k4][jj], lane), lane);
#pragma unroll
      for (int kb = 1; kb < KS; kb <<= 1)    // strides 32, 64, 128: channel bits 5-7
#pragma unroll
        for (int k4 = 0; k4 < KS; ++k4)
          if (!(k4 & kb)) {
#pragma unroll
            for (int jj = 0; jj < 8; ++jj) {
              const float a = qv[k4][jj], b = qv[k4 | kb][jj];
              qv[k4][jj] = a + b;
              qv[k4 | kb][jj] = a - b;
            }
          }
#pragma unroll
      for (int k4 = 0; k4 < KS; ++k4)
#pragma unroll
        for (int jj = 0; jj < 8; ++jj) qv[k4][jj] *= wht_scale<DW>();
    }
  }
  // q' of row n scaled into (-1, 1) by 2^-eq, as fp16 hi + lo pairs
  float qmax = 0.0f;
#pragma unroll
  for (int k4 = 0; k4 < KS; ++k4)
#pragma unroll
    for (int j = 0; j < 8; ++j) qmax = fmaxf(qmax, fabsf(qv[k4][j]));
  const int eq = exp_floor(rows_max(qmax), -100, 99) + 1;
  const float beta = pow2i(eq);
  uint32_t qh[KS][4], ql[KS][4];   // [k4][pair]: channels 32 k4 + 8 g + 2 i, + 1
  {
    const float inv = pow2i(-eq);
#pragma unroll
    for (int k4 = 0; k4 < KS; ++k4)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = qv[k4][2 * i] * inv, b = qv[k4][2 * i + 1] * inv;
        const _Float16 ha = (_Float16)a, hb = (_Float16)b;
        qh[k4][i] = pack_h2(ha, hb);
        ql[k4][i] = pack_h2((_Float16)(a - (float)ha), (_Float16)(b - (float)hb));
      }
  }
  // operand read offsets (16-byte units) of lane (g, n): K blocks 4 hx + bb,
  // V blocks by the parity of the 64-channel block
  int offk[2][4], offv[2];
#pragma unroll
  for (int hx = 0; hx < 2; ++hx)
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) offk[hx][bb] = 16 * g + (n ^ swk(4 * hx + bb, n));
#pragma unroll
  for (int h = 0; h < 2; ++h) offv[h] = 16 * g + (n ^ swv(4 * h, n));

  float m_run = -INFINITY, l_run = 0.0f;   // softmax state of row n (log2 domain)
  floatx4 O[QB][4];                         // row n; channel 64 qb + 16 g + 4 i + kk in O[qb][kk][i]
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) O[qb][kk] = (floatx4){0.f, 0.f, 0.f, 0.f};

  for (int j = ja; j < jend; ++j) {
    if (j > ja) __syncthreads();   // every wave is done with tile j - 1's operands
    unpack_tile(tr, s_lds + kLdsK, s_lds + kLdsV, s_lds + kLdsC, lane, wv, scale_log2);
    if (j + 1 < jend) load_tile<H>(recs + (int64_t)(j + 1) * rstride, lane, wv, tr);
    __syncthreads();               // tile j is in place
    if (j >= T_wave) continue;
    const int* ex = reinterpret_cast<const int*>(cst + cExp);
    const int ek = __builtin_amdgcn_readfirstlane(ex[0]);
    const int ev = __builtin_amdgcn_readfirstlane(ex[1]);
    const int em = __builtin_amdgcn_readfirstlane(ex[2]);
    // bias b = sum_c q'_c kmin_c: every row of A is kmin 2^(13 - em) (hi, lo),
    // B is q' 2^-eq (hi, lo); rescaled to the score accumulator's 2^(-7 - ek - eq)
    __builtin_amdgcn_s_setprio(1);
    floatx4 bacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k4 = 0; k4 < KS; ++k4) {
      const uint4 mh4 = *reinterpret_cast<const uint4*>(cst + cMh + 2 * (32 * k4 + 8 * g));
      const uint4 ml4 = *reinterpret_cast<const uint4*>(cst + cMl + 2 * (32 * k4 + 8 * g));
      const half8 Amh = as_half8(mh4.x, mh4.y, mh4.z, mh4.w);
      const half8 Aml = as_half8(ml4.x, ml4.y, ml4.z, ml4.w);
      const half8 Qh = as_half8(qh[k4][0], qh[k4][1], qh[k4][2], qh[k4][3]);
      const half8 Ql = as_half8(ql[k4][0], ql[k4][1], ql[k4][2], ql[k4][3]);
      bacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Amh, Qh, bacc, 0, 0, 0);
      bacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Amh, Ql, bacc, 0, 0, 0);
      bacc = __builtin_amdgcn_mfma_f32_16x16x32_f16(Aml, Qh, bacc, 0, 0, 0);
    }
    const int bexp = em - 20 - ek;
    const float bsc = pow2i(bexp < -126 ? -126 : (bexp > 127 ? 127 : bexp));
    const floatx4 acc0 = {bacc[0] * bsc, bacc[1] * bsc, bacc[2] * bsc, bacc[3] * bsc};
    // scores of both token halves, channel step k4 outermost: the q~ B operands
    // of step k4, q~ = q' kscale 2^(13 - ek - eq) = (qh + ql)(kh + kl) as hi + lo
    // by packed fp16 arithmetic (hi rounded, lo = exact product rest + cross
    // terms), formed just before its matrix ops; each block sums its steps in
    // k4 order, hi before lo
    floatx4 acc[2][4];
#pragma unroll
    for (int hx = 0; hx < 2; ++hx)
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) acc[hx][bb] = acc0;
#pragma unroll
    for (int k4 = 0; k4 < KS; ++k4) {
      const uint4 kh4 = *reinterpret_cast<const uint4*>(cst + cKh + 2 * (32 * k4 + 8 * g));
      const uint4 kl4 = *reinterpret_cast<const uint4*>(cst + cKl + 2 * (32 * k4 + 8 * g));
      const uint32_t khv[4] = {kh4.x, kh4.y, kh4.z, kh4.w};
      const uint32_t klv[4] = {kl4.x, kl4.y, kl4.z, kl4.w};
      uint32_t bh[4], bl[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const h2v a = as_h2(qh[k4][i]), a2 = as_h2(ql[k4][i]), k = as_h2(khv[i]), k2 = as_h2(klv[i]);
        const h2v hi = a * k;
        h2v lo = __builtin_elementwise_fma(a, k, -hi);
        lo = __builtin_elementwise_fma(a, k2, lo);
        lo = __builtin_elementwise_fma(a2, k, lo);
        bh[i] = as_u(hi);
        bl[i] = as_u(lo);
      }
      const half8 Bh = as_half8(bh[0], bh[1], bh[2], bh[3]);
      const half8 Bl = as_half8(bl[0], bl[1], bl[2], bl[3]);
#pragma unroll
      for (int hx = 0; hx < 2; ++hx)
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const uint4 a = kop[(k4 * 8 + 4 * hx + bb) * 64 + offk[hx][bb]];
          const half8 A = as_half8(a.x, a.y, a.z, a.w);
          acc[hx][bb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bh, acc[hx][bb], 0, 0, 0);
          acc[hx][bb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bl, acc[hx][bb], 0, 0, 0);
        }
    }
    // y = alpha_t acc / beta (log2 domain): token 16 b + 4 g + i of row n; one
    // running-maximum update for the tile, then per half the probabilities and
    // the value aggregate
    const float* alp = reinterpret_cast<const float*>(cst + cAlpha);
    float y[2][4][4];
    float ymax = -INFINITY;
#pragma unroll
    for (int hx = 0; hx < 2; ++hx)
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const float4 al = *reinterpret_cast<const float4*>(alp + 16 * (4 * hx + bb) + 4 * g);
        y[hx][bb][0] = acc[hx][bb][0] * al.x;
        y[hx][bb][1] = acc[hx][bb][1] * al.y;
        y[hx][bb][2] = acc[hx][bb][2] * al.z;
        y[hx][bb][3] = acc[hx][bb][3] * al.w;
        ymax = fmaxf(fmaxf(ymax, y[hx][bb][0]), y[hx][bb][1]);
        ymax = fmaxf(fmaxf(ymax, y[hx][bb][2]), y[hx][bb][3]);
      }
    __builtin_amdgcn_s_setprio(0);
    // lazy running maximum: raised only when the tile exceeds it by > tau
    const bool vis = j < T_row;
    const float tmax = rows_max(ymax) * beta;
    const bool raise = vis && !(tmax <= m_run + kTau);
    const float m_new = raise ? tmax : m_run;
    const float alpha = raise ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.0f;   // 0 from -inf
    m_run = m_new;
    const float negm = vis ? -m_run : -INFINITY;
    l_run *= alpha;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int i = 0; i < 4; ++i) O[qb][kk][i] *= alpha;
    }
    const float* vsf = reinterpret_cast<const float*>(cst + cVsf);
    const float* vmn = reinterpret_cast<const float*>(cst + cVmin);
    const float* vcu = reinterpret_cast<const float*>(cst + cVcu);
#pragma unroll
    for (int hx = 0; hx < 2; ++hx) {
      // probabilities p (<= 2^tau) and their sum
      float p[4][4];
      float psum = 0.0f;
#pragma unroll
      for (int bb = 0; bb < 4; ++bb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          p[bb][i] = __builtin_amdgcn_exp2f(fmaf(beta, y[hx][bb][i], negm));
          psum += p[bb][i];
        }
      l_run += rows_sum(psum);
      // per value group: u = sum_t p vmin_g, w = p vsf_g as hi / lo B operands,
      // and the aggregate of the group's two 64-channel blocks
#pragma unroll
      for (int gv = 0; gv < 2; ++gv) {
        float upart = 0.0f;
        uint32_t wh[4][2], wl[4][2];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const int b = 4 * hx + bb;
          const float4 va = *reinterpret_cast<const float4*>(vsf + 128 * gv + 16 * b + 4 * g);
          const float4 ma = *reinterpret_cast<const float4*>(vmn + 128 * gv + 16 * b + 4 * g);
          const float vs4[4] = {va.x, va.y, va.z, va.w};
          const float vm4[4] = {ma.x, ma.y, ma.z, ma.w};
          float w4[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            upart = fmaf(p[bb][i], vm4[i], upart);
            w4[i] = p[bb][i] * vs4[i];
          }
#pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
            const fp16x2 h = __builtin_amdgcn_cvt_pkrtz(w4[2 * pr], w4[2 * pr + 1]);
            const fp16x2 l = __builtin_amdgcn_cvt_pkrtz(w4[2 * pr] - (float)h.x, w4[2 * pr + 1] - (float)h.y);
            wh[bb][pr] = __builtin_bit_cast(uint32_t, h);
            wl[bb][pr] = __builtin_bit_cast(uint32_t, l);
          }
        }
        const float u = rows_sum(upart);
        // O'^T[c][n] += vcu_c z_c, z_c starting at u fv 2^-(24 - shift(c)) so that
        // vcu_c z_c = vchan_c (sum_t p_t vscale_t zV_tc + sum_t p_t vmin_t)
        const float ufv = u * pow2i(13 - (int)kTau - ev);
        const float zi0 = ufv * pow2i(-20), zi1 = ufv * pow2i(-18);
        half8 Wh[2], Wl[2];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          Wh[tt] = as_half8(wh[2 * tt][0], wh[2 * tt][1], wh[2 * tt + 1][0], wh[2 * tt + 1][1]);
          Wl[tt] = as_half8(wl[2 * tt][0], wl[2 * tt][1], wl[2 * tt + 1][0], wl[2 * tt + 1][1]);
        }
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
          const int qb = 2 * gv + qq;
          float4 vc[4];   // channels 64 qb + 16 g + 4 i .. + 3
#pragma unroll
          for (int i = 0; i < 4; ++i) vc[i] = *reinterpret_cast<const float4*>(vcu + 64 * qb + 16 * g + 4 * i);
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const int q8 = 4 * qb + kk;
            const float zi = (kk & 1) ? zi1 : zi0;
            floatx4 z = {zi, zi, zi, zi};
#pragma unroll
            for (int tt = 0; tt < 2; ++tt) {
              const uint4 av = vop[((2 * hx + tt) * 16 + q8) * 64 + offv[qb & 1]];
              const half8 Av = as_half8(av.x, av.y, av.z, av.w);
              z = __builtin_amdgcn_mfma_f32_16x16x32_f16(Av, Wh[tt], z, 0, 0, 0);
              z = __builtin_amdgcn_mfma_f32_16x16x32_f16(Av, Wl[tt], z, 0, 0, 0);
            }
            const float vk[4] = {kk == 0 ? vc[0].x : kk == 1 ? vc[0].y : kk == 2 ? vc[0].z : vc[0].w,
                                 kk == 0 ? vc[1].x : kk == 1 ? vc[1].y : kk == 2 ? vc[1].z : vc[1].w,
                                 kk == 0 ? vc[2].x : kk == 1 ? vc[2].y : kk == 2 ? vc[2].z : vc[2].w,
                                 kk == 0 ? vc[3].x : kk == 1 ? vc[3].y : kk == 2 ? vc[3].z : vc[3].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) O[qb][kk][i] = fmaf(vk[i], z[i], O[qb][kk][i]);
          }
        }
        __builtin_amdgcn_s_setprio(0);
      }
    }
  }

  // ---- the partial of each row that sees a tile of this split ----
  if (!row_ok || T_row <= ja) return;
  const int nsp = P.n_tsplit + P.n_wsplit;
  float* o = P.part + (((int64_t)(r0 + n) * P.n_q + hq) * nsp + s) * (DW + 4);
  if (g == 0) *reinterpret_cast<float2*>(o + DW) = make_float2(m_run * kLn2, l_run);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<float4*>(o + 64 * qb + 16 * g + 4 * i) =
          make_float4(O[qb][0][i], O[qb][1][i], O[qb][2][i], O[qb][3][i]);
}

}  // namespace

hipError_t launch_prefill_tiles256(const DecodeParams& P, int chunk, hipStream_t stream) {
  if (P.n_tsplit < 1) return hipSuccess;
  const int n_blk = ((chunk + 15) / 16) * P.G;
  const dim3 grid((n_blk + 7) / 8, P.n_kv, P.n_tsplit);
  if (P.h16)
    hipLaunchKernelGGL(prefill_tiles256_kernel<true>, grid, dim3(kThr), 0, stream, P, chunk);
  else
    hipLaunchKernelGGL(prefill_tiles256_kernel<false>, grid, dim3(kThr), 0, stream, P, chunk);
  return hipGetLastError();
}

}  // namespace kvarn
