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
// Work split: a row group is 16 consecutive positions of one query head (one
// MFMA column block); a workgroup of 8 waves serves row groups of one KV head
// in one of two layouts:
//   - split layout (prefill_split_kernel, the chunked prefill with a
//     workspace): eight row groups, one per wave, each wave over all 128
//     tokens of every tile (the tile's q~ operands and bias computed once; the
//     scores of both 64-token halves, one running-maximum update, then per
//     half the probabilities and the value aggregate, so that the vector work
//     of one half meets the matrix work of the other) and over both raw
//     16-token blocks of every staging step.  The workgroup's tiles and raw tokens are
//     cut into S equal shares (blockIdx.z), so that the 128-row-head
//     workgroups fill the chip; each share's raw-domain partial goes to the
//     workspace and a combine launch merges them;
//   - half layout (prefill_mfma_kernel without a workspace, and multi-query
//     verify): four row groups, wave (r, h) over tokens 64 h .. 64 h + 63 of
//     every tile and the raw blocks of parity h; the two halves of a row group
//     merge at the end.
// Each wave keeps a streaming softmax of its own.  Two waves per SIMD (w and
// w + 4) let the matrix work of one run under the vector work of the other.
//
// Per compressed tile the 8 waves first unpack the tile once, together, into
// LDS operand tiles in the fp16 layout the MFMAs read (one 16-byte read per
// operand) plus a few per-tile constants; the split layout thus serves 128
// row-heads per unpack, the half layout 64.  Each wave computes, for its 16
// rows r and each 64-token half t of its share,
//   S^T[t][r] = sum_c zK[t][c] q~[c][r] + b[r]     (fp16 MFMA; q~ = q' kscale
//               as hi + lo parts, b = sum_c q'_c kmin_c by a small MFMA too)
//   O^T[c][r] += sum_t zV[t][c] w[r][t]            (fp16 MFMA; w = p vscale
//               as hi + lo parts)
// The score layout of the first product (lane (g, r) holds tokens
// 16 b + 4 g .. + 3 of row r) is the B-operand layout of the second once the
// V operands list their tokens in that order, and the second leaves row r in
// lane r again, so the softmax state of a row never moves between lanes.
// After the last tile each row's O' is rotated back with the WHT butterflies
// (in-lane, and across the four 16-lane rows with the gfx950 permlane swaps),
// then the raw tokens are added with fp32 MFMAs (v_mfma_f32_16x16x4_f32):
// scores from the raw query and raw keys, and the aggregate of raw values
// straight into the same accumulator.
#include <float.h>

#include "kvarn_launch.h"
#include "kvarn_mfma.h"

namespace kvarn {
namespace {

using namespace mfma;

typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef __fp16 fp16x2 __attribute__((ext_vector_type(2)));   // cvt_pkrtz result

constexpr int kRows = 16;                          // query rows per wave
constexpr int kThreads = 512;                      // 8 waves
constexpr int kRawTok = 32;                        // raw tokens staged per step
constexpr int kRawRow = D + 4;                     // padded LDS row of raw K / V (floats)
constexpr int kOpBytes = 32768;                    // one tile's K or V operands (fp16)
// LDS: K operands of buffers 0 and 1, V operands of buffers 0 and 1, then the
// two constant areas, so that every read of a tile is a lane offset plus an
// immediate below 64 KB.  Constants: f32 alpha, vsf, vmin, vcu; f16 kh, kl, mh, ml
constexpr int kCAlpha = 0, kCVsf = 512, kCVmin = 1024, kCVcu = 1536;
constexpr int kCKh = 2048, kCKl = 2304, kCMh = 2560, kCMl = 2816;
constexpr int kCExp = 3072;                        // int ek, ev, em
constexpr int kConstBytes = 3088;
constexpr int kLdsK = 0, kLdsV = 2 * kOpBytes, kLdsC = 4 * kOpBytes;
constexpr int kLdsBytes = kLdsC + 2 * kConstBytes;
constexpr int kLdsRaw = 2 * kRawTok * kRawRow * 4; // raw K and V rows (over the tiles)
constexpr int kMergeO = 4 * 8 * 64 * 16;           // merge: O of the h = 1 waves, then (m, l)
static_assert(kLdsRaw <= kLdsBytes && kMergeO + 4 * 64 * 8 <= kLdsBytes, "staging fits");
// Lazy softmax rescaling: a row's running maximum is raised only when a tile's
// maximum exceeds it by more than kTau (log2 units), so probabilities stay
// below 2^kTau and the output is rescaled only on those tiles.
constexpr float kTau = 8.0f;

// floor(log2 x) of a non-negative float, clamped to [lo, hi] (zero -> lo)
__device__ __forceinline__ int exp_floor(float x, int lo, int hi) {
  const int e = (int)((__float_as_uint(x) >> 23) & 0xff) - 127;
  return e < lo ? lo : (e > hi ? hi : e);
}

// Sums and maxima over the four 16-lane rows of a wave (lanes n, n + 16,
// n + 32, n + 48); every lane gets the result.  A permlane swap of a value
// with itself gives each lane its own and its partner's value.
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
// WHT butterfly across lanes 16 (M = 16) or 32 (M = 32) apart: the lower lane
// gets a + b, the upper a - b.
template <int M>
__device__ __forceinline__ float bfly_rows(float x, int lane) {
  const auto r = (M == 32) ? __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false)
                           : __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float sg = (lane & M) ? -1.0f : 1.0f;
  return fmaf(sg, __uint_as_float(r[1]), __uint_as_float(r[0]));
}
// Maximum of a non-negative value over the wave (bit order = float order).
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

// Operand tiles in LDS, 16-byte chunks, one tile (128 tokens x 128 channels)
// each.  K (A operand of the scores): chunk (k4, b, g, n) holds token
// 16 b + n, channels 32 k4 + 8 g .. + 7, at 16-byte index
//   (k4 * 8 + b) * 64 + 16 g + (n ^ swk(b, n)).
// V (A operand of the aggregate): chunk (s, q, g, n) holds channel
// 64 (q / 4) + 4 n + q % 4 of tokens 32 s + 16 (j / 4) + 4 g + j % 4 (K slot
// j = 0..7), at (s * 8 + q) * 64 + 16 g + (n ^ swv(q, n)).  A 4-bit code sits
// in bits 4-7 of its fp16 half, a 2-bit code in bits 4-5 (crumbs 0, 2 of a
// byte) or 6-7 (crumbs 1, 3).  The XOR swizzles keep both the cooperative
// writes and the per-lane MFMA reads free of LDS bank conflicts (each group of
// 16 lanes touches 16 distinct 16-byte bank groups).
__device__ __forceinline__ int swk(int b, int n) { return ((b & 3) << 1) | ((n >> 3) & 1) | (((b >> 2) & 1) << 3); }
__device__ __forceinline__ int swv(int q, int n) { return ((q >> 2) & 1) ^ ((n >> 3) & 1); }

// What one thread loads of a record for the unpack: waves 0-3 one dword of
// 8 K channel rows, waves 4-7 two bytes of 8 V token rows; every lane the
// pair(s) of the scale array(s) whose tile maximum its wave needs and the
// input(s) of its share of the constants.  Constant work by wave:
//   0, 1: alpha (needs ek)         2, 3: kh, kl (ek)
//   4, 5: vsf, vmin (ev)           6, 7: vcu (ev), mh, ml (em)
struct TileRegs {
  uint32_t c[8];
  float2 xa, xb;
  float c0, c1, c2;
};

template <bool H>
__device__ __forceinline__ void load_tile(const uint8_t* rec, int lane, int wv, TileRegs& r) {
  using R = Rec<D, H>;
  const int hi4 = lane >> 4, lo4 = lane & 15;
  if (wv < 4) {
    const uint32_t* src = reinterpret_cast<const uint32_t*>(rec + (8 * (4 * wv + hi4)) * 64) + lo4;
#pragma unroll
    for (int e = 0; e < 8; ++e) r.c[e] = src[16 * e];
  } else {
    const uint8_t* vcode = rec + R::vcode;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        r.c[4 * h + i] = *reinterpret_cast<const uint16_t*>(vcode + (32 * (wv - 4) + 16 * h + 4 * hi4 + i) * (D / 4) + 2 * lo4);
  }
  const int idx = 64 * (wv & 1) + lane;
  const int role = wv >> 1;
  r.xa = sc_ld2<H>(rec + (role < 2 ? R::kscale : R::vscale), 2 * lane);
  r.xb = sc_ld2<H>(rec + R::kmin, 2 * lane);
  r.c0 = sc_ld<H>(rec + (role == 0 ? R::ktok : role == 1 ? R::kscale : role == 2 ? R::vscale : R::vchan), idx);
  r.c1 = sc_ld<H>(rec + (role == 2 ? R::vmin : R::kmin), idx);
  r.c2 = 0.0f;
}

// Unpack one tile (from TileRegs) into K / V operand buffers and a constant area:
//   alpha[t] = scale log2(e) ktok[t] 2^(7 + ek)        (score factor)
//   vsf[t]   = vscale[t] 2^(13 - tau - ev)             (w = p vsf < 2^14)
//   vmin[t]  = vmin[t]
//   vcu[c]   = vchan[c] 2^(24 - shift(c)) / 2^(13 - tau - ev)
//   kh + kl  = kscale[c] 2^(13 - ek)                   (fp16 hi, lo)
//   mh + ml  = kmin[c] 2^(13 - em)                     (fp16 hi, lo)
// with ek, ev, em the floor(log2) of the tile's largest kscale, vscale, |kmin|
// (stored for the compute), shift 4 for even channels and 6 for odd ones (the
// crumb's bit position).  Waves 0-3 unpack K channel groups 4 w + lane/16,
// tokens 8 (lane % 16) .. + 7; waves 4-7 V token step w - 4, token group
// lane/16, channels 8 (lane % 16) .. + 7.
__device__ __forceinline__ void unpack_tile(const TileRegs& r, uint8_t* kdst, uint8_t* vdst, uint8_t* buf,
                                            int lane, int wv, float scale_log2) {
  const int hi4 = lane >> 4, lo4 = lane & 15;
  if (wv < 4) {
    const int b0 = lo4 >> 1, n3 = lo4 & 1;   // token 8 lo4 + tt: block lo4 / 2, n = 8 n3 + tt
    uint4* dst = reinterpret_cast<uint4*>(kdst) + (wv * 8 + b0) * 64 + 16 * hi4;
    const int sw = swk(b0, 8 * n3);
    uint32_t lo[8], hi[8];   // low / high nibbles of every byte, in bits 4-7
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      lo[e] = (r.c[e] << 4) & 0xF0F0F0F0u;
      hi[e] = r.c[e] & 0xF0F0F0F0u;
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
  } else {
    uint4* dst = reinterpret_cast<uint4*>(vdst) + ((wv - 4) * 8) * 64 + 16 * hi4;
#pragma unroll
    for (int bb = 0; bb < 2; ++bb) {
      const uint32_t sel = (uint32_t)bb | (0x0Cu << 8) | ((uint32_t)(4 + bb) << 16) | (0x0Cu << 24);
      uint32_t x[4];   // pair p: tokens of K slots 2p, 2p + 1
#pragma unroll
      for (int pq = 0; pq < 4; ++pq) x[pq] = __builtin_amdgcn_perm(r.c[2 * pq + 1], r.c[2 * pq], sel);
      const int n = (2 * lo4 + bb) & 15;
#pragma unroll
      for (int kc = 0; kc < 4; ++kc) {
        const uint32_t mask = (kc & 1) ? 0x00C000C0u : 0x00300030u;
        uint32_t d[4];
#pragma unroll
        for (int pq = 0; pq < 4; ++pq) d[pq] = ((kc < 2) ? (x[pq] << 4) : x[pq]) & mask;
        const int q8 = 4 * (lo4 >> 3) + kc;
        dst[q8 * 64 + (n ^ swv(q8, n))] = make_uint4(d[0], d[1], d[2], d[3]);
      }
    }
  }
  // constants: each wave needs one or two tile maxima
  const int role = wv >> 1;
  const int idx = 64 * (wv & 1) + lane;
  const int ea = exp_floor(wave_max_nn(fmaxf(r.xa.x, r.xa.y)), role < 2 ? -114 : -100, role < 2 ? 120 : 100);
  int* ex = reinterpret_cast<int*>(buf + kCExp);
  if (role == 0) {
    reinterpret_cast<float*>(buf + kCAlpha)[idx] = scale_log2 * r.c0 * pow2i(7 + ea);
    if (wv == 0 && lane == 0) ex[0] = ea;
  } else if (role == 1) {
    const float x = r.c0 * pow2i(13 - ea);
    const _Float16 h = (_Float16)x;
    reinterpret_cast<_Float16*>(buf + kCKh)[idx] = h;
    reinterpret_cast<_Float16*>(buf + kCKl)[idx] = (_Float16)(x - (float)h);
  } else if (role == 2) {
    reinterpret_cast<float*>(buf + kCVsf)[idx] = r.c0 * pow2i(13 - (int)kTau - ea);
    reinterpret_cast<float*>(buf + kCVmin)[idx] = r.c1;
    if (wv == 4 && lane == 0) ex[1] = ea;
  } else {
    reinterpret_cast<float*>(buf + kCVcu)[idx] = r.c0 * pow2i(24 - ((idx & 1) ? 6 : 4) - (13 - (int)kTau - ea));
    const int em = exp_floor(wave_max_nn(fmaxf(fabsf(r.xb.x), fabsf(r.xb.y))), -100, 100);
    const float x = r.c1 * pow2i(13 - em);
    const _Float16 h = (_Float16)x;
    reinterpret_cast<_Float16*>(buf + kCMh)[idx] = h;
    reinterpret_cast<_Float16*>(buf + kCMl)[idx] = (_Float16)(x - (float)h);
    if (wv == 6 && lane == 0) ex[2] = em;
  }
}

__device__ __forceinline__ int tiles_at(int64_t p, int window) {
  const int64_t ahead = p + 1 - window;
  return ahead > 0 ? (int)(ahead / kTile) : 0;
}

__device__ __forceinline__ half2v as_h2(uint32_t x) { return __builtin_bit_cast(half2v, x); }
__device__ __forceinline__ uint32_t as_u(half2v x) { return __builtin_bit_cast(uint32_t, x); }

// One thread's share of a raw staging step: floats 4 c4 .. + 3 and 4 c4 + 64 .. + 67
// of the key and value rows of token t.  The load always reads a row of the
// range (t clamped below r_hi) and ok marks whether t itself is in it, so that
// no branch has to wait on the load.
struct RawShare {
  float4 k0, k1, v0, v1;
  bool ok;
};

__device__ __forceinline__ float4 keep4(bool ok, float4 x) {
  return make_float4(ok ? x.x : 0.0f, ok ? x.y : 0.0f, ok ? x.z : 0.0f, ok ? x.w : 0.0f);
}

__device__ __forceinline__ RawShare raw_fetch(const float* kbase, const float* vbase, int64_t tok_stride,
                                              int64_t raw_base, int64_t t, int64_t r_hi, int c4) {
  RawShare x;
  x.ok = t < r_hi;
  const int64_t tc = x.ok ? t : r_hi - 1;
  const float4* rk = reinterpret_cast<const float4*>(kbase + (tc - raw_base) * tok_stride);
  const float4* rv = reinterpret_cast<const float4*>(vbase + (tc - raw_base) * tok_stride);
  x.k0 = rk[c4];
  x.k1 = rk[c4 + 16];
  x.v0 = rv[c4];
  x.v1 = rv[c4 + 16];
  return x;
}

// What one workgroup computes: the query rows [0, chunk) of one sequence at
// positions pos0 + r, against its tiles [ja, jb) (clipped to the tiles the
// rows see) and, if raw, its raw rows; either the final output or, with part
// set, the unnormalised partial (m, l, o') of each row and head.
struct Ctx {
  const float* q;                  // row r, head h at (r * n_q + h) * D
  const float* q_rot;
  float* out;
  const uint8_t* records;          // tile j, KV head h at (j * n_kv + h) * tile bytes
  const float* k;                  // raw row of position p, KV head h at
  const float* v;                  //   (p - raw_base) * tok_stride + h * head_stride
  int64_t tok_stride, head_stride;
  int64_t pos0, raw_base;
  float scale;
  int chunk, window, n_q, n_kv, G;
  int ja, jb;
  bool raw;
  bool rotate;                     // q_rot absent: rotate q in registers
  int64_t ra, rb;                  // raw positions [ra, rb) of this workgroup
  float* part;                     // row r, head h at part + r * part_row + h * part_head
  int64_t part_row, part_head;
  bool pack;                       // row groups of 8 positions x 2 query heads (chunk <= 8, G >= 2)
};

// FR = false: four row groups of 16 rows, wave (r, h) takes the token half h
// of every tile and the 16-token raw blocks of parity h, and the two halves
// of a row group merge at the end.  FR = true: eight row groups, each wave
// takes all 128 tokens of every tile (the scores of both halves, one running-
// maximum update, then softmax and values per half; the tile's q~ operands
// and bias computed once) and both raw blocks of every staging step; each
// tile's unpack then serves twice the rows.  The next tile is unpacked by
// waves 0-3 at the start of an iteration and by waves 4-7 at its end in the
// half layout, by every wave at the end in the split layout.
template <bool H, bool FR>
__device__ __forceinline__ void prefill_body(const Ctx& P) {
  constexpr int RG = FR ? 8 : 4;          // row groups (column blocks) per workgroup
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int rg = FR ? wv : (wv & 3), th = wv >> 2;   // row group; token half (FR: unpack slot)
  const int n = lane & 15, g = lane >> 4;
  const int kvh = blockIdx.y;
  const int G = P.G;
  // a row group (MFMA column block) is PPG positions of HPG query heads:
  // 16 x 1, or with P.pack 8 x 2 (lane n: position n % 8, head n / 8), so
  // that a short chunk fills the columns
  const int PPG = P.pack ? 8 : kRows, HPG = P.pack ? 2 : 1;
  const int GB = G / HPG;                                   // row groups per position group
  const int n_blk = ((P.chunk + PPG - 1) / PPG) * GB;       // (position group, head group) column blocks
  const int blk_first = blockIdx.x * RG;
  const int blk_last = min(blk_first + RG - 1, n_blk - 1);
  const int blk = blk_first + rg;
  const bool active = blk < n_blk;
  const int pg = (active ? blk : blk_last) / GB;
  const int rn = P.pack ? (n & 7) : n;                      // this lane's position in the group
  const int hq = kvh * G + ((active ? blk : blk_last) % GB) * HPG + (P.pack ? (n >> 3) : 0);
  const int r0 = PPG * pg;                                  // chunk row of position 0 of the group
  const int64_t prow = P.pos0 + r0 + rn;                    // position of this lane's row
  const bool row_ok = active && (r0 + rn < P.chunk);
  const int T_row = row_ok ? tiles_at(prow, P.window) : 0;
  const int64_t p_wlast = P.pos0 + min(r0 + PPG - 1, P.chunk - 1);
  const int T_wave = active ? tiles_at(p_wlast, P.window) : 0;
  // positions spanned by the workgroup
  const int64_t p_first = P.pos0 + PPG * (blk_first / GB);
  const int64_t p_last = P.pos0 + min(PPG * (blk_last / GB) + PPG - 1, P.chunk - 1);
  const int ja = P.ja;
  const int jend = min(P.jb, tiles_at(p_last, P.window));   // tiles [ja, jend)
  const bool partial = P.part != nullptr;

  __shared__ __attribute__((aligned(16))) uint8_t s_lds[kLdsBytes];
  const float scale_log2 = P.scale * kLog2e;
  const uint8_t* recs = P.records + (int64_t)kvh * Rec<D, H>::bytes;
  const int64_t rstride = (int64_t)P.n_kv * Rec<D, H>::bytes;

  // ---- tile 0 unpacked, tile 1 in registers; this lane's rotated query:
  // row n, channels 32 k4 + 8 g .. + 7 ----
  TileRegs tr;
  if (ja < jend) load_tile<H>(recs + (int64_t)ja * rstride, lane, wv, tr);
  float qv[4][8];
  {
    const float* qp = (P.rotate ? P.q : P.q_rot) + ((int64_t)(row_ok ? r0 + rn : 0) * P.n_q + hq) * D + 8 * g;
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4) {
      float4 a = make_float4(0.f, 0.f, 0.f, 0.f), b = a;
      if (row_ok) {
        a = *reinterpret_cast<const float4*>(qp + 32 * k4);
        b = *reinterpret_cast<const float4*>(qp + 32 * k4 + 4);
      }
      qv[k4][0] = a.x; qv[k4][1] = a.y; qv[k4][2] = a.z; qv[k4][3] = a.w;
      qv[k4][4] = b.x; qv[k4][5] = b.y; qv[k4][6] = b.z; qv[k4][7] = b.w;
    }
  }
  if (ja < jend) {
    unpack_tile(tr, s_lds + kLdsK, s_lds + kLdsV, s_lds + kLdsC, lane, wv, scale_log2);
    if (ja + 1 < jend) load_tile<H>(recs + (int64_t)(ja + 1) * rstride, lane, wv, tr);
  }
  __syncthreads();
  if (P.rotate) {   // q' = H q in registers: channel 32 k4 + 8 g + jj (g = lane bits 4, 5),
                    // butterfly strides in ascending order, then one scale: the rounding of
                    // the separate rotation (and of the oracle's fp32 transform), bit for bit
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4)
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
    for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj)       // strides 8, 16: channel bits 3, 4 across the 16-lane rows
        qv[k4][jj] = bfly_rows<32>(bfly_rows<16>(qv[k4][jj], lane), lane);
#pragma unroll
    for (int kb = 1; kb < 4; kb <<= 1)     // strides 32, 64: channel bits 5, 6
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4)
        if (!(k4 & kb)) {
#pragma unroll
          for (int jj = 0; jj < 8; ++jj) {
            const float a = qv[k4][jj], b = qv[k4 | kb][jj];
            qv[k4][jj] = a + b;
            qv[k4 | kb][jj] = a - b;
          }
        }
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
      for (int jj = 0; jj < 8; ++jj) qv[k4][jj] *= wht_scale<D>();
  }
  // q' of row n scaled into (-1, 1) by 2^-eq, as fp16 hi + lo pairs
  float qmax = 0.0f;
#pragma unroll
  for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
    for (int j = 0; j < 8; ++j) qmax = fmaxf(qmax, fabsf(qv[k4][j]));
  const int eq = exp_floor(rows_max(qmax), -100, 99) + 1;
  const float beta = pow2i(eq);
  uint32_t qh[4][4], ql[4][4];   // [k4][pair]: channels 32 k4 + 8 g + 2 i, + 1
  {
    const float inv = pow2i(-eq);
#pragma unroll
    for (int k4 = 0; k4 < 4; ++k4)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = qv[k4][2 * i] * inv, b = qv[k4][2 * i + 1] * inv;
        const _Float16 ha = (_Float16)a, hb = (_Float16)b;
        qh[k4][i] = pack_h2(ha, hb);
        ql[k4][i] = pack_h2((_Float16)(a - (float)ha), (_Float16)(b - (float)hb));
      }
  }
  // operand read offsets (16-byte units) of lane (g, n): K blocks 4 hh + bb of the
  // token half(s) hh the wave takes, V channel halves
  constexpr int NH = FR ? 2 : 1;   // token halves per wave
  int offk[NH][4], offv[2];
#pragma unroll
  for (int hx = 0; hx < NH; ++hx)
#pragma unroll
    for (int bb = 0; bb < 4; ++bb) offk[hx][bb] = 16 * g + (n ^ swk(4 * (FR ? hx : th) + bb, n));
#pragma unroll
  for (int h = 0; h < 2; ++h) offv[h] = 16 * g + (n ^ swv(4 * h, n));

  float m_run = -INFINITY, l_run = 0.0f;   // softmax state of row n (log2 domain)
  floatx4 O[2][4];                          // row n; channel 64 qb + 16 g + 4 i + kk in O[qb][kk][i]
#pragma unroll
  for (int qb = 0; qb < 2; ++qb)
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) O[qb][kk] = (floatx4){0.f, 0.f, 0.f, 0.f};

  // ---- compressed tiles: compute tile j while unpacking tile j + 1 into the
  // other buffer and loading tile j + 2.  In the half layout the two waves on a
  // SIMD (waves w and w + 4) unpack at opposite ends of the iteration, so the
  // matrix work of one meets the vector work of the other; in the split layout,
  // where each wave's two token halves already interleave vector and matrix
  // work, every wave unpacks at the end (measured faster than either split of
  // the waves). ----
  for (int j = ja; j < jend; ++j) {
    const int pb = (j - ja) & 1;   // buffer of tile j
    const uint8_t* cst = s_lds + kLdsC + pb * kConstBytes;
    const uint4* kop = reinterpret_cast<const uint4*>(s_lds + kLdsK + pb * kOpBytes);
    const uint4* vop = reinterpret_cast<const uint4*>(s_lds + kLdsV + pb * kOpBytes);
    const bool next = j + 1 < jend;
    auto unpack_next = [&]() {
      const int nb = pb ^ 1;
      unpack_tile(tr, s_lds + kLdsK + nb * kOpBytes, s_lds + kLdsV + nb * kOpBytes, s_lds + kLdsC + nb * kConstBytes,
                  lane, wv, scale_log2);
      if (j + 2 < jend) load_tile<H>(recs + (int64_t)(j + 2) * rstride, lane, wv, tr);
    };
    if (!FR && th == 0 && next) unpack_next();
    if (j < T_wave) {
      const int* ex = reinterpret_cast<const int*>(cst + kCExp);
      const int ek = __builtin_amdgcn_readfirstlane(ex[0]);
      const int ev = __builtin_amdgcn_readfirstlane(ex[1]);
      const int em = __builtin_amdgcn_readfirstlane(ex[2]);
      // bias b = sum_c q'_c kmin_c: every row of A is kmin 2^(13 - em) (hi, lo),
      // B is q' 2^-eq (hi, lo); rescaled to the score accumulator's 2^(-7 - ek - eq).
      // Matrix-core blocks run at raised wave priority, so the arbiter issues them
      // while the other wave of the SIMD works through its vector blocks; the
      // bias ops run first, under the forming of the first q~ operands.
      __builtin_amdgcn_s_setprio(1);
      floatx4 bacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const uint4 mh4 = *reinterpret_cast<const uint4*>(cst + kCMh + 2 * (32 * k4 + 8 * g));
        const uint4 ml4 = *reinterpret_cast<const uint4*>(cst + kCMl + 2 * (32 * k4 + 8 * g));
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
      // scores of the wave's token half(s), channel step k4 outermost: the q~ B
      // operands of step k4, q~ = q' kscale 2^(13 - ek - eq) = (qh + ql)(kh + kl) as
      // hi + lo by packed fp16 arithmetic (hi rounded, lo = exact product rest +
      // cross terms), are formed just before its matrix ops, under those of step
      // k4 - 1; each block still sums its steps in k4 order, hi before lo
      floatx4 acc[NH][4];
#pragma unroll
      for (int hx = 0; hx < NH; ++hx)
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) acc[hx][bb] = acc0;
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        const uint4 kh4 = *reinterpret_cast<const uint4*>(cst + kCKh + 2 * (32 * k4 + 8 * g));
        const uint4 kl4 = *reinterpret_cast<const uint4*>(cst + kCKl + 2 * (32 * k4 + 8 * g));
        const uint32_t khv[4] = {kh4.x, kh4.y, kh4.z, kh4.w};
        const uint32_t klv[4] = {kl4.x, kl4.y, kl4.z, kl4.w};
        uint32_t bh[4], bl[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const half2v a = as_h2(qh[k4][i]), a2 = as_h2(ql[k4][i]), k = as_h2(khv[i]), k2 = as_h2(klv[i]);
          const half2v hi = a * k;
          half2v lo = __builtin_elementwise_fma(a, k, -hi);
          lo = __builtin_elementwise_fma(a, k2, lo);
          lo = __builtin_elementwise_fma(a2, k, lo);
          bh[i] = as_u(hi);
          bl[i] = as_u(lo);
        }
        const half8 Bh = as_half8(bh[0], bh[1], bh[2], bh[3]);
        const half8 Bl = as_half8(bl[0], bl[1], bl[2], bl[3]);
#pragma unroll
        for (int hx = 0; hx < NH; ++hx) {
          const int hh = FR ? hx : th;
#pragma unroll
          for (int bb = 0; bb < 4; ++bb) {
            const uint4 a = kop[(k4 * 8 + 4 * hh + bb) * 64 + offk[hx][bb]];
            const half8 A = as_half8(a.x, a.y, a.z, a.w);
            acc[hx][bb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bh, acc[hx][bb], 0, 0, 0);
            acc[hx][bb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(A, Bl, acc[hx][bb], 0, 0, 0);
          }
        }
      }
      // y = alpha_t acc / beta (log2 domain): token 16 b + 4 g + i of row n; then
      // one running-maximum update for the tile, then per half the probabilities
      // and the value aggregate, so that the vector work of one half meets the
      // matrix work of the other
      const float* alp = reinterpret_cast<const float*>(cst + kCAlpha);
      float y[NH][4][4];
      float ymax = -INFINITY;
#pragma unroll
      for (int hx = 0; hx < NH; ++hx) {
        const int hh = FR ? hx : th;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const float4 al = *reinterpret_cast<const float4*>(alp + 16 * (4 * hh + bb) + 4 * g);
          y[hx][bb][0] = acc[hx][bb][0] * al.x;
          y[hx][bb][1] = acc[hx][bb][1] * al.y;
          y[hx][bb][2] = acc[hx][bb][2] * al.z;
          y[hx][bb][3] = acc[hx][bb][3] * al.w;
          ymax = fmaxf(fmaxf(ymax, y[hx][bb][0]), y[hx][bb][1]);
          ymax = fmaxf(fmaxf(ymax, y[hx][bb][2]), y[hx][bb][3]);
        }
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
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int kk = 0; kk < 4; ++kk)
#pragma unroll
            for (int i = 0; i < 4; ++i) O[qb][kk][i] *= alpha;
      }
      const float* vsf = reinterpret_cast<const float*>(cst + kCVsf);
      const float* vmn = reinterpret_cast<const float*>(cst + kCVmin);
      const float* vcu = reinterpret_cast<const float*>(cst + kCVcu);
#pragma unroll
      for (int hx = 0; hx < NH; ++hx) {
        const int hh = FR ? hx : th;
        // probabilities p (<= 2^tau), their sums, and w = p vsf as hi / lo B operands
        float psum = 0.0f, upart = 0.0f;
        uint32_t wh[4][2], wl[4][2];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const int b = 4 * hh + bb;
          const float4 va = *reinterpret_cast<const float4*>(vsf + 16 * b + 4 * g);
          const float4 ma = *reinterpret_cast<const float4*>(vmn + 16 * b + 4 * g);
          const float vs4[4] = {va.x, va.y, va.z, va.w};
          const float vm4[4] = {ma.x, ma.y, ma.z, ma.w};
          float w4[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float pj = __builtin_amdgcn_exp2f(fmaf(beta, y[hx][bb][i], negm));
            psum += pj;
            upart = fmaf(pj, vm4[i], upart);
            w4[i] = pj * vs4[i];
          }
#pragma unroll
          for (int pr = 0; pr < 2; ++pr) {
            const fp16x2 h = __builtin_amdgcn_cvt_pkrtz(w4[2 * pr], w4[2 * pr + 1]);
            const fp16x2 l = __builtin_amdgcn_cvt_pkrtz(w4[2 * pr] - (float)h.x, w4[2 * pr + 1] - (float)h.y);
            wh[bb][pr] = __builtin_bit_cast(uint32_t, h);
            wl[bb][pr] = __builtin_bit_cast(uint32_t, l);
          }
        }
        l_run += rows_sum(psum);
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
        for (int qb = 0; qb < 2; ++qb) {
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
              const uint4 av = vop[((2 * hh + tt) * 8 + q8) * 64 + offv[qb]];
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
        if (hx + 1 < NH) __builtin_amdgcn_s_setprio(0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
    if ((FR || th == 1) && next) unpack_next();
    // tile j + 1 is in place and every wave is done with tile j's buffer
    __syncthreads();
  }

  // ---- inverse rotation of the tile part: channel bits kk (0, 1), i (2, 3),
  // g (4, 5: across 16-lane rows), qb (6).  The partials of FR = false stay
  // rotated (a verify split holds tiles or raw tokens, never both); those of
  // FR = true hold both and are in the raw domain. ----
  if (T_wave > 0 && (FR || !partial)) {
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a0 = O[qb][0][i], a1 = O[qb][1][i], a2 = O[qb][2][i], a3 = O[qb][3][i];
        const float b0 = a0 + a1, b1 = a0 - a1, b2 = a2 + a3, b3 = a2 - a3;
        O[qb][0][i] = b0 + b2;
        O[qb][1][i] = b1 + b3;
        O[qb][2][i] = b0 - b2;
        O[qb][3][i] = b1 - b3;
      }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        const float a0 = O[qb][kk][0], a1 = O[qb][kk][1], a2 = O[qb][kk][2], a3 = O[qb][kk][3];
        const float b0 = a0 + a1, b1 = a0 - a1, b2 = a2 + a3, b3 = a2 - a3;
        O[qb][kk][0] = b0 + b2;
        O[qb][kk][1] = b1 + b3;
        O[qb][kk][2] = b0 - b2;
        O[qb][kk][3] = b1 - b3;
      }
#pragma unroll
    for (int kk = 0; kk < 4; ++kk)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float a = O[0][kk][i], b = O[1][kk][i];
        O[0][kk][i] = a + b;
        O[1][kk][i] = a - b;
      }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int kk = 0; kk < 4; ++kk)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float x = bfly_rows<16>(O[qb][kk][i], lane);
          O[qb][kk][i] = bfly_rows<32>(x, lane) * wht_scale<D>();
        }
  }

  // ---- raw tokens [128 T(p), p] on fp32 MFMA, 16-token blocks of parity th ----
  float4 qr[8];   // raw query of row n, channels 16 jj + 4 g .. + 3
#pragma unroll
  for (int jj = 0; jj < 8; ++jj) {
    qr[jj] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (row_ok)
      qr[jj] = *reinterpret_cast<const float4*>(P.q + ((int64_t)(r0 + rn) * P.n_q + hq) * D + 16 * jj + 4 * g);
  }
  float* s_k = reinterpret_cast<float*>(s_lds);   // over the tile buffers
  float* s_v = s_k + kRawTok * kRawRow;
  const int64_t raw_lo = (int64_t)kTile * tiles_at(p_first, P.window);
  const int64_t wave_lo = (int64_t)kTile * tiles_at(P.pos0 + r0, P.window);
  const int64_t row_lo = (int64_t)kTile * T_row;
  const float* kbase = P.k + (int64_t)kvh * P.head_stride;
  const float* vbase = P.v + (int64_t)kvh * P.head_stride;
  // raw tokens of this workgroup: [r_lo, r_hi)
  const int64_t r_lo = raw_lo > P.ra ? raw_lo : P.ra;
  const int64_t r_hi = p_last + 1 < P.rb ? p_last + 1 : P.rb;
  // this thread's staging share of a step: token t0 + tid / 16, floats 4 (tid % 16) and
  // 4 (tid % 16) + 64 of its key and value rows; the next step's share is loaded
  // into registers while the current step is computed
  const int sr = tid >> 4, sc4 = tid & 15;
  RawShare xs;
  if (P.raw && r_lo < r_hi) xs = raw_fetch(kbase, vbase, P.tok_stride, P.raw_base, r_lo + sr, r_hi, sc4);
  for (int64_t t0 = r_lo; P.raw && t0 < r_hi; t0 += kRawTok) {
    __syncthreads();   // previous readers of the staging rows are done
    *reinterpret_cast<float4*>(s_k + sr * kRawRow + 4 * sc4) = keep4(xs.ok, xs.k0);
    *reinterpret_cast<float4*>(s_k + sr * kRawRow + 4 * (sc4 + 16)) = keep4(xs.ok, xs.k1);
    *reinterpret_cast<float4*>(s_v + sr * kRawRow + 4 * sc4) = keep4(xs.ok, xs.v0);
    *reinterpret_cast<float4*>(s_v + sr * kRawRow + 4 * (sc4 + 16)) = keep4(xs.ok, xs.v1);
    if (t0 + kRawTok < r_hi) xs = raw_fetch(kbase, vbase, P.tok_stride, P.raw_base, t0 + kRawTok + sr, r_hi, sc4);
    __syncthreads();
#pragma unroll
    for (int sx = 0; sx < NH; ++sx) {   // the wave's 16-token block(s) of the step
      const int sb = FR ? sx : th;
      const int64_t tb = t0 + 16 * sb;
      if (!active || tb > p_wlast || tb >= r_hi || tb + 15 < wave_lo) continue;   // wave-uniform
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
        const bool vis = row_ok && t >= row_lo && t <= prow && t < r_hi;
        sv[i] = vis ? sacc[i] * scale_log2 : -INFINITY;
        tmax = fmaxf(tmax, sv[i]);
      }
      tmax = rows_max(tmax);
      const float m_new = fmaxf(m_run, tmax);
      const float m_use = (m_new == -INFINITY) ? 0.0f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
      float pv[4], psum = 0.0f;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        pv[i] = __builtin_amdgcn_exp2f(sv[i] - m_use);
        psum += pv[i];
      }
      l_run = l_run * alpha + rows_sum(psum);
      m_run = m_new;
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
#pragma unroll
          for (int i = 0; i < 4; ++i) O[qb][kk][i] *= alpha;
      // O^T[c][n] += sum_t v[t][c] p[n][t]; step i: K slot g is token tb + 4 g + i,
      // A row n' is channel 64 qb + 4 n' + kk
#pragma unroll
      for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int qb = 0; qb < 2; ++qb) {
          const float4 vv = *reinterpret_cast<const float4*>(s_v + (16 * sb + 4 * g + i) * kRawRow + 64 * qb + 4 * n);
          O[qb][0] = __builtin_amdgcn_mfma_f32_16x16x4f32(vv.x, pv[i], O[qb][0], 0, 0, 0);
          O[qb][1] = __builtin_amdgcn_mfma_f32_16x16x4f32(vv.y, pv[i], O[qb][1], 0, 0, 0);
          O[qb][2] = __builtin_amdgcn_mfma_f32_16x16x4f32(vv.z, pv[i], O[qb][2], 0, 0, 0);
          O[qb][3] = __builtin_amdgcn_mfma_f32_16x16x4f32(vv.w, pv[i], O[qb][3], 0, 0, 0);
        }
      }
    }
  }

  if constexpr (FR) {   // ---- normalise (or keep the partial), store ----
    if (!row_ok) return;
    float ca = 1.0f;
    float* o;
    if (partial) {
      o = P.part + (int64_t)(r0 + rn) * P.part_row + (int64_t)hq * P.part_head;
      if (g == 0) *reinterpret_cast<float2*>(o + D) = make_float2(m_run, l_run);
    } else {
      ca = 1.0f / l_run;   // every row of a final output sees its own position
      o = P.out + ((int64_t)(r0 + rn) * P.n_q + hq) * D;
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<float4*>(o + 64 * qb + 16 * g + 4 * i) =
            make_float4(O[qb][0][i] * ca, O[qb][1][i] * ca, O[qb][2][i] * ca, O[qb][3][i] * ca);
  } else {   // ---- merge the two token halves of each row group, normalise, store ----
    __syncthreads();   // the raw staging rows are free
    float4* mo = reinterpret_cast<float4*>(s_lds);
    float2* mml = reinterpret_cast<float2*>(s_lds + kMergeO);
    if (th == 1 && active) {
#pragma unroll
      for (int qb = 0; qb < 2; ++qb)
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          mo[(rg * 8 + 4 * qb + kk) * 64 + lane] = make_float4(O[qb][kk][0], O[qb][kk][1], O[qb][kk][2], O[qb][kk][3]);
      mml[rg * 64 + lane] = make_float2(m_run, l_run);
    }
    __syncthreads();
    if (th == 1 || !row_ok) return;
    const float2 ml2 = mml[rg * 64 + lane];
    const float M = fmaxf(m_run, ml2.x);   // -inf only for a partial that sees nothing
    const float fa = (m_run == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m_run - M);
    const float fb = (ml2.x == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(ml2.x - M);
    const float lsum = l_run * fa + ml2.y * fb;
    float ca = fa, cb = fb;
    float* o;
    if (partial) {
      o = P.part + (int64_t)(r0 + rn) * P.part_row + (int64_t)hq * P.part_head;
      if (g == 0) *reinterpret_cast<float2*>(o + D) = make_float2(M, lsum);
    } else {
      const float inv = 1.0f / lsum;   // every row of a final output sees its own position
      ca *= inv;
      cb *= inv;
      o = P.out + ((int64_t)(r0 + rn) * P.n_q + hq) * D;
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float4 ob[4];
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) ob[kk] = mo[(rg * 8 + 4 * qb + kk) * 64 + lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float b0 = i == 0 ? ob[0].x : i == 1 ? ob[0].y : i == 2 ? ob[0].z : ob[0].w;
        const float b1 = i == 0 ? ob[1].x : i == 1 ? ob[1].y : i == 2 ? ob[1].z : ob[1].w;
        const float b2 = i == 0 ? ob[2].x : i == 1 ? ob[2].y : i == 2 ? ob[2].z : ob[2].w;
        const float b3 = i == 0 ? ob[3].x : i == 1 ? ob[3].y : i == 2 ? ob[3].z : ob[3].w;
        *reinterpret_cast<float4*>(o + 64 * qb + 16 * g + 4 * i) =
            make_float4(O[qb][0][i] * ca + b0 * cb, O[qb][1][i] * ca + b1 * cb,
                        O[qb][2][i] * ca + b2 * cb, O[qb][3][i] * ca + b3 * cb);
      }
    }
  }
}

template <bool H>
__global__ void __launch_bounds__(kThreads) prefill_mfma_kernel(PrefillParams P) {
  Ctx c;
  c.q = P.q;
  c.q_rot = P.q_rot;
  c.out = P.out;
  c.records = P.records;
  c.k = P.k;
  c.v = P.v;
  c.tok_stride = P.tok_stride;
  c.head_stride = P.head_stride;
  c.pos0 = P.pos0;
  c.raw_base = P.raw_base;
  c.scale = P.scale;
  c.chunk = P.chunk;
  c.window = P.window;
  c.n_q = P.n_q;
  c.n_kv = P.n_kv;
  c.G = P.G;
  c.ja = 0;
  c.jb = 0x7fffffff;
  c.raw = true;
  c.rotate = P.q_rot == nullptr;   // no rotated query given: rows rotate q in registers
  if (c.rotate) c.q_rot = P.q;
  c.ra = 0;
  c.rb = INT64_MAX;
  c.part = nullptr;
  c.part_row = c.part_head = 0;
  c.pack = false;
  prefill_body<H, false>(c);
}

// Chunked prefill with whole tiles per wave (FR layout: 128 row-heads per
// workgroup).  blockIdx.z = split s of S takes the s-th S-th of its
// workgroup's tiles and of its raw tokens (in 32-token staging steps), so the
// splits carry equal shares of both kinds of work; with S > 1 each writes the
// raw-domain partial of its rows at part + ((r n_q + h) S + s) (D + 4), and
// prefill_combine_kernel merges them.
template <bool H>
__global__ void __launch_bounds__(kThreads) prefill_split_kernel(PrefillParams P, float* part, int S) {
  Ctx c;
  c.q = P.q;
  c.q_rot = P.q_rot;
  c.out = P.out;
  c.records = P.records;
  c.k = P.k;
  c.v = P.v;
  c.tok_stride = P.tok_stride;
  c.head_stride = P.head_stride;
  c.pos0 = P.pos0;
  c.raw_base = P.raw_base;
  c.scale = P.scale;
  c.chunk = P.chunk;
  c.window = P.window;
  c.n_q = P.n_q;
  c.n_kv = P.n_kv;
  c.G = P.G;
  c.rotate = P.q_rot == nullptr;   // no rotated query given: rows rotate q in registers
  if (c.rotate) c.q_rot = P.q;
  const int s = blockIdx.z;
  const int n_blk = ((P.chunk + kRows - 1) / kRows) * P.G;
  const int blk_first = blockIdx.x * 8;
  const int blk_last = min(blk_first + 7, n_blk - 1);
  const int64_t p_first = P.pos0 + kRows * (blk_first / P.G);
  const int64_t p_last = P.pos0 + min(kRows * (blk_last / P.G) + kRows - 1, P.chunk - 1);
  const int Tw = tiles_at(p_last, P.window);
  const int64_t r_lo = (int64_t)kTile * tiles_at(p_first, P.window);
  const int64_t steps = (p_last + 1 - r_lo + kRawTok - 1) / kRawTok;
  c.ja = (int)((int64_t)Tw * s / S);
  c.jb = (int)((int64_t)Tw * (s + 1) / S);
  c.raw = true;
  c.ra = r_lo + kRawTok * (steps * s / S);
  c.rb = r_lo + kRawTok * (steps * (s + 1) / S);
  c.part = S > 1 ? part + (int64_t)s * (D + 4) : nullptr;
  c.part_head = (int64_t)S * (D + 4);
  c.part_row = (int64_t)P.n_q * c.part_head;
  c.pack = false;
  prefill_body<H, true>(c);
}

// Multi-query verify: sequence b's q_len query rows are the q_len newest
// window tokens; row i sees the n_tiles[b] tiles and window tokens
// [0, n_win[b] - q_len + i].  That is the chunked-prefill view at positions
// 128 T + n_win - q_len + i with window parameter n_win - q_len + 1, so the
// prefill workgroup computes it.  blockIdx.z = b (n_tsplit + n_wsplit) + s:
// split s < n_tsplit takes tiles [tps s, tps s + tps), split n_tsplit + r the
// window tokens [wchunk r, wchunk r + wchunk).  Partials: row r = b q_len + i,
// head h, split s at part + ((r n_q + h) (n_tsplit + n_wsplit) + s) (D + 4).
template <bool H>
__global__ void __launch_bounds__(kThreads) verify_mfma_kernel(DecodeParams P) {
  const int ns = P.n_tsplit, nsp = P.n_tsplit + P.n_wsplit;
  const int b = blockIdx.z / nsp, s = blockIdx.z % nsp;
  const int w = P.q_len;
  const int T = P.n_tiles[b], nw = P.n_win[b];
  // the arguments this workgroup reads, pinned together: one round of scalar
  // loads instead of a chain
  const int64_t rs0 = P.rec_start[b], ws0 = P.win_start[b];
  const int64_t seq_st = P.win_seq_stride, tok_st = P.win_tok_stride;
  const float* p_q = P.q;
  const float* p_qrot = P.q_rot;
  asm volatile("" ::"s"(ns), "s"(nsp), "s"(w), "s"(T), "s"(nw), "s"(rs0), "s"(ws0), "s"(seq_st),
               "s"(tok_st), "s"(p_q), "s"(p_qrot));
  Ctx c;
  const int64_t row0 = (int64_t)b * w * P.n_q * D;
  c.q = p_q + row0;
  c.rotate = p_qrot == nullptr;
  c.q_rot = c.rotate ? c.q : p_qrot + row0;
  c.out = P.out;   // unused: partial output
  c.records = P.records + rs0 * (int64_t)P.n_kv * Rec<D, H>::bytes;
  c.k = P.k_win + (int64_t)b * seq_st + ws0 * tok_st;
  c.v = P.v_win + (int64_t)b * seq_st + ws0 * tok_st;
  c.tok_stride = tok_st;
  c.head_stride = P.win_head_stride;
  c.raw_base = (int64_t)kTile * T;
  c.pos0 = c.raw_base + nw - w;
  c.window = nw - w + 1;
  c.scale = P.scale;
  c.chunk = w;
  c.n_q = P.n_q;
  c.n_kv = P.n_kv;
  c.G = P.G;
  c.ja = s < ns ? P.tps * s : 0;
  c.jb = s < ns ? P.tps * (s + 1) : 0;
  c.raw = s >= ns;
  c.ra = c.raw_base + (int64_t)P.wchunk * (s - ns);
  c.rb = c.ra + P.wchunk;
  c.part_head = (int64_t)nsp * (D + 4);
  c.part_row = (int64_t)P.n_q * c.part_head;
  c.part = P.part + (int64_t)b * w * c.part_row + (int64_t)s * (D + 4);
  c.pack = P.G >= 2;   // q_len <= 8 rows: a row group holds them for two heads
  prefill_body<H, false>(c);
}

// Verify combine: one wave per (row, query head), lane l owns channels l and
// l + 64.  Lane j first reads split j's (m, l); the tile partials merge with
// log-sum-exp weights, the sum gets one inverse WHT, then the window partials
// join the same way and the result is divided by L.  Splits: at most 64.
__global__ void __launch_bounds__(256) verify_combine_kernel(DecodeParams P, int n_rows) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);   // (row, head)
  if (item >= n_rows * P.n_q) return;   // wave-uniform
  const int ns = P.n_tsplit, nsp = P.n_tsplit + P.n_wsplit;
  const float* pp = P.part + (int64_t)item * nsp * (D + 4);
  float2 ml = make_float2(-INFINITY, 0.0f);
  if (lane < nsp) ml = *reinterpret_cast<const float2*>(pp + (int64_t)lane * (D + 4) + D);
  // weights of the tile splits and of the window splits, each against its own maximum
  const bool tile = lane < ns;
  float mt = tile ? ml.x : -INFINITY, mr = tile ? -INFINITY : ml.x;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    mt = fmaxf(mt, __shfl_xor(mt, m, 64));
    mr = fmaxf(mr, __shfl_xor(mr, m, 64));
  }
  const float mg = tile ? mt : mr;
  const float wgt = (ml.x == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(ml.x - mg);
  float lt = tile ? wgt * ml.y : 0.0f, lr = tile ? 0.0f : wgt * ml.y;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) {
    lt += __shfl_xor(lt, m, 64);
    lr += __shfl_xor(lr, m, 64);
  }
  float o0 = 0.0f, o1 = 0.0f, r0 = 0.0f, r1 = 0.0f;
  for (int j0 = 0; j0 < nsp; j0 += 8) {
    float x0[8], x1[8], wj[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int j = j0 + k < nsp ? j0 + k : 0;
      wj[k] = __shfl(wgt, j, 64);
      x0[k] = pp[(int64_t)j * (D + 4) + lane];
      x1[k] = pp[(int64_t)j * (D + 4) + lane + 64];
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const int j = j0 + k;
      const float wk = j < nsp ? wj[k] : 0.0f;
      if (j < ns) {
        o0 = fmaf(wk, x0[k], o0);
        o1 = fmaf(wk, x1[k], o1);
      } else {
        r0 = fmaf(wk, x0[k], r0);
        r1 = fmaf(wk, x1[k], r1);
      }
    }
  }
  // inverse WHT of the rotated tile sum: element lane in o0, lane + 64 in o1
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) {
    const float y0 = __shfl_xor(o0, m, 64), y1 = __shfl_xor(o1, m, 64);
    const bool up = (lane & m) != 0;
    o0 = up ? (y0 - o0) : (o0 + y0);
    o1 = up ? (y1 - o1) : (o1 + y1);
  }
  {
    const float a = o0, c = o1;
    o0 = (a + c) * wht_scale<D>();
    o1 = (a - c) * wht_scale<D>();
  }
  const float M = fmaxf(mt, mr);   // finite: every row sees window token 0
  const float a = (mt == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mt - M);
  const float bw = (mr == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(mr - M);
  const float inv = 1.0f / (lt * a + lr * bw);
  float* o = P.out + (int64_t)item * D;
  o[lane] = (o0 * a + r0 * bw) * inv;
  o[lane + 64] = (o1 * a + r1 * bw) * inv;
}

// Merge of the S raw-domain split partials of a chunked prefill: one wave per
// (row, query head), lane l owns channels 2l, 2l + 1; log-sum-exp weights
// against the largest running maximum, then the division by L.
__global__ void __launch_bounds__(256) prefill_combine_kernel(const float* part, float* out, int n_items, int S) {
  const int lane = threadIdx.x & 63;
  const int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item >= n_items) return;   // wave-uniform
  const float* pp = part + (int64_t)item * S * (D + 4);
  float M = -INFINITY;
  for (int s = 0; s < S; ++s) M = fmaxf(M, pp[(int64_t)s * (D + 4) + D]);
  float L = 0.0f, x = 0.0f, y = 0.0f;
  for (int s = 0; s < S; ++s) {
    const float2 ml = *reinterpret_cast<const float2*>(pp + (int64_t)s * (D + 4) + D);
    const float2 o = *reinterpret_cast<const float2*>(pp + (int64_t)s * (D + 4) + 2 * lane);
    const float w = (ml.x == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(ml.x - M);   // a split that sees nothing
    L = fmaf(w, ml.y, L);
    x = fmaf(w, o.x, x);
    y = fmaf(w, o.y, y);
  }
  const float inv = 1.0f / L;   // finite: every row sees its own position in one split
  *reinterpret_cast<float2*>(out + (int64_t)item * D + 2 * lane) = make_float2(x * inv, y * inv);
}

}  // namespace

hipError_t launch_prefill_mfma(const PrefillParams& P, hipStream_t stream) {
  const int n_blk = ((P.chunk + kRows - 1) / kRows) * P.G;
  dim3 grid((n_blk + 3) / 4, P.n_kv);
  if (P.h16)
    hipLaunchKernelGGL(prefill_mfma_kernel<true>, grid, dim3(kThreads), 0, stream, P);
  else
    hipLaunchKernelGGL(prefill_mfma_kernel<false>, grid, dim3(kThreads), 0, stream, P);
  return hipGetLastError();
}

hipError_t launch_prefill_split(const PrefillParams& P, float* part, int S, hipStream_t stream) {
  const int n_blk = ((P.chunk + kRows - 1) / kRows) * P.G;
  dim3 grid((n_blk + 7) / 8, P.n_kv, S);
  if (P.h16)
    hipLaunchKernelGGL(prefill_split_kernel<true>, grid, dim3(kThreads), 0, stream, P, part, S);
  else
    hipLaunchKernelGGL(prefill_split_kernel<false>, grid, dim3(kThreads), 0, stream, P, part, S);
  if (S > 1) {
    const int items = P.chunk * P.n_q;
    hipLaunchKernelGGL(prefill_combine_kernel, dim3((items + 3) / 4), dim3(256), 0, stream,
                       static_cast<const float*>(part), P.out, items, S);
  }
  return hipGetLastError();
}

hipError_t launch_verify_mfma(const DecodeParams& P, int batch, hipStream_t stream) {
  // row groups of 8 rows x 2 heads when G >= 2 (q_len <= 8), else 16 x 1
  const int n_blk = P.G >= 2 ? ((P.q_len + 7) / 8) * (P.G / 2) : (P.q_len + kRows - 1) / kRows;
  dim3 grid((n_blk + 3) / 4, P.n_kv, batch * (P.n_tsplit + P.n_wsplit));
  if (P.h16)
    hipLaunchKernelGGL(verify_mfma_kernel<true>, grid, dim3(kThreads), 0, stream, P);
  else
    hipLaunchKernelGGL(verify_mfma_kernel<false>, grid, dim3(kThreads), 0, stream, P);
  const int items = batch * P.q_len * P.n_q;
  hipLaunchKernelGGL(verify_combine_kernel, dim3((items + 3) / 4), dim3(256), 0, stream, P, batch * P.q_len);
  return hipGetLastError();
}

}  // namespace kvarn
