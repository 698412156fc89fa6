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
#include "kvarn_mfma.h"

namespace kvarn {
namespace {

using namespace mfma;

__device__ __forceinline__ void st_part(float* p, float v) { *p = v; }

// fp16 hi/lo MFMA operands of one tile in LDS, [32-step][hi, lo][row group g]
// [head] x 8 halves.  Scores: q~ = q' kscale, channels 32 step + 8 g .. + 7 of
// one head (B operand).  Values: w = p vscale, tokens 32 step + 8 g .. + 7 of
// one head (A operand).  The two uses never overlap in time, so they share
// the storage.
template <int G>
struct OpTile {
  uint4 v[4][2][4][G];
};

// Step 1 of a tile, all 256 threads: q~ hi/lo for the G real heads into the
// operand tile, and the bias b_h = sum_c q'_c kmin_c.  fp16 scale per head
// from a bound on |q~|: max|q'| of the head times the tile's max kscale
// (kscale >= 0); the bound only has to keep the hi part finite, the hi/lo
// split keeps each element's relative precision.
template <int G>
__device__ __forceinline__ void tile_qtilde(const uint8_t* rec, const float* qrot, const float* qmax,
                                            float kmx, int tid, OpTile<G>& Q, float* s_bias) {
  const float* ks = reinterpret_cast<const float*>(rec + kOffKscale);
  const float* km = reinterpret_cast<const float*>(rec + kOffKmin);
  constexpr int kItems = G * 32;   // (head, 4 channels)
  for (int e = tid; e < kItems; e += 256) {
    const int h = e >> 5, c0 = 4 * (e & 31);
    const float4 q = *reinterpret_cast<const float4*>(qrot + h * D + c0);
    const float4 sc = *reinterpret_cast<const float4*>(ks + c0);
    const float4 mn = *reinterpret_cast<const float4*>(km + c0);
    float bias = q.x * mn.x + q.y * mn.y + q.z * mn.z + q.w * mn.w;
    const float f16inv = pow2i(fp16_scale_exp(kmx * qmax[h]) - 4);   // q~ * f / 16
    const float x0 = q.x * sc.x * f16inv, x1 = q.y * sc.y * f16inv;
    const float x2 = q.z * sc.z * f16inv, x3 = q.w * sc.w * f16inv;
    const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1, h2 = (_Float16)x2, h3 = (_Float16)x3;
    const int k4 = c0 >> 5, g = (c0 >> 3) & 3, part = (c0 >> 2) & 1;
    reinterpret_cast<uint2*>(&Q.v[k4][0][g][h])[part] = make_uint2(pack_h2(h0, h1), pack_h2(h2, h3));
    reinterpret_cast<uint2*>(&Q.v[k4][1][g][h])[part] =
        make_uint2(pack_h2((_Float16)(x0 - (float)h0), (_Float16)(x1 - (float)h1)),
                   pack_h2((_Float16)(x2 - (float)h2), (_Float16)(x3 - (float)h3)));
#pragma unroll
    for (int m = 1; m < 32; m <<= 1) bias += __shfl_xor(bias, m, 64);   // the head's 32 items
    if ((e & 31) == 0) s_bias[h] = bias;
  }
}

// Scores of one tile held in LDS at `rec` for the 32 tokens [32w, 32w + 32)
// of wave w: lane (g, n) gets s[j][i] = log2-domain score of token
// 32w + 8g + 2i + j for query head n (columns n >= G are padding).
//   S^T[t][h] = sum_c zK[t][c] * q~[h][c]
// on v_mfma_f32_16x16x32_f16, 16 tokens (the low or the high nibble of one
// code byte) per MFMA row block.
template <int G>
__device__ __forceinline__ void tile_scores(const uint8_t* rec, const OpTile<G>& Q, const float* s_bias,
                                            float qmax_n, float kmx, float scale_log2, int lane, int w,
                                            float (&s)[2][4]) {
  const int n = lane & 15;   // MFMA row (A: code byte 16w + n) / column (query head)
  const int g = lane >> 4;   // K group
  const float unscale = pow2i(24 - fp16_scale_exp(kmx * qmax_n));   // S = acc * 2^24 / f
  floatx4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
  // byte (n & 3) of two channels' code dwords into the low bytes of two halves
  const uint32_t nb = (uint32_t)(n & 3);
  const uint32_t sel = nb | (12u << 8) | ((4u + nb) << 16) | (12u << 24);
  const int boff = 16 * w + 4 * (n >> 2);
#pragma unroll
  for (int k4 = 0; k4 < 4; ++k4) {
    uint4 bh = make_uint4(0, 0, 0, 0), bl = make_uint4(0, 0, 0, 0);
    if (n < G) {
      bh = Q.v[k4][0][g][n];
      bl = Q.v[k4][1][g][n];
    }
    const half8 Bh = as_half8(bh.x, bh.y, bh.z, bh.w);
    const half8 Bl = as_half8(bl.x, bl.y, bl.z, bl.w);
    uint32_t ae[4], ao[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int c = 32 * k4 + 8 * g + 2 * p;
      const uint32_t c0 = *reinterpret_cast<const uint32_t*>(rec + c * 64 + boff);
      const uint32_t c1 = *reinterpret_cast<const uint32_t*>(rec + (c + 1) * 64 + boff);
      ae[p] = __builtin_amdgcn_perm(c1 << 4, c0 << 4, sel) & 0x00F000F0u;   // 16 z, token 32w + 2n
      ao[p] = __builtin_amdgcn_perm(c1, c0, sel) & 0x00F000F0u;             // 16 z, token 32w + 2n + 1
    }
    const half8 Ae = as_half8(ae[0], ae[1], ae[2], ae[3]);
    const half8 Ao = as_half8(ao[0], ao[1], ao[2], ao[3]);
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ae, Bh, acc0, 0, 0, 0);
    acc0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ae, Bl, acc0, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ao, Bh, acc1, 0, 0, 0);
    acc1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ao, Bl, acc1, 0, 0, 0);
  }
  const float bias = (n < G) ? s_bias[n] : 0.0f;
  const float* ktok = reinterpret_cast<const float*>(rec + kOffKtok) + 32 * w + 8 * g;
  const float4 k0 = *reinterpret_cast<const float4*>(ktok);
  const float4 k1 = *reinterpret_cast<const float4*>(ktok + 4);
  const float kt[8] = {k0.x, k0.y, k0.z, k0.w, k1.x, k1.y, k1.z, k1.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    s[0][i] = scale_log2 * kt[2 * i] * (acc0[i] * unscale + bias);
    s[1][i] = scale_log2 * kt[2 * i + 1] * (acc1[i] * unscale + bias);
  }
}

// Value aggregate of one tile for wave w's two channel blocks: channels
// 4(16 qb + n) + kk with qb = w / 2 and kk = 2 (w % 2) + {0, 1}, over all 128
// tokens (four 32-token steps):  O[h][c] = sum_t w[h][t] zV[t][c].  z2 gets
// the raw MFMA sums (2-bit codes in bits 4-5 / 6-7 of an fp16 subnormal).
template <int G>
__device__ __forceinline__ void tile_values(const uint8_t* rec, const OpTile<G>& W, int lane, int w,
                                            floatx4& z0, floatx4& z1) {
  const int n = lane & 15, g = lane >> 4;
  const uint8_t* vcode = rec + kOffV;
  const int qb = w >> 1;
  const uint32_t bsel = (uint32_t)(n & 3);
  const uint32_t vsel = bsel | (12u << 8) | ((4u + bsel) << 16) | (12u << 24);
  const int doff = 16 * qb + 4 * (n >> 2);
  const bool shift = (w & 1) == 0;   // crumbs 0, 1 move up by 4; crumbs 2, 3 are in place
  z0 = (floatx4){0.f, 0.f, 0.f, 0.f};
  z1 = (floatx4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ts = 0; ts < 4; ++ts) {
    uint4 ah = make_uint4(0, 0, 0, 0), al = make_uint4(0, 0, 0, 0);
    if (n < G) {
      ah = W.v[ts][0][g][n];
      al = W.v[ts][1][g][n];
    }
    const half8 Ah = as_half8(ah.x, ah.y, ah.z, ah.w);
    const half8 Al = as_half8(al.x, al.y, al.z, al.w);
    uint32_t pr[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int t = 32 * ts + 8 * g + 2 * q;
      const uint32_t da = *reinterpret_cast<const uint32_t*>(vcode + t * (D / 4) + doff);
      const uint32_t db = *reinterpret_cast<const uint32_t*>(vcode + (t + 1) * (D / 4) + doff);
      const uint32_t x = __builtin_amdgcn_perm(db, da, vsel);
      pr[q] = shift ? (x << 4) : x;
    }
    const half8 B0 = as_half8(pr[0] & 0x00300030u, pr[1] & 0x00300030u, pr[2] & 0x00300030u, pr[3] & 0x00300030u);
    const half8 B1 = as_half8(pr[0] & 0x00C000C0u, pr[1] & 0x00C000C0u, pr[2] & 0x00C000C0u, pr[3] & 0x00C000C0u);
    z0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, B0, z0, 0, 0, 0);
    z0 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Al, B0, z0, 0, 0, 0);
    z1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Ah, B1, z1, 0, 0, 0);
    z1 = __builtin_amdgcn_mfma_f32_16x16x32_f16(Al, B1, z1, 0, 0, 0);
  }
}

constexpr int kRow = D + 4;                 // padded window row (528 bytes)
constexpr int kWinRowsLds = kWinChunkFused; // window rows staged per workgroup
constexpr int kMax(int a, int b) { return a > b ? a : b; }
// tile path: double-buffered records + operand tile; window path: K and V rows
template <int G>
constexpr int lds_bytes() { return kMax(2 * kRecBytes + (int)sizeof(OpTile<G>), 2 * kWinRowsLds * kRow * 4); }

template <int G>
__global__ void __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4, 4))) decode_fused_kernel(DecodeParams P) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = tid >> 6;
  const int split = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int n_split = P.n_tsplit + P.n_wsplit;

  __shared__ __attribute__((aligned(16))) uint8_t s_buf[lds_bytes<G>()];   // records + w / window rows
  __shared__ __attribute__((aligned(16))) float s_q[G][D];
  __shared__ float s_red[3][4][G];   // per wave: tile max, sum p, sum p * vmin
  __shared__ float s_ml[G][2];
  __shared__ float s_qmax[G];
  __shared__ float s_bias[G];

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
    for (int h = wv; h < G; h += 4) {
      float x0 = qsrc[h * D + lane], x1 = qsrc[h * D + lane + 64];
      if (!P.q_rot) {
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) {
          const bool up = (lane & m) != 0;
          const float p0 = __shfl_xor(x0, m, 64), p1 = __shfl_xor(x1, m, 64);
          x0 = up ? (p0 - x0) : (x0 + p0);
          x1 = up ? (p1 - x1) : (x1 + p1);
        }
        const float a = x0, c = x1;
        x0 = (a + c) * wht_scale<D>();
        x1 = (a - c) * wht_scale<D>();
      }
      s_q[h][lane] = x0;
      s_q[h][lane + 64] = x1;
      // max |q'| per head (bound for the fp16 operand scale)
      const float mq = wave_max(fmaxf(fabsf(x0), fabsf(x1)));
      if (lane == 0) s_qmax[h] = mq;
    }
    KVARN_STORE_REC(0);
    __syncthreads();
    const int n = lane & 15, g = lane >> 4;
    const float qmax_n = (n < G) ? s_qmax[n] : 0.0f;
    const float scale_log2 = P.scale * kLog2e;
    OpTile<G>& Op = *reinterpret_cast<OpTile<G>*>(s_buf + 2 * kRecBytes);
    float m_run = -INFINITY, l_run = 0.0f;   // softmax state of head n (same in every wave)
    floatx4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};   // o'[head 4g + i][channel block]
    int cur = 0;
    for (int tile = t_begin; tile < t_end; ++tile) {
      const bool more = tile + 1 < t_end;
      if (more) KVARN_LOAD_REC(tile + 1);            // in flight during the compute
      const uint8_t* rec = s_buf + cur * kRecBytes;
      const float2 kk2 = *reinterpret_cast<const float2*>(rec + kOffKscale + 8 * lane);
      const float kmx = wave_max(fmaxf(kk2.x, kk2.y));   // tile max kscale
      tile_qtilde<G>(rec, &s_q[0][0], s_qmax, kmx, tid, Op, s_bias);
      __syncthreads();
      float s[2][4];
      tile_scores<G>(rec, Op, s_bias, qmax_n, kmx, scale_log2, lane, wv, s);
      float tmax = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                         fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
      tmax = wave_max16(tmax);
      if (g == 0 && n < G) s_red[0][wv][n] = tmax;
      // tile-wide fp16 scale for w = p * vscale (p <= 1): max vscale over 128 tokens
      const float* vsc = reinterpret_cast<const float*>(rec + kOffVscale);
      const float* vmn = reinterpret_cast<const float*>(rec + kOffVmin);
      const float2 vv = *reinterpret_cast<const float2*>(vsc + 2 * lane);
      const int vexp = fp16_scale_exp(wave_max(fmaxf(vv.x, vv.y)));
      const float fv = pow2i(vexp);
      __syncthreads();
      float m_new = m_run;
      if (n < G) {
#pragma unroll
        for (int k = 0; k < 4; ++k) m_new = fmaxf(m_new, s_red[0][k][n]);
      }
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);   // 0 on the first tile
      const float* vs8 = vsc + 32 * wv + 8 * g;
      const float* vm8 = vmn + 32 * wv + 8 * g;
      const float4 va = *reinterpret_cast<const float4*>(vs8), vb = *reinterpret_cast<const float4*>(vs8 + 4);
      const float4 ma = *reinterpret_cast<const float4*>(vm8), mb = *reinterpret_cast<const float4*>(vm8 + 4);
      const float vsv[8] = {va.x, va.y, va.z, va.w, vb.x, vb.y, vb.z, vb.w};
      const float vmv[8] = {ma.x, ma.y, ma.z, ma.w, mb.x, mb.y, mb.z, mb.w};
      float psum = 0.0f, upart = 0.0f;
      uint32_t wh[4], wl[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const float pj = __builtin_amdgcn_exp2f(s[j][i] - m_new);
          psum += pj;
          upart += pj * vmv[2 * i + j];
          x[j] = pj * vsv[2 * i + j] * fv;
        }
        const _Float16 h0 = (_Float16)x[0], h1 = (_Float16)x[1];
        wh[i] = pack_h2(h0, h1);
        wl[i] = pack_h2((_Float16)(x[0] - (float)h0), (_Float16)(x[1] - (float)h1));
      }
      psum = wave_sum16(psum);
      upart = wave_sum16(upart);
      if (n < G) {
        Op.v[wv][0][g][n] = make_uint4(wh[0], wh[1], wh[2], wh[3]);
        Op.v[wv][1][g][n] = make_uint4(wl[0], wl[1], wl[2], wl[3]);
        if (g == 0) {
          s_red[1][wv][n] = psum;
          s_red[2][wv][n] = upart;
        }
      }
      __syncthreads();
      float lsum = 0.0f, u = 0.0f;
      if (n < G) {
#pragma unroll
        for (int k = 0; k < 4; ++k) { lsum += s_red[1][k][n]; u += s_red[2][k][n]; }
      }
      l_run = l_run * alpha + lsum;
      m_run = m_new;
      floatx4 z0, z1;
      tile_values<G>(rec, Op, lane, wv, z0, z1);
      // o' = o' alpha_h + vchan_c (O 2^24 / (fv 2^shift) + u_h), shift 4 / 6 for the two crumbs
      const float4 vc4 = *reinterpret_cast<const float4*>(
          reinterpret_cast<const float*>(rec + kOffVchan) + 4 * (16 * (wv >> 1) + n));
      const int kk0 = 2 * (wv & 1);
      const float vc0 = (wv & 1) ? vc4.z : vc4.x, vc1 = (wv & 1) ? vc4.w : vc4.y;
      const float un0 = pow2i(24 - vexp - 4), un1 = pow2i(24 - vexp - 6);
      (void)kk0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float ar = __shfl(alpha, 4 * g + i, 64);
        const float ur = __shfl(u, 4 * g + i, 64);
        o0[i] = o0[i] * ar + vc0 * (z0[i] * un0 + ur);
        o1[i] = o1[i] * ar + vc1 * (z1[i] * un1 + ur);
      }
      if (more) KVARN_STORE_REC(cur ^ 1);
      __syncthreads();
      cur ^= 1;
    }
#undef KVARN_LOAD_REC
#undef KVARN_STORE_REC
    // ---- the workgroup's partial: o' through LDS for coalesced stores ----
    float* s_o = reinterpret_cast<float*>(s_buf);   // [G][D]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int h = 4 * g + i;
      const int c = 4 * (16 * (wv >> 1) + n) + 2 * (wv & 1);
      if (h < G) {
        s_o[h * D + c] = o0[i];
        s_o[h * D + c + 1] = o1[i];
      }
    }
    if (wv == 0 && g == 0 && n < G) {
      s_ml[n][0] = m_run;
      s_ml[n][1] = l_run;
    }
    __syncthreads();
    for (int i = tid; i < G * D; i += 256) {
      const int h = i / D, c = i % D;
      st_part(&part[h * hs + c], s_o[i]);
      if (c == 0) {
        st_part(&part[h * hs + D], s_ml[h][0]);        // log2 domain
        st_part(&part[h * hs + D + 1], s_ml[h][1]);
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
      if (lane == 0) { s_ml[h][0] = m; s_ml[h][1] = l; }
    }
    __syncthreads();
    for (int i = tid; i < G * D; i += 256) {
      const int h = i / D, c = i % D;
      float o = 0.0f;
#pragma unroll 8
      for (int t = 0; t < kWinRowsLds; ++t) o += s_sc[h * kWinRowsLds + t] * s_v[t * kRow + c];
      st_part(&part[h * hs + c], o);
      if (c == 0) {
        st_part(&part[h * hs + D], s_ml[h][0]);
        st_part(&part[h * hs + D + 1], s_ml[h][1]);
      }
    }
  }

}

// ---------------------------------------------------------------------------
// Combine: one workgroup per (query head, sequence).  Thread (quarter sq,
// channel pair c2) folds the splits sq, sq + 4, ... with an online
// log-sum-exp, 128 splits per pass: the pass's (m, l) go through LDS while
// every thread's 32 partial loads are in flight, so a pass costs one memory
// round trip.  The four quarters are merged in LDS; the rotated tile part
// gets one inverse WHT, the raw window part is added, and the result is
// divided by L.
// ---------------------------------------------------------------------------
constexpr int kCombinePass = 128;

__global__ void __launch_bounds__(256) decode_combine128_kernel(DecodeParams P) {
  const int hq = blockIdx.x;
  const int b = blockIdx.y;
  const int tid = threadIdx.x;
  const int sq = tid >> 6, c2 = (tid & 63) * 2;
  const int n_split = P.n_tsplit + P.n_wsplit;
  const float* ph = P.part + ((int64_t)b * P.n_q + hq) * (int64_t)n_split * (D + 4);
  __shared__ float s_pm[kCombinePass], s_pl[kCombinePass];
  __shared__ float s_m[4][64], s_l[4][64];
  __shared__ __attribute__((aligned(16))) float s_o[4][2][D];

  float M = -INFINITY, L = 0.0f;
  float t0 = 0.f, t1 = 0.f, w0 = 0.f, w1 = 0.f;
  for (int base = 0; base < n_split; base += kCombinePass) {
    float2 v[kCombinePass / 4];
#pragma unroll
    for (int j = 0; j < kCombinePass / 4; ++j) {
      const int s = base + sq + 4 * j;
      v[j] = (s < n_split) ? *reinterpret_cast<const float2*>(ph + (int64_t)s * (D + 4) + c2)
                           : make_float2(0.f, 0.f);
    }
    if (tid < kCombinePass) {
      const int s = base + tid;
      s_pm[tid] = (s < n_split) ? ph[(int64_t)s * (D + 4) + D] : -INFINITY;
      s_pl[tid] = (s < n_split) ? ph[(int64_t)s * (D + 4) + D + 1] : 0.0f;
    }
    __syncthreads();
    float mc = -INFINITY;
#pragma unroll
    for (int j = 0; j < kCombinePass / 4; ++j) mc = fmaxf(mc, s_pm[sq + 4 * j]);
    if (mc > M) {
      const float r = __builtin_amdgcn_exp2f(M - mc);   // 0 when M = -inf
      L *= r; t0 *= r; t1 *= r; w0 *= r; w1 *= r;
      M = mc;
    }
#pragma unroll
    for (int j = 0; j < kCombinePass / 4; ++j) {
      const float m = s_pm[sq + 4 * j];
      const float wt = (m == -INFINITY) ? 0.0f : __builtin_amdgcn_exp2f(m - M);
      L += wt * s_pl[sq + 4 * j];
      if (base + sq + 4 * j < P.n_tsplit) { t0 += wt * v[j].x; t1 += wt * v[j].y; }
      else { w0 += wt * v[j].x; w1 += wt * v[j].y; }
    }
    __syncthreads();   // s_pm / s_pl are rewritten by the next pass
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
