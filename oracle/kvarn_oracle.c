/*
 * kvarn_oracle.c -- plain, slow CPU oracle for the KVarN KV-cache hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may load, call or
 * link this file; only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or constant with the
 * HIP library.
 *
 * What it computes, and where the method is stated:
 *   - SharpInference issue #180 "Implement KVarN variance-normalized KV-cache
 *     quantization (2-bit values)", section "Algorithm (per 128-token tile)":
 *     step 1 Hadamard rotation along the channel dim (orthonormal), step 2
 *     dual-axis "Sinkhorn" variance normalisation (alternating per-channel /
 *     per-token std normalisation), step 3 asymmetric RTN (per-channel keys,
 *     per-token values, group 128), step 4 scales folded at read time,
 *     preset kvarn_k4v2_g128 (4-bit K / 2-bit V).
 *   - SharpInference PR #434 "KVarN variance-normalized KV-cache quantization:
 *     CPU + CUDA (#180)", commit list: channel-major K / token-major V packing
 *     in 128-token tiles, 2-bit bit packing; "Measured" table: the capacity
 *     figure that fixes the record size.
 *   - gmlx PR #116 "KVarN variance-normalized KV cache", commit list: mixed
 *     key / value widths ("k6v5"-style arms, widths set per side): the
 *     *_w functions take kb-bit keys and vb-bit values (1..8 bits each),
 *     packed as LSB-first bit streams.
 *
 * Precision.  Compression is an encoding: the packed codes are decided in
 * fp32, and both this oracle and the GPU path must make every decision in the
 * same precision with the same operation order.  So the compressor below is a
 * literal fp32 program with a fixed order: one IEEE operation per line, no
 * fused multiply-add (compile with -ffp-contract=off), no reassociation.
 * The dequantised cache and attention are evaluated in fp64.
 *
 * Readings of the pages (the pages give no formulas; these are the plain
 * readings, listed in the design notes):
 *   WHT: Sylvester Hadamard, butterfly stages in ascending stride h = 1..d/2,
 *        then one multiply by fp32(1/sqrt(d)); no random signs (self-inverse).
 *   Sum order: every fp32 sum is a pairwise sum over contiguous halves.
 *   Sinkhorn: std read as RMS about zero; alternation written as
 *        Sinkhorn-Knopp scaling of the squared tile X*X to unit row and column
 *        means (the log-space alternation is the same map without logs);
 *        8 iterations, channel step then token step; a mean below FLT_MIN
 *        (all-zero row or column) is replaced by 1.
 *   RTN: delta = (max-min)/(2^b-1), code = clamp(rint((x-min)*(1/delta))),
 *        round half to even; delta below FLT_MIN gives all codes 0; a zero
 *        min or max is taken as +0.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define TILE 128 /* tokens per tile */

/* ------------------------------------------------------------------ */
/* Sizes and record layout (byte offsets inside one tile-head record)   */
/* ------------------------------------------------------------------ */

static int valid_dim(int d) { return d == 128 || d == 256 || d == 512; }

/* Scale formats of the record: 0 = fp32 scales (116 d + 512 bytes), 1 = f16
 * scales, each fp32 scale rounded to nearest-even half precision (SharpInference
 * issue #433 item 3, "f16 scales": 106 d + 256 bytes, 108 B per token per KV
 * head at d = 128).  The codes are the same in both formats. */
long long oracle_tile_bytes_fmt(int d, int fmt) {
  if (!valid_dim(d) || (fmt != 0 && fmt != 1)) return 0;
  return fmt ? 106LL * d + 256 : 116LL * d + 512;
}
long long oracle_tile_bytes(int d) { return oracle_tile_bytes_fmt(d, 0); }

/* Code widths (SharpInference gmlx PR #116 commit list: mixed-width "k6v5"
 * arms, key and value widths set on their own): kb-bit keys and vb-bit values,
 * 1 <= kb, vb <= 8, levels 2^b - 1.  Codes are an LSB-first bit stream: the
 * code of token t in channel c's key stream starts at bit kb*t, the code of
 * channel c in token t's value stream at bit vb*c.  K4V2 is kb = 4, vb = 2:
 * 64 bytes per channel, d/4 bytes per token. */
static int valid_bits(int b) { return b >= 1 && b <= 8; }

long long oracle_tile_bytes_w(int d, int fmt, int kb, int vb) {
  if (!valid_dim(d) || (fmt != 0 && fmt != 1) || !valid_bits(kb) || !valid_bits(vb)) return 0;
  const long long w = fmt ? 2 : 4;
  return 16LL * d * (kb + vb) + w * (128 + 5LL * d);
}

/* offsets: K codes, V codes, ktok, kscale, kmin, vchan, vscale, vmin, end */
static void layout_w(int d, int fmt, int kb, int vb, long long off[9]) {
  const long long w = fmt ? 2 : 4;   /* bytes per scale */
  off[0] = 0;                 /* K codes  [d][16 kb] bytes     */
  off[1] = 16LL * kb * d;     /* V codes  [128][d vb / 8]      */
  off[2] = off[1] + 16LL * vb * d;   /* ktok [128]             */
  off[3] = off[2] + 128 * w;  /* kscale   [d]                  */
  off[4] = off[3] + d * w;    /* kmin     [d]                  */
  off[5] = off[4] + d * w;    /* vchan    [d]                  */
  off[6] = off[5] + d * w;    /* vscale   [128][d/128]         */
  off[7] = off[6] + d * w;    /* vmin     [128][d/128]         */
  off[8] = off[7] + d * w;    /* end                           */
}
static void layout_fmt(int d, int fmt, long long off[9]) { layout_w(d, fmt, 4, 2, off); }
static void layout(int d, long long off[9]) { layout_fmt(d, 0, off); }

void oracle_layout(int d, long long* off) { layout(d, off); }
void oracle_layout_fmt(int d, int fmt, long long* off) { layout_fmt(d, fmt, off); }
void oracle_layout_w(int d, int fmt, int kb, int vb, long long* off) { layout_w(d, fmt, kb, vb, off); }

/* IEEE binary32 -> binary16 bits, round to nearest, ties to even (overflow
 * to infinity, NaN stays NaN), and back (exact). */
static uint32_t rshift_rne(uint32_t x, int s) {
  if (s <= 0) return x;
  if (s >= 32) return 0;
  const uint32_t q = x >> s, rem = x & ((1u << s) - 1), half = 1u << (s - 1);
  return q + ((rem > half || (rem == half && (q & 1))) ? 1u : 0u);
}
uint16_t oracle_f32_to_f16(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  const uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
  const int e = (int)((u >> 23) & 0xff);
  const uint32_t m = u & 0x7fffffu;
  if (e == 255) return (uint16_t)(sign | 0x7c00u | (m ? 0x200u : 0u));
  const int E = e - 127 + 15;
  if (E >= 31) return (uint16_t)(sign | 0x7c00u);
  if (E <= 0) {   /* subnormal half (or zero): value = M 2^-24 */
    if (e == 0) return sign;   /* fp32 zero or subnormal: far below half's range */
    const uint32_t M = rshift_rne(m | 0x800000u, 14 - E);
    return (uint16_t)(sign | M);   /* M = 0x400 is the smallest normal: still correct bits */
  }
  uint32_t mh = rshift_rne(m, 13);
  uint32_t eh = (uint32_t)E;
  if (mh == 0x400u) { mh = 0; eh += 1; }
  if (eh >= 31) return (uint16_t)(sign | 0x7c00u);
  return (uint16_t)(sign | (eh << 10) | mh);
}
float oracle_f16_to_f32(uint16_t h) {
  const int e = (h >> 10) & 31, m = h & 1023;
  float v;
  if (e == 0) v = ldexpf((float)m, -24);
  else if (e == 31) v = m ? NAN : INFINITY;
  else v = ldexpf((float)(1024 + m), e - 25);
  return (h & 0x8000) ? -v : v;
}

/* ------------------------------------------------------------------ */
/* Walsh-Hadamard transform (fp32, fixed order)                         */
/* ------------------------------------------------------------------ */

/* fp32(1/sqrt(d)) for d = 2^k: 2^(-k/2) exactly when k is even, otherwise
 * fp32(sqrt(2)) * 2^(-(k+1)/2), which is exact scaling of the rounded sqrt(2)
 * and therefore the correctly rounded value of 2^(-k/2). */
float oracle_wht_scale(int d) {
  int k = 0;
  while ((1 << k) < d) k++;
  if ((k & 1) == 0) return ldexpf(1.0f, -k / 2);
  return ldexpf(0x1.6a09e6p+0f, -(k + 1) / 2);
}

void oracle_wht_f32(float* x, int d) {
  for (int h = 1; h < d; h <<= 1) {
    for (int i = 0; i < d; i++) {
      if ((i & h) == 0) {
        float a = x[i];
        float b = x[i + h];
        x[i] = a + b;
        x[i + h] = a - b;
      }
    }
  }
  float c = oracle_wht_scale(d);
  for (int i = 0; i < d; i++) x[i] = x[i] * c;
}

/* ------------------------------------------------------------------ */
/* Pairwise sum over contiguous halves (n a power of two)               */
/* ------------------------------------------------------------------ */

float oracle_pairwise_sum_f32(const float* y, int n) {
  if (n == 1) return y[0];
  float left = oracle_pairwise_sum_f32(y, n / 2);
  float right = oracle_pairwise_sum_f32(y + n / 2, n / 2);
  return left + right;
}

/* ------------------------------------------------------------------ */
/* Sinkhorn variance normalisation of one rotated tile X[128][d]        */
/* ------------------------------------------------------------------ */

/* Outputs the per-token spread r[128] and the per-channel spread s[d] such
 * that X[t][c] / (r[t] * s[c]) has unit mean square along both axes (the
 * token axis exactly after the last step, the channel axis to convergence). */
void oracle_sinkhorn_f32(const float* X, int d, int iters, float* r, float* s) {
  float* Q = (float*)malloc(sizeof(float) * TILE * d);
  float* buf = (float*)malloc(sizeof(float) * (d > TILE ? d : TILE));
  float u[TILE];   /* 1 / r^2 */
  float mt[TILE];  /* token mean squares (r^2) */
  float* v = (float*)malloc(sizeof(float) * d);   /* 1 / s^2 */
  float* mc = (float*)malloc(sizeof(float) * d);  /* channel mean squares (s^2) */
  const float inv_t = 1.0f / (float)TILE; /* exact power of two */
  const float inv_d = 1.0f / (float)d;    /* exact power of two */

  for (int t = 0; t < TILE; t++)
    for (int c = 0; c < d; c++) Q[t * d + c] = X[t * d + c] * X[t * d + c];
  for (int t = 0; t < TILE; t++) { u[t] = 1.0f; mt[t] = 1.0f; }
  for (int c = 0; c < d; c++) { v[c] = 1.0f; mc[c] = 1.0f; }

  for (int it = 0; it < iters; it++) {
    /* channel step: mean over tokens of Q * u */
    for (int c = 0; c < d; c++) {
      for (int t = 0; t < TILE; t++) buf[t] = Q[t * d + c] * u[t];
      float m = oracle_pairwise_sum_f32(buf, TILE) * inv_t;
      if (!(m >= FLT_MIN)) m = 1.0f;
      mc[c] = m;
      v[c] = 1.0f / m;
    }
    /* token step: mean over channels of Q * v */
    for (int t = 0; t < TILE; t++) {
      for (int c = 0; c < d; c++) buf[c] = Q[t * d + c] * v[c];
      float m = oracle_pairwise_sum_f32(buf, d) * inv_d;
      if (!(m >= FLT_MIN)) m = 1.0f;
      mt[t] = m;
      u[t] = 1.0f / m;
    }
  }
  for (int c = 0; c < d; c++) s[c] = sqrtf(mc[c]);
  for (int t = 0; t < TILE; t++) r[t] = sqrtf(mt[t]);
  free(Q); free(buf); free(v); free(mc);
}

/* Xn[t][c] = (X[t][c] * (1/r[t])) * (1/s[c]) */
void oracle_normalise_f32(const float* X, int d, const float* r, const float* s,
                          float* Xn) {
  for (int t = 0; t < TILE; t++) {
    float ir = 1.0f / r[t];
    for (int c = 0; c < d; c++) {
      float is = 1.0f / s[c];
      Xn[t * d + c] = (X[t * d + c] * ir) * is;
    }
  }
}

/* ------------------------------------------------------------------ */
/* Asymmetric round-to-nearest over one group                           */
/* ------------------------------------------------------------------ */

/* x[i * stride] for i < n; levels = 2^bits - 1.  Writes codes[i * cstride]. */
void oracle_rtn_group(const float* x, int n, int stride, int levels,
                      float* lo_out, float* delta_out,
                      uint8_t* codes, int cstride) {
  float lo = x[0], hi = x[0];
  for (int i = 1; i < n; i++) {
    float e = x[i * stride];
    if (e < lo) lo = e;
    if (e > hi) hi = e;
  }
  /* -0 and +0 compare equal; adding +0 makes a zero endpoint +0 so the
   * stored min and step have one bit pattern whatever order found it. */
  lo = lo + 0.0f;
  hi = hi + 0.0f;
  float delta = (hi - lo) / (float)levels;
  float inv = (delta >= FLT_MIN) ? 1.0f / delta : 0.0f;
  for (int i = 0; i < n; i++) {
    float q = (x[i * stride] - lo) * inv;
    float z = rintf(q); /* round half to even in the default rounding mode */
    if (!(z >= 0.0f)) z = 0.0f;
    if (z > (float)levels) z = (float)levels;
    codes[i * cstride] = (uint8_t)z;
  }
  *lo_out = lo;
  *delta_out = delta;
}

/* ------------------------------------------------------------------ */
/* Whole-tile compression into one record                               */
/* ------------------------------------------------------------------ */

/* Everything the compressor decides for one tile-head, before packing. */
typedef struct {
  float rK[TILE], sK[512], rV[TILE], sV[512];
  float loK[512], dK[512];
  float loV[TILE * 4], dV[TILE * 4];
  uint8_t zK[TILE * 512], zV[TILE * 512]; /* [t][c] */
} tile_parts;

static void compress_one(const float* src, long long tok_stride, int d, int iters,
                         float* r, float* s, uint8_t* z, float* lo, float* dl,
                         int is_key, int levels) {
  float* X = (float*)malloc(sizeof(float) * TILE * d);
  float* Xn = (float*)malloc(sizeof(float) * TILE * d);
  for (int t = 0; t < TILE; t++) {
    for (int c = 0; c < d; c++) X[t * d + c] = src[(long long)t * tok_stride + c];
    oracle_wht_f32(X + t * d, d);
  }
  oracle_sinkhorn_f32(X, d, iters, r, s);
  oracle_normalise_f32(X, d, r, s, Xn);
  if (is_key) {
    /* per channel over the tile's 128 tokens */
    for (int c = 0; c < d; c++)
      oracle_rtn_group(Xn + c, TILE, d, levels, &lo[c], &dl[c], z + c, d);
  } else {
    /* per token over each group of 128 channels */
    int ng = d / 128;
    for (int t = 0; t < TILE; t++)
      for (int g = 0; g < ng; g++)
        oracle_rtn_group(Xn + t * d + 128 * g, 128, 1, levels, &lo[t * ng + g],
                         &dl[t * ng + g], z + t * d + 128 * g, 1);
  }
  free(X);
  free(Xn);
}

static void put_scale(uint8_t* rec, long long off, int i, float v, int fmt) {
  if (fmt) {
    const uint16_t h = oracle_f32_to_f16(v);
    memcpy(rec + off + 2LL * i, &h, 2);
  } else {
    memcpy(rec + off + 4LL * i, &v, 4);
  }
}

/* Everything the compressor decides for one tile-head: RTN with 2^kb - 1
 * levels for the keys and 2^vb - 1 for the values.  Caller frees. */
static tile_parts* tile_decide(const float* k, const float* v, long long tok_stride, int d,
                               int iters, int kb, int vb) {
  tile_parts* P = (tile_parts*)calloc(1, sizeof(tile_parts));
  compress_one(k, tok_stride, d, iters, P->rK, P->sK, P->zK, P->loK, P->dK, 1, (1 << kb) - 1);
  compress_one(v, tok_stride, d, iters, P->rV, P->sV, P->zV, P->loV, P->dV, 0, (1 << vb) - 1);
  return P;
}

/* folded scales: single fp32 multiplies */
static void put_scales(uint8_t* rec, const long long off[9], const tile_parts* P, int d, int fmt) {
  for (int t = 0; t < TILE; t++) put_scale(rec, off[2], t, P->rK[t], fmt);
  for (int c = 0; c < d; c++) {
    put_scale(rec, off[3], c, P->dK[c] * P->sK[c], fmt);
    put_scale(rec, off[4], c, P->loK[c] * P->sK[c], fmt);
    put_scale(rec, off[5], c, P->sV[c], fmt);
  }
  int ng = d / 128;
  for (int t = 0; t < TILE; t++)
    for (int g = 0; g < ng; g++) {
      put_scale(rec, off[6], t * ng + g, P->dV[t * ng + g] * P->rV[t], fmt);
      put_scale(rec, off[7], t * ng + g, P->loV[t * ng + g] * P->rV[t], fmt);
    }
}

/* K4V2 packing, nibble by nibble and crumb by crumb. */
static void pack_k4v2(uint8_t* rec, const long long off[9], const tile_parts* P, int d) {
  /* K codes, channel-major: byte j of channel c = tokens 2j (low), 2j+1 (high) */
  for (int c = 0; c < d; c++)
    for (int j = 0; j < TILE / 2; j++)
      rec[off[0] + 64LL * c + j] =
          (uint8_t)(P->zK[(2 * j) * d + c] | (P->zK[(2 * j + 1) * d + c] << 4));
  /* V codes, token-major: byte j of token t = channels 4j+i at bits 2i */
  for (int t = 0; t < TILE; t++)
    for (int j = 0; j < d / 4; j++) {
      int b = 0;
      for (int i = 0; i < 4; i++) b |= P->zV[t * d + 4 * j + i] << (2 * i);
      rec[off[1] + (long long)t * (d / 4) + j] = (uint8_t)b;
    }
}

/* Any widths: a b-bit code goes one bit at a time into an LSB-first stream
 * (bit i of the stream is bit i % 8 of byte i / 8). */
static void put_code(uint8_t* stream, long long bit0, int b, unsigned code) {
  for (int i = 0; i < b; i++)
    if ((code >> i) & 1u) stream[(bit0 + i) >> 3] |= (uint8_t)(1u << ((bit0 + i) & 7));
}
static unsigned get_code(const uint8_t* stream, long long bit0, int b) {
  unsigned code = 0;
  for (int i = 0; i < b; i++) code |= (unsigned)((stream[(bit0 + i) >> 3] >> ((bit0 + i) & 7)) & 1u) << i;
  return code;
}
static void pack_bits(uint8_t* rec, const long long off[9], const tile_parts* P, int d, int kb,
                      int vb) {
  /* K: channel c's stream of 16 kb bytes, token t at bit kb t */
  for (int c = 0; c < d; c++)
    for (int t = 0; t < TILE; t++)
      put_code(rec + off[0] + 16LL * kb * c, (long long)kb * t, kb, P->zK[t * d + c]);
  /* V: token t's stream of d vb / 8 bytes, channel c at bit vb c */
  for (int t = 0; t < TILE; t++)
    for (int c = 0; c < d; c++)
      put_code(rec + off[1] + (long long)t * d * vb / 8, (long long)vb * c, vb, P->zV[t * d + c]);
}

/* Compress the K and V tiles of one (tile, kv head).  k and v point at token
 * 0 channel 0; token t starts tok_stride floats later.  Writes
 * oracle_tile_bytes_fmt(d, fmt) bytes to rec.  Returns 0 on success, -1 for
 * an unsupported head_dim or format. */
int oracle_compress_tile_fmt(const float* k, const float* v, long long tok_stride,
                             int d, int iters, int fmt, uint8_t* rec) {
  if (!valid_dim(d) || (fmt != 0 && fmt != 1)) return -1;
  tile_parts* P = tile_decide(k, v, tok_stride, d, iters, 4, 2);
  long long off[9];
  layout_fmt(d, fmt, off);
  memset(rec, 0, (size_t)off[8]);
  pack_k4v2(rec, off, P, d);
  put_scales(rec, off, P, d, fmt);
  free(P);
  return 0;
}

int oracle_compress_tile(const float* k, const float* v, long long tok_stride,
                         int d, int iters, uint8_t* rec) {
  return oracle_compress_tile_fmt(k, v, tok_stride, d, iters, 0, rec);
}

/* The same with kb-bit keys and vb-bit values, packed by the bit-stream
 * writer.  Writes oracle_tile_bytes_w(d, fmt, kb, vb) bytes. */
int oracle_compress_tile_w(const float* k, const float* v, long long tok_stride, int d,
                           int iters, int fmt, int kb, int vb, uint8_t* rec) {
  if (!oracle_tile_bytes_w(d, fmt, kb, vb)) return -1;
  tile_parts* P = tile_decide(k, v, tok_stride, d, iters, kb, vb);
  long long off[9];
  layout_w(d, fmt, kb, vb, off);
  memset(rec, 0, (size_t)off[8]);
  pack_bits(rec, off, P, d, kb, vb);
  put_scales(rec, off, P, d, fmt);
  free(P);
  return 0;
}

/* The unpacked codes of a K4V2 record: zK[t][c] and zV[t][c]. */
void oracle_unpack_codes(const uint8_t* rec, int d, uint8_t* zK, uint8_t* zV) {
  long long off[9];
  layout(d, off);
  for (int c = 0; c < d; c++)
    for (int j = 0; j < TILE / 2; j++) {
      uint8_t b = rec[off[0] + 64LL * c + j];
      zK[(2 * j) * d + c] = b & 15;
      zK[(2 * j + 1) * d + c] = b >> 4;
    }
  for (int t = 0; t < TILE; t++)
    for (int c = 0; c < d; c++) {
      uint8_t b = rec[off[1] + (long long)t * (d / 4) + c / 4];
      zV[t * d + c] = (b >> (2 * (c % 4))) & 3;
    }
}

/* The unpacked codes of a record with kb-bit keys and vb-bit values. */
void oracle_unpack_codes_w(const uint8_t* rec, int d, int kb, int vb, uint8_t* zK, uint8_t* zV) {
  long long off[9];
  layout_w(d, 0, kb, vb, off);   /* code sections do not depend on the scale format */
  for (int c = 0; c < d; c++)
    for (int t = 0; t < TILE; t++)
      zK[t * d + c] = (uint8_t)get_code(rec + off[0] + 16LL * kb * c, (long long)kb * t, kb);
  for (int t = 0; t < TILE; t++)
    for (int c = 0; c < d; c++)
      zV[t * d + c] = (uint8_t)get_code(rec + off[1] + (long long)t * d * vb / 8, (long long)vb * c, vb);
}

/* ------------------------------------------------------------------ */
/* Dequantised cache in fp64                                            */
/* ------------------------------------------------------------------ */

static double get_scale(const uint8_t* rec, long long off, int i, int fmt) {
  if (fmt) {
    uint16_t h;
    memcpy(&h, rec + off + 2LL * i, 2);
    return (double)oracle_f16_to_f32(h);
  }
  float v;
  memcpy(&v, rec + off + 4LL * i, 4);
  return (double)v;
}


/* H[i][j] = (-1)^popcount(i & j) / sqrt(d), applied to one fp64 row. */
static void hadamard_f64(const double* x, double* y, int d) {
  double c = 1.0 / sqrt((double)d);
  for (int i = 0; i < d; i++) {
    double acc = 0.0;
    for (int j = 0; j < d; j++) {
      double h = (__builtin_popcount((unsigned)(i & j)) & 1) ? -1.0 : 1.0;
      acc += h * x[j];
    }
    y[i] = acc * c;
  }
}

/* Dequantise one record to the raw (unrotated) domain from its codes:
 *   k'[t][c] = ktok[t] * (zK[t][c] * kscale[c] + kmin[c])
 *   v'[t][c] = vchan[c] * (zV[t][c] * vscale[t][g] + vmin[t][g])
 *   khat = H k', vhat = H v'  (H is its own inverse)
 * If rotated_only is nonzero the rotation is skipped (k', v' are returned). */
static void dequant_codes(const uint8_t* rec, const long long off[9], int d, int fmt,
                          const uint8_t* zK, const uint8_t* zV, int rotated_only,
                          double* khat, double* vhat) {
  double* row = (double*)malloc(sizeof(double) * d);
  int ng = d / 128;
  for (int t = 0; t < TILE; t++) {
    double ktok = get_scale(rec, off[2], t, fmt);
    for (int c = 0; c < d; c++)
      row[c] = ktok * ((double)zK[t * d + c] * get_scale(rec, off[3], c, fmt) +
                       get_scale(rec, off[4], c, fmt));
    if (rotated_only) memcpy(khat + (long long)t * d, row, sizeof(double) * d);
    else hadamard_f64(row, khat + (long long)t * d, d);
    for (int c = 0; c < d; c++) {
      int g = c / 128;
      row[c] = get_scale(rec, off[5], c, fmt) *
               ((double)zV[t * d + c] * get_scale(rec, off[6], t * ng + g, fmt) +
                get_scale(rec, off[7], t * ng + g, fmt));
    }
    if (rotated_only) memcpy(vhat + (long long)t * d, row, sizeof(double) * d);
    else hadamard_f64(row, vhat + (long long)t * d, d);
  }
  free(row);
}

void oracle_dequant_f64_fmt(const uint8_t* rec, int d, int fmt, int rotated_only,
                            double* khat, double* vhat) {
  long long off[9];
  layout_fmt(d, fmt, off);
  uint8_t* zK = (uint8_t*)malloc((size_t)TILE * d);
  uint8_t* zV = (uint8_t*)malloc((size_t)TILE * d);
  oracle_unpack_codes(rec, d, zK, zV);
  dequant_codes(rec, off, d, fmt, zK, zV, rotated_only, khat, vhat);
  free(zK); free(zV);
}

void oracle_dequant_f64(const uint8_t* rec, int d, int rotated_only, double* khat, double* vhat) {
  oracle_dequant_f64_fmt(rec, d, 0, rotated_only, khat, vhat);
}

void oracle_dequant_f64_w(const uint8_t* rec, int d, int fmt, int kb, int vb, int rotated_only,
                          double* khat, double* vhat) {
  long long off[9];
  layout_w(d, fmt, kb, vb, off);
  uint8_t* zK = (uint8_t*)malloc((size_t)TILE * d);
  uint8_t* zV = (uint8_t*)malloc((size_t)TILE * d);
  oracle_unpack_codes_w(rec, d, kb, vb, zK, zV);
  dequant_codes(rec, off, d, fmt, zK, zV, rotated_only, khat, vhat);
  free(zK); free(zV);
}

/* ------------------------------------------------------------------ */
/* Textbook softmax attention in fp64                                   */
/* ------------------------------------------------------------------ */

/* One query over n keys/values (rows of d doubles):
 *   s_j = scale * (q . k_j),  p = softmax(s),  out = sum_j p_j v_j.
 * Writes the natural-log LSE of the scaled scores to *lse if non-null. */
void oracle_attend_f64(const double* q, const double* keys, const double* vals,
                       long long n, int d, double scale, double* out, double* lse) {
  double* s = (double*)malloc(sizeof(double) * (size_t)(n > 0 ? n : 1));
  double m = -INFINITY;
  for (long long j = 0; j < n; j++) {
    double acc = 0.0;
    for (int c = 0; c < d; c++) acc += q[c] * keys[j * d + c];
    s[j] = scale * acc;
    if (s[j] > m) m = s[j];
  }
  double l = 0.0;
  for (int c = 0; c < d; c++) out[c] = 0.0;
  for (long long j = 0; j < n; j++) {
    double p = exp(s[j] - m);
    l += p;
    for (int c = 0; c < d; c++) out[c] += p * vals[j * d + c];
  }
  for (int c = 0; c < d; c++) out[c] /= l;
  if (lse) *lse = m + log(l);
  free(s);
}
