/*
 * kvarn.h -- C ABI of the KVarN hot path on AMD Instinct MI355X (gfx950).
 *
 * KVarN is calibration-free KV-cache quantisation with 4-bit keys and 2-bit
 * values.  Method statement: SharpInference issue #180 "Implement KVarN
 * variance-normalized KV-cache quantization (2-bit values)", section
 * "Algorithm (per 128-token tile)": (1) Hadamard rotation along the channel
 * dim, (2) dual-axis Sinkhorn variance normalisation, (3) asymmetric RTN,
 * per-channel keys / per-token values, group 128, (4) scales folded at read
 * time, preset kvarn_k4v2_g128.  The four calls below are the kernels the
 * SharpInference PR #434 commit list names (rotate query, compress tile,
 * decode attention, chunked prefill attention).
 *
 * Conventions for every call:
 *   - Device pointers are HIP device memory; "host" arrays are read during
 *     the call and not retained.  The library never allocates, frees or
 *     synchronises and keeps no pointer after returning.
 *   - Arguments are validated on the host before anything is enqueued; a
 *     non-zero status means nothing was launched.  KVARN_OK means the kernels
 *     were enqueued on `stream` (a hipStream_t; NULL is the null stream).
 *     A launch failure reported by HIP returns KVARN_E_DEVICE.
 *   - Device pointers and strides (in bytes) must be 16-byte aligned.
 *   - fp32 throughout; non-finite inputs give undefined results (not checked).
 *   - Results are bitwise reproducible run to run for the same arguments.
 *   - The method's parameters are not call arguments: the group (128 tokens
 *     per tile, 128 channels per value group) and the 8 Sinkhorn iterations
 *     are fixed by issue #180's preset kvarn_k4v2_g128; the record format
 *     (head_dim, f16 scales, code widths) is one head_dim word (below).
 *     Records are written contiguously, [tile][KV head], and decode reads
 *     them through per-sequence start rows of a pool.
 *
 * Tile record (one per 128-token tile and KV head), kvarn_tile_bytes(d) =
 * 116*d + 512 bytes, every section 16-byte aligned:
 *     [0, 64d)            K codes, channel-major: 64 bytes per channel c; byte j
 *                         holds token 2j in bits 0-3 and token 2j+1 in bits 4-7
 *     [64d, 96d)          V codes, token-major: d/4 bytes per token t; byte j
 *                         holds channel 4j+i in bits 2i..2i+1
 *     [96d, +512)         ktok[128]    per-token key spread r_t
 *     [96d+512, +4d)      kscale[d]    delta_c * s_c  (key step times channel spread)
 *     [100d+512, +4d)     kmin[d]      min_c * s_c
 *     [104d+512, +4d)     vchan[d]     value channel spread s_c
 *     [108d+512, +4d)     vscale[128][d/128]  delta_{t,g} * r_t
 *     [112d+512, +4d)     vmin[128][d/128]    min_{t,g} * r_t
 *   Rotated-domain dequantisation: k'[t][c] = ktok_t (z*kscale_c + kmin_c),
 *   v'[t][c] = vchan_c (z*vscale_{t,g} + vmin_{t,g}); keys and values in the
 *   original domain are H k', H v' with H the orthonormal Walsh-Hadamard
 *   matrix (its own inverse).  The record size is the one the capacity figure
 *   in PR #434's "Measured" table implies (six fp32 vectors per tile-head).
 *
 * Record with f16 scales (issue #433 item 3, "f16 scales in the packed tile
 * layout"): a head_dim argument OR-ed with KVARN_SCALES_F16 selects it in
 * every call.  Same codes and section order; each scale is the fp32 value
 * above rounded to the nearest binary16 (ties to even), so the sections are
 * half as long and the record is 106*d + 256 bytes (108 bytes per token at
 * d = 128 instead of 120).  The codes are those of the fp32 record: only the
 * stored scales are rounded.
 *
 * Code widths (gmlx PR #116 commit list: mixed-width "k6v5"-style arms, key
 * and value widths set on their own): a head_dim argument OR-ed with
 * KVARN_KEY_BITS(kb) and KVARN_VALUE_BITS(vb), 1 <= kb, vb <= 8, selects RTN
 * with 2^kb - 1 key levels and 2^vb - 1 value levels.  The code sections become
 * LSB-first bit streams: key channel c's stream is 16*kb bytes at 16*kb*c with
 * token t at bit kb*t; value token t's stream is d*vb/8 bytes at 16*kb*d +
 * t*d*vb/8 with channel c at bit vb*c (for kb = 4, vb = 2: the layout above).
 * The six scale sections follow at 16*d*(kb+vb) in the same order, so the
 * record is 16*d*(kb+vb) + 20*d + 512 bytes (10*d + 256 with f16 scales).
 * K4V2 records run on the matrix units (at head_dim 256 and 512 the raw
 * window part of decode runs on the vector units, and prefill needs a
 * workspace); other widths run decode and prefill on the vector-unit
 * kernels (a q_rot is then required, prefill needs a workspace, and
 * multi-query verify is unsupported).
 *
 * FP32 window and promotion (PR #434 commit list: "the FP32 window is the
 * staging; whole-tile promotion"): with a window of W tokens, the oldest 128
 * raw tokens are compressed into one tile when the window reaches W+128, so
 * after token p a sequence holds T(p) = max(0, floor((p+1-W)/128)) tiles and
 * raw tokens [128*T(p), p].
 */
#ifndef KVARN_H
#define KVARN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVARN_TILE_TOKENS 128
#define KVARN_MAX_BATCH 64
/* OR into any head_dim argument: records carry f16 scales (see above). */
#define KVARN_SCALES_F16 0x10000
/* OR into any head_dim argument: key / value code widths 1..8 (see above);
 * a zero field means the default (4-bit keys, 2-bit values). */
#define KVARN_KEY_BITS(b) (((b) & 0xF) << 20)
#define KVARN_VALUE_BITS(b) (((b) & 0xF) << 24)

typedef enum kvarn_status {
  KVARN_OK = 0,
  KVARN_E_INVALID = 1,     /* null pointer, negative or inconsistent sizes   */
  KVARN_E_UNSUPPORTED = 2, /* head_dim not 128/256/512 (with or without the
                              format flags), a code width above 8, GQA not
                              integral, or a size beyond a documented limit  */
  KVARN_E_ALIGN = 3,       /* pointer or stride not 16-byte aligned          */
  KVARN_E_WORKSPACE = 4,   /* workspace missing or smaller than required     */
  KVARN_E_DEVICE = 5       /* HIP reported an error at launch                */
} kvarn_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* kvarn_status_string(int status);

/* Bytes of one (tile, KV head) record: 116*d + 512 (106*d + 256 with
 * KVARN_SCALES_F16), d = head_dim without the flags; 16*d*(kb+vb) + 20*d + 512
 * (+ 10*d + 256 with f16 scales) for other code widths; 0 when d is not 128,
 * 256 or 512, a width is above 8, or an unknown bit is set. */
size_t kvarn_tile_bytes(int32_t head_dim);

/*
 * kvarn_compress_tile -- compress whole 128-token tiles of raw K and V.
 * Issue #180 "Algorithm (per 128-token tile)" steps 1-4, preset k4v2 g128,
 * 8 Sinkhorn iterations; PR #434 commit list (channel-major K, token-major V,
 * 2-bit packing).
 *
 *   k, v        device fp32.  Row t (0..127) of tile j, KV head h starts at
 *               k + (128*j + t)*tok_stride + h*head_stride (floats); its
 *               head_dim channels are contiguous.  Same for v.
 *   records     device, n_tiles*n_kv_heads*kvarn_tile_bytes(head_dim) bytes;
 *               record (j, h) is written at (j*n_kv_heads + h)*tile_bytes.
 * Codes and scales are a pure function of the tile's 128 rows, so they do not
 * depend on how a prompt is chunked.  n_tiles == 0 is a no-op.
 * Errors: KVARN_E_UNSUPPORTED (head_dim), KVARN_E_INVALID (null pointer,
 * n_tiles < 0, n_kv_heads < 1, strides < head_dim when n_tiles > 0),
 * KVARN_E_ALIGN.
 */
int kvarn_compress_tile(int32_t head_dim, int32_t n_tiles, int32_t n_kv_heads,
                        const float* k, const float* v,
                        int64_t tok_stride, int64_t head_stride,
                        void* records, void* stream);

/*
 * kvarn_rotate_query -- q_rot = H q per row (orthonormal Walsh-Hadamard along
 * head_dim).  PR #434 commit list (llm_kvarn_rotate_query); issue #180
 * Algorithm step 1 (the rotation preserves attention scores).
 *   q, q_rot    device fp32 [n_rows][head_dim], contiguous; may alias.
 * KVARN_SCALES_F16 in head_dim is accepted and has no effect here.
 * Errors: KVARN_E_UNSUPPORTED, KVARN_E_INVALID (null, n_rows < 0), KVARN_E_ALIGN.
 */
int kvarn_rotate_query(int32_t head_dim, int64_t n_rows, const float* q,
                       float* q_rot, void* stream);

/*
 * kvarn_decode_attention -- one query per (sequence, query head) over that
 * sequence's compressed tiles plus its raw FP32 window.  Issue #180 Algorithm
 * step 4 (scales folded at read time); PR #434 commit list (single streaming
 * softmax over compressed tiles + FP32 window, deferred inverse WHT); issue
 * #433 item 2 (split-tile decode: fixed worst-case grid, early exit, LSE
 * combine, inverse WHT after combining the rotated tile partials).
 *
 * For query head h the KV head is h / (n_q_heads / n_kv_heads).  Tile scores
 * use q_rot (from kvarn_rotate_query) against the rotated-domain records;
 * window scores use the raw q against raw keys.  out = softmax-weighted sum
 * in the original domain.
 */
typedef struct kvarn_decode_args {
  int32_t head_dim;        /* 128, 256 or 512, | KVARN_SCALES_F16 (f16 scales),
                              | KVARN_KEY_BITS / KVARN_VALUE_BITS (widths)      */
  int32_t batch;           /* 1..KVARN_MAX_BATCH sequences                      */
  int32_t n_q_heads;       /* multiple of n_kv_heads                            */
  int32_t n_kv_heads;
  float softmax_scale;     /* tau: scores are tau * q.k                         */
  int32_t max_tiles;       /* grid bound: >= n_tiles[b] for every b             */
  const float* q;          /* device [batch][n_q_heads][head_dim] raw query     */
  const float* q_rot;      /* device [batch][n_q_heads][head_dim] rotated query;
                              may be NULL with K4V2 records (any head_dim):
                              the kernels then rotate q themselves              */
  const void* records;     /* device record pool; record (b, j, h) at
                              ((rec_start[b] + j)*n_kv_heads + h)*tile_bytes    */
  int64_t n_record_rows;   /* rows in the pool (a row = n_kv_heads records)     */
  const int64_t* rec_start;/* host [batch]                                      */
  const int32_t* n_tiles;  /* host [batch] compressed tiles per sequence        */
  float* k_win;            /* device raw window keys: token i of sequence b,
                              KV head h at k_win + b*win_seq_stride +
                              (win_start[b] + i)*win_tok_stride +
                              h*win_head_stride (floats); written only at token
                              n_win[b] - 1, and only when k_new is given        */
  float* v_win;            /* device raw window values, same strides            */
  int64_t win_seq_stride, win_tok_stride, win_head_stride;
  const int64_t* win_start;/* host [batch] first window row of each sequence, or
                              NULL for all zero                                 */
  const int32_t* n_win;    /* host [batch] window tokens per sequence           */
  int32_t max_win;         /* grid bound: >= n_win[b] for every b               */
  float* out;              /* device [batch][n_q_heads][head_dim]               */
  int32_t q_len;           /* query rows per sequence, 0 or 1: one decode query;
                              2..8: multi-query verify (head_dim 128, K4V2
                              records).  Then q,
                              q_rot and out are [batch][q_len][n_q_heads][head_dim]
                              and row i of sequence b is the query of window token
                              n_win[b] - q_len + i: it sees the n_tiles[b] tiles
                              and window tokens [0, n_win[b] - q_len + i]
                              (n_win[b] >= q_len).  gmlx PR #116 commit list:
                              verify widths 2-8 attend the records on the matrix
                              units at about the cost of one decode step.       */
  const float* k_new;      /* device [batch][n_kv_heads][head_dim] keys of each
                              sequence's newest token, or NULL.  Given (with
                              v_new, q_len <= 1, n_win[b] >= 1), the call stores
                              them and v_new as window token n_win[b] - 1 of
                              sequence b (the window append of the PR #434
                              commit list: FP32 window staging) and attends them
                              as part of the window, so a decode step needs no
                              separate copy: the head_dim-128 K4V2 kernel
                              appends in the same launch, the other paths with
                              one small copy launch first.                      */
  const float* v_new;      /* device values of the newest token, same layout    */
} kvarn_decode_args;

/* Workspace bytes kvarn_decode_attention needs for these arguments (0 on
 * invalid arguments).  The workspace is device memory owned by the caller;
 * its contents need no initialisation and are scratch after the call.  Calls
 * that share a workspace must not overlap in time. */
size_t kvarn_decode_workspace_bytes(const kvarn_decode_args* args);

/* Errors: KVARN_E_INVALID (null pointers, counts out of range, a sequence with
 * no visible key, rec_start[b] + n_tiles[b] > n_record_rows, n_tiles[b] >
 * max_tiles, n_win[b] > max_win, win_start[b] < 0, q_len outside 0..8,
 * n_win[b] < q_len), KVARN_E_UNSUPPORTED (head_dim, GQA ratio, batch >
 * KVARN_MAX_BATCH, group of more than 8 query heads per KV head, q_len >= 2
 * with head_dim other than 128 or with other code widths),
 * KVARN_E_ALIGN, KVARN_E_WORKSPACE. */
int kvarn_decode_attention(const kvarn_decode_args* args, void* workspace,
                           size_t workspace_bytes, void* stream);

/*
 * kvarn_decode_attention_noalloc -- kvarn_decode_attention for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): the same kernels and the same
 * result, with the split partials in a library-owned device array of
 * KVARN_NOALLOC_SCRATCH_BYTES per GPU instead of a caller workspace.  The
 * caller still passes the inputs and the output in `args`.
 *
 *   - The array is a static device variable of the library: each GPU the
 *     library runs on holds its own copy from the first call on that device
 *     (its address is looked up once per device, with the device current)
 *     until the process ends.  The call allocates and frees nothing.
 *   - The current device must be the device of `stream` and of the pointers.
 *   - Every call on one GPU shares that GPU's array, which keeps the last
 *     call's partials; the kernels write every partial before they read it,
 *     so nothing needs clearing.  Calls that overlap in time on one GPU (two
 *     streams, two host threads) race on the array and give undefined
 *     results: serialise them.
 *   - Errors: those of kvarn_decode_attention, KVARN_E_WORKSPACE when
 *     kvarn_decode_workspace_bytes(args) exceeds KVARN_NOALLOC_SCRATCH_BYTES
 *     (checked before anything is enqueued), KVARN_E_DEVICE when the array's
 *     address cannot be obtained.
 */
#define KVARN_NOALLOC_SCRATCH_BYTES (16u << 20)
int kvarn_decode_attention_noalloc(const kvarn_decode_args* args, void* stream);

/*
 * kvarn_prefill_attention -- causal attention of one chunk of C consecutive
 * query positions [pos0, pos0+C) of one sequence.  PR #434 commit list
 * (chunked batched prefill: single streaming softmax over compressed tiles +
 * FP32 window, deferred inverse WHT, schedule-independent tiles); issue #433
 * item 1 (the Q.K score block of compressed tiles on the matrix units).
 *
 * Query position p sees the tiles [0, T(p)) compressed and the raw tokens
 * [128*T(p), p] (the decode view at p, so the output does not depend on how
 * the prompt is chunked).  The caller compresses every tile the chunk makes
 * due (tiles < T(pos0+C-1)) before this call.
 *
 * head_dim 128 over K4V2 records runs on the matrix units, in workgroups of
 * query-row blocks that read each tile once for 128 row-heads.  Over K4V2
 * records at head_dim 256 and 512 (issue #433 item 3: prefill at the wider
 * heads) the tiles run on the matrix units, at 256 in such workgroups (in
 * tile splits), at 512 every chunk row as a decode query with that view; the
 * raw windows run on the fp32 matrix units.  Records with other code widths
 * run the decode view on the vector-unit split kernels.  All of these need a
 * workspace for the partials.
 */
typedef struct kvarn_prefill_args {
  int32_t head_dim;        /* 128, 256 or 512, | KVARN_SCALES_F16 (f16 scales),
                              | KVARN_KEY_BITS / KVARN_VALUE_BITS (widths)      */
  int32_t n_q_heads;
  int32_t n_kv_heads;
  int32_t window;          /* W of the promotion rule, >= 0                     */
  int64_t pos0;            /* absolute position of the chunk's first query      */
  int32_t chunk;           /* C >= 1 query positions                            */
  float softmax_scale;
  const float* q;          /* device [C][n_q_heads][head_dim] raw               */
  const float* q_rot;      /* device [C][n_q_heads][head_dim] rotated; NULL
                              over K4V2 records (any head_dim): the kernels
                              then rotate each row themselves (the vector-unit
                              paths of other code widths require it)           */
  const void* records;     /* device: record (j, h) at (j*n_kv_heads+h)*tile_bytes */
  int64_t n_record_rows;   /* tiles available; must be >= T(pos0 + C - 1)       */
  const float* k;          /* device raw keys: absolute position p, KV head h at
                              k + (p - raw_base)*tok_stride + h*head_stride     */
  const float* v;          /* device raw values, same strides                   */
  int64_t tok_stride, head_stride;
  int64_t raw_base;        /* first raw position provided; <= 128*T(pos0)       */
  float* out;              /* device [C][n_q_heads][head_dim]                   */
} kvarn_prefill_args;

/* Workspace bytes kvarn_prefill_attention needs (0 on invalid arguments).
 * head_dim 128 over K4V2 records: the partials of the S tile-and-raw splits
 * that fill the CUs (S = 256 / workgroups of 128 row-heads, 1..4; 0 bytes when
 * S = 1).  The workspace may also be NULL there: the call then runs one
 * launch that keeps every partial result on chip, with half as many row-heads
 * per unpacked tile (slower).  head_dim 256 / 512 and other code widths: the
 * per-row split partials, required.  Device memory owned by the caller,
 * scratch after the call (no initialisation needed); calls sharing a
 * workspace must not overlap in time. */
size_t kvarn_prefill_workspace_bytes(const kvarn_prefill_args* args);

/* Errors: KVARN_E_INVALID (null pointers, chunk < 1, pos0 < 0, missing tiles
 * or raw rows), KVARN_E_UNSUPPORTED (head_dim, GQA ratio), KVARN_E_ALIGN,
 * KVARN_E_WORKSPACE (a workspace smaller than kvarn_prefill_workspace_bytes;
 * NULL only at head_dim 128 over K4V2 records).  The raw rows
 * [raw_base, pos0 + C) must be readable. */
int kvarn_prefill_attention(const kvarn_prefill_args* args, void* workspace,
                            size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVARN_H */
