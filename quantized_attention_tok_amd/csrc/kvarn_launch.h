// kvarn_launch.h -- host/device interface between the C ABI layer and the
// HIP kernels: parameter blocks and launch entry points.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvarn_device.h"

namespace kvarn {

constexpr int kDecThreads = 256;
constexpr int kWinChunk = 64;      // window tokens per split (vector-unit kernels)
constexpr int kWinPerSplit = 16;   // most window tokens per split (head_dim-128 matrix-core kernel)

struct DecodeParams {
  const float* q;
  const float* q_rot;
  const uint8_t* records;
  const float* k_win;
  const float* v_win;
  float* part;                     // [B][Hq][n_split][D + 4]
  float* out;                      // [B][Hq][D]
  int64_t win_seq_stride, win_tok_stride, win_head_stride;
  float scale;
  int n_q, n_kv, G;
  int tps, n_tsplit, n_wsplit;
  int wchunk;                      // window tokens per window split
  // prefill view (mode 1): "sequence" b is query position pos0 + b of one
  // sequence; it sees T(p) tiles and raw rows [128 T(p), p] of k_win/v_win,
  // where raw row p lives at (p - raw_base) * win_tok_stride.
  int mode;
  int q_len;                       // query rows per sequence (multi-query verify)
  int h16;                         // records carry f16 scales
  int kb, vb;                      // key / value code widths (4 / 2: the K4V2 record)
  int window;
  int64_t pos0, raw_base;
  int64_t rec_start[64];
  int64_t win_start[64];
  int n_tiles[64];
  int n_win[64];
  int wparts;                      // prefill: the window kernel's parts (the combine reads them all), or 0
  const float* k_new;              // newest token's rows [B][n_kv][D] to append, or NULL
  const float* v_new;
};

// Chunked prefill of one sequence (head_dim 128 matrix-core kernel).
struct PrefillParams {
  const float* q;                  // [chunk][n_q][128] raw
  const float* q_rot;              // [chunk][n_q][128] rotated
  const uint8_t* records;          // record (j, h) at (j * n_kv + h) * tile bytes
  const float* k;                  // raw row of position p, KV head h at
  const float* v;                  //   (p - raw_base) * tok_stride + h * head_stride
  float* out;                      // [chunk][n_q][128]
  int64_t tok_stride, head_stride;
  int64_t pos0, raw_base;
  float scale;
  int chunk, window, n_q, n_kv, G;
  int h16;                         // records carry f16 scales
};

// Tiles, window tokens, first record row and window base of sequence b.
struct SeqView {
  int nt, nw;
  int64_t rec_row0;
  int64_t win_off;   // float offset of window token 0, KV head 0
};

__device__ __forceinline__ SeqView seq_view(const DecodeParams& P, int b) {
  SeqView v;
  if (P.mode == 0) {
    v.nt = P.n_tiles[b];
    v.nw = P.n_win[b];
    v.rec_row0 = P.rec_start[b];
    v.win_off = (int64_t)b * P.win_seq_stride + P.win_start[b] * P.win_tok_stride;
  } else {
    const int64_t p = P.pos0 + b;
    const int64_t ahead = p + 1 - P.window;
    const int64_t T = ahead > 0 ? ahead / kTile : 0;
    v.nt = (int)T;
    v.nw = (int)(p + 1 - kTile * T);
    v.rec_row0 = 0;
    v.win_off = (kTile * T - P.raw_base) * P.win_tok_stride;
  }
  return v;
}

// The decode view (mode 0) alone: no branch on the mode, so the compiler can
// issue every kernel-argument load at once.
__device__ __forceinline__ SeqView seq_view_decode(const DecodeParams& P, int b) {
  SeqView v;
  v.nt = P.n_tiles[b];
  v.nw = P.n_win[b];
  v.rec_row0 = P.rec_start[b];
  v.win_off = (int64_t)b * P.win_seq_stride + P.win_start[b] * P.win_tok_stride;
  return v;
}

hipError_t launch_compress(int d, bool h16, int kb, int vb, int n_tiles, int n_kv, const float* k,
                           const float* v, int64_t tok_stride, int64_t head_stride, void* records,
                           hipStream_t stream);
hipError_t launch_rotate(int d, int64_t n_rows, const float* q, float* q_rot, hipStream_t stream);
hipError_t launch_decode(int d, const DecodeParams& P, int batch, hipStream_t stream);
// Store k_new / v_new (P.k_new, P.v_new) as window token n_win[b] - 1 of each
// sequence: the append for the decode paths that do not take it in-kernel.
hipError_t launch_append_window(int d, const DecodeParams& P, float* k_win, float* v_win, int batch,
                                hipStream_t stream);
hipError_t launch_decode_fused(const DecodeParams& P, int batch, hipStream_t stream);
// Head_dim 256 / 512 over K4V2 records: the tile splits on the matrix cores,
// and in decode (P.mode 0) the P.n_wsplit window splits of kWinChunk tokens
// after them in the same grid ((n_tsplit + n_wsplit) x n_kv x batch); in
// prefill the tile splits alone.  With P.q_rot NULL the kernel rotates q.
hipError_t launch_decode_wide(int d, const DecodeParams& P, int batch, hipStream_t stream);
// Head_dim 256 chunked prefill over K4V2 records (P.mode 1): the compressed-
// tile partials of the chunk's rows, P.n_tsplit tile splits of P.tps tiles,
// on the matrix cores (8 row groups of 16 rows per workgroup).
hipError_t launch_prefill_tiles256(const DecodeParams& P, int chunk, hipStream_t stream);
hipError_t launch_prefill_mfma(const PrefillParams& P, hipStream_t stream);
// The same over the FR layout in S tile-and-raw splits (1 <= S <= 4): with
// S > 1, part holds chunk * n_q * S partials of 128 + 4 floats and a combine
// launch writes the output; with S = 1 the output is written directly.
hipError_t launch_prefill_split(const PrefillParams& P, float* part, int S, hipStream_t stream);
// The raw-window part of chunked prefill (P.mode 1) at head_dim 256 / 512 on
// the fp32 matrix cores, each 16-row block's raw tokens in P.n_wsplit parts
// (grid z): one raw-domain partial per part, chunk row and query head, written
// as split P.n_tsplit + part of P.n_tsplit + P.n_wsplit (P.wparts = P.n_wsplit
// tells the combine to read every part).
hipError_t launch_window_mfma(int d, const DecodeParams& P, int chunk, hipStream_t stream);
// Multi-query verify (head_dim 128): P.part holds batch * q_len * n_q *
// (n_tsplit + n_wsplit) partials of D + 4 floats (n_wsplit window splits of
// wchunk tokens); with P.q_rot NULL the kernel rotates q itself.
hipError_t launch_verify_mfma(const DecodeParams& P, int batch, hipStream_t stream);

}  // namespace kvarn
