// kvarn_api.hip -- the C ABI declared in include/kvarn.h: host-side argument
// validation (before anything is enqueued), split planning, and launches.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <string.h>

#include <mutex>

#include "../../include/kvarn.h"
#include "kvarn_launch.h"


namespace {

// A head_dim argument is a format word: the head dimension in bits 0-15,
// KVARN_SCALES_F16 (records with f16 scales), the key code width in bits
// 20-23 and the value code width in bits 24-27 (0 = the K4V2 default); no
// other bits.
constexpr int32_t kFieldMask = 0xFFFF | KVARN_SCALES_F16 | (0xF << 20) | (0xF << 24);
int dim_of(int32_t hd) { return hd & 0xFFFF; }
bool f16_of(int32_t hd) { return (hd & KVARN_SCALES_F16) != 0; }
int kbits_of(int32_t hd) { const int b = (hd >> 20) & 0xF; return b ? b : 4; }
int vbits_of(int32_t hd) { const int b = (hd >> 24) & 0xF; return b ? b : 2; }
bool k4v2(int32_t hd) { return kbits_of(hd) == 4 && vbits_of(hd) == 2; }
bool dim_ok(int32_t hd) {
  const int d = dim_of(hd);
  return (hd & ~kFieldMask) == 0 && (d == 128 || d == 256 || d == 512) && kbits_of(hd) <= 8 &&
         vbits_of(hd) <= 8;
}
bool al16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool st16(int64_t floats) { return (floats % 4) == 0; }

// Work target for the vector-unit split plan: one workgroup per tile range,
// enough to cover the 256 CUs several times.
constexpr int64_t kTargetGroups = 2048;
constexpr int64_t kPrefillTarget512 = 512;
// Matrix-core tile splits of K4V2 decode at head_dim 256 / 512: the split
// kernels keep the next tile's loads in flight, so longer splits pay more
// at 512 (two workgroups per CU); measured fastest on the 16-sequence batch
// against targets of 1024-8192 (256) and 1024-4096 (512).
int64_t wide_target(int d) { return d >= 512 ? 512 : 4096; }

struct DecodePlan {
  int tps, n_tsplit, n_wsplit, wchunk;
};

// target: number of tile workgroups; wchunk: window tokens per window split
DecodePlan plan_decode(int batch, int n_kv, int max_tiles, int max_win, int64_t target, int wchunk) {
  DecodePlan p;
  const int64_t units = (int64_t)batch * n_kv * (max_tiles > 0 ? max_tiles : 0);
  int64_t tps = (units + target - 1) / target;
  if (tps < 1) tps = 1;
  p.tps = (int)tps;
  p.n_tsplit = max_tiles > 0 ? (int)((max_tiles + tps - 1) / tps) : 0;
  p.n_wsplit = max_win > 0 ? (max_win + wchunk - 1) / wchunk : 0;
  p.wchunk = wchunk;
  return p;
}

// head_dim 128 decode over K4V2 records runs the matrix-core split kernel
// plus its combine; other widths and head dims run the vector-unit kernels.
bool fused_decode(int32_t hd) { return dim_of(hd) == 128 && k4v2(hd); }

// Matrix-core split plan: TPW tiles per workgroup (4 waves per tile): 2 once
// the batch has 256 tile-heads (measured fastest at the 8B shape for
// contexts 4096, 15488 and 32768, against 1 and 4, and with 1 below 256
// tile-heads on the 0.6B-shaped layer), else 1.  The window
// tokens are spread over the tile splits (at most 16 per split; more splits
// when the window needs them), so that no split carries many of them.
DecodePlan plan_fused(int batch, int n_kv, int max_tiles, int max_win) {
  const int64_t units = (int64_t)batch * n_kv * (max_tiles > 0 ? max_tiles : 0);
  const int tpw = units >= 256 ? 2 : 1;
  DecodePlan p;
  p.tps = tpw;
  const int nt = max_tiles > 0 ? (max_tiles + tpw - 1) / tpw : 0;
  int wps = nt > 0 ? (max_win + nt - 1) / nt : kvarn::kWinPerSplit;
  if (wps < 1) wps = 1;
  if (wps > kvarn::kWinPerSplit) wps = kvarn::kWinPerSplit;
  const int nw = max_win > 0 ? (max_win + wps - 1) / wps : 0;
  p.n_tsplit = nt > nw ? nt : nw;
  p.n_wsplit = 0;
  p.wchunk = wps;
  return p;
}

int q_rows(const kvarn_decode_args* a) { return a->q_len > 1 ? a->q_len : 1; }

// Multi-query verify plan (head_dim 128 prefill workgroups of 8 waves, one per
// CU): window splits of 128 raw tokens (at most 16 of them; measured faster
// than 64 and 256 at the 8B shape, where a split of 128 raw tokens takes about
// as long as one of 4 tiles), and tiles per split so that all splits of all
// (sequence, KV head, row block) groups fit on the 256 CUs at once; at most 64
// splits in all (the combine's limit).
DecodePlan plan_verify(int batch, int n_kv, int G, int max_tiles, int max_win) {
  // row blocks of 4 row groups; a row group holds the <= 8 rows of 2 query
  // heads when G >= 2, of one head when G = 1
  const int64_t groups = (int64_t)batch * n_kv * (G >= 2 ? (G / 2 + 3) / 4 : 1);
  int wchunk = 128;
  int nr = (max_win + wchunk - 1) / wchunk;
  if (nr > 16) {
    wchunk = ((max_win + 15) / 16 + 31) / 32 * 32;
    nr = (max_win + wchunk - 1) / wchunk;
  }
  if (nr < 1) nr = 1;
  int64_t per = 256 / groups;
  int64_t avail = per - nr;
  if (avail < 1) avail = 1;
  if (avail > 64 - nr) avail = 64 - nr;
  int64_t tps = max_tiles > 0 ? (max_tiles + avail - 1) / avail : 1;
  if (tps < 1) tps = 1;
  DecodePlan p;
  p.tps = (int)tps;
  p.n_tsplit = max_tiles > 0 ? (int)((max_tiles + tps - 1) / tps) : 0;
  p.n_wsplit = nr;
  p.wchunk = wchunk;
  return p;
}

int validate_decode(const kvarn_decode_args* a, DecodePlan* plan) {
  if (!a) return KVARN_E_INVALID;
  if (!dim_ok(a->head_dim)) return KVARN_E_UNSUPPORTED;
  if (a->q_len < 0 || a->q_len > 8) return KVARN_E_INVALID;
  const int w = q_rows(a);
  if (w > 1 && !fused_decode(a->head_dim)) return KVARN_E_UNSUPPORTED;
  if (a->batch < 1 || a->n_q_heads < 1 || a->n_kv_heads < 1) return KVARN_E_INVALID;
  if (a->batch > KVARN_MAX_BATCH) return KVARN_E_UNSUPPORTED;
  if (a->n_q_heads % a->n_kv_heads != 0) return KVARN_E_UNSUPPORTED;
  const int G = a->n_q_heads / a->n_kv_heads;
  if (!(G == 1 || G == 2 || G == 4 || G == 8)) return KVARN_E_UNSUPPORTED;
  if (a->max_tiles < 0 || a->max_win < 0 || a->n_record_rows < 0) return KVARN_E_INVALID;
  if (!a->q || !a->out || !a->n_tiles || !a->n_win || !a->rec_start) return KVARN_E_INVALID;
  if (!a->q_rot && !k4v2(a->head_dim)) return KVARN_E_INVALID;   // K4V2 kernels rotate q themselves
  bool any_tiles = false, any_win = false;
  for (int b = 0; b < a->batch; ++b) {
    const int nt = a->n_tiles[b], nw = a->n_win[b];
    if (nt < 0 || nw < 0 || nt > a->max_tiles || nw > a->max_win) return KVARN_E_INVALID;
    if (a->win_start && a->win_start[b] < 0) return KVARN_E_INVALID;
    if (nt + nw == 0) return KVARN_E_INVALID;
    if (nw < w && w > 1) return KVARN_E_INVALID;
    if (nt > 0) {
      if (a->rec_start[b] < 0 || a->rec_start[b] + nt > a->n_record_rows) return KVARN_E_INVALID;
      any_tiles = true;
    }
    if (nw > 0) any_win = true;
  }
  if ((a->k_new == nullptr) != (a->v_new == nullptr)) return KVARN_E_INVALID;
  if (a->k_new) {   // the appended token is window token n_win[b] - 1 of a single-query decode
    if (w > 1) return KVARN_E_INVALID;
    for (int b = 0; b < a->batch; ++b)
      if (a->n_win[b] < 1) return KVARN_E_INVALID;
    if (!al16(a->k_new) || !al16(a->v_new)) return KVARN_E_ALIGN;
  }
  if (any_tiles && !a->records) return KVARN_E_INVALID;
  if (any_win && (!a->k_win || !a->v_win)) return KVARN_E_INVALID;
  if (any_win && (a->win_tok_stride < dim_of(a->head_dim) || a->win_head_stride < 0 ||
                  a->win_seq_stride < 0))
    return KVARN_E_INVALID;
  if (!al16(a->q) || !al16(a->q_rot) || !al16(a->out) || !al16(a->records) ||
      !al16(a->k_win) || !al16(a->v_win))
    return KVARN_E_ALIGN;
  if (!st16(a->win_seq_stride) || !st16(a->win_tok_stride) || !st16(a->win_head_stride))
    return KVARN_E_ALIGN;
  if (plan) {
    *plan = w > 1 ? plan_verify(a->batch, a->n_kv_heads, G, a->max_tiles, a->max_win)
          : fused_decode(a->head_dim)
                ? plan_fused(a->batch, a->n_kv_heads, a->max_tiles, a->max_win)
                : plan_decode(a->batch, a->n_kv_heads, a->max_tiles, a->max_win,
                              k4v2(a->head_dim) && dim_of(a->head_dim) >= 256 ? wide_target(dim_of(a->head_dim))
                                                                              : kTargetGroups,
                              kvarn::kWinChunk);
  }
  return KVARN_OK;
}

size_t decode_part_floats(int rows, int n_q, int d, const DecodePlan& p) {
  return (size_t)rows * n_q * (size_t)(p.n_tsplit + p.n_wsplit) * (size_t)(d + 4);
}
size_t decode_ws(const kvarn_decode_args* a, const DecodePlan& p) {
  return decode_part_floats(a->batch * q_rows(a), a->n_q_heads, dim_of(a->head_dim), p) * sizeof(float);
}

int64_t prefill_tiles_at(int64_t pos, int window) {
  const int64_t ahead = pos + 1 - window;
  return ahead > 0 ? ahead / KVARN_TILE_TOKENS : 0;
}

// Splits of the head_dim-128 matrix-core prefill: the workgroups of 128
// row-heads (8 row groups of 16 positions of one query head) times S should
// fill the 256 CUs once (one workgroup per CU), with at most 4 shares.
int prefill_splits(const kvarn_prefill_args* a) {
  const int G = a->n_q_heads / a->n_kv_heads;
  const int64_t n_blk = (int64_t)((a->chunk + 15) / 16) * G;
  const int64_t wgs = (n_blk + 7) / 8 * a->n_kv_heads;
  const int64_t S = 256 / wgs;
  return S < 1 ? 1 : (S > 4 ? 4 : (int)S);
}
size_t prefill_split_bytes(const kvarn_prefill_args* a) {
  const int S = prefill_splits(a);
  return S > 1 ? (size_t)a->chunk * a->n_q_heads * S * (128 + 4) * sizeof(float) : 0;   // o, m, l, pad
}

int validate_prefill(const kvarn_prefill_args* a, DecodePlan* plan) {
  if (!a) return KVARN_E_INVALID;
  if (!dim_ok(a->head_dim)) return KVARN_E_UNSUPPORTED;
  if (a->n_q_heads < 1 || a->n_kv_heads < 1 || a->chunk < 1 || a->pos0 < 0 || a->window < 0)
    return KVARN_E_INVALID;
  if (a->n_q_heads % a->n_kv_heads != 0) return KVARN_E_UNSUPPORTED;
  const int G = a->n_q_heads / a->n_kv_heads;
  if (!(G == 1 || G == 2 || G == 4 || G == 8)) return KVARN_E_UNSUPPORTED;
  if (!a->q || !a->out || !a->k || !a->v) return KVARN_E_INVALID;
  if (!a->q_rot && !k4v2(a->head_dim)) return KVARN_E_INVALID;   // K4V2 kernels rotate q themselves
  const int64_t last = a->pos0 + a->chunk - 1;
  const int64_t t_first = prefill_tiles_at(a->pos0, a->window);
  const int64_t t_last = prefill_tiles_at(last, a->window);
  if (t_last > 0 && !a->records) return KVARN_E_INVALID;
  if (a->n_record_rows < t_last) return KVARN_E_INVALID;
  if (a->raw_base < 0 || a->raw_base > KVARN_TILE_TOKENS * t_first) return KVARN_E_INVALID;
  if (a->tok_stride < dim_of(a->head_dim) || a->head_stride < 0) return KVARN_E_INVALID;
  if (!al16(a->q) || !al16(a->q_rot) || !al16(a->out) || !al16(a->records) || !al16(a->k) ||
      !al16(a->v))
    return KVARN_E_ALIGN;
  if (!st16(a->tok_stride) || !st16(a->head_stride)) return KVARN_E_ALIGN;
  if (plan) {
    // window tokens of a row are at most W + 127 (fewer when the prompt is short)
    int64_t max_win = a->window + KVARN_TILE_TOKENS - 1;
    if (last + 1 < max_win) max_win = last + 1;
    // head_dim 512 over K4V2 records: one row (or row pair) per workgroup of
    // each tile split; a target of 512 row-tile units gives one split per row
    // at 512-row chunks (measured fastest on the 4096-token prompt against
    // 1024-8192)
    *plan = plan_decode(a->chunk, a->n_kv_heads, (int)t_last, (int)max_win,
                        k4v2(a->head_dim) && dim_of(a->head_dim) == 512 ? kPrefillTarget512 : kTargetGroups,
                        kvarn::kWinChunk);
    // K4V2 records at head_dim 256 / 512: the raw windows run on the window
    // kernel, in R parts of each 16-row block's raw tokens, one partial per
    // part, row and head; R so that the workgroups fill the CUs twice
    // (measured fastest on the 4096-token prompts against 1, 3 and 4 parts)
    if (k4v2(a->head_dim) && dim_of(a->head_dim) >= 256) {
      const int d = dim_of(a->head_dim);
      const int G = a->n_q_heads / a->n_kv_heads;
      const int64_t wgs = (int64_t)((a->chunk + 15) / 16) * (d == 256 && G % 2 == 0 ? a->n_q_heads / 2 : a->n_q_heads);
      const int64_t R = 2 * 256 / wgs;
      plan->n_wsplit = R < 1 ? 1 : (R > 4 ? 4 : (int)R);
      // head_dim 256: the tile kernel's workgroups of 8 row groups, one per
      // CU; tile splits so that they fill the 256 CUs once
      if (d == 256 && t_last > 0) {
        const int64_t groups = ((int64_t)(a->chunk + 15) / 16 * G + 7) / 8 * a->n_kv_heads;
        int64_t ns = (256 + groups - 1) / groups;
        if (ns > t_last) ns = t_last;
        const int64_t tps = (t_last + ns - 1) / ns;
        plan->tps = (int)tps;
        plan->n_tsplit = (int)((t_last + tps - 1) / tps);
      }
    }
  }
  return KVARN_OK;
}

// Split partials of kvarn_decode_attention_noalloc: one array per GPU that
// the library runs on, held until the process ends.  Host code never passes
// the array's name to a kernel (on the host it is a stand-in, not a device
// address): it uses the device address that hipGetSymbolAddress returns.
static __device__ __align__(256) uint8_t scratch[KVARN_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::once_flag g_scratch_once[kMaxDevices];
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];

// The current device's copy of `scratch`, looked up once per device (with
// that device current) and kept; NULL when the lookup failed.
void* scratch_on_current_device(hipError_t* err) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    *err = e != hipSuccess ? e : hipErrorInvalidDevice;
    return nullptr;
  }
  std::call_once(g_scratch_once[dev], [dev] {
    void* ptr = nullptr;
    g_scratch_err[dev] = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? ptr : nullptr;
  });
  *err = g_scratch_err[dev];
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" {

const char* kvarn_status_string(int status) {
  switch (status) {
    case KVARN_OK: return "KVARN_OK";
    case KVARN_E_INVALID: return "KVARN_E_INVALID";
    case KVARN_E_UNSUPPORTED: return "KVARN_E_UNSUPPORTED";
    case KVARN_E_ALIGN: return "KVARN_E_ALIGN";
    case KVARN_E_WORKSPACE: return "KVARN_E_WORKSPACE";
    case KVARN_E_DEVICE: return "KVARN_E_DEVICE";
    default: return "KVARN_E_UNKNOWN";
  }
}

size_t kvarn_tile_bytes(int32_t head_dim) {
  return dim_ok(head_dim) ? (size_t)kvarn::rec_rt(dim_of(head_dim), f16_of(head_dim),
                                                  kbits_of(head_dim), vbits_of(head_dim)).bytes
                          : 0;
}

int kvarn_compress_tile(int32_t head_dim, int32_t n_tiles, int32_t n_kv_heads, const float* k,
                        const float* v, int64_t tok_stride, int64_t head_stride, void* records,
                        void* stream) {
  if (!dim_ok(head_dim)) return KVARN_E_UNSUPPORTED;
  if (n_tiles < 0 || n_kv_heads < 1) return KVARN_E_INVALID;
  if (n_tiles == 0) return KVARN_OK;
  if (!k || !v || !records) return KVARN_E_INVALID;
  if (tok_stride < dim_of(head_dim) || head_stride < 0) return KVARN_E_INVALID;
  if (n_kv_heads > 65535) return KVARN_E_UNSUPPORTED;
  if (!al16(k) || !al16(v) || !al16(records) || !st16(tok_stride) || !st16(head_stride))
    return KVARN_E_ALIGN;
  hipError_t e = kvarn::launch_compress(dim_of(head_dim), f16_of(head_dim), kbits_of(head_dim),
                                        vbits_of(head_dim), n_tiles, n_kv_heads, k, v, tok_stride,
                                        head_stride, records, (hipStream_t)stream);
  return e == hipSuccess ? KVARN_OK : KVARN_E_DEVICE;
}

int kvarn_rotate_query(int32_t head_dim, int64_t n_rows, const float* q, float* q_rot,
                       void* stream) {
  if (!dim_ok(head_dim)) return KVARN_E_UNSUPPORTED;
  if (n_rows < 0) return KVARN_E_INVALID;
  if (n_rows == 0) return KVARN_OK;
  if (!q || !q_rot) return KVARN_E_INVALID;
  if (!al16(q) || !al16(q_rot)) return KVARN_E_ALIGN;
  if ((n_rows + 3) / 4 > 0x7fffffffLL) return KVARN_E_UNSUPPORTED;
  hipError_t e = kvarn::launch_rotate(dim_of(head_dim), n_rows, q, q_rot, (hipStream_t)stream);
  return e == hipSuccess ? KVARN_OK : KVARN_E_DEVICE;
}

size_t kvarn_decode_workspace_bytes(const kvarn_decode_args* a) {
  DecodePlan p;
  if (validate_decode(a, &p) != KVARN_OK) return 0;
  return decode_ws(a, p);
}

int kvarn_decode_attention_noalloc(const kvarn_decode_args* a, void* stream) {
  DecodePlan p;
  int st = validate_decode(a, &p);
  if (st != KVARN_OK) return st;
  if (decode_ws(a, p) > (size_t)KVARN_NOALLOC_SCRATCH_BYTES) return KVARN_E_WORKSPACE;
  hipError_t e = hipSuccess;
  void* ws = scratch_on_current_device(&e);
  if (!ws) return KVARN_E_DEVICE;
  return kvarn_decode_attention(a, ws, KVARN_NOALLOC_SCRATCH_BYTES, stream);
}

int kvarn_decode_attention(const kvarn_decode_args* a, void* workspace, size_t ws_bytes,
                           void* stream) {
  DecodePlan p;
  int st = validate_decode(a, &p);
  if (st != KVARN_OK) return st;
  const bool fused = fused_decode(a->head_dim);
  const int w = q_rows(a);
  const size_t need = decode_ws(a, p);
  if (!workspace || ws_bytes < need) return KVARN_E_WORKSPACE;
  if (!al16(workspace)) return KVARN_E_ALIGN;
  kvarn::DecodeParams P;
  memset(&P, 0, sizeof(P));
  P.q = a->q;
  P.q_rot = a->q_rot;
  P.records = static_cast<const uint8_t*>(a->records);
  P.k_win = a->k_win;
  P.v_win = a->v_win;
  P.part = static_cast<float*>(workspace);
  P.out = a->out;
  P.win_seq_stride = a->win_seq_stride;
  P.win_tok_stride = a->win_tok_stride;
  P.win_head_stride = a->win_head_stride;
  P.scale = a->softmax_scale;
  P.n_q = a->n_q_heads;
  P.n_kv = a->n_kv_heads;
  P.G = a->n_q_heads / a->n_kv_heads;
  P.tps = p.tps;
  P.n_tsplit = p.n_tsplit;
  P.n_wsplit = p.n_wsplit;
  P.wchunk = p.wchunk;
  P.mode = 0;
  P.h16 = f16_of(a->head_dim);
  P.kb = kbits_of(a->head_dim);
  P.vb = vbits_of(a->head_dim);
  for (int b = 0; b < a->batch; ++b) {
    P.rec_start[b] = a->rec_start[b];
    P.win_start[b] = a->win_start ? a->win_start[b] : 0;
    P.n_tiles[b] = a->n_tiles[b];
    P.n_win[b] = a->n_win[b];
  }
  hipError_t e;
  if (a->k_new) {   // the newest token's rows into the window (a single-query decode)
    P.k_new = a->k_new;
    P.v_new = a->v_new;
    if (!fused) {   // the split kernel of head_dim-128 K4V2 appends them itself; the others copy first
      e = kvarn::launch_append_window(dim_of(a->head_dim), P, a->k_win, a->v_win, a->batch, (hipStream_t)stream);
      if (e != hipSuccess) return KVARN_E_DEVICE;
      P.k_new = P.v_new = nullptr;
    }
  }
  if (w > 1) {
    P.q_len = w;   // without q_rot the workgroups rotate the rows themselves
    e = kvarn::launch_verify_mfma(P, a->batch, (hipStream_t)stream);
  } else {
    e = fused ? kvarn::launch_decode_fused(P, a->batch, (hipStream_t)stream)
              : kvarn::launch_decode(dim_of(a->head_dim), P, a->batch, (hipStream_t)stream);
  }
  return e == hipSuccess ? KVARN_OK : KVARN_E_DEVICE;
}

// head_dim 128 over K4V2 records: the matrix-core prefill in S splits, whose
// raw-domain partials the workspace holds (S = 1: none); without a workspace
// the single-launch kernel, which keeps its whole state on chip.  head_dim
// 256 / 512 and other code widths: the split kernels run every chunk row as a
// decode query with the prefill view (T(p) tiles, raw rows [128 T(p), p]) and
// need their partials in the workspace.
size_t kvarn_prefill_workspace_bytes(const kvarn_prefill_args* a) {
  DecodePlan p;
  if (validate_prefill(a, &p) != KVARN_OK) return 0;
  if (fused_decode(a->head_dim)) return prefill_split_bytes(a);
  return decode_part_floats(a->chunk, a->n_q_heads, dim_of(a->head_dim), p) * sizeof(float);
}

int kvarn_prefill_attention(const kvarn_prefill_args* a, void* workspace, size_t ws_bytes,
                            void* stream) {
  DecodePlan plan;
  int st = validate_prefill(a, &plan);
  if (st != KVARN_OK) return st;
  if (!fused_decode(a->head_dim)) {
    const size_t need =
        decode_part_floats(a->chunk, a->n_q_heads, dim_of(a->head_dim), plan) * sizeof(float);
    if (!workspace || ws_bytes < need) return KVARN_E_WORKSPACE;
    if (!al16(workspace)) return KVARN_E_ALIGN;
    kvarn::DecodeParams P;
    memset(&P, 0, sizeof(P));
    P.q = a->q;
    P.q_rot = a->q_rot;
    P.records = static_cast<const uint8_t*>(a->records);
    P.k_win = a->k;
    P.v_win = a->v;
    P.part = static_cast<float*>(workspace);
    P.out = a->out;
    P.win_tok_stride = a->tok_stride;
    P.win_head_stride = a->head_stride;
    P.scale = a->softmax_scale;
    P.n_q = a->n_q_heads;
    P.n_kv = a->n_kv_heads;
    P.G = a->n_q_heads / a->n_kv_heads;
    P.tps = plan.tps;
    P.n_tsplit = plan.n_tsplit;
    P.n_wsplit = plan.n_wsplit;
    P.wchunk = plan.wchunk;
    P.mode = 1;
    P.wparts = (k4v2(a->head_dim) && dim_of(a->head_dim) >= 256) ? plan.n_wsplit : 0;
    P.h16 = f16_of(a->head_dim);
    P.kb = kbits_of(a->head_dim);
    P.vb = vbits_of(a->head_dim);
    P.window = a->window;
    P.pos0 = a->pos0;
    P.raw_base = a->raw_base;
    hipError_t e = kvarn::launch_decode(dim_of(a->head_dim), P, a->chunk, (hipStream_t)stream);
    return e == hipSuccess ? KVARN_OK : KVARN_E_DEVICE;
  }
  kvarn::PrefillParams P;
  memset(&P, 0, sizeof(P));
  P.q = a->q;
  P.q_rot = a->q_rot;
  P.records = static_cast<const uint8_t*>(a->records);
  P.k = a->k;
  P.v = a->v;
  P.out = a->out;
  P.tok_stride = a->tok_stride;
  P.head_stride = a->head_stride;
  P.pos0 = a->pos0;
  P.raw_base = a->raw_base;
  P.scale = a->softmax_scale;
  P.chunk = a->chunk;
  P.window = a->window;
  P.n_q = a->n_q_heads;
  P.n_kv = a->n_kv_heads;
  P.G = a->n_q_heads / a->n_kv_heads;
  P.h16 = f16_of(a->head_dim);
  const int S = prefill_splits(a);
  hipError_t e;
  if (S == 1) {   // the workgroups fill the chip unsplit: no partials
    e = kvarn::launch_prefill_split(P, nullptr, 1, (hipStream_t)stream);
  } else if (workspace) {
    if (ws_bytes < prefill_split_bytes(a)) return KVARN_E_WORKSPACE;
    if (!al16(workspace)) return KVARN_E_ALIGN;
    e = kvarn::launch_prefill_split(P, static_cast<float*>(workspace), S, (hipStream_t)stream);
  } else {        // no workspace: the half layout, 64 row-heads per workgroup, one launch
    e = kvarn::launch_prefill_mfma(P, (hipStream_t)stream);
  }
  return e == hipSuccess ? KVARN_OK : KVARN_E_DEVICE;
}

}  // extern "C"
