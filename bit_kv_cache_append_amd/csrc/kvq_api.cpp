// Host side of the kvq C ABI: argument validation, buffer sizes, launch setup.
// Nothing here allocates memory; every launch goes onto the caller's stream.

#include <math.h>
#include <algorithm>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "kvq_internal.h"

using namespace kvq;

namespace {

thread_local char g_err[512] = "";

kvq_status fail(kvq_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

kvq_status hip_fail(hipError_t e, const char* what) {
  return fail(KVQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

bool valid_fmt(int f) { return f == KVQ_INT4 || f == KVQ_INT8 || f == KVQ_INT2 || f == KVQ_FP4; }

int eff_group(int fmt, int g) { return fmt_group(fmt, g); }

// shape/enum checks common to every call
kvq_status check_params(const kvq_params* p) {
  if (!p) return fail(KVQ_ERR_INVALID_ARG, "params is NULL");
  if (p->head_dim != D) return fail(KVQ_ERR_UNSUPPORTED, "head_dim must be 128 (got %d)", p->head_dim);
  if (p->batch < 1 || p->batch > MAX_BATCH) return fail(KVQ_ERR_INVALID_ARG, "batch must be 1..%d", MAX_BATCH);
  if (p->n_kv_heads < 1 || p->n_q_heads < 1 || p->n_q_heads % p->n_kv_heads)
    return fail(KVQ_ERR_INVALID_ARG, "n_q_heads (%d) must be a positive multiple of n_kv_heads (%d)", p->n_q_heads,
                p->n_kv_heads);
  if (p->max_ctx < TILE || p->max_ctx % TILE)
    return fail(KVQ_ERR_INVALID_ARG, "max_ctx must be a positive multiple of 64 (got %d)", p->max_ctx);
  if (p->in_dtype != KVQ_F16 && p->in_dtype != KVQ_BF16) return fail(KVQ_ERR_INVALID_ARG, "bad in_dtype");
  if (!valid_fmt(p->k_fmt) || !valid_fmt(p->v_fmt)) return fail(KVQ_ERR_INVALID_ARG, "bad k_fmt/v_fmt");
  if (p->v_fmt == KVQ_INT8) return fail(KVQ_ERR_UNSUPPORTED, "INT8 values are not supported");
  if (p->k_fmt == KVQ_INT8 && p->k_group != 32 && p->k_group != 128)
    return fail(KVQ_ERR_INVALID_ARG, "INT8 k_group must be 32 or 128");
  if (p->k_fmt == KVQ_INT4 && p->k_group != 16 && p->k_group != 32 && p->k_group != 128)
    return fail(KVQ_ERR_INVALID_ARG, "INT4 k_group must be 16, 32 or 128");
  if (p->v_fmt == KVQ_INT4 && p->v_group != 16 && p->v_group != 32 && p->v_group != 128)
    return fail(KVQ_ERR_INVALID_ARG, "v_group must be 16, 32 or 128");
  if (p->scale_mode != KVQ_SCALE_ABSMAX && p->scale_mode != KVQ_SCALE_SEARCH9 &&
      p->scale_mode != KVQ_SCALE_SEARCH_OFFSETS)
    return fail(KVQ_ERR_INVALID_ARG, "bad scale_mode");
  if (p->rotation != KVQ_ROT_NONE && p->rotation != KVQ_ROT_SIGN_FWHT && p->rotation != KVQ_ROT_DENSE &&
      p->rotation != KVQ_ROT_SRFT)
    return fail(KVQ_ERR_INVALID_ARG, "bad rotation");
  if (!(p->softmax_scale >= 0.0f) || isinf(p->softmax_scale)) return fail(KVQ_ERR_INVALID_ARG, "bad softmax_scale");
  if (p->sink_blocks < 0 || p->recent_blocks < 0 || (long)p->sink_blocks + p->recent_blocks > p->max_ctx / TILE)
    return fail(KVQ_ERR_INVALID_ARG, "sink_blocks (%d) and recent_blocks (%d) must be >= 0 with sum <= max_ctx / 64",
                p->sink_blocks, p->recent_blocks);
  return KVQ_OK;
}

kvq_status check_cache(const kvq_params* p, const kvq_cache* c, bool need_desc) {
  if (!c) return fail(KVQ_ERR_INVALID_ARG, "cache is NULL");
  if (!c->k_codes || !c->k_meta || !c->v_codes || !c->v_meta)
    return fail(KVQ_ERR_INVALID_ARG, "code/metadata buffers must be non-NULL");
  if (!aligned16(c->k_codes) || !aligned16(c->k_meta) || !aligned16(c->v_codes) || !aligned16(c->v_meta))
    return fail(KVQ_ERR_INVALID_ARG, "code/metadata buffers must be 16-byte aligned");
  if ((p->rotation == KVQ_ROT_SIGN_FWHT || p->rotation == KVQ_ROT_SRFT) && !c->signs)
    return fail(KVQ_ERR_INVALID_ARG, "signs required for SIGN_FWHT and SRFT");
  if (p->rotation == KVQ_ROT_DENSE && (!c->rot_f16 || !aligned16(c->rot_f16)))
    return fail(KVQ_ERR_INVALID_ARG, "rot_f16 (16-byte aligned) required for DENSE");
  if (p->keep_fp16_copy) {
    if (!c->blk_desc || !c->k_orig || !c->v_orig)
      return fail(KVQ_ERR_INVALID_ARG, "keep_fp16_copy needs blk_desc, k_orig and v_orig");
    if (!aligned16(c->k_orig) || !aligned16(c->v_orig))
      return fail(KVQ_ERR_INVALID_ARG, "k_orig/v_orig must be 16-byte aligned");
  } else if (need_desc) {
    return fail(KVQ_ERR_INVALID_ARG, "this call needs keep_fp16_copy");
  }
  // The descriptors are residual norms in the rotated basis; they bound original-basis
  // errors only for an orthogonal rotation, and the fp16-rounded dense matrix is not one.
  if (p->keep_fp16_copy && p->rotation == KVQ_ROT_DENSE)
    return fail(KVQ_ERR_UNSUPPORTED, "keep_fp16_copy (certified descriptors) is not supported with the dense rotation");
  if (p->sink_blocks + p->recent_blocks > 0 &&
      (!c->k_win || !c->v_win || !aligned16(c->k_win) || !aligned16(c->v_win)))
    return fail(KVQ_ERR_INVALID_ARG, "a window (sink_blocks + recent_blocks > 0) needs k_win and v_win, 16-byte aligned");
  return KVQ_OK;
}

kvq_status check_seq(const kvq_params* p, const int32_t* seq_host, SeqArray& out) {
  if (!seq_host) return fail(KVQ_ERR_INVALID_ARG, "seq_len_host is NULL");
  for (int b = 0; b < p->batch; ++b) {
    if (seq_host[b] < 0 || seq_host[b] > p->max_ctx)
      return fail(KVQ_ERR_INVALID_ARG, "seq_len_host[%d] = %d outside [0, %d]", b, seq_host[b], p->max_ctx);
    out.v[b] = seq_host[b];
  }
  return KVQ_OK;
}

// SRFT twiddles W128^k = (fl32(cos(2 pi k / 128)), fl32(-sin(2 pi k / 128))), k = 0..64: the
// fp64 values (angle computed as (2 pi) k / 128) rounded once
void srft_twiddles(float* re, float* im) {
  for (int k = 0; k <= 64; ++k) {
    const double ang = 2.0 * M_PI * (double)k / 128.0;
    re[k] = (float)cos(ang);
    im[k] = (float)(-sin(ang));
  }
}
// cos(2 pi k / 128), k = 0..127: entries of the SRFT matrix (query and output rotations)
void srft_cos_table(float* c) {
  for (int k = 0; k < 128; ++k) c[k] = (float)cos(2.0 * M_PI * (double)k / 128.0);
}

float softmax_scale(const kvq_params* p) { return p->softmax_scale > 0.0f ? p->softmax_scale : 1.0f / sqrtf((float)D); }

// split count for decode: about two workgroups per CU (256 CUs), at
// least 8 chunks (512 tokens) per workgroup, at most MAX_SPLITS
// Context splits per (sequence, kv head, group of 4 query heads): enough workgroups
// to fill the GPU (quantized path: 8-wave workgroups, one per CU; fp16 baseline:
// 4-wave workgroups, two per CU), each with at least 2 chunks per wave.
int choose_splits(const kvq_params* p, int max_chunks, bool dense = false) {
  const int G = p->n_q_heads / p->n_kv_heads;
  const int hg = (G + 3) / 4;
  const long units = (long)p->batch * p->n_kv_heads * hg;
  const long wgs = dense ? 512 : 256;
  long target = (wgs + units - 1) / units;
  long by_len = max_chunks / (dense ? 8 : 16);
  if (by_len < 1) by_len = 1;
  long s = target < by_len ? target : by_len;
  if (s < 1) s = 1;
  if (s > MAX_SPLITS) s = MAX_SPLITS;
  return (int)s;
}

int units_of(const kvq_params* p) {
  const int G = p->n_q_heads / p->n_kv_heads;
  return p->batch * p->n_kv_heads * ((G + 3) / 4);
}

// The dense fallback recomputes a few rows, so it splits each of their sequences finely
// (chunks of 8 or more 64-token blocks, at most 16 splits) to spread them over the CUs.
// The dense fallback runs only the units with a row to recompute, usually a few: more
// splits spread them over more CUs (32 measured best on the certified shape with 26 of
// 256 units falling back: 16 splits 148 us, 32 splits 125 us, 64 splits 139 us).
int fallback_splits(int max_chunks) {
  int s = max_chunks / 8;
  if (s < 1) s = 1;
  if (s > 32) s = 32;
  return s;
}

int max_splits_for(const kvq_params* p) {
  const int a = choose_splits(p, p->max_ctx / TILE, false), b = choose_splits(p, p->max_ctx / TILE, true);
  const int c = p->keep_fp16_copy ? fallback_splits(p->max_ctx / TILE) : 1;
  return std::max(a, std::max(b, c));
}

}  // namespace

extern "C" {

int32_t kvq_abi_version(void) { return KVQ_ABI_VERSION; }

kvq_status kvq_debug_status(uint32_t* out, int32_t clear) {
  if (!out) return fail(KVQ_ERR_INVALID_ARG, "out is NULL");
#ifdef KVQ_DEBUG
  // the four translation units keep their own records; the first one with a failure names it
  hipError_t (*const readers[4])(uint32_t*, bool) = {dbg_read_append, dbg_read_decode, dbg_read_bound,
                                                     dbg_read_adaptive};
  out[0] = out[1] = out[2] = out[3] = 0;
  for (auto rd : readers) {
    uint32_t w[4];
    const hipError_t e = rd(w, clear != 0);
    if (e != hipSuccess) return hip_fail(e, "debug record");
    if (out[0] == 0 && w[0] != 0) {
      out[0] = w[0];
      out[1] = w[1];
      out[2] = w[2];
    }
    out[3] += w[3];
  }
  return KVQ_OK;
#else
  (void)clear;
  out[0] = out[1] = out[2] = out[3] = 0;
  return fail(KVQ_ERR_UNSUPPORTED, "layout checks exist only in the debug library (libkvq_debug.so)");
#endif
}

const char* kvq_status_str(kvq_status s) {
  switch (s) {
    case KVQ_OK: return "KVQ_OK";
    case KVQ_ERR_INVALID_ARG: return "KVQ_ERR_INVALID_ARG";
    case KVQ_ERR_UNSUPPORTED: return "KVQ_ERR_UNSUPPORTED";
    case KVQ_ERR_WORKSPACE: return "KVQ_ERR_WORKSPACE";
    case KVQ_ERR_HIP: return "KVQ_ERR_HIP";
    default: return "KVQ_UNKNOWN_STATUS";
  }
}

const char* kvq_last_error(void) { return g_err; }

kvq_status kvq_buffer_bytes(const kvq_params* p, size_t* out) {
  kvq_status st = check_params(p);
  if (st) return st;
  if (!out) return fail(KVQ_ERR_INVALID_ARG, "out_bytes is NULL");
  const size_t streams = (size_t)p->batch * p->n_kv_heads;
  const size_t T = (size_t)p->max_ctx, nt = T / TILE;
  const int kg = eff_group(p->k_fmt, p->k_group), vg = eff_group(p->v_fmt, p->v_group);
  out[KVQ_BUF_K_CODES] = streams * T * row_bytes(p->k_fmt);
  out[KVQ_BUF_K_META] = streams * T * meta_bytes(p->k_fmt, kg);
  out[KVQ_BUF_V_CODES] = streams * nt * D * chan_bytes(p->v_fmt);
  out[KVQ_BUF_V_META] = streams * nt * TILE * meta_bytes(p->v_fmt, vg);
  const bool keep = p->keep_fp16_copy != 0;
  out[KVQ_BUF_BLK_DESC] = keep ? streams * nt * 3 * sizeof(float) : 0;
  out[KVQ_BUF_K_ORIG] = keep ? streams * T * D * 2 : 0;
  out[KVQ_BUF_V_ORIG] = keep ? streams * T * D * 2 : 0;
  const size_t win = (size_t)(p->sink_blocks + p->recent_blocks) * TILE;
  out[KVQ_BUF_K_WIN] = streams * win * D * 2;
  out[KVQ_BUF_V_WIN] = streams * win * D * 2;
  return KVQ_OK;
}

int32_t kvq_decode_splits(const kvq_params* p, const int32_t* seq_len_host) {
  if (check_params(p) || !seq_len_host) return 0;
  int max_chunks = 0;
  for (int b = 0; b < p->batch; ++b) {
    const int32_t t = seq_len_host[b];
    if (t < 0 || t > p->max_ctx) return 0;
    const int ch = (t + TILE - 1) / TILE;
    if (ch > max_chunks) max_chunks = ch;
  }
  return choose_splits(p, max_chunks > 0 ? max_chunks : 1);
}

// workspace: [arrival counters, one int32 per unit (sequence, kv head, group of 4 query
// heads), padded to 256 bytes][split records]
static size_t ctr_bytes(const kvq_params* p) {
  const size_t n = (size_t)units_of(p);
  return (n * sizeof(int32_t) + 255) & ~(size_t)255;
}

size_t kvq_decode_workspace_bytes(const kvq_params* p) {
  if (check_params(p)) return 0;
  return ctr_bytes(p) + (size_t)p->batch * p->n_q_heads * max_splits_for(p) * PART_FLOATS * sizeof(float);
}

kvq_status kvq_append(const kvq_params* p, const kvq_cache* c, const void* k_new, const void* v_new,
                      const int32_t* start_pos_host, int32_t n_new, void* stream) {
  kvq_status st = check_params(p);
  if (st) return st;
  if ((st = check_cache(p, c, false))) return st;
  if (n_new < 0) return fail(KVQ_ERR_INVALID_ARG, "n_new < 0");
  if (n_new == 0) return KVQ_OK;
  if (!k_new || !v_new || !aligned16(k_new) || !aligned16(v_new))
    return fail(KVQ_ERR_INVALID_ARG, "k_new/v_new must be non-NULL and 16-byte aligned");
  if (!start_pos_host) return fail(KVQ_ERR_INVALID_ARG, "start_pos_host is NULL");
  AppendArgs a;
  memset(&a, 0, sizeof(a));
  int max_tiles = 0;
  for (int b = 0; b < p->batch; ++b) {
    const int s0 = start_pos_host[b];
    if (s0 < 0 || (long)s0 + n_new > p->max_ctx)
      return fail(KVQ_ERR_INVALID_ARG, "start_pos_host[%d] = %d: [start, start + %d) exceeds max_ctx %d", b, s0, n_new,
                  p->max_ctx);
    a.start.v[b] = s0;
    const int tiles = (s0 + n_new - 1) / TILE - s0 / TILE + 1;
    if (tiles > max_tiles) max_tiles = tiles;
  }
  a.k_new = (const uint16_t*)k_new;
  a.v_new = (const uint16_t*)v_new;
  a.k_codes = (uint8_t*)c->k_codes;
  a.k_meta = (uint8_t*)c->k_meta;
  a.v_codes = (uint8_t*)c->v_codes;
  a.v_meta = (uint8_t*)c->v_meta;
  if (p->keep_fp16_copy) {
    a.desc = c->blk_desc;
    a.k_orig = (uint16_t*)c->k_orig;
    a.v_orig = (uint16_t*)c->v_orig;
  }
  a.signs = c->signs;
  a.rot = c->rot_f16;
  a.clip_k = p->k_fmt == KVQ_INT2 ? c->clip_k : nullptr;
  a.clip_v = p->v_fmt == KVQ_INT2 ? c->clip_v : nullptr;
  a.lam_k = c->lambda_k;
  a.lam_v = c->lambda_v;
  a.B = p->batch;
  a.H = p->n_kv_heads;
  a.Tmax = p->max_ctx;
  a.n_new = n_new;
  a.in_bf16 = p->in_dtype == KVQ_BF16;
  a.k_fmt = p->k_fmt;
  a.v_fmt = p->v_fmt;
  a.k_group = eff_group(p->k_fmt, p->k_group);
  a.v_group = eff_group(p->v_fmt, p->v_group);
  a.scale_mode = p->scale_mode;
  a.rotation = p->rotation;
  if (p->rotation == KVQ_ROT_SRFT) srft_twiddles(a.tw_re, a.tw_im);
  hipError_t e = launch_append(a, max_tiles, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "append launch");
  if (p->sink_blocks + p->recent_blocks > 0) {
    a.k_win = (uint16_t*)c->k_win;
    a.v_win = (uint16_t*)c->v_win;
    a.n_sink = p->sink_blocks;
    a.n_recent = p->recent_blocks;
    e = launch_window_copy(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "window copy launch");
  }
  return KVQ_OK;
}

kvq_status kvq_calibrate_clip(const kvq_params* p, const kvq_cache* c, const void* calib_k, const void* calib_v,
                              int32_t n_tokens, float ratio, float* clip_k_out, float* clip_v_out, void* stream) {
  kvq_status st = check_params(p);
  if (st) return st;
  if (!c) return fail(KVQ_ERR_INVALID_ARG, "cache is NULL");
  if ((p->rotation == KVQ_ROT_SIGN_FWHT || p->rotation == KVQ_ROT_SRFT) && !c->signs)
    return fail(KVQ_ERR_INVALID_ARG, "signs required");
  if (p->rotation == KVQ_ROT_DENSE && !c->rot_f16) return fail(KVQ_ERR_INVALID_ARG, "rot_f16 required");
  if (n_tokens < 1) return fail(KVQ_ERR_INVALID_ARG, "n_tokens must be >= 1");
  if (!(ratio > 0.0f) || isinf(ratio)) return fail(KVQ_ERR_INVALID_ARG, "ratio must be positive and finite");
  if (!calib_k || !calib_v || !clip_k_out || !clip_v_out || !aligned16(calib_k) || !aligned16(calib_v))
    return fail(KVQ_ERR_INVALID_ARG, "calibration buffers must be non-NULL (inputs 16-byte aligned)");
  CalibArgs a;
  memset(&a, 0, sizeof(a));
  a.signs = c->signs;
  a.rot = c->rot_f16;
  a.H = p->n_kv_heads;
  a.n = n_tokens;
  a.in_bf16 = p->in_dtype == KVQ_BF16;
  a.rotation = p->rotation;
  a.ratio = ratio;
  if (p->rotation == KVQ_ROT_SRFT) srft_twiddles(a.tw_re, a.tw_im);
  hipStream_t s = (hipStream_t)stream;
  a.x = (const uint16_t*)calib_k;
  a.out = clip_k_out;
  a.lam = c->lambda_k;
  hipError_t e = launch_calibrate(a, s);
  if (e != hipSuccess) return hip_fail(e, "calibrate launch");
  a.x = (const uint16_t*)calib_v;
  a.out = clip_v_out;
  a.lam = c->lambda_v;
  e = launch_calibrate(a, s);
  if (e != hipSuccess) return hip_fail(e, "calibrate launch");
  return KVQ_OK;
}

kvq_status kvq_calibrate_lambda(const kvq_params* p, const kvq_cache* c, const void* calib_k, const void* calib_v,
                                int32_t n_tokens, float* lambda_k_out, float* lambda_v_out, void* stream) {
  kvq_status st = check_params(p);
  if (st) return st;
  if (!c) return fail(KVQ_ERR_INVALID_ARG, "cache is NULL");
  if ((p->rotation == KVQ_ROT_SIGN_FWHT || p->rotation == KVQ_ROT_SRFT) && !c->signs)
    return fail(KVQ_ERR_INVALID_ARG, "signs required");
  if (p->rotation == KVQ_ROT_DENSE && !c->rot_f16) return fail(KVQ_ERR_INVALID_ARG, "rot_f16 required");
  if (n_tokens < 1) return fail(KVQ_ERR_INVALID_ARG, "n_tokens must be >= 1");
  if (!calib_k || !calib_v || !lambda_k_out || !lambda_v_out || !aligned16(calib_k) || !aligned16(calib_v))
    return fail(KVQ_ERR_INVALID_ARG, "calibration buffers must be non-NULL (inputs 16-byte aligned)");
  CalibArgs a;
  memset(&a, 0, sizeof(a));
  a.signs = c->signs;
  a.rot = c->rot_f16;
  a.H = p->n_kv_heads;
  a.n = n_tokens;
  a.in_bf16 = p->in_dtype == KVQ_BF16;
  a.rotation = p->rotation;
  a.mode = 1;
  if (p->rotation == KVQ_ROT_SRFT) srft_twiddles(a.tw_re, a.tw_im);
  hipStream_t s = (hipStream_t)stream;
  a.x = (const uint16_t*)calib_k;
  a.out = lambda_k_out;
  hipError_t e = launch_calibrate(a, s);
  if (e != hipSuccess) return hip_fail(e, "calibrate launch");
  a.x = (const uint16_t*)calib_v;
  a.out = lambda_v_out;
  e = launch_calibrate(a, s);
  if (e != hipSuccess) return hip_fail(e, "calibrate launch");
  return KVQ_OK;
}

kvq_status kvq_error_bound(const kvq_params* p, const kvq_cache* c, const void* q, const int32_t* seq_len_host,
                           float tau, float* block_bound, uint8_t* block_flags, void* stream) {
  kvq_status st = check_params(p);
  if (st) return st;
  if ((st = check_cache(p, c, true))) return st;
  if (!q || !block_bound || !block_flags) return fail(KVQ_ERR_INVALID_ARG, "q/block_bound/block_flags are NULL");
  if (isnan(tau) || tau < 0.0f) return fail(KVQ_ERR_INVALID_ARG, "tau must be >= 0");
  BoundArgs a;
  memset(&a, 0, sizeof(a));
  if ((st = check_seq(p, seq_len_host, a.seq))) return st;
  a.q = (const uint16_t*)q;
  a.desc = c->blk_desc;
  a.bound = block_bound;
  a.flags = block_flags;
  a.B = p->batch;
  a.Hq = p->n_q_heads;
  a.H = p->n_kv_heads;
  a.nt = p->max_ctx / TILE;
  a.in_bf16 = p->in_dtype == KVQ_BF16;
  a.scale = softmax_scale(p);
  a.tau = tau;
  hipError_t e = launch_bound(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "bound launch");
  return KVQ_OK;
}

// ws == nullptr with noalloc: the library's fixed per-device workspace (no allocation)
static kvq_status decode_common(const kvq_params* p, const kvq_cache* c, const void* q, const int32_t* seq_len_host,
                                const uint8_t* flags, float* out, float* cert, void* ws, size_t ws_bytes,
                                void* stream, bool dense, const void* kd, const void* vd, bool noalloc = false) {
  kvq_status st = check_params(p);
  if (st) return st;
  if (!q || !out) return fail(KVQ_ERR_INVALID_ARG, "q/out are NULL");
  DecodeArgs a;
  memset(&a, 0, sizeof(a));
  if ((st = check_seq(p, seq_len_host, a.seq))) return st;
  int max_chunks = 0;
  for (int b = 0; b < p->batch; ++b) {
    const int ch = (a.seq.v[b] + TILE - 1) / TILE;
    if (ch > max_chunks) max_chunks = ch;
  }
  const int n_splits = choose_splits(p, max_chunks > 0 ? max_chunks : 1, dense);
  if (noalloc) {
    const size_t nctr = ctr_bytes(p);
    const size_t nrec = (size_t)p->batch * p->n_q_heads * n_splits * PART_FLOATS * sizeof(float);
    if (nctr > SCRATCH_CTR_BYTES)
      return fail(KVQ_ERR_WORKSPACE, "the fixed workspace holds %zu bytes of split counters; this call needs %zu",
                  SCRATCH_CTR_BYTES, nctr);
    if (nrec > SCRATCH_BYTES - SCRATCH_CTR_BYTES)
      return fail(KVQ_ERR_WORKSPACE, "the fixed workspace holds %zu bytes of split records; this call needs %zu",
                  SCRATCH_BYTES - SCRATCH_CTR_BYTES, nrec);
  } else {
    const size_t need = kvq_decode_workspace_bytes(p);
    if (!ws || ws_bytes < need) return fail(KVQ_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, ws_bytes);
    if (((uintptr_t)ws & 255u) != 0) return fail(KVQ_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  }
  a.q = (const uint16_t*)q;
  if (dense) {
    if (!kd || !vd || !aligned16(kd) || !aligned16(vd))
      return fail(KVQ_ERR_INVALID_ARG, "k/v must be non-NULL and 16-byte aligned");
    a.k_orig = (const uint16_t*)kd;
    a.v_orig = (const uint16_t*)vd;
  } else {
    if ((st = check_cache(p, c, flags != nullptr || cert != nullptr))) return st;
    a.k_codes = (const uint8_t*)c->k_codes;
    a.k_meta = (const uint8_t*)c->k_meta;
    a.v_codes = (const uint8_t*)c->v_codes;
    a.v_meta = (const uint8_t*)c->v_meta;
    if (p->keep_fp16_copy) {
      a.desc = c->blk_desc;
      a.k_orig = (const uint16_t*)c->k_orig;
      a.v_orig = (const uint16_t*)c->v_orig;
    }
    a.flags = flags;
    a.lam_k = c->lambda_k;
    a.lam_v = c->lambda_v;
    if (p->sink_blocks + p->recent_blocks > 0) {
      a.k_win = (const uint16_t*)c->k_win;
      a.v_win = (const uint16_t*)c->v_win;
      a.n_sink = p->sink_blocks;
      a.n_recent = p->recent_blocks;
    }
    a.signs = c->signs;
    a.rot = c->rot_f16;
  }
  hipStream_t s = (hipStream_t)stream;
  if (noalloc) {
    void* base = nullptr;
    hipError_t e = decode_scratch(&base, s);
    if (e != hipSuccess) return hip_fail(e, "fixed decode workspace");
    a.ctr = (int*)base;
    a.part = (float*)((char*)base + SCRATCH_CTR_BYTES);
  } else {
    a.ctr = (int*)ws;
    a.part = (float*)((char*)ws + ctr_bytes(p));
  }
  a.U = units_of(p);
  a.out = out;
  a.cert = dense ? nullptr : cert;
  a.B = p->batch;
  a.Hq = p->n_q_heads;
  a.H = p->n_kv_heads;
  a.G = p->n_q_heads / p->n_kv_heads;
  a.Tmax = p->max_ctx;
  a.nt = p->max_ctx / TILE;
  a.in_bf16 = p->in_dtype == KVQ_BF16;
  a.rotation = dense ? KVQ_ROT_NONE : p->rotation;
  a.k_group = eff_group(p->k_fmt, p->k_group);
  a.v_group = eff_group(p->v_fmt, p->v_group);
  a.n_splits = n_splits;
  a.chunks_per_split = (max_chunks + n_splits - 1) / n_splits;
  if (a.chunks_per_split < 1) a.chunks_per_split = 1;
  a.scale = softmax_scale(p);
  if (a.rotation == KVQ_ROT_SRFT) srft_cos_table(a.cos128);
  hipError_t e = launch_decode(a, p->k_fmt, p->v_fmt, dense, s);
  if (e == hipErrorNotSupported) return fail(KVQ_ERR_UNSUPPORTED, "format combination not supported by decode");
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return KVQ_OK;
}

static void adapt_common(const kvq_params* p, AdaptArgs& a) {
  a.B = p->batch;
  a.Hq = p->n_q_heads;
  a.H = p->n_kv_heads;
  a.G = p->n_q_heads / p->n_kv_heads;
  a.Tmax = p->max_ctx;
  a.nt = p->max_ctx / TILE;
  a.in_bf16 = p->in_dtype == KVQ_BF16;
  a.rotation = p->rotation;
  a.k_fmt = p->k_fmt;
  a.k_group = eff_group(p->k_fmt, p->k_group);
  a.scale = softmax_scale(p);
  if (p->rotation == KVQ_ROT_SRFT) srft_cos_table(a.cos128);
}

kvq_status kvq_block_mass(const kvq_params* p, const kvq_cache* c, const void* q, const int32_t* seq_len_host,
                          float* mass, void* stream) {
  kvq_status st = check_params(p);
  if (st) return st;
  if ((st = check_cache(p, c, false))) return st;
  if (!q || !mass) return fail(KVQ_ERR_INVALID_ARG, "q/mass are NULL");
  AdaptArgs a;
  memset(&a, 0, sizeof(a));
  if ((st = check_seq(p, seq_len_host, a.seq))) return st;
  adapt_common(p, a);
  a.q = (const uint16_t*)q;
  a.k_codes = (const uint8_t*)c->k_codes;
  a.k_meta = (const uint8_t*)c->k_meta;
  a.signs = c->signs;
  a.rot = c->rot_f16;
  a.lam_k = c->lambda_k;
  a.mass = mass;
  hipError_t e = launch_block_mass(a, (hipStream_t)stream);
  if (e == hipErrorNotSupported) return fail(KVQ_ERR_UNSUPPORTED, "key format not supported by the scoring pass");
  if (e != hipSuccess) return hip_fail(e, "block mass launch");
  return KVQ_OK;
}

kvq_status kvq_select_blocks(const kvq_params* p, const float* mass, const int32_t* seq_len_host, float tau_cov,
                             const uint8_t* flags_in, uint8_t* flags_out, void* stream) {
  kvq_status st = check_params(p);
  if (st) return st;
  if (!mass || !flags_out) return fail(KVQ_ERR_INVALID_ARG, "mass/flags_out are NULL");
  if (!(tau_cov >= 0.0f && tau_cov <= 1.0f)) return fail(KVQ_ERR_INVALID_ARG, "tau_cov must be in [0, 1]");
  if (p->max_ctx / TILE > MAX_SELECT_BLOCKS)
    return fail(KVQ_ERR_UNSUPPORTED, "selection supports max_ctx / 64 <= %d blocks", MAX_SELECT_BLOCKS);
  AdaptArgs a;
  memset(&a, 0, sizeof(a));
  if ((st = check_seq(p, seq_len_host, a.seq))) return st;
  adapt_common(p, a);
  a.mass = const_cast<float*>(mass);
  a.flags_in = flags_in;
  a.flags_out = flags_out;
  a.tau_cov = tau_cov;
  hipError_t e = launch_select(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "select launch");
  return KVQ_OK;
}

kvq_status kvq_promote_values(const kvq_params* p, const kvq_cache* c, const float* mass,
                              const int32_t* seq_len_host, float tau_v, uint8_t* flags, void* stream) {
  kvq_status st = check_params(p);
  if (st) return st;
  if ((st = check_cache(p, c, true))) return st;
  if (!mass || !flags) return fail(KVQ_ERR_INVALID_ARG, "mass/flags are NULL");
  if (!(tau_v >= 0.0f)) return fail(KVQ_ERR_INVALID_ARG, "tau_v must be >= 0");
  AdaptArgs a;
  memset(&a, 0, sizeof(a));
  if ((st = check_seq(p, seq_len_host, a.seq))) return st;
  adapt_common(p, a);
  a.mass = const_cast<float*>(mass);
  a.desc = c->blk_desc;
  a.flags_out = flags;
  a.tau_v = tau_v;
  hipError_t e = launch_promote_values(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "value promotion launch");
  return KVQ_OK;
}

kvq_status kvq_ranking_check(const kvq_params* p, const kvq_cache* c, const void* q, const int32_t* seq_len_host,
                             const float* mass, float tau_cov, float margin, int32_t max_inversions,
                             int32_t* inversions, uint8_t* fail_out, void* stream) {
  kvq_status st = check_params(p);
  if (st) return st;
  if ((st = check_cache(p, c, true))) return st;
  if (!q || !mass || !inversions || !fail_out) return fail(KVQ_ERR_INVALID_ARG, "q/mass/inversions/fail are NULL");
  if (!(tau_cov >= 0.0f && tau_cov <= 1.0f)) return fail(KVQ_ERR_INVALID_ARG, "tau_cov must be in [0, 1]");
  if (!(margin >= 0.0f) || margin == INFINITY) return fail(KVQ_ERR_INVALID_ARG, "margin must be finite and >= 0");
  if (max_inversions < 0) return fail(KVQ_ERR_INVALID_ARG, "max_inversions must be >= 0");
  if (p->max_ctx / TILE > MAX_SELECT_BLOCKS)
    return fail(KVQ_ERR_UNSUPPORTED, "the ranking check supports max_ctx / 64 <= %d blocks", MAX_SELECT_BLOCKS);
  AdaptArgs a;
  memset(&a, 0, sizeof(a));
  if ((st = check_seq(p, seq_len_host, a.seq))) return st;
  adapt_common(p, a);
  a.q = (const uint16_t*)q;
  a.k_orig = (const uint16_t*)c->k_orig;
  a.mass = const_cast<float*>(mass);
  a.tau_cov = tau_cov;
  a.margin = margin;
  a.max_inv = max_inversions;
  a.inv = inversions;
  a.fail = fail_out;
  hipError_t e = launch_ranking_check(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "ranking check launch");
  return KVQ_OK;
}

kvq_status kvq_dense_fallback(const kvq_params* p, const kvq_cache* c, const void* q, const int32_t* seq_len_host,
                              float eps, const uint8_t* head_fail, float* out, float* certificate, void* workspace,
                              size_t workspace_bytes, void* stream) {
  kvq_status st = check_params(p);
  if (st) return st;
  if ((st = check_cache(p, c, true))) return st;
  if (!q || !out) return fail(KVQ_ERR_INVALID_ARG, "q/out are NULL");
  if (!certificate && !head_fail) return fail(KVQ_ERR_INVALID_ARG, "certificate and fail are both NULL");
  if (!(eps >= 0.0f)) return fail(KVQ_ERR_INVALID_ARG, "eps must be >= 0");
  const size_t need = kvq_decode_workspace_bytes(p);
  if (!workspace || workspace_bytes < need)
    return fail(KVQ_ERR_WORKSPACE, "workspace needs %zu bytes (got %zu)", need, workspace_bytes);
  if (((uintptr_t)workspace & 255u) != 0) return fail(KVQ_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  DecodeArgs a;
  memset(&a, 0, sizeof(a));
  if ((st = check_seq(p, seq_len_host, a.seq))) return st;
  int max_chunks = 0;
  for (int b = 0; b < p->batch; ++b) max_chunks = std::max(max_chunks, (a.seq.v[b] + TILE - 1) / TILE);
  a.q = (const uint16_t*)q;
  a.k_orig = (const uint16_t*)c->k_orig;
  a.v_orig = (const uint16_t*)c->v_orig;
  a.part = (float*)((char*)workspace + ctr_bytes(p));
  a.out = out;
  a.fb_cert = certificate;
  a.fb_fail = head_fail;
  a.fb_eps = eps;
  a.B = p->batch;
  a.Hq = p->n_q_heads;
  a.H = p->n_kv_heads;
  a.G = p->n_q_heads / p->n_kv_heads;
  a.Tmax = p->max_ctx;
  a.nt = p->max_ctx / TILE;
  a.in_bf16 = p->in_dtype == KVQ_BF16;
  a.rotation = KVQ_ROT_NONE;
  a.n_splits = fallback_splits(max_chunks > 0 ? max_chunks : 1);
  a.chunks_per_split = std::max(1, (max_chunks + a.n_splits - 1) / a.n_splits);
  a.U = units_of(p);
  a.scale = softmax_scale(p);
  hipError_t e = launch_dense_fallback(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "fallback launch");
  return KVQ_OK;
}

kvq_status kvq_decode_attn(const kvq_params* p, const kvq_cache* c, const void* q, const int32_t* seq_len_host,
                           const uint8_t* block_flags, float* out, float* certificate, void* workspace,
                           size_t workspace_bytes, void* stream) {
  return decode_common(p, c, q, seq_len_host, block_flags, out, certificate, workspace, workspace_bytes, stream, false,
                       nullptr, nullptr);
}

kvq_status kvq_decode_attn_noalloc(const kvq_params* p, const kvq_cache* c, const void* q,
                                   const int32_t* seq_len_host, const uint8_t* block_flags, float* out,
                                   float* certificate, void* stream) {
  return decode_common(p, c, q, seq_len_host, block_flags, out, certificate, nullptr, 0, stream, false, nullptr,
                       nullptr, true);
}

kvq_status kvq_decode_attn_dense(const kvq_params* p, const void* k, const void* v, const void* q,
                                 const int32_t* seq_len_host, float* out, void* workspace, size_t workspace_bytes,
                                 void* stream) {
  return decode_common(p, nullptr, q, seq_len_host, nullptr, out, nullptr, workspace, workspace_bytes, stream, true, k,
                       v);
}

}  // extern "C"
