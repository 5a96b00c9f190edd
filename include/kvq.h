/*
 * kvq.h -- rotate-then-quantize KV cache with fused single-token decode attention
 * for AMD Instinct MI355X (gfx950).  C ABI; all compute runs in HIP kernels that
 * are enqueued on the caller's stream.
 *
 * What the calls compute (the pages, by title and section):
 *  - kvq_append: each new K/V head vector is widened to fp32, sign-flipped and
 *    rotated by a fast orthogonal transform, scaled per group and rounded to
 *    signed int4/int8 with two int4 codes per byte ("When Quantization Is Free:
 *    An int4 KV Cache That Outruns fp16 on Apple Silicon", Methodology sections
 *    1-3); or rotated by a fixed dense matrix, clipped per channel and coded in
 *    2 bits ("OSCAR: Offline Spectral Covariance-Aware Rotation for 2-bit KV
 *    Cache Quantization", section 2.2); or coded as FP4 E2M1 with one E4M3 scale
 *    per 16 elements whose value is searched around the absmax scale ("Search
 *    Your Block Floating Point Scales!", Methodology, ScaleSearch).  With
 *    keep_fp16_copy it also stores the original vectors and per-block error
 *    descriptors ("Runtime-Certified Bounded-Error Quantized Attention",
 *    Methodology section 1).
 *  - kvq_error_bound: per 64-token block, a certified bound on the logit and
 *    value errors from the query norm and the descriptors, and the blocks it
 *    flags for exact recompute ("Runtime-Certified ...", Methodology section 2).
 *  - kvq_decode_attn: rotates the query once, streams the packed cache,
 *    dequantizes in registers and computes softmax(q k^T * scale) v for the
 *    newest token with grouped-query heads; flagged blocks are recomputed from
 *    the stored originals; the output is rotated back to the original basis
 *    ("OSCAR", section 2.2B: unpack, dequantize, inverse rotation, attention).
 *  - kvq_decode_attn_dense: the same decode over uncompressed fp16/bf16 K/V
 *    (the baseline the compressed cache is compared against, and the full
 *    dense rung of the fallback).
 *  - kvq_calibrate_clip: per-channel clipping thresholds from rotated
 *    calibration vectors ("OSCAR", section 2.2A, clipping thresholds).
 *
 * Conventions for every call:
 *  - Ownership: the caller allocates and frees every buffer; the library never
 *    allocates device or host memory.  It keeps no state between calls, except
 *    for kvq_decode_attn_noalloc: a fixed device array per device (part of the
 *    library's code object) and its looked-up address.
 *    Pointers named *_host are host memory, all others device memory.
 *  - Asynchrony: work is enqueued on `stream` (0 = the null stream); results are
 *    valid once the stream has synchronised.  Calls that share buffers must be
 *    ordered by the caller (same stream or events).
 *  - Errors: arguments are validated on the host before anything is enqueued; a
 *    failure returns a negative kvq_status, enqueues nothing, and leaves a
 *    message for kvq_last_error() (thread-local).  A failed kernel launch
 *    returns KVQ_ERR_HIP.  No C++ exception crosses this interface.
 *  - Sizes: head_dim must be 128; max_ctx a positive multiple of 64; batch at
 *    most 256; n_q_heads a multiple of n_kv_heads (the group size G =
 *    n_q_heads / n_kv_heads; query head hq reads kv head hq / G).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_ABI_VERSION 5

typedef int32_t kvq_status;
#define KVQ_OK 0
#define KVQ_ERR_INVALID_ARG (-1)  /* bad shape, enum, pointer, alignment or range */
#define KVQ_ERR_UNSUPPORTED (-2)  /* valid but not implemented combination */
#define KVQ_ERR_WORKSPACE (-3)    /* workspace missing or too small */
#define KVQ_ERR_HIP (-4)          /* a HIP runtime call or launch failed */

/* input dtype of K/V/q vectors */
#define KVQ_F16 0
#define KVQ_BF16 1

/* code formats (K and V independently) */
#define KVQ_INT4 0 /* symmetric, codes -7..7, fp16 scale per group (16, 32 or 128) */
#define KVQ_INT8 1 /* symmetric, codes -127..127, fp16 scale per group (32 or 128) */
#define KVQ_INT2 2 /* asymmetric, codes 0..3, fp16 scale + fp16 offset per 32 */
#define KVQ_FP4 3  /* E2M1 codes, one E4M3 scale per 16 */

/* rotation applied before quantization (and to the query / output) */
#define KVQ_ROT_NONE 0
#define KVQ_ROT_SIGN_FWHT 1 /* y = fl32(FWHT(s * x) * fl32(1/sqrt(128))) */
#define KVQ_ROT_DENSE 2     /* y_j = sum_k R16[j][k] x_k, fp32 chain in k order */
/* y = pack(F diag(s) x), F the unitary DFT ("When Quantization Is Free", Methodology
 * sections 1-2): signs, the 64-point FFT of the channel pairs (x_2n + i x_2n+1) by
 * six radix-2 Stockham passes, Hermitian unpack to the real DFT X_0..X_64, then
 * y_0 = X_0 / sqrt(128), y_1 = X_64 / sqrt(128), y_2k = Re X_k / 8, y_2k+1 = Im X_k / 8
 * (an orthonormal packing), all in fp32 in a fixed order with twiddles
 * fl32(cos), fl32(-sin) of 2 pi k / 128 */
#define KVQ_ROT_SRFT 3

/* FP4 scale selection */
#define KVQ_SCALE_ABSMAX 0  /* S = E4M3(absmax / 6) */
#define KVQ_SCALE_SEARCH9 1 /* best of E4M3(absmax/6 * m), m = 0.900, 0.925, ..., 1.100 */
/* best of the E4M3 bit patterns c0 + f, c0 = E4M3(absmax/6), f = -2, ..., 6 (patterns
 * 0x00..0x7E only): the bit-offset search of "Search Your Block Floating Point Scales!",
 * Methodology, ScaleSearch */
#define KVQ_SCALE_SEARCH_OFFSETS 2

/* indices into the array filled by kvq_buffer_bytes */
#define KVQ_BUF_K_CODES 0
#define KVQ_BUF_K_META 1
#define KVQ_BUF_V_CODES 2
#define KVQ_BUF_V_META 3
#define KVQ_BUF_BLK_DESC 4
#define KVQ_BUF_K_ORIG 5
#define KVQ_BUF_V_ORIG 6
#define KVQ_BUF_K_WIN 7
#define KVQ_BUF_V_WIN 8
#define KVQ_NUM_BUFS 9

/* Shapes and formats of one cache (one layer).  Plain values, passed by pointer. */
typedef struct kvq_params {
  int32_t batch;          /* B, 1..256 */
  int32_t n_q_heads;      /* Hq */
  int32_t n_kv_heads;     /* Hkv; Hq % Hkv == 0 */
  int32_t head_dim;       /* must be 128 */
  int32_t max_ctx;        /* Tmax positions per sequence, multiple of 64 */
  int32_t in_dtype;       /* KVQ_F16 | KVQ_BF16 */
  int32_t k_fmt, v_fmt;   /* KVQ_INT4 | KVQ_INT8 | KVQ_INT2 | KVQ_FP4 (V: not INT8) */
  int32_t k_group;        /* INT4: 16, 32 or 128; INT8: 32 or 128; ignored otherwise */
  int32_t v_group;        /* INT4: 16, 32 or 128; ignored otherwise */
  int32_t scale_mode;     /* KVQ_SCALE_*: FP4 only */
  int32_t rotation;       /* KVQ_ROT_* (SIGN_FWHT and SRFT need signs) */
  int32_t keep_fp16_copy; /* nonzero: store originals + per-block descriptors */
  float softmax_scale;    /* 0 => 1/sqrt(head_dim) */
  /* Full-precision window ("OSCAR", section 2.2B, mixed-precision layout; "Search Your
   * Block Floating Point Scales!", attention-sink-aware mixed-precision caching): the
   * first sink_blocks and the last recent_blocks 64-token blocks of every sequence
   * are attended from their in_dtype originals, the blocks between from the codes.
   * Both 0 = no window.  sink_blocks + recent_blocks <= max_ctx / 64. */
  int32_t sink_blocks;
  int32_t recent_blocks;
} kvq_params;

/*
 * Device buffers of one cache.  Byte layouts (little-endian; b batch, h kv head,
 * t position, c channel, nt = max_ctx / 64):
 *   k_codes [B][Hkv][Tmax][KB]      KB = 64 (INT4, FP4), 128 (INT8), 32 (INT2):
 *                                   element c at nibble c%2 of byte c/2 (INT4/FP4,
 *                                   even element low), bits 2*(c%4) of byte c/4
 *                                   (INT2), byte c (INT8); INT4/INT8 two's complement
 *   k_meta  [B][Hkv][Tmax][KM]      fp16 scales per group (INT4/INT8: 128/group of
 *                                   them; groups of 16 follow "When Quantization Is
 *                                   Free", Methodology section 3), INT2: 4 fp16 scales then 4 fp16 offsets,
 *                                   FP4: 8 E4M3 bytes
 *   v_codes [B][Hkv][nt][128][CB]   per 64-token tile, channel-major: channel c's 64
 *                                   codes packed along tokens with the rules above
 *                                   (CB = 32 for INT4/FP4, 16 for INT2)
 *   v_meta  [B][Hkv][nt][NM][64]    per tile, metadata element m of token tau
 *                                   (fp16, or E4M3 bytes for FP4)
 *   blk_desc[B][Hkv][nt][3]         fp32 (ek, ev, vn) per 64-token block: max key /
 *                                   value reconstruction error norm and max value
 *                                   norm; combined by max, so zero it when a cache
 *                                   is (re)started.  Needed iff keep_fp16_copy.
 *   k_orig, v_orig [B][Hkv][Tmax][128]  in_dtype originals; needed iff keep_fp16_copy
 *   signs   [128] int8 of +1/-1                 needed for KVQ_ROT_SIGN_FWHT
 *   rot_f16 [128][128] fp16 bits, row-major     needed for KVQ_ROT_DENSE
 *   clip_k, clip_v [Hkv][128] fp32 thresholds   optional, INT2 only (NULL = none)
 *   k_win, v_win [B][Hkv][NW * 64][128]  in_dtype originals of the window blocks,
 *                                   NW = sink_blocks + recent_blocks; block j sits
 *                                   in slot j if j < sink_blocks, else in slot
 *                                   sink_blocks + j % recent_blocks (a ring), at row
 *                                   position % 64; needed iff NW > 0
 *   lambda_k, lambda_v [Hkv][128] fp32  per-channel rescale factors or NULL: the
 *                                   rotated vector is multiplied by them (fp32) before
 *                                   clipping and the group scales ("When Quantization
 *                                   Is Free", Methodology sections 2 and 3; one scale per
 *                                   coordinate with per-group scales), and decode
 *                                   divides them out; with keep_fp16_copy the
 *                                   descriptors hold the residuals taken back to
 *                                   the unscaled basis (times 1 / lambda)
 * Code, metadata, original and window buffers must be 16-byte aligned.
 */
typedef struct kvq_cache {
  void* k_codes;
  void* k_meta;
  void* v_codes;
  void* v_meta;
  float* blk_desc;
  void* k_orig;
  void* v_orig;
  const int8_t* signs;
  const uint16_t* rot_f16;
  const float* clip_k;
  const float* clip_v;
  void* k_win;
  void* v_win;
  const float* lambda_k;
  const float* lambda_v;
} kvq_cache;

/* Returns KVQ_ABI_VERSION. */
int32_t kvq_abi_version(void);

/* Human-readable name of a status code (static string). */
const char* kvq_status_str(kvq_status s);

/* Detail of the last error on the calling thread ("" if none). */
const char* kvq_last_error(void);

/* Layout checks of the debug library (libkvq_debug.so, the same sources compiled with
 * KVQ_DEBUG; not for production use).  Its kernels check every stream, position,
 * chunk, block, split-record and counter index they address against the sizes the call
 * was validated with; a failed check does not stop the kernel but is recorded per
 * device.  This call waits for the current device, then writes out[0] = code of the
 * first recorded failure (0 = none; the codes name the index kind: 1 stream, 2 chunk or
 * block, 3 split record, 4 counter, 5 window slot, 6 appended position, 7 query row),
 * out[1], out[2] = the two indices it recorded, out[3] = failures counted; clear != 0
 * resets the record.  out: host, 4 words.  The release library returns
 * KVQ_ERR_UNSUPPORTED without touching a device; a HIP failure returns
 * KVQ_ERR_HIP. */
kvq_status kvq_debug_status(uint32_t* out, int32_t clear);

/* Bytes of each cache buffer for these params, written to out_bytes[KVQ_NUM_BUFS]
 * (0 for buffers the configuration does not use).  Host only. */
kvq_status kvq_buffer_bytes(const kvq_params* p, size_t* out_bytes);

/* Workspace bytes kvq_decode_attn / kvq_decode_attn_dense / kvq_dense_fallback need
 * for these params (depends on batch, heads, max_ctx and keep_fp16_copy only).  Host
 * only; 0 on invalid params.
 * The workspace holds one arrival counter per unit (sequence, kv head, group of 4
 * query heads), through which the last of the unit's workgroups learns that it is
 * last and merges the others' results, and one partial-result record per (sequence,
 * query head, split).  It must be zero-filled before its
 * first use; every call leaves the counters zero again (the records' contents
 * do not matter), so one workspace serves call after call.  Calls that share a
 * workspace must not overlap (order them on one stream).  The split workgroups
 * share out 64-token chunks at run time, so the fp32 summation order, and with
 * it the last bits of the output, can differ from call to call. */
size_t kvq_decode_workspace_bytes(const kvq_params* p);

/* Number of context splits kvq_decode_attn uses for these params and sequence
 * lengths: each unit (sequence, kv head, group of 4 query heads) is served by that many
 * workgroups, each taking a range of its 64-token chunks.  Host only, informational; 0 on
 * invalid input. */
int32_t kvq_decode_splits(const kvq_params* p, const int32_t* seq_len_host);

/*
 * Append n_new tokens to every sequence: positions [start_pos_host[b],
 * start_pos_host[b] + n_new) of sequence b are (over)written.
 *   k_new, v_new: device [B][Hkv][n_new][128] in_dtype, contiguous.
 *   start_pos_host: host [B]; 0 <= start < start + n_new <= max_ctx.
 * Codes and scales are bit-exact functions of the inputs (fp32 arithmetic in a
 * fixed order, round-half-to-even of exact quotients).  Other positions of the
 * cache are left unchanged.  n_new == 0 is a no-op.
 * With a window, every position is still quantized; in addition the originals of
 * the positions in blocks j < sink_blocks, and in the last recent_blocks blocks
 * that this call reaches (blocks j > (start + n_new - 1) / 64 - recent_blocks),
 * are copied into the window.  Appending in position order therefore keeps the
 * window holding the sink blocks and the most recent blocks appended.
 */
kvq_status kvq_append(const kvq_params* p, const kvq_cache* cache, const void* k_new, const void* v_new,
                      const int32_t* start_pos_host, int32_t n_new, void* stream);

/*
 * Per-block error bound (needs keep_fp16_copy and descriptors).  For block j of
 * kv head h of sequence b (tokens [64j, 64j+64) below seq_len_host[b]):
 *   bound = max_{hq in group h} ||q_hq|| * scale * ek_j + ev_j,  flag = bound > tau;
 * blocks at or beyond seq_len get bound 0 and flag 0.
 *   q: device [B][Hq][128] in_dtype; seq_len_host: host [B], 0..max_ctx.
 *   block_bound: device fp32 [B][Hkv][max_ctx/64]; block_flags: device uint8, same shape.
 */
kvq_status kvq_error_bound(const kvq_params* p, const kvq_cache* cache, const void* q,
                           const int32_t* seq_len_host, float tau, float* block_bound,
                           uint8_t* block_flags, void* stream);

/*
 * Decode attention of one query token per (b, hq) over positions [0, seq_len_host[b]).
 *   q: device [B][Hq][128] in_dtype.
 *   block_flags: device uint8 [B][Hkv][max_ctx/64] or NULL (needs keep_fp16_copy):
 *     bit 0 set makes the block use k_orig/v_orig exactly; bit 1 set with bit 0
 *     clear keeps its logits from the codes and takes its values from v_orig
 *     (value promotion, "Runtime-Certified Bounded-Error Quantized Attention",
 *     Methodology section 3, rung 2); other bits are ignored.
 *   out: device fp32 [B][Hq][128], original (unrotated) basis.  Rows with
 *     seq_len 0 are written as zeros.
 *   certificate: device fp32 [B][Hq] or NULL (needs keep_fp16_copy): an upper bound
 *     on ||out - dense attention over the originals||_2 for that row (blocks with
 *     quantized keys enter its key term, blocks with quantized values its value sum).
 *   workspace: device, >= kvq_decode_workspace_bytes(p) bytes, 256-byte aligned,
 *     zero-filled before its first use (see kvq_decode_workspace_bytes).
 * With a window (sink_blocks + recent_blocks > 0), blocks j < sink_blocks and
 * j >= ceil(seq_len / 64) - recent_blocks are attended exactly from k_win/v_win in
 * the original basis (like flagged blocks), so seq_len must be the number of
 * positions appended in order (the ring holds the most recent blocks appended).
 * Attention output differs from exact fp64 attention over the decoded cache by
 * fp16 rounding of the query/probabilities and fp32 accumulation only.
 */
kvq_status kvq_decode_attn(const kvq_params* p, const kvq_cache* cache, const void* q,
                           const int32_t* seq_len_host, const uint8_t* block_flags, float* out,
                           float* certificate, void* workspace, size_t workspace_bytes, void* stream);

/*
 * kvq_decode_attn without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc): the same computation and the same q/out/certificate/flags
 * contract as kvq_decode_attn, with the split counters and records kept in a fixed
 * device array of the library (8 MiB per device: 64 KiB of counters, the rest for
 * records), which each device holds until the process ends.  It calls no
 * hipMalloc/hipFree.  The first call on a device looks the array's address up (with
 * that device current) and clears its counters with a fill kernel on `stream`.
 * A call needing more than the array holds (B * Hkv * ceil(G/4) * 4 bytes of
 * counters above 64 KiB, or B * Hq * splits * 1056 bytes of records above
 * 8 MiB - 64 KiB; splits as kvq_decode_splits reports) returns KVQ_ERR_WORKSPACE
 * and enqueues nothing.  All calls on one device share the array: calls that
 * overlap in time on one device (different streams, no ordering) race and give
 * wrong results; order them (one stream or events).
 */
kvq_status kvq_decode_attn_noalloc(const kvq_params* p, const kvq_cache* cache, const void* q,
                                   const int32_t* seq_len_host, const uint8_t* block_flags, float* out,
                                   float* certificate, void* stream);

/*
 * Adaptive precision ("Runtime-Certified Bounded-Error Quantized Attention",
 * Methodology section 3): a scoring pass over the quantized keys estimates each
 * block's attention mass; the blocks covering a fraction tau_cov of it are
 * promoted to exact recompute (kvq_select_blocks), blocks whose value error is
 * large against their estimated mass take exact values (kvq_promote_values, the
 * ladder's rung 2), kvq_decode_attn runs with those flags, and a head whose
 * promoted blocks rank differently under the originals (kvq_ranking_check), or
 * whose certificate still exceeds eps, is recomputed densely (kvq_dense_fallback,
 * rung 3).  Flags: device uint8 [B][Hkv][max_ctx/64], bits as for kvq_decode_attn.
 *
 * kvq_block_mass: mass[b][hq][j] = sum over the tokens t of block j of
 *   softmax_t(scale * (R q) . k_hat_t), the softmax over positions [0,
 *   seq_len_host[b]) of the quantized keys alone (fp32; 0 past the sequence).
 *   q: device [B][Hq][128] in_dtype; mass: device fp32 [B][Hq][max_ctx/64].
 *   Key formats as for kvq_decode_attn.
 */
kvq_status kvq_block_mass(const kvq_params* p, const kvq_cache* cache, const void* q,
                          const int32_t* seq_len_host, float* mass, void* stream);

/*
 * kvq_select_blocks: flags_out[b][h][j] = flags_in[b][h][j] (0 if flags_in is NULL)
 * with bit 0 set if block j is among the top-K* blocks of any query head of kv head
 * h (flags_in may equal flags_out).  Top-K* of a query head: its blocks below
 * seq_len sorted by decreasing mass (equal masses: lower index first), K* the
 * shortest prefix whose fp32 running sum, accumulated in that order, reaches
 * tau_cov (all blocks if it never does).  mass: device fp32 [B][Hq][max_ctx/64]
 * (from kvq_block_mass); tau_cov in [0, 1].
 * max_ctx / 64 must not exceed 4096 (KVQ_ERR_UNSUPPORTED otherwise).
 */
kvq_status kvq_select_blocks(const kvq_params* p, const float* mass, const int32_t* seq_len_host,
                             float tau_cov, const uint8_t* flags_in, uint8_t* flags_out, void* stream);

/*
 * kvq_promote_values (rung 2): in place, every block j below seq_len of kv head h
 * whose flag has bit 0 clear gets bit 1 if mass[b][hq][j] * ev_j > tau_v (one fp32
 * product) for some query head hq of h; ev_j is the block's value error descriptor
 * (blk_desc[..][1]).  Needs keep_fp16_copy.  mass: from kvq_block_mass; tau_v >= 0.
 */
kvq_status kvq_promote_values(const kvq_params* p, const kvq_cache* cache, const float* mass,
                              const int32_t* seq_len_host, float tau_v, uint8_t* flags, void* stream);

/*
 * kvq_ranking_check: for every (b, hq), its top-K* blocks (as kvq_select_blocks
 * chooses them from mass, in that order: the ranking by the quantized keys) are
 * scored from k_orig, score_j = log sum_t exp(scale * q . k_t) over the block's
 * positions below seq_len (fp32, original basis); inversions[b][hq] = the number of
 * pairs (i, j), i ranked before j, with score_j > score_i + margin, and
 * fail[b][hq] = inversions > max_inversions.  Needs keep_fp16_copy.
 *   q: device [B][Hq][128] in_dtype; mass: device fp32 [B][Hq][max_ctx/64];
 *   inversions: device int32 [B][Hq]; fail: device uint8 [B][Hq].
 *   tau_cov in [0, 1], margin >= 0, max_inversions >= 0.  max_ctx / 64 <= 4096.
 * The page prints no criterion for a consistent ranking: margin = 0 and
 * max_inversions = 0 (any pair out of order) is the strict reading.
 */
kvq_status kvq_ranking_check(const kvq_params* p, const kvq_cache* cache, const void* q,
                             const int32_t* seq_len_host, const float* mass, float tau_cov, float margin,
                             int32_t max_inversions, int32_t* inversions, uint8_t* fail, void* stream);

/*
 * kvq_dense_fallback: for every (b, hq) with certificate[b][hq] > eps, or with
 * fail[b][hq] != 0, out[b][hq] is replaced by attention over k_orig/v_orig
 * (positions [0, seq_len_host[b]), original basis; the same arithmetic as
 * kvq_decode_attn_dense) and certificate[b][hq] is set to 0; other rows are left
 * unchanged.  Needs keep_fp16_copy.  out/certificate: device, as written by
 * kvq_decode_attn; certificate may be NULL (then only fail triggers), fail may be
 * NULL (then only the certificate), not both.  eps >= 0.  workspace: as for
 * kvq_decode_attn (its records are overwritten; its counters are not used).
 */
kvq_status kvq_dense_fallback(const kvq_params* p, const kvq_cache* cache, const void* q,
                              const int32_t* seq_len_host, float eps, const uint8_t* fail, float* out,
                              float* certificate, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decode attention over uncompressed K/V in the layout of k_orig/v_orig
 * ([B][Hkv][Tmax][128] in_dtype); no rotation.  Same q/out/workspace contract as
 * kvq_decode_attn.  Only the shape fields and in_dtype of p are used.  Logits: the
 * fp32 query times scale (split into an fp16 high part and the fp16 rounding of the
 * remainder) against the keys in fp16 (bf16 keys rounded to fp16), fp32 accumulation;
 * softmax and the value sums in fp32.
 */
kvq_status kvq_decode_attn_dense(const kvq_params* p, const void* k, const void* v, const void* q,
                                 const int32_t* seq_len_host, float* out, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * Clipping thresholds for KVQ_INT2: t[h][c] = fl32(ratio * max_t |y_t,c|), with y
 * the same fp32 rotation kvq_append applies (times the cache's lambda_k / lambda_v
 * when given).
 *   calib_k, calib_v: device [Hkv][n_tokens][128] in_dtype; n_tokens >= 1.
 *   clip_k_out, clip_v_out: device fp32 [Hkv][128].
 */
kvq_status kvq_calibrate_clip(const kvq_params* p, const kvq_cache* cache, const void* calib_k,
                              const void* calib_v, int32_t n_tokens, float ratio, float* clip_k_out,
                              float* clip_v_out, void* stream);

/*
 * Per-channel rescale factors (calibrated): lambda[h][c] = fl32(1 / max_t |y_t,c|), 1
 * where the maximum is 0, with y the same fp32 rotation kvq_append applies (before
 * any rescale).  Same buffers as kvq_calibrate_clip; the results go into
 * kvq_cache.lambda_k / lambda_v.  (kvq_calibrate_clip applies a cache's factors
 * before taking its maxima, so calibrate the factors first.)
 */
kvq_status kvq_calibrate_lambda(const kvq_params* p, const kvq_cache* cache, const void* calib_k,
                                const void* calib_v, int32_t n_tokens, float* lambda_k_out,
                                float* lambda_v_out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
