// Internal declarations shared by the kvq HIP translation units (not installed).
// gfx950 only: wave64, MFMA, 160 KiB LDS per CU.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/kvq.h"

namespace kvq {

constexpr int D = 128;         // head dim
constexpr int TILE = 64;       // tokens per V tile / descriptor block / decode chunk
constexpr int MAX_BATCH = 256;

// ----------------------------------------------------------------- format facts
__host__ __device__ constexpr int fmt_bits(int f) { return f == KVQ_INT8 ? 8 : (f == KVQ_INT2 ? 2 : 4); }
__host__ __device__ constexpr int row_bytes(int f) { return D * fmt_bits(f) / 8; }  // KB
__host__ __device__ constexpr int chan_bytes(int f) { return TILE * fmt_bits(f) / 8; }  // CB
// group size of a format: INT4/INT8 take the configured group, INT2 32, FP4 16
__host__ __device__ constexpr int fmt_group(int f, int g) { return f == KVQ_INT2 ? 32 : (f == KVQ_FP4 ? 16 : g); }
// metadata elements per vector and bytes per element
__host__ __device__ constexpr int meta_elems(int f, int g) {
  return f == KVQ_INT2 ? 8 : (f == KVQ_FP4 ? 8 : D / g);
}
__host__ __device__ constexpr int meta_esize(int f) { return f == KVQ_FP4 ? 1 : 2; }
__host__ __device__ constexpr int meta_bytes(int f, int g) { return meta_elems(f, g) * meta_esize(f); }  // KM

// ----------------------------------------------------------------- kernel args
struct SeqArray {
  int32_t v[MAX_BATCH];
};

struct AppendArgs {
  const uint16_t* k_new;  // [B][H][n][128]
  const uint16_t* v_new;
  uint8_t* k_codes;
  uint8_t* k_meta;
  uint8_t* v_codes;
  uint8_t* v_meta;
  float* desc;  // may be null
  uint16_t* k_orig;  // may be null
  uint16_t* v_orig;
  const int8_t* signs;
  const uint16_t* rot;  // fp16 bits [128][128]
  const float* clip_k;
  const float* clip_v;
  uint16_t* k_win;  // may be null
  uint16_t* v_win;
  const float* lam_k;  // [H][128] per-channel rescale, or null
  const float* lam_v;
  int32_t B, H, Tmax, n_new;
  int32_t in_bf16;
  int32_t k_fmt, v_fmt, k_group, v_group, scale_mode, rotation;
  int32_t n_sink, n_recent;  // window blocks
  float tw_re[65], tw_im[65];  // SRFT twiddles W128^k = (fl32(cos), fl32(-sin)) of 2 pi k / 128
  SeqArray start;
};

struct CalibArgs {
  const uint16_t* x;  // [H][n][128]
  float* out;         // [H][128]
  const float* lam;   // [H][128] rescale applied before the maxima (clip mode), or null
  int32_t mode;       // 0: ratio * max |y| (clip thresholds), 1: 1 / max |y| (rescale factors)
  const int8_t* signs;
  const uint16_t* rot;
  int32_t H, n, in_bf16, rotation;
  float ratio;
  float tw_re[65], tw_im[65];  // SRFT twiddles
};

struct BoundArgs {
  const uint16_t* q;  // [B][Hq][128]
  const float* desc;  // [B][H][nt][3]
  float* bound;       // [B][H][nt]
  uint8_t* flags;
  int32_t B, Hq, H, nt, in_bf16;
  float scale, tau;
  SeqArray seq;
};

// Adaptive precision: scoring pass, top-K* selection, per-head dense fallback.
struct AdaptArgs {
  const uint16_t* q;  // [B][Hq][128]
  const uint8_t* k_codes;
  const uint8_t* k_meta;
  const uint16_t* k_orig;  // [B][H][Tmax][128] (ranking check)
  const int8_t* signs;
  const uint16_t* rot;
  const float* lam_k;        // [H][128] per-channel rescale of the keys, or null
  float* mass;               // [B][Hq][nt]
  const uint8_t* flags_in;   // [B][H][nt] or null
  uint8_t* flags_out;        // [B][H][nt]
  const float* desc;         // [B][H][nt][3] (ek, ev, vn) (value promotion)
  int32_t* inv;              // [B][Hq] inverted pairs (ranking check)
  uint8_t* fail;             // [B][Hq] ranking check result
  int32_t B, Hq, H, G, Tmax, nt;
  int32_t in_bf16, rotation, k_fmt, k_group;
  int32_t max_inv;
  int32_t score_splits, score_cps;  // scoring pass: splits per unit, blocks per split
  float scale, tau_cov, tau_v, margin;
  float cos128[128];  // fl32(cos(2 pi k / 128)): the SRFT matrix entries
  SeqArray seq;
};
constexpr int MAX_SELECT_BLOCKS = 4096;  // selection sorts one head's blocks in LDS

// Workspace of a decode call: one partial-result record per (b, hq, split),
// written by the split kernel and read by the combine kernel:
// [0] m: running max (log2 domain), [1] l: sum of exp2, [2] eta: sum of p * ev
// (certified), [3] ekmax, [4] vnmax: maxima over this split's blocks,
// [5] ||q|| * softmax_scale, [8..8+D) o: rotated-basis accumulator,
// [8+D..8+2D) oo: original-basis accumulator of exactly recomputed blocks.
constexpr int PART_FLOATS = 8 + 2 * D;
constexpr int MAX_SPLITS = 128;
// The allocation-free decode's fixed workspace: 8 MiB per device, counters in the first
// 64 KiB (16384 of them), records in the rest.
constexpr size_t SCRATCH_BYTES = size_t(8) << 20;
constexpr size_t SCRATCH_CTR_BYTES = size_t(64) << 10;
constexpr int MAX_DEVICES = 64;

struct DecodeArgs {
  const uint16_t* q;  // [B][Hq][128]
  const uint8_t* k_codes;
  const uint8_t* k_meta;
  const uint8_t* v_codes;
  const uint8_t* v_meta;
  const float* desc;
  const uint16_t* k_orig;
  const uint16_t* v_orig;
  const uint8_t* flags;  // [B][H][nt] or null
  const uint16_t* k_win;  // [B][H][(n_sink + n_recent) * 64][128] or null
  const uint16_t* v_win;
  const float* lam_k;  // [H][128] per-channel rescale, or null
  const float* lam_v;
  const int8_t* signs;
  const uint16_t* rot;
  float* part;              // [B][Hq][n_splits][PART_FLOATS]
  int* ctr;                 // [U] split arrival counters per unit, zero between calls
  float* out;               // [B][Hq][128]
  float* cert;              // [B][Hq] or null
  float* fb_cert;           // dense fallback: rows with fb_cert > fb_eps ... (or null)
  const uint8_t* fb_fail;   // ... or fb_fail != 0 (or null) are recomputed; the others untouched
  float fb_eps;
  int32_t B, Hq, H, G, Tmax, nt;
  int32_t in_bf16, rotation, k_group, v_group;
  int32_t n_splits, chunks_per_split;
  int32_t U;  // units (sequence, kv head, group of 4 query heads)
  int32_t n_sink, n_recent;  // window blocks (0, 0 = none)
  float scale;  // softmax scale
  float cos128[128];  // fl32(cos(2 pi k / 128)): the SRFT matrix entries
  SeqArray seq;
};


// ----------------------------------------------------------------- debug build
// Compiled with -DKVQ_DEBUG (libkvq_debug.so), the kernels check the layout as they address
// memory: every stream, position, chunk, block, split record and counter index against the
// sizes the call was validated with.  A failed check does not stop the kernel: the first one
// in a translation unit records its code and two indices in that unit's word array, and
// every failure is counted; kvq_debug_status reads and clears them.  The release library
// compiles the checks out.
enum DbgCode : uint32_t {
  DBG_NONE = 0,
  DBG_STREAM = 1,  // (sequence, kv head) stream index outside [0, B * Hkv)
  DBG_CHUNK = 2,   // decode chunk / 64-token block outside [0, Tmax / 64)
  DBG_RECORD = 3,  // split record (row, split) outside [0, B * Hq) x [0, n_splits)
  DBG_COUNTER = 4, // split arrival counter outside [0, units)
  DBG_WINDOW = 5,  // window slot outside [0, sink + recent) or a position outside its block
  DBG_POS = 6,     // appended position outside [0, Tmax) or outside the input's n_new rows
  DBG_ROW = 7,     // (sequence, query head) row outside [0, B * Hq)
};
#ifdef KVQ_DEBUG
static __device__ uint32_t dbg_word[4];  // first code, its two indices, failures counted
__device__ __noinline__ static void dbg_fail(uint32_t code, uint32_t i0, uint32_t i1) {
  uint64_t p = (uint64_t)(uintptr_t)&dbg_word[0];
  asm volatile("" : "+v"(p));  // a per-lane address: vector memory atomics
  uint32_t* w = reinterpret_cast<uint32_t*>(p);
  uint32_t expect = 0;
  if (__hip_atomic_compare_exchange_strong(w, &expect, code, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT)) {
    __hip_atomic_store(w + 1, i0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(w + 2, i1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __hip_atomic_fetch_add(w + 3, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
#define KVQ_DCHECK(cond, code, i0, i1)                                            \
  do {                                                                           \
    if (__builtin_expect(!(cond), 0)) kvq::dbg_fail((code), (uint32_t)(i0), (uint32_t)(i1)); \
  } while (0)
// the host reader of this translation unit's record (waits for the device first)
#define KVQ_DBG_READER(name)                                                                  \
  hipError_t name(uint32_t out[4], bool clear) {                                              \
    hipError_t e = hipDeviceSynchronize();                                                    \
    if (e == hipSuccess) e = hipMemcpyFromSymbol(out, HIP_SYMBOL(dbg_word), 4 * sizeof(uint32_t)); \
    if (e == hipSuccess && clear) {                                                           \
      const uint32_t z[4] = {0u, 0u, 0u, 0u};                                                 \
      e = hipMemcpyToSymbol(HIP_SYMBOL(dbg_word), z, sizeof(z));                              \
    }                                                                                         \
    return e;                                                                                 \
  }
hipError_t dbg_read_append(uint32_t out[4], bool clear);
hipError_t dbg_read_decode(uint32_t out[4], bool clear);
hipError_t dbg_read_bound(uint32_t out[4], bool clear);
hipError_t dbg_read_adaptive(uint32_t out[4], bool clear);
#else
#define KVQ_DCHECK(cond, code, i0, i1) ((void)0)
#endif
// a token a lane writes in an append: inside its stream, the cache and the input rows
#define KVQ_DCHECK_APPEND(a, stream, pos, start)                                               \
  do {                                                                                        \
    KVQ_DCHECK((stream) < (size_t)(a).B * (a).H, DBG_STREAM, (stream), (pos));                \
    KVQ_DCHECK((pos) >= 0 && (pos) < (a).Tmax && (pos) - (start) >= 0 && (pos) - (start) < (a).n_new, DBG_POS, \
               (stream), (pos));                                                              \
  } while (0)

// host-side launchers (defined in the .hip files)
hipError_t launch_append(const AppendArgs& a, int grid_x, hipStream_t s);
hipError_t launch_window_copy(const AppendArgs& a, hipStream_t s);
hipError_t launch_calibrate(const CalibArgs& a, hipStream_t s);
hipError_t launch_bound(const BoundArgs& a, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int k_fmt, int v_fmt, bool dense, hipStream_t s);
hipError_t decode_scratch(void** ptr, hipStream_t s);
hipError_t launch_block_mass(const AdaptArgs& a, hipStream_t s);
hipError_t launch_select(const AdaptArgs& a, hipStream_t s);
hipError_t launch_dense_fallback(const DecodeArgs& a, hipStream_t s);
hipError_t launch_promote_values(const AdaptArgs& a, hipStream_t s);
hipError_t launch_ranking_check(const AdaptArgs& a, hipStream_t s);

}  // namespace kvq
