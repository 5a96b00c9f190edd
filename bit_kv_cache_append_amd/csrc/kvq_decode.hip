// Read side: single-token decode attention over the packed cache.
//
// Split kernel: one workgroup (8 waves, one workgroup per CU) per (context
// split, kv head, group of 4 query heads, sequence).  The waves share out the
// 64-token chunks of the split through a counter in LDS (the chunk is also the
// V tile and the descriptor block).  Per chunk:
//
//  QK^T  -- 4x4x4 (16-block) int8 MFMA.  Lane 4s+r loads the packed K row of
//           token pi(s, r); the query is rotated once, prescaled by
//           softmax_scale * log2(e), quantized to 16 bits per head and split into
//           two int8 halves, so every K code x query product is an exact
//           integer and the group scale is applied to the exact group dot
//           product in fp32.  Output: lane 4s+j holds head j's logits of the
//           four tokens pi(s, 0..3).
//  softmax -- online (running max / sum in the exp2 domain), max over the 16
//           lanes of a head by lane exchange.
//  PV    -- 4x4x4 fp16 MFMA.  V tiles are channel-major, so lane l reads the
//           64 tokens of channels 2l and 2l+1 as a few 16-byte loads and turns
//           nibbles/crumbs into exact fp16 codes with magic-number bit tricks;
//           probabilities are broadcast from lane 4s+h and scaled per token by
//           the V group scale (fp16).  Output: lane l holds o[h][2l], o[h][2l+1].
//
// The token order pi within a chunk is chosen so that the fp16 pairs produced
// by the V bit tricks line up with the probability pairs of the QK output.
//
// Certified mode: a flagged chunk is recomputed from the fp16 originals in the
// original basis ("Runtime-Certified Bounded-Error Quantized Attention",
// Methodology sections 1 and 3) into a separate accumulator; the value-error
// mass sum p * ev and the descriptor maxima are tracked for the certificate.
//
// Merge: log-sum-exp merge of the splits, inverse rotation back to the original
// basis ("OSCAR", section 2.2B), certificate; done by the last split workgroup of
// each (sequence, kv head, query-head group) to finish, found with an arrival
// counter, on records written and read with agent-coherent accesses.  The fp16
// baseline uses a separate combine launch for the same merge.

#include <mutex>

#include "kvq_common.h"

namespace kvq {

namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef float f2 __attribute__((ext_vector_type(2)));
typedef int i4 __attribute__((ext_vector_type(4)));

constexpr int NT = 256;   // combine kernel, fp16 baseline split kernel
constexpr int NTS = 512;  // quantized split kernel: 8 waves, one workgroup per CU
constexpr int NWS = NTS / 64;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float NEG_INF = -__builtin_huge_valf();

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u(h2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ h4 cat(h2 a, h2 b) { return h4{a.x, a.y, b.x, b.y}; }

// ------------------------------------------------------------------ token order
// QK slice s (lanes 4s..4s+3) covers tokens pi(s, 0..3) of the chunk.
template <int VF>
__device__ __forceinline__ int tok_of(int s, int r) {
  if constexpr (VF == KVQ_INT2) return 4 * s + 2 * (r & 1) + (r >> 1);  // even, then odd codes of a byte
  if constexpr (VF == KVQ_FP4) return 4 * s + r;  // the hardware FP4 pair conversion keeps token order
  return 8 * (s >> 1) + 2 * (s & 1) + ((r & 1) << 2) + (r >> 1);
}

// ------------------------------------------------------------------ K formats
template <int KF>
struct KFmt;
template <>
struct KFmt<KVQ_INT4> {
  static constexpr int DW = 16;  // dwords per row
  static constexpr int MDW = 2;  // metadata dwords per token (g32: 4 fp16); g128 uses 1 fp16
  // offset-binary nibbles (code + 8) as bytes: the low or the high nibble of each byte
  __device__ static __forceinline__ int a_op(const uint32_t* row, int n) {
    const uint32_t t = (n & 1) ? (row[n >> 1] >> 4) : row[n >> 1];
    return (int)((t & 0x0F0F0F0Fu) ^ 0x08080808u);
  }
  __device__ static __forceinline__ int chan(int n, int m) { return 8 * (n >> 1) + 2 * m + (n & 1); }
  __device__ static __forceinline__ int slot(int c) { return 4 * (2 * (c >> 3) + (c & 1)) + ((c & 7) >> 1); }
};
template <>
struct KFmt<KVQ_INT8> {
  static constexpr int DW = 32;
  static constexpr int MDW = 2;
  __device__ static __forceinline__ int a_op(const uint32_t* row, int n) { return (int)row[n]; }
  __device__ static __forceinline__ int chan(int n, int m) { return 4 * n + m; }
  __device__ static __forceinline__ int slot(int c) { return c; }
};
template <>
struct KFmt<KVQ_FP4> {
  static constexpr int DW = 16;  // 128 E2M1 nibbles
  static constexpr int MDW = 2;  // 8 E4M3 block scales
  // fp16 values of channels 4n..4n+3 (E2M1 is exact in fp16)
  __device__ static __forceinline__ h4 a_op_f16(const uint32_t* row, int n) {
    const uint32_t w = row[n >> 1];
    const h2 lo = (n & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2)
                          : __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
    const h2 hi = (n & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3)
                          : __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
    return h4{lo.x, lo.y, hi.x, hi.y};
  }
  // the integer-operand interface is not used for FP4 keys (fp16 operands instead)
  __device__ static __forceinline__ int a_op(const uint32_t*, int) { return 0; }
  __device__ static __forceinline__ int slot(int c) { return c; }
};
template <>
struct KFmt<KVQ_INT2> {
  static constexpr int DW = 8;
  static constexpr int MDW = 4;  // 4 scales + 4 offsets
  __device__ static __forceinline__ int a_op(const uint32_t* row, int n) {
    return (int)((row[n >> 2] >> (2 * (n & 3))) & 0x03030303u);
  }
  __device__ static __forceinline__ int chan(int n, int m) { return 16 * (n >> 2) + 4 * m + (n & 3); }
  __device__ static __forceinline__ int slot(int c) { return 4 * (4 * (c >> 4) + (c & 3)) + ((c & 15) >> 2); }
};

// ------------------------------------------------------------------ V formats
// exact fp16 codes of one dword of a channel's token run, as fp16 pairs
// (the nibble n of a two's complement code c is placed in an fp16 mantissa as
// n ^ 8 = c + 8 under exponent 2^10: one and-xor per pair, then one packed op)
__device__ __forceinline__ void v_int4_pairs(uint32_t w, h2 out[4]) {
  const uint32_t w8 = w >> 8;
  const h2 k1032 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const h2 k16 = {(_Float16)0.0625f, (_Float16)0.0625f};
  const h2 k72 = {(_Float16)-72.0f, (_Float16)-72.0f};
  out[0] = as_h2((w & 0x000F000Fu) ^ 0x64086408u) + k1032;                     // tokens 0, 4
  out[1] = as_h2((w & 0x00F000F0u) ^ 0x64806480u) * k16 + k72;                 // tokens 1, 5
  out[2] = as_h2((w8 & 0x000F000Fu) ^ 0x64086408u) + k1032;                    // tokens 2, 6
  out[3] = as_h2((w8 & 0x00F000F0u) ^ 0x64806480u) * k16 + k72;                // tokens 3, 7
}
// int2: the 16 codes of a dword (token i in bits 2i, 2i+1), codes 0..3.  A code in the low
// two bits of an E2M1 nibble (high bits clear) is c / 2 exactly (0, 0.5 as a subnormal, 1,
// 1.5), so masking the even and the odd codes into nibbles and running the gfx950 pair
// conversion with scale 2 gives the exact fp16 code, one instruction per two codes.
// out[2b] = tokens (4b, 4b + 2), out[2b + 1] = tokens (4b + 1, 4b + 3).
__device__ __forceinline__ void v_int2_pairs(uint32_t w, h2 out[8]) {
  const uint32_t ev = w & 0x33333333u, od = (w >> 2) & 0x33333333u;
  out[0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ev, 2.0f, 0);
  out[1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(od, 2.0f, 0);
  out[2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ev, 2.0f, 1);
  out[3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(od, 2.0f, 1);
  out[4] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ev, 2.0f, 2);
  out[5] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(od, 2.0f, 2);
  out[6] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ev, 2.0f, 3);
  out[7] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(od, 2.0f, 3);
}

template <int VF>
struct VFmt;
template <>
struct VFmt<KVQ_INT4> {
  static constexpr int CDW = 8;   // dwords per channel per tile
  static constexpr int NMAX = 4;  // metadata elements per token (g32)
};
template <>
struct VFmt<KVQ_INT2> {
  static constexpr int CDW = 4;
  static constexpr int NMAX = 8;
};
template <>
struct VFmt<KVQ_FP4> {
  static constexpr int CDW = 8;
  static constexpr int NMAX = 8;  // 8 blocks of 16 channels, one E4M3 scale each
};

// E4M3 (non-negative) byte pair -> fp16 pair, exact: the byte shifted into an
// fp16 is the value / 2^8 (normal and subnormal codes alike), so one packed
// multiply by 256 finishes it
__device__ __forceinline__ h2 e4m3x2_to_h2(uint32_t b0, uint32_t b1) {
  const uint32_t bits = (b0 << 7) | (b1 << 23);
  return as_h2(bits) * h2{(_Float16)256.0f, (_Float16)256.0f};
}

// ------------------------------------------------------------------ reductions
// v of lane l ^ M: DPP moves for masks inside a row of 16 (quad permutes; (l ^ 3) then a
// half-row mirror (l ^ 7) is l ^ 4; (l ^ 7) then a row mirror (l ^ 15) is l ^ 8), a
// shuffle through the LDS crossbar otherwise
// {v of lane l, v of lane l ^ M} in every lane, M = 16 or 32 (the gfx950 row and
// half-wave swaps: the first result holds the lower rows, the second the upper ones)
template <int M>
__device__ __forceinline__ void lane_pair(float v, float& lo, float& hi) {
  const int vi = __float_as_int(v);
  if constexpr (M == 16) {
    const auto p = __builtin_amdgcn_permlane16_swap(vi, vi, false, false);
    lo = __int_as_float(p[0]);
    hi = __int_as_float(p[1]);
  } else {
    const auto p = __builtin_amdgcn_permlane32_swap(vi, vi, false, false);
    lo = __int_as_float(p[0]);
    hi = __int_as_float(p[1]);
  }
}
template <int M>
__device__ __forceinline__ float lane_xor(float v) {
  if constexpr (M == 1) return dpp_f<0xB1>(v);
  else if constexpr (M == 2) return dpp_f<0x4E>(v);
  else if constexpr (M == 4) return dpp_f<0x141>(dpp_f<0x1B>(v));
  else if constexpr (M == 8) return dpp_f<0x140>(dpp_f<0x141>(v));
  else {
    float lo, hi;
    lane_pair<M>(v, lo, hi);
    return (__lane_id() & M) ? lo : hi;
  }
}
// one Walsh-Hadamard stage across lanes on two values per lane: the lower lane of each
// pair keeps own + partner, the upper partner - own
template <int M>
__device__ __forceinline__ void wht_stage(float& y0, float& y1, int l) {
  const float p0 = lane_xor<M>(y0), p1 = lane_xor<M>(y1);
  const bool up = (l & M) != 0;
  y0 = up ? p0 - y0 : y0 + p0;
  y1 = up ? p1 - y1 : y1 + p1;
}
__device__ __forceinline__ void wht_lanes(float& y0, float& y1, int l) {  // h = 2, 4, ..., 64 (masks 1..32)
  wht_stage<1>(y0, y1, l);
  wht_stage<2>(y0, y1, l);
  wht_stage<4>(y0, y1, l);
  wht_stage<8>(y0, y1, l);
  wht_stage<16>(y0, y1, l);
  wht_stage<32>(y0, y1, l);
}
// one radix-2 stage of the wave FFT below (span H)
template <int H>
__device__ __forceinline__ void fft_stage(float& re, float& im, int l, const float* ctab, bool inverse) {
  const float pr = lane_xor<H>(re), pi = lane_xor<H>(im);
  const bool up = (l & H) != 0;
  const float sr = up ? pr - re : re + pr;
  const float si = up ? pi - im : im + pi;
  const int e2 = 2 * (l & (H - 1)) * (32 / H);  // W64^e = W128^(2e)
  const float c = ctab[e2 & 127], sn = ctab[(e2 + 96) & 127];
  const float wi = inverse ? sn : -sn;
  re = up ? sr * c - si * wi : sr;
  im = up ? sr * wi + si * c : si;
}

// max / sum with lane l ^ M for M = 16, 32: both lanes of a pair form the same value
template <int M>
__device__ __forceinline__ float max_with(float v) {
  float lo, hi;
  lane_pair<M>(v, lo, hi);
  return fmaxf(lo, hi);
}
template <int M>
__device__ __forceinline__ float sum_with(float v) {
  float lo, hi;
  lane_pair<M>(v, lo, hi);
  return lo + hi;
}
__device__ __forceinline__ float max_same_head(float v) {  // over lanes with equal (lane & 3)
  v = fmaxf(v, lane_xor<4>(v));
  v = fmaxf(v, lane_xor<8>(v));
  return max_with<32>(max_with<16>(v));
}
__device__ __forceinline__ float sum_same_head(float v) {
  v += lane_xor<4>(v);
  v += lane_xor<8>(v);
  return sum_with<32>(sum_with<16>(v));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, lane_xor<1>(v));
  v = fmaxf(v, lane_xor<2>(v));
  v = fmaxf(v, lane_xor<4>(v));
  v = fmaxf(v, lane_xor<8>(v));
  return max_with<32>(max_with<16>(v));
}
__device__ __forceinline__ float wave_sum(float v) {
  v += lane_xor<1>(v);
  v += lane_xor<2>(v);
  v += lane_xor<4>(v);
  v += lane_xor<8>(v);
  return sum_with<32>(sum_with<16>(v));
}
template <int H>
__device__ __forceinline__ float quad_bcast(float v) {
  return dpp_f<H * 0x55>(v);
}
template <int H>
__device__ __forceinline__ uint32_t quad_bcast_u(uint32_t v) {
  return (uint32_t)dpp_i<H * 0x55>((int)v);
}

__device__ __forceinline__ void lds_wait() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Per-wave partial results merged in LDS at the end of a split kernel.
template <int NW>
struct MergeArea {
  float o[NW][4][D];   // rotated-basis accumulator by wave, head, channel
  float oo[NW][4][D];  // original-basis accumulator of exactly recomputed chunks
  float m[NW][4], l[NW][4], e[NW][4];
  float ek[NW], vn[NW];
};

constexpr int MAX_VG = 8;  // V scale groups per token (groups of 16 and FP4 blocks)

struct __align__(16) DecodeSmem {
  float ctab[128];                   // cos(2 pi k / 128) for the SRFT rotation
  float qo[4][D];                    // original query * scale * log2e, per head (exact recompute)
  uint32_t qh[4][32];                // high int8 halves: dword 4n + c = MFMA operand of chain c, step n
  uint32_t ql[4][32];                // low int8 halves, same order
  uint32_t qf4[4][32][4];            // FP4 keys: per head and 4-channel step, fp16 query high then low parts
  float qs[4];                       // per head: dequantization of the 16-bit query
  float qsum[4][8];                  // per head and key group: sum of the 16-bit query codes
  uint16_t vmeta[NWS][8][16][4];     // per wave: V metadata by (element, slice, r)
  float zt[NWS][4][4];               // INT2 values: per wave, head, group: sum of p * offset
  union {
    struct {
      float pb[NWS][TILE][4];                 // per wave: probabilities by token (exact recompute)
      uint4 pw[NWS][MAX_VG][16][4];           // per wave: PV weights by (V group, step, head): 4 hi + 4 lo fp16
    } loop;
    struct {
      float qf[NWS][D];                       // per wave: prologue scratch (dense rotation)
      float qr[NWS][D];
    } pro;
    MergeArea<NWS> mrg;
    float zsw[NWS][D];                        // per wave: merge scratch (dense inverse rotation)
  } u;
  int next;                          // next chunk (offset from the split's first) to claim
  int last;                          // this workgroup is the last of its unit's to finish
};

// The fp16/bf16 decode's shared memory (the same-shape baseline and the dense fallback
// of the adaptive ladder), padded so that at most two of its workgroups share a CU (160
// KiB of LDS): with more of them resident at once their streams of rows compete for the
// CU's memory pipeline.
struct __align__(16) DenseSmem {
  float qo[4][D];
  uint4 qhl[4][32];  // per head and 4-channel step: fp16 high parts, then fp16 low parts
  float pb[4][TILE][4];
  MergeArea<4> mrg;
  int nlist;                // dense fallback: units in the list below
  uint8_t pad[52 * 1024];   // (dense fallback: the list of units with a row to recompute)
};

// ------------------------------------------------------------------ prologue
// 64-point complex FFT across the lanes of a wave (lane l holds point l), radix 2,
// decimation in frequency: stage h pairs lanes l and l ^ h, the lower takes a + b, the
// upper (a - b) W64^((l mod h) 32 / h).  The result is in bit-reversed order: lane p
// holds point rev6(p).  Forward: W64 = e^(-2 pi i / 64); inverse (unnormalised): e^(+...).
// ctab: cos(2 pi k / 128), k = 0..127 (sin x = cos(x - pi/2): index + 96).
__device__ __forceinline__ void wave_fft64(float& re, float& im, int l, const float* ctab, bool inverse) {
  fft_stage<32>(re, im, l, ctab, inverse);
  fft_stage<16>(re, im, l, ctab, inverse);
  fft_stage<8>(re, im, l, ctab, inverse);
  fft_stage<4>(re, im, l, ctab, inverse);
  fft_stage<2>(re, im, l, ctab, inverse);
  fft_stage<1>(re, im, l, ctab, inverse);
}
__device__ __forceinline__ int rev6(int l) { return (int)(__builtin_bitreverse32((uint32_t)l) >> 26); }

// Rotate one query head (the whole wave: lane l holds channels 2l and 2l+1), prescale by
// softmax_scale * log2(e), and publish it as head h: the original (scaled) query
// for exact recompute, and the key operands: a 16-bit quantization split into int8 halves
// in MFMA operand order plus per-group code sums (integer keys), or two fp16 parts (FP4
// keys).  Wave-local: the caller holds the workgroup barrier that publishes the results.
// The Walsh-Hadamard butterflies run in the order h = 1, 2, ..., 64 with the in-lane pair
// first and lane exchanges after.
// The loads of one head's query and sign bits, issued before the first chunk's loads.
struct QueryIn {
  uint32_t q01;  // channels 2l, 2l+1 (bits)
  uint16_t sg;   // sign bytes of those channels
};
__device__ __forceinline__ QueryIn query_loads(const DecodeArgs& a, int b, int hq) {
  const int l = threadIdx.x & 63;
  QueryIn r;
  r.q01 = *reinterpret_cast<const uint32_t*>(a.q + ((size_t)b * a.Hq + hq) * D + 2 * l);
  r.sg = a.signs != nullptr ? *reinterpret_cast<const uint16_t*>(a.signs + 2 * l) : (uint16_t)0;
  return r;
}

template <int KF>
__device__ void query_head(const DecodeArgs& a, DecodeSmem& sm, const QueryIn& qin, int wv, int h, bool live,
                           int kgroup, int hkv) {
  const int l = threadIdx.x & 63;
  const bool bf16 = a.in_bf16 != 0;
  float x0 = 0.0f, x1 = 0.0f;
  if (live) {
    x0 = widen((uint16_t)(qin.q01 & 0xFFFF), bf16);
    x1 = widen((uint16_t)(qin.q01 >> 16), bf16);
  }
  const float pre = a.scale * LOG2E;
  sm.qo[h][2 * l] = x0 * pre;
  sm.qo[h][2 * l + 1] = x1 * pre;
  float y0 = x0, y1 = x1;
  if (a.rotation == KVQ_ROT_SIGN_FWHT || a.rotation == KVQ_ROT_SRFT) {
    x0 = (qin.sg & 0x80u) ? -x0 : x0;
    x1 = (qin.sg & 0x8000u) ? -x1 : x1;
  }
  if (a.rotation == KVQ_ROT_SIGN_FWHT) {
    y0 = x0 + x1;
    y1 = x0 - x1;
    wht_lanes(y0, y1, l);
  } else if (a.rotation == KVQ_ROT_SRFT) {
    // y = R q with R the packed unitary DFT times diag(s): the 64-point FFT of
    // z_n = u_2n + i u_2n+1 (u = s * q) across the wave, then X_l = E + W128^l O from
    // Z_l and conj Z_(64-l); lane l keeps channels 2l, 2l + 1 (lane 0: X_0 and X_64)
    float re = x0, im = x1;
    wave_fft64(re, im, l, sm.ctab, false);
    const int ka = rev6(l), kb = rev6((64 - l) & 63);
    const float a_re = __shfl(re, ka), a_im = __shfl(im, ka);   // Z_l
    const float b_re = __shfl(re, kb), b_im = -__shfl(im, kb);  // conj Z_(64-l)
    const float e_re = 0.5f * (a_re + b_re), e_im = 0.5f * (a_im + b_im);
    const float o_re = 0.5f * (a_im - b_im), o_im = -0.5f * (a_re - b_re);
    const float c = sm.ctab[l], sn = sm.ctab[(l + 96) & 127];  // W128^l = (c, -sn)
    y0 = (e_re + (o_re * c + o_im * sn)) * 0.125f;
    y1 = (e_im + (o_im * c - o_re * sn)) * 0.125f;
    if (l == 0) {
      const float c0 = bits_to_f32(KVQ_INV_SQRT_D_BITS);
      y0 = (a_re + a_im) * c0;  // X_0
      y1 = (a_re - a_im) * c0;  // X_64
    }
  } else if (a.rotation == KVQ_ROT_DENSE) {
    float* qf = sm.u.pro.qf[wv];
    float* qr = sm.u.pro.qr[wv];
    qf[2 * l] = x0;
    qf[2 * l + 1] = x1;
    __builtin_amdgcn_wave_barrier();
    lds_wait();
    for (int rr = 0; rr < 2; ++rr) {
      const int row = l + 64 * rr;
      const uint16_t* rp = a.rot + (size_t)row * D;
      float acc = 0.0f;
      for (int k = 0; k < D; ++k) acc = fmaf(f16_bits_to_f32(rp[k]), qf[k], acc);
      qr[row] = acc;
    }
    __builtin_amdgcn_wave_barrier();
    lds_wait();
    y0 = qr[2 * l];
    y1 = qr[2 * l + 1];
    __builtin_amdgcn_wave_barrier();  // the scratch is reused by the next head
  }
  if (a.lam_k != nullptr) {  // keys were stored times lambda_k: q . y = (q / lambda) . (lambda y)
    y0 = y0 / a.lam_k[(size_t)hkv * D + 2 * l];
    y1 = y1 / a.lam_k[(size_t)hkv * D + 2 * l + 1];
  }
  const float norm = a.rotation == KVQ_ROT_SIGN_FWHT ? bits_to_f32(KVQ_INV_SQRT_D_BITS) : 1.0f;
  y0 = y0 * norm * pre;
  y1 = y1 * norm * pre;
  const float mx = wave_max(fmaxf(fabsf(y0), fabsf(y1)));
  if constexpr (KF == KVQ_FP4) {
    // FP4 keys: the query as two fp16 parts (high + residual) after an exact
    // power-of-two scaling to |y| < 2^14; products with E2M1 codes are exact
    int ex = 0;
    frexpf(mx, &ex);  // mx = f 2^ex, f in [0.5, 1)
    const float qs = mx > 0.0f ? ldexpf(1.0f, ex - 14) : 1.0f;
    const float inv = mx > 0.0f ? ldexpf(1.0f, 14 - ex) : 1.0f;
    uint16_t* qq = reinterpret_cast<uint16_t*>(&sm.qf4[h][0][0]);
    const float ys[2] = {y0 * inv, y1 * inv};
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int c = 2 * l + e, n = c >> 2, mm = c & 3;
      const _Float16 hh = (_Float16)ys[e];
      const _Float16 ll = (_Float16)(ys[e] - (float)hh);
      qq[n * 8 + mm] = __builtin_bit_cast(uint16_t, hh);
      qq[n * 8 + 4 + mm] = __builtin_bit_cast(uint16_t, ll);
    }
    if (l == 0) sm.qs[h] = qs;
    return;
  }
  const float qs = mx > 0.0f ? mx / 32000.0f : 1.0f;
  const int q0 = (int)rintf(y0 / qs), q1 = (int)rintf(y1 / qs);
  // scatter int8 halves into MFMA operand order
  uint8_t* hb = reinterpret_cast<uint8_t*>(&sm.qh[h][0]);
  uint8_t* lb = reinterpret_cast<uint8_t*>(&sm.ql[h][0]);
  const int qv[2] = {q0, q1};
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int c = 2 * l + e;
    const int hi = (qv[e] + 128) >> 8;
    const int lo = qv[e] - 256 * hi;
    // operand dword d = 8 c + n of the QK chains is stored at 4 n + c, so that one 16-byte
    // LDS read gives step n of all four chains
    const int sl = KFmt<KF>::slot(c);
    const int d = sl >> 2, ps = (((d & 7) << 2) | (d >> 3)) * 4 + (sl & 3);
    hb[ps] = (uint8_t)(hi & 0xFF);
    lb[ps] = (uint8_t)(lo & 0xFF);
  }
  // per-group sums of the 16-bit codes (groups of 16 channels = 8 lanes, 32 = 16 lanes)
  float gs = (float)(q0 + q1);
  gs += lane_xor<1>(gs);
  gs += lane_xor<2>(gs);
  gs += lane_xor<4>(gs);
  if (kgroup == 16) {
    if ((l & 7) == 0) sm.qsum[h][l >> 3] = gs;
  } else {
    gs += lane_xor<8>(gs);
    if (kgroup == 128) gs = sum_with<32>(sum_with<16>(gs));
    if ((l & 15) == 0) sm.qsum[h][l >> 4] = gs;
  }
  if (l == 0) sm.qs[h] = qs;
}

// ------------------------------------------------------------------ coherent record access
// Split records read by the last workgroup of a stream (on any XCD) are written and
// read with agent-scope atomic accesses, which the hardware keeps coherent across
// the L2s of all XCDs; plain accesses when a separate launch does the merge.
template <bool COH>
__device__ __forceinline__ void rec_st(float* p, float v) {
  if constexpr (COH) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else *p = v;
}
template <bool COH>
__device__ __forceinline__ float rec_ld(const float* p) {
  if constexpr (COH) return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  else return *p;
}
// two adjacent record words (8-byte aligned) in one access
template <bool COH>
__device__ __forceinline__ void rec_st2(float* p, float v0, float v1) {
  if constexpr (COH) {
    const uint64_t w = (uint64_t)__float_as_uint(v0) | ((uint64_t)__float_as_uint(v1) << 32);
    __hip_atomic_store(reinterpret_cast<uint64_t*>(p), w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  } else {
    *reinterpret_cast<float2*>(p) = make_float2(v0, v1);
  }
}
template <bool COH>
__device__ __forceinline__ float2 rec_ld2(const float* p) {
  if constexpr (COH) {
    const uint64_t w = __hip_atomic_load(reinterpret_cast<const uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return make_float2(__uint_as_float((uint32_t)w), __uint_as_float((uint32_t)(w >> 32)));
  } else {
    return *reinterpret_cast<const float2*>(p);
  }
}

// ------------------------------------------------------------------ split record
// Merges waves [w0, w0 + nw) of this workgroup (log-sum-exp weights) and writes head hh's
// record of (sequence b, query head hq0 + hh, split) for the merge; qo: the unit's
// scaled original query (certificate: ||q|| * scale).  Called by 64 threads per head
// (l = lane); heads at or beyond nh are skipped.
template <bool CERT, int NW, bool COH>
__device__ void write_record(const DecodeArgs& a, const MergeArea<NW>& mg, const float (*qo)[D], int w0, int nw,
                             int b, int hq0, int nh, int split, int hh, int l) {
  const int c = 2 * l;
  if (hh >= nh) return;
  float M = NEG_INF;
  for (int w = w0; w < w0 + nw; ++w) M = fmaxf(M, mg.m[w][hh]);
  KVQ_DCHECK(b < a.B && hq0 + hh < a.Hq && split >= 0 && split < a.n_splits, DBG_RECORD, b * a.Hq + hq0 + hh, split);
  float* rec = a.part + (((size_t)b * a.Hq + hq0 + hh) * a.n_splits + split) * PART_FLOATS;
  float o0 = 0.0f, o1 = 0.0f, p0 = 0.0f, p1 = 0.0f, L = 0.0f, E = 0.0f, ek = 0.0f, vn = 0.0f;
  for (int w = w0; w < w0 + nw; ++w) {
    const float wgt = (M == NEG_INF) ? 0.0f : exp2f(mg.m[w][hh] - M);
    o0 += wgt * mg.o[w][hh][c];
    o1 += wgt * mg.o[w][hh][c + 1];
    if constexpr (CERT) {
      p0 += wgt * mg.oo[w][hh][c];
      p1 += wgt * mg.oo[w][hh][c + 1];
    }
    L += wgt * mg.l[w][hh];
    E += wgt * mg.e[w][hh];
    ek = fmaxf(ek, mg.ek[w]);
    vn = fmaxf(vn, mg.vn[w]);
  }
  rec_st2<COH>(rec + 8 + c, o0, o1);
  if constexpr (CERT) rec_st2<COH>(rec + 8 + D + c, p0, p1);
  float qn = 0.0f;
  if constexpr (CERT) {
    // ||q|| * scale from the prologue's q * scale * log2(e)
    const float q0 = qo[hh][c], q1 = qo[hh][c + 1];
    float sq = q0 * q0 + q1 * q1;
    sq = wave_sum(sq);
    qn = sqrtf(sq) / LOG2E;
  }
  if (l == 0) {
    rec_st2<COH>(rec, M, L);
    rec_st2<COH>(rec + 2, E, ek);
    rec_st2<COH>(rec + 4, vn, qn);
  }
}

// ------------------------------------------------------------------ combine
// One wave per (sequence, query head): log-sum-exp merge of the split records,
// inverse rotation back to the original basis ("OSCAR", section 2.2B), and the
// certificate.  zsw: 128 floats of LDS private to the wave.
template <bool CERT, bool COH, int SB = 8>
__device__ void combine_row(const DecodeArgs& a, int row, float* zsw, const float* ctab) {
  const int l = threadIdx.x & 63, c = 2 * l;
  const int b = row / a.Hq;
  KVQ_DCHECK(row >= 0 && row < a.B * a.Hq, DBG_ROW, row, a.n_splits);
  float* out = a.out + (size_t)row * D;
  if (a.seq.v[b] == 0) {
    *reinterpret_cast<float2*>(out + c) = make_float2(0.0f, 0.0f);
    if (CERT && a.cert && l == 0) a.cert[row] = 0.0f;
    return;
  }
  // Records in batches of SB splits (2 when a unit has at most 2, else 8): all loads
  // of a batch are issued together (indices past the last split reload it and get
  // weight 0), then merged with a running maximum.  Adjacent record words travel in
  // pairs (one 64-bit access each).
  const float* rec0 = a.part + (size_t)row * a.n_splits * PART_FLOATS;
  float M = NEG_INF, L = 0.0f, E = 0.0f, ek = 0.0f, vn = 0.0f, o0 = 0.0f, o1 = 0.0f, p0 = 0.0f, p1 = 0.0f;
  for (int s0 = 0; s0 < a.n_splits; s0 += SB) {
    float4 hd[SB];
    float vs[SB];
    float2 ov[SB], pv[SB];
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      const float* rec = rec0 + (size_t)min(s0 + i, a.n_splits - 1) * PART_FLOATS;
      if constexpr (COH) {
        const float2 h01 = rec_ld2<true>(rec), h23 = rec_ld2<true>(rec + 2);
        hd[i] = make_float4(h01.x, h01.y, h23.x, h23.y);
        vs[i] = rec_ld<true>(rec + 4);
        ov[i] = rec_ld2<true>(rec + 8 + c);
        if constexpr (CERT) pv[i] = rec_ld2<true>(rec + 8 + D + c);
      } else {
        hd[i] = *reinterpret_cast<const float4*>(rec);
        vs[i] = rec[4];
        ov[i] = *reinterpret_cast<const float2*>(rec + 8 + c);
        if constexpr (CERT) pv[i] = *reinterpret_cast<const float2*>(rec + 8 + D + c);
      }
    }
    float Mb = M;
#pragma unroll
    for (int i = 0; i < SB; ++i)
      if (s0 + i < a.n_splits) Mb = fmaxf(Mb, hd[i].x);
    const float sc = (M == NEG_INF) ? 0.0f : exp2f(M - Mb);
    L *= sc;
    E *= sc;
    o0 *= sc;
    o1 *= sc;
    if constexpr (CERT) {
      p0 *= sc;
      p1 *= sc;
    }
#pragma unroll
    for (int i = 0; i < SB; ++i) {
      if (s0 + i >= a.n_splits) continue;
      const float wt = (hd[i].x == NEG_INF) ? 0.0f : exp2f(hd[i].x - Mb);
      L += wt * hd[i].y;
      E += wt * hd[i].z;
      ek = fmaxf(ek, hd[i].w);
      vn = fmaxf(vn, vs[i]);
      o0 += wt * ov[i].x;
      o1 += wt * ov[i].y;
      if constexpr (CERT) {
        p0 += wt * pv[i].x;
        p1 += wt * pv[i].y;
      }
    }
    M = Mb;
  }
  const float inv = 1.0f / L;
  o0 *= inv;
  o1 *= inv;
  if (a.lam_v != nullptr) {  // values were stored times lambda_v
    const float* lp = a.lam_v + (size_t)((row % a.Hq) / a.G) * D;
    o0 = o0 / lp[c];
    o1 = o1 / lp[c + 1];
  }
  float r0 = o0, r1 = o1;
  if (a.rotation == KVQ_ROT_SIGN_FWHT) {
    // R^T o = diag(s) H o / sqrt(128): the butterflies over this head's 64 lanes
    r0 = o0 + o1;
    r1 = o0 - o1;
    wht_lanes(r0, r1, l);
    const float cn = bits_to_f32(KVQ_INV_SQRT_D_BITS);
    r0 *= a.signs[c] < 0 ? -cn : cn;
    r1 *= a.signs[c + 1] < 0 ? -cn : cn;
  } else if (a.rotation == KVQ_ROT_SRFT) {
    // R^T o = s * IDFT128(V), V the Hermitian spectrum V_0 = o_0 c0, V_64 = o_1 c0,
    // V_k = (o_2k + i o_2k+1) / 16, V_(128-k) = conj V_k.  Its even and odd samples are
    // z_n = x_2n + i x_2n+1 = IDFT64(G)_n with G_k = (V_k + conj V_(64-k)) + i W128^(-k)
    // (V_k - conj V_(64-k)); lane l forms G_l, the wave runs the inverse FFT, and lane l
    // takes z_l from lane rev6(l).  (zsw is not needed: everything stays in registers.)
    (void)zsw;
    const float c0 = bits_to_f32(KVQ_INV_SQRT_D_BITS);
    const float vr = l == 0 ? o0 * c0 : o0 * 0.0625f, vi = l == 0 ? 0.0f : o1 * 0.0625f;
    float qr = __shfl(vr, (64 - l) & 63), qi = __shfl(vi, (64 - l) & 63);  // V_(64-l)
    if (l == 0) {
      qr = o1 * c0;  // V_64
      qi = 0.0f;
    }
    const float pr = vr + qr, pi = vi - qi;  // V + conj Q
    const float dr = vr - qr, di = vi + qi;  // V - conj Q
    const float cw = ctab[l], sw = ctab[(l + 96) & 127];  // W128^(-l) = (cw, sw)
    float gr = pr - (dr * sw + di * cw), gi = pi + (dr * cw - di * sw);
    wave_fft64(gr, gi, l, ctab, true);
    r0 = __shfl(gr, rev6(l));
    r1 = __shfl(gi, rev6(l));
    if (a.signs[c] < 0) r0 = -r0;
    if (a.signs[c + 1] < 0) r1 = -r1;
  } else if (a.rotation == KVQ_ROT_DENSE) {
    zsw[c] = o0;
    zsw[c + 1] = o1;
    __builtin_amdgcn_wave_barrier();
    lds_wait();
    float acc0 = 0.0f, acc1 = 0.0f;
    for (int k = 0; k < D; ++k) {
      const float z = zsw[k];
      const uint32_t rr = *reinterpret_cast<const uint32_t*>(a.rot + (size_t)k * D + c);
      acc0 = fmaf(f16_bits_to_f32((uint16_t)(rr & 0xFFFF)), z, acc0);
      acc1 = fmaf(f16_bits_to_f32((uint16_t)(rr >> 16)), z, acc1);
    }
    r0 = acc0;
    r1 = acc1;
  }
  if constexpr (CERT) {
    r0 += p0 * inv;
    r1 += p1 * inv;
  }
  *reinterpret_cast<float2*>(out + c) = make_float2(r0, r1);
  if (CERT && a.cert && l == 0) {
    const float dstar = rec_ld<COH>(rec0 + 5) * ek;
    // key term: total-variation distance under logit moves of at most dstar is at most
    // tanh(dstar / 2), times twice the largest value norm; value term: mass-weighted
    // reconstruction errors of the blocks read from codes
    a.cert[row] = 2.0f * tanhf(0.5f * dstar) * vn + E * inv;
  }
}

// Rows the dense fallback recomputes: certificate above eps, or failed the ranking check.
__device__ __forceinline__ bool fallback_row(const DecodeArgs& a, size_t row) {
  return (a.fb_cert != nullptr && a.fb_cert[row] > a.fb_eps) || (a.fb_fail != nullptr && a.fb_fail[row] != 0);
}

// The separate combine launch of the fp16/bf16 decode: one wave per row, ordered after
// every split workgroup by the stream.  FB: the dense fallback, which writes only the
// rows it recomputes and sets their certificate to 0.
template <bool FB>
__global__ __launch_bounds__(NT) void combine_kernel(DecodeArgs a) {
  __shared__ float zs[4][D];
  const int w = threadIdx.x >> 6;
  const int row = blockIdx.x * 4 + w;
  if (row >= a.B * a.Hq) return;  // whole waves; no barrier in combine_row
  if constexpr (FB) {
    if (!fallback_row(a, (size_t)row)) return;
  }
  combine_row<false, false>(a, row, zs[w], nullptr);  // no rotation on this path
  if constexpr (FB) {
    if (a.fb_cert != nullptr && (threadIdx.x & 63) == 0) a.fb_cert[row] = 0.0f;
  }
}

// ------------------------------------------------------------------ split kernel
// V metadata dwords per lane and chunk: 8 elements x 64 tokens x 2 bytes (INT2 scales and
// offsets, INT4 groups of 16) is 16 bytes; the others fit in 8.
__host__ __device__ constexpr int vmeta_words(int vf, int vg) {
  return (vf == KVQ_INT2 || (vf == KVQ_INT4 && vg == 16)) ? 4 : 2;
}

// Registers holding one chunk of packed data for one lane.
template <int KF, int VF, int VMW>
struct ChunkRegs {
  uint32_t krow[KFmt<KF>::DW];            // K row of token pi(s_a, r_a)
  uint32_t kmeta[4];                      // its metadata (scales [, offsets])
  uint32_t vw[2 * VFmt<VF>::CDW];         // V codes of channels 2*lane, 2*lane+1
  uint32_t vmeta[VMW];                    // this lane's share of the V metadata tile
};

// Flag and error descriptor of one chunk (exact-recompute kernels only).
template <bool CERT>
struct ChunkAux {};
template <>
struct ChunkAux<true> {
  uint32_t flag;
  float ek, ev, vn;
};

// Issue the loads of chunk ch (no waits: the caller consumes them one chunk later).
template <int KF, int KG, int VF, int VG>
__device__ __forceinline__ void load_chunk(const DecodeArgs& a, size_t stream, int ch, int lane, int tok_a,
                                           ChunkRegs<KF, VF, vmeta_words(VF, VG)>& R) {
  constexpr int KDW = KFmt<KF>::DW;
  constexpr int KM = meta_bytes(KF, KG);
  constexpr int CDW = VFmt<VF>::CDW;
  const int tok0 = ch * TILE;
  KVQ_DCHECK(stream < (size_t)a.B * a.H, DBG_STREAM, stream, ch);
  KVQ_DCHECK(ch >= 0 && ch < a.nt, DBG_CHUNK, stream, ch);
  const uint4* rp = reinterpret_cast<const uint4*>(a.k_codes + (stream * a.Tmax + tok0 + tok_a) * (KDW * 4));
#pragma unroll
  for (int i = 0; i < KDW / 4; ++i) {
    const uint4 u = rp[i];
    R.krow[4 * i] = u.x; R.krow[4 * i + 1] = u.y; R.krow[4 * i + 2] = u.z; R.krow[4 * i + 3] = u.w;
  }
  const uint8_t* mp = a.k_meta + (stream * a.Tmax + tok0 + tok_a) * KM;
  if constexpr (KM == 16) {
    const uint4 u = *reinterpret_cast<const uint4*>(mp);
    R.kmeta[0] = u.x; R.kmeta[1] = u.y; R.kmeta[2] = u.z; R.kmeta[3] = u.w;
  } else if constexpr (KM == 8) {
    const uint2 u = *reinterpret_cast<const uint2*>(mp);
    R.kmeta[0] = u.x; R.kmeta[1] = u.y;
  } else {
    R.kmeta[0] = *reinterpret_cast<const uint16_t*>(mp);
  }
  const uint4* vp = reinterpret_cast<const uint4*>(a.v_codes + (stream * a.nt + ch) * (size_t)(D * CDW * 4) +
                                                   (size_t)(2 * lane) * CDW * 4);
#pragma unroll
  for (int i = 0; i < CDW / 2; ++i) {
    const uint4 u = vp[i];
    R.vw[4 * i] = u.x; R.vw[4 * i + 1] = u.y; R.vw[4 * i + 2] = u.z; R.vw[4 * i + 3] = u.w;
  }
  constexpr int NM = meta_elems(VF, VG);
  const uint8_t* vm = a.v_meta + (stream * a.nt + ch) * (size_t)(NM * TILE * meta_esize(VF));
  if constexpr (VF == KVQ_INT2 || (VF == KVQ_INT4 && NM == 8)) {  // 8 elements x 64 tokens: 16 bytes per lane
    const uint4 u = reinterpret_cast<const uint4*>(vm)[lane];
    R.vmeta[0] = u.x; R.vmeta[1] = u.y; R.vmeta[2] = u.z; R.vmeta[3] = u.w;
  } else if constexpr (NM == 4 || VF == KVQ_FP4) {  // 8 bytes per lane
    const uint2 u = reinterpret_cast<const uint2*>(vm)[lane];
    R.vmeta[0] = u.x; R.vmeta[1] = u.y;
  } else {  // one scale per token
    R.vmeta[0] = reinterpret_cast<const uint16_t*>(vm)[lane];
  }
}

// V metadata of a chunk -> this wave's LDS area, laid out [element][slice][pair][half]
// so that slice s of element m is two dwords: (pi(s,0), pi(s,1)) and (pi(s,2), pi(s,3)).
template <int VF, int VG>
__device__ __forceinline__ void stage_vmeta(uint16_t* L, int lane, const uint32_t* vmeta) {
  constexpr int NM = meta_elems(VF, VG);
  if constexpr (VF == KVQ_FP4) {  // block mm = lane / 8, tokens 8u..8u+7 (natural order), E4M3 -> fp16
    const int mm = lane >> 3, u = lane & 7;
    uint4 o;
    const uint32_t w0 = vmeta[0], w1 = vmeta[1];
    o.x = as_u(e4m3x2_to_h2(w0 & 0xFF, (w0 >> 8) & 0xFF));
    o.y = as_u(e4m3x2_to_h2((w0 >> 16) & 0xFF, w0 >> 24));
    o.z = as_u(e4m3x2_to_h2(w1 & 0xFF, (w1 >> 8) & 0xFF));
    o.w = as_u(e4m3x2_to_h2((w1 >> 16) & 0xFF, w1 >> 24));
    *reinterpret_cast<uint4*>(L + mm * 64 + 8 * u) = o;
  } else if constexpr (VF == KVQ_INT2) {  // tokens 8u..8u+7 of element mm: slices 2u, 2u+1
    const int mm = lane >> 3, u = lane & 7;
    uint4 o;
    o.x = (vmeta[0] & 0xFFFFu) | (vmeta[1] << 16);          // tokens 0, 2
    o.y = (vmeta[0] >> 16) | (vmeta[1] & 0xFFFF0000u);      // tokens 1, 3
    o.z = (vmeta[2] & 0xFFFFu) | (vmeta[3] << 16);          // tokens 4, 6
    o.w = (vmeta[2] >> 16) | (vmeta[3] & 0xFFFF0000u);      // tokens 5, 7
    *reinterpret_cast<uint4*>(L + mm * 64 + 8 * u) = o;
  } else if constexpr (NM == 8) {  // INT4, groups of 16: tokens 8u..8u+7 of group mm, placed as below
    const int mm = lane >> 3, u = lane & 7;
    const int base = (mm * 16 + 2 * u) * 4;
#pragma unroll
    for (int e = 0; e < 8; ++e) L[base + ((e >> 2) & 1) + 2 * (e & 3)] = (uint16_t)(vmeta[e >> 1] >> (16 * (e & 1)));
  } else if constexpr (NM == 4) {
    const int mm = lane >> 4, t0 = 4 * (lane & 15);  // tokens t0..t0+3 of group mm
    const int base = (mm * 16 + 2 * (t0 >> 3)) * 4 + ((t0 >> 2) & 1);
#pragma unroll
    for (int e = 0; e < 4; ++e) L[base + 2 * e] = (uint16_t)(vmeta[e >> 1] >> (16 * (e & 1)));
  } else {
    const int tau = lane, e = tau & 7;
    L[(2 * (tau >> 3)) * 4 + ((e >> 2) & 1) + 2 * (e & 3)] = (uint16_t)vmeta[0];
  }
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// max over the 16 lanes sharing (lane & 3): rotate within rows of 16, then across rows
// (per chunk, in the main loop: the shuffles go through the LDS crossbar and cost no
// vector issue slots there, which the row swaps would; measured ≈3 % on the FP4 decode)
__device__ __forceinline__ float max_same_head_fast(float v) {
  v = fmaxf(v, dpp_f<0x124>(v));  // row_ror:4
  v = fmaxf(v, dpp_f<0x128>(v));  // row_ror:8
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
}

// V scale groups per token whose PV weights are formed on the QK side
__host__ __device__ constexpr int v_groups(int vf, int vg) {
  return (vf == KVQ_FP4 || vg == 16) ? 8 : (vf == KVQ_INT2 || vg == 32) ? 4 : 1;
}

// MODE 0: codes only.  MODE 1: blocks of the full-precision window recomputed
// exactly from their originals.  MODE 2: certified cache: window blocks and blocks
// flagged by the error bound recomputed exactly, per-block descriptors for the
// certificate.
//
// Work layout.  A unit is (sequence, kv head, group of 4 query heads).  Workgroup g of
// the 1-D grid takes split g % S of unit g / S: a range of its 64-token chunks.  Its 8
// waves share the range out through a counter in LDS: wave w starts with the range's
// chunk w, and every further chunk is claimed after the visit before it, its loads in
// flight while the chunk loaded before it is visited.  The two waves that
// share a SIMD do not progress equally (the older one wins issue slots), so the faster
// one simply claims more chunks.
template <int KF, int KG, int VF, int VG, int MODE>
__global__ __launch_bounds__(NTS) void decode_split(DecodeArgs a) {
  constexpr bool EXACT = MODE != 0;  // exact recompute of some chunks
  constexpr bool CERT = MODE == 2;   // flags and descriptors
  __shared__ DecodeSmem sm;
  {
    // every kernel argument the start-up needs, loaded in one batch (the empty asm makes
    // them all available at one point, so none is loaded later behind a branch)
    const uint16_t* p0 = a.q;
    const int8_t* p1 = a.signs;
    const uint8_t* p2 = a.k_codes;
    const uint8_t* p3 = a.k_meta;
    const uint8_t* p4 = a.v_codes;
    const uint8_t* p5 = a.v_meta;
    int i0 = a.G, i1 = a.Hq, i2 = a.H, i3 = a.Tmax, i4 = a.nt, i5 = a.chunks_per_split, i6 = a.rotation,
        i7 = a.seq.v[blockIdx.x / a.n_splits / ((a.G + 3) / 4) / a.H], i8 = a.n_splits;
    asm volatile("" ::"s"(p0), "s"(p1), "s"(p2), "s"(p3), "s"(p4), "s"(p5));
    asm volatile("" ::"s"(i0), "s"(i1), "s"(i2), "s"(i3), "s"(i4), "s"(i5), "s"(i6), "s"(i7), "s"(i8));
  }
  const int t = threadIdx.x, lane = t & 63;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);  // wave-uniform: the chunk walk is scalar
  const int S = a.n_splits;
  const int u = blockIdx.x / S, split = blockIdx.x % S;
  const int HG = (a.G + 3) >> 2;
  const int b = u / (a.H * HG), hkv = (u / HG) % a.H, hg = u % HG;
  const int hq0 = hkv * a.G + hg * 4;
  const int nh = min(4, a.G - hg * 4);
  const int T = a.seq.v[b];
  const int nchunks = (T + TILE - 1) / TILE;
  const int c0 = split * a.chunks_per_split;
  const int c1 = min(nchunks, c0 + a.chunks_per_split);
  const int j = lane & 3;     // head of this lane (QK output / softmax role, PV operand row)
  const int s_a = lane >> 2;  // QK slice of this lane (A role)
  const int r_a = lane & 3;
  const int tok_a = tok_of<VF>(s_a, r_a);
  const size_t stream = (size_t)b * a.H + hkv;
  constexpr int CDW = VFmt<VF>::CDW;
  constexpr int NGV = v_groups(VF, VG);
  // PV weights p * s in two fp16 parts (about 2^-22 of themselves) for integer values, one
  // fp16 rounding for FP4 values: with it their worst attention rows are ~3e-4 (the bar is
  // 2e-3), and the second pair of products cost ~7 % of their decode time
  constexpr bool PV_LO = VF != KVQ_FP4;
  float neg_one = -1.0f;
  asm volatile("" : "+v"(neg_one));  // opaque: fma(hi, -1, x) is not turned into x - hi
  // V scale group of channels 2*lane, 2*lane+1: 32-channel group, one per token, or 16-channel block
  const int vgrp = (VF == KVQ_FP4 || VG == 16) ? (lane >> 3) : (VG == 128) ? 0 : (lane >> 4);
  uint16_t* vml = &sm.vmeta[wv][0][0][0];

  if (t == 0) sm.next = NWS;  // published by the prologue's barrier
  auto claim = [&]() -> int {
    int v = 0;
    if (lane == 0) v = atomicAdd(&sm.next, 1);
    return v;
  };
  // With exact recompute, a chunk's flag and descriptor are loaded right after its
  // codes, unconditionally (from a stand-in address when the buffer is absent), so
  // that the wait for them is the wait for the chunk itself, never for the chunk
  // loaded after it.
  auto load_aux = [&](int ch, ChunkAux<CERT>& X) {
    if constexpr (CERT) {
      // The offset is taken through an empty asm: the loaded values are then not
      // known to be wave-uniform, so they stay in vector registers (no read into a
      // scalar register, and no wait, at the load) until the visit reads them.
      uint32_t blk = (uint32_t)(stream * a.nt + ch);
      asm volatile("" : "+v"(blk));
      const uint8_t* fp = a.flags != nullptr ? a.flags + blk : a.k_meta;
      const float* dp = a.desc != nullptr ? a.desc + (size_t)blk * 3 : reinterpret_cast<const float*>(a.k_meta);
      X.flag = *fp;
      X.ek = dp[0];
      X.ev = dp[1];
      X.vn = dp[2];
    }
  };
  // The first chunk's loads are in flight during the query prologue.  Every prefetch is
  // unconditional (a wave past its last chunk reloads a chunk index that is always
  // inside the cache), so the number of loads in flight is the same on every path.
  const int hw = wv < nh ? wv : 0;  // waves 0..3 rotate query heads 0..3 (others load a valid head)
  const QueryIn qin = query_loads(a, b, hq0 + hw);
  __builtin_amdgcn_sched_barrier(0);
  ChunkRegs<KF, VF, vmeta_words(VF, VG)> RA, RB;
  ChunkAux<CERT> XA, XB;
  int cA = c0 + wv;
  load_chunk<KF, KG, VF, VG>(a, stream, cA < c1 ? cA : 0, lane, tok_a, RA);
  load_aux(cA < c1 ? cA : 0, XA);
  __builtin_amdgcn_sched_barrier(0);
  if (a.rotation == KVQ_ROT_SRFT) {
    if (t < 128) sm.ctab[t] = a.cos128[t];
    __syncthreads();
  }
  if (wv < 4) query_head<KF>(a, sm, qin, wv, wv, wv < nh, KG, hkv);
  __syncthreads();
  int pB = claim();

  const float qs = sm.qs[j];
  float qsum[4];  // (groups of 16 read theirs from LDS when needed: registers are short there)
#pragma unroll
  for (int g = 0; g < 4; ++g) qsum[g] = sm.qsum[j][g];

  float m = NEG_INF, lsum = 0.0f, eta = 0.0f, ekmax = 0.0f, vnmax = 0.0f;
  float zacc[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // INT2 values: sum of p * offset per group (this lane's tokens)
  f4 o[2], oo[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    o[hf] = f4{0, 0, 0, 0};
    oo[hf] = f4{0, 0, 0, 0};
  }

  // ---------------------------------------------------------------- chunks read from the originals
  // Window blocks: the first n_sink and the last n_recent blocks of the sequence,
  // kept at full precision in k_win/v_win ("OSCAR", section 2.2B, mixed-precision
  // layout).  They are attended exactly, like blocks flagged by the error bound.
  auto in_window = [&](int ch) -> bool {
    return a.k_win != nullptr && (ch < a.n_sink || ch >= nchunks - a.n_recent);
  };
  // first row of chunk ch's originals: its window slot, else the full copy
  auto orig_rows = [&](const uint16_t* full, const uint16_t* win, int ch) -> const uint16_t* {
    if (in_window(ch)) {
      const int wslot = ch < a.n_sink ? ch : a.n_sink + ch % a.n_recent;
      KVQ_DCHECK(wslot >= 0 && wslot < a.n_sink + a.n_recent, DBG_WINDOW, stream, ch);
      return win + (stream * (size_t)(a.n_sink + a.n_recent) + wslot) * TILE * D;
    }
    KVQ_DCHECK(ch >= 0 && ch < a.nt, DBG_CHUNK, stream, ch);
    return full + (stream * a.Tmax + (size_t)ch * TILE) * D;
  };
  // Original values of one chunk into oo: lane l holds channels 2l, 2l+1 of every token
  // (vp = the chunk's first row + lane, in dwords), the weights of (token, head) in the
  // wave's pb (written and waited for by the caller); vr[0] holds the first 16 rows.  The
  // value rows go in batches of 16, the next batch in flight while one is accumulated.
  // Rows at or past the sequence end count as zeros (their weights are 0, and whatever
  // bits the buffer holds there must not turn 0 * x into a NaN).
  auto pv_orig = [&](int ch, const uint32_t* vp, uint32_t(&vr)[2][16]) {
    const bool bf16 = a.in_bf16 != 0;
    const float(*pb)[4] = sm.u.loop.pb[wv];
    const int nlive = T - ch * TILE;  // rows of the chunk below the sequence end (>= 1)
#pragma unroll
    for (int bt = 0; bt < TILE / 16; ++bt) {
      if (bt + 1 < TILE / 16) {
#pragma unroll
        for (int k = 0; k < 16; ++k) vr[(bt + 1) & 1][k] = vp[(size_t)(16 * (bt + 1) + k) * (D / 2)];
      }
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const uint32_t vv = 16 * bt + k < nlive ? vr[bt & 1][k] : 0u;
        const float v0 = widen((uint16_t)(vv & 0xFFFF), bf16), v1 = widen((uint16_t)(vv >> 16), bf16);
        const float4 pp = *reinterpret_cast<const float4*>(&pb[16 * bt + k][0]);
        oo[0] += f4{pp.x, pp.y, pp.z, pp.w} * v0;
        oo[1] += f4{pp.x, pp.y, pp.z, pp.w} * v1;
      }
    }
    lds_wait();
  };

  // ---------------------------------------------------------------- one quantized chunk
  auto quant_chunk = [&](const ChunkRegs<KF, VF, vmeta_words(VF, VG)>& R, int ch, float ev_c, bool vexact) {
    const int tok0 = ch * TILE;
    stage_vmeta<VF, VG>(vml, lane, R.vmeta);
    float l[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if constexpr (KF == KVQ_FP4) {
      // ---- QK^T with E2M1 keys in fp16 (exact) against the two fp16 query
      // parts, one fp32 accumulator per 16-channel block (8 chains), then the
      // E4M3 block scales of tokens 4s + r (quad broadcast)
      f4 ab[8];
#pragma unroll
      for (int bk = 0; bk < 8; ++bk) ab[bk] = f4{0, 0, 0, 0};
      const uint4* qrow = reinterpret_cast<const uint4*>(&sm.qf4[j][0][0]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int bk = 0; bk < 8; ++bk) {
          const int n = 4 * bk + i;
          const uint4 qv = qrow[n];
          const h4 av = KFmt<KVQ_FP4>::a_op_f16(R.krow, n);
          ab[bk] = __builtin_amdgcn_mfma_f32_4x4x4f16(av, cat(as_h2(qv.x), as_h2(qv.y)), ab[bk], 0, 0, 0);
          ab[bk] = __builtin_amdgcn_mfma_f32_4x4x4f16(av, cat(as_h2(qv.z), as_h2(qv.w)), ab[bk], 0, 0, 0);
        }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint32_t sw[2];
#pragma unroll
        for (int w = 0; w < 2; ++w)
          sw[w] = r == 0 ? quad_bcast_u<0>(R.kmeta[w]) : r == 1 ? quad_bcast_u<1>(R.kmeta[w])
                : r == 2 ? quad_bcast_u<2>(R.kmeta[w]) : quad_bcast_u<3>(R.kmeta[w]);
        // the token's 8 E4M3 block scales, exactly, by the gfx950 fp8 -> fp32 conversion
        // (scale 1), two per instruction; blocks 0..7 in order
        float sf[8];
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const f2 lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sw[w], 1.0f, false);
          const f2 hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(sw[w], 1.0f, true);
          sf[4 * w] = lo.x;
          sf[4 * w + 1] = lo.y;
          sf[4 * w + 2] = hi.x;
          sf[4 * w + 3] = hi.y;
        }
#pragma unroll
        for (int bk = 0; bk < 8; ++bk) l[r] = fmaf(ab[bk][r], sf[bk], l[r]);
      }
    } else {
      // ---- QK^T: exact integer dot products.  Four independent accumulator
      // chains per query half (chain c covers channels 32c..32c+31, i.e. one
      // 32-channel group); each K operand is unpacked once and feeds both halves.
      // With groups of 16 each chain is read out, scaled and added after its first
      // four steps (channels 32c..32c+15, group 2c) and restarted for group 2c + 1.
      constexpr int NG = (KG == 128) ? 1 : 4;  // groups whose sums wait for the scale step below
      constexpr int NC = 4, PER = 32 / NC;
      constexpr int NPH = (KG == 16) ? 2 : 1, PPH = PER / NPH;  // phases per chain, steps per phase
      i4 ah[NC], al[NC], acc[NG];
      auto kscale_word = [&](int r, int w) -> uint32_t {  // metadata dword w of token pi(s, r)
        return r == 0 ? quad_bcast_u<0>(R.kmeta[w]) : r == 1 ? quad_bcast_u<1>(R.kmeta[w])
             : r == 2 ? quad_bcast_u<2>(R.kmeta[w]) : quad_bcast_u<3>(R.kmeta[w]);
      };
      static_assert(NC == 4, "query operand layout: 4 chains per 16-byte LDS read");
#pragma unroll
      for (int ph = 0; ph < NPH; ++ph) {
#pragma unroll
        for (int c = 0; c < NC; ++c) {
          // the offset-binary correction -8 * sum(q16) of the chain's group rides in the low half
          int corr = 0;
          if constexpr (KF == KVQ_INT4)
            corr = (KG == 16) ? -8 * (int)sm.qsum[j][2 * c + ph]
                 : (NG == 1) ? (c == 0 ? -8 * (int)qsum[0] : 0) : -8 * (int)qsum[c];
          ah[c] = i4{0, 0, 0, 0};
          al[c] = i4{corr, corr, corr, corr};
        }
#pragma unroll
        for (int n = ph * PPH; n < (ph + 1) * PPH; ++n) {
          // the query operands stay in LDS (registers go to the chunk prefetch)
          const uint4 qhv = *reinterpret_cast<const uint4*>(&sm.qh[j][4 * n]);
          const uint4 qlv = *reinterpret_cast<const uint4*>(&sm.ql[j][4 * n]);
          const int qhc[4] = {(int)qhv.x, (int)qhv.y, (int)qhv.z, (int)qhv.w};
          const int qlc[4] = {(int)qlv.x, (int)qlv.y, (int)qlv.z, (int)qlv.w};
#pragma unroll
          for (int c = 0; c < NC; ++c) {
            const int av = KFmt<KF>::a_op(R.krow, c * PER + n);
            ah[c] = __builtin_amdgcn_mfma_i32_4x4x4i8(av, qhc[c], ah[c], 0, 0, 0);
            al[c] = __builtin_amdgcn_mfma_i32_4x4x4i8(av, qlc[c], al[c], 0, 0, 0);
          }
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          if constexpr (KG == 16) {
            // group 2c + ph: its fp16 scale is half ph of metadata dword c
#pragma unroll
            for (int c = 0; c < NC; ++c) {
              const uint16_t sb = (uint16_t)(kscale_word(r, c) >> (16 * ph));
              l[r] += (float)(ah[c][r] * 256 + al[c][r]) * f16_bits_to_f32(sb);
            }
          } else if constexpr (NG == 1) {
            acc[0][r] = 0;
#pragma unroll
            for (int c = 0; c < NC; ++c) acc[0][r] += ah[c][r] * 256 + al[c][r];
          } else {
#pragma unroll
            for (int c = 0; c < NC; ++c) acc[c][r] = ah[c][r] * 256 + al[c][r];
          }
        }
        // keep the next phase's chains from starting before this one is read out (both
        // sets of accumulators live at once would cost 32 registers)
        if constexpr (NPH > 1) __builtin_amdgcn_sched_barrier(0);
      }
      // ---- group scales of tokens pi(s, r), held by lanes 4s + r (A role): quad broadcast
#pragma unroll
      for (int r = 0; r < 4 && KG != 16; ++r) {
        uint32_t sw[2], zw[2] = {0u, 0u};
#pragma unroll
        for (int w = 0; w < (NG == 1 ? 1 : 2); ++w) {
          sw[w] = kscale_word(r, w);
          if constexpr (KF == KVQ_INT2) zw[w] = kscale_word(r, 2 + w);
        }
        // each group's sum times its fp16 scale (and the int2 offset times the query's
        // group sum) accumulated by fmas that read the fp16 halves directly
#pragma unroll
        for (int g = 0; g < NG; ++g) {
          const uint16_t sb = (uint16_t)(sw[g >> 1] >> (16 * (g & 1)));
          l[r] = fmaf((float)acc[g][r], f16_bits_to_f32(sb), l[r]);
          if constexpr (KF == KVQ_INT2) {
            const uint16_t zb = (uint16_t)(zw[g >> 1] >> (16 * (g & 1)));
            l[r] = fmaf(f16_bits_to_f32(zb), qsum[g], l[r]);
          }
        }
      }
    }
    const bool tail = tok0 + TILE > T;  // the chunk holds positions at or past the sequence end
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      l[r] *= qs;
      if (tok0 + tok_of<VF>(s_a, r) >= T) l[r] = NEG_INF;
    }
    // ---- online softmax (exp2 domain)
    const float cmax = max_same_head_fast(fmaxf(fmaxf(l[0], l[1]), fmaxf(l[2], l[3])));
    const float m_new = fmaxf(m, cmax);
    const bool none = m_new == NEG_INF;
    const float alpha = none ? 1.0f : fast_exp2(m - m_new);
    float p[4], ps = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = none ? 0.0f : fast_exp2(l[r] - m_new);
      ps += p[r];
    }
    lsum = lsum * alpha + ps;
    if constexpr (CERT) eta = eta * alpha + ps * ev_c;
    m = m_new;
    const f4 av = {quad_bcast<0>(alpha), quad_bcast<1>(alpha), quad_bcast<2>(alpha), quad_bcast<3>(alpha)};
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      o[hf] *= av;
      if constexpr (EXACT) oo[hf] *= av;
    }
    if constexpr (CERT) {
      if (vexact) {
        // value promotion: the logits above came from the codes, the values come from the
        // originals, accumulated like those of an exactly recomputed chunk (weights p of
        // token tok_of(s_a, r), head j, through LDS)
        const uint32_t* vp = reinterpret_cast<const uint32_t*>(orig_rows(a.v_orig, a.v_win, ch)) + lane;
        uint32_t vr[2][16];
#pragma unroll
        for (int k = 0; k < 16; ++k) vr[0][k] = vp[(size_t)k * (D / 2)];
        float(*pb)[4] = sm.u.loop.pb[wv];
#pragma unroll
        for (int r = 0; r < 4; ++r) pb[tok_of<VF>(s_a, r)][j] = p[r];
        if constexpr (VF == KVQ_INT2) {
#pragma unroll
          for (int g = 0; g < 4; ++g) zacc[g] *= alpha;
        }
        lds_wait();
        pv_orig(ch, vp, vr);
        return;
      }
    }
    // ---- PV weights, formed here once per (token, V group): p * s in fp32 for this lane's
    // four tokens (slice s_a, head j), rounded to fp16 and (PV_LO) the fp16 rounding of the
    // remainder, so that the fp16 matrix products carry each weight to about 2^-22 of
    // itself.  Positions past the sequence end have p = 0 and weight 0 (their metadata may
    // be anything).
    // (scales are never negative, so max(p s, 0) changes no weight and turns the 0 * NaN of
    // a position past the end into 0)
    // (hi is formed by packed conversions; the remainder x - hi by one mixed-precision fma per
    // weight that reads hi's fp16 half directly, with an opaque -1 so that it stays an fma)
    const uint2* vmw = reinterpret_cast<const uint2*>(vml) + s_a;
    uint2 sc[NGV];
#pragma unroll
    for (int g = 0; g < NGV; ++g) sc[g] = vmw[g * 16];
#pragma unroll
    for (int g = 0; g < NGV; ++g) {
      const h2 s01 = as_h2(sc[g].x), s23 = as_h2(sc[g].y);
      const float x0 = fmaxf(fmaf(p[0], (float)s01.x, 0.0f), 0.0f), x1 = fmaxf(fmaf(p[1], (float)s01.y, 0.0f), 0.0f);
      const float x2 = fmaxf(fmaf(p[2], (float)s23.x, 0.0f), 0.0f), x3 = fmaxf(fmaf(p[3], (float)s23.y, 0.0f), 0.0f);
      const h2 hi01 = __builtin_convertvector(f2{x0, x1}, h2), hi23 = __builtin_convertvector(f2{x2, x3}, h2);
      if constexpr (PV_LO) {
        // the remainder x - hi is exact in fp32 (hi is x rounded to 11 bits)
        const f2 r01 = {fmaf((float)hi01.x, neg_one, x0), fmaf((float)hi01.y, neg_one, x1)};
        const f2 r23 = {fmaf((float)hi23.x, neg_one, x2), fmaf((float)hi23.y, neg_one, x3)};
        const h2 lo01 = __builtin_convertvector(r01, h2), lo23 = __builtin_convertvector(r23, h2);
        sm.u.loop.pw[wv][g][s_a][j] = make_uint4(as_u(hi01), as_u(hi23), as_u(lo01), as_u(lo23));
      } else {
        sm.u.loop.pw[wv][g][s_a][j] = make_uint4(as_u(hi01), as_u(hi23), 0u, 0u);
      }
    }
    if constexpr (VF == KVQ_INT2) {
      // zero points: sum_t p_t z_(t, g) per group in fp32, added to every channel of the
      // group at the end (z is constant over the group's channels; offsets may be negative,
      // so positions past the end are masked by p)
      uint2 zc[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) zc[g] = vmw[(4 + g) * 16];
      // one fma per token on the fp16 offsets; the chunk holding the sequence end (rare,
      // wave-uniform) takes the masked sums in a branch of its own (the empty asm keeps the
      // compiler from evaluating both forms on every chunk and selecting)
      float zs[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const h2 z01 = as_h2(zc[g].x), z23 = as_h2(zc[g].y);
        zs[g] = fmaf(p[3], (float)z23.y, fmaf(p[2], (float)z23.x, fmaf(p[1], (float)z01.y, p[0] * (float)z01.x)));
      }
      if (tail) {
        asm volatile("");
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const h2 z01 = as_h2(zc[g].x), z23 = as_h2(zc[g].y);
          zs[g] = (p[0] > 0.0f ? p[0] * (float)z01.x : 0.0f) + (p[1] > 0.0f ? p[1] * (float)z01.y : 0.0f) +
                  (p[2] > 0.0f ? p[2] * (float)z23.x : 0.0f) + (p[3] > 0.0f ? p[3] * (float)z23.y : 0.0f);
        }
      }
#pragma unroll
      for (int g = 0; g < 4; ++g) zacc[g] = fmaf(zacc[g], alpha, zs[g]);
    }
    // ---- PV: step s takes the weights of tokens pi(s, 0..3) for this lane's head row and
    // V group, high and low parts through two products each
    const uint4* pwv = &sm.u.loop.pw[wv][vgrp][0][j];
    auto pv_step = [&](int s, h4 B0, h4 B1) {
      const uint4 w = pwv[4 * s];
      const h4 Ah = cat(as_h2(w.x), as_h2(w.y));
      o[0] = __builtin_amdgcn_mfma_f32_4x4x4f16(Ah, B0, o[0], 0, 0, 0);
      o[1] = __builtin_amdgcn_mfma_f32_4x4x4f16(Ah, B1, o[1], 0, 0, 0);
      if constexpr (PV_LO) {
        const h4 Al = cat(as_h2(w.z), as_h2(w.w));
        o[0] = __builtin_amdgcn_mfma_f32_4x4x4f16(Al, B0, o[0], 0, 0, 0);
        o[1] = __builtin_amdgcn_mfma_f32_4x4x4f16(Al, B1, o[1], 0, 0, 0);
      }
    };
    if constexpr (VF == KVQ_FP4) {
      // tokens 4s..4s+3 of step s are the byte pairs 2(s&1), 2(s&1)+1 of word s/2
#pragma unroll
      for (int s = 0; s < 16; ++s) {
        const uint32_t w0 = R.vw[s >> 1], w1 = R.vw[CDW + (s >> 1)];
        const h2 c00 = (s & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 2) : __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 0);
        const h2 c01 = (s & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 3) : __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w0, 1.0f, 1);
        const h2 c10 = (s & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 2) : __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 0);
        const h2 c11 = (s & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 3) : __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w1, 1.0f, 1);
        pv_step(s, cat(c00, c01), cat(c10, c11));
      }
    } else if constexpr (VF == KVQ_INT4) {
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        h2 c0[4], c1[4];
        v_int4_pairs(R.vw[d], c0);
        v_int4_pairs(R.vw[CDW + d], c1);
#pragma unroll
        for (int x = 0; x < 2; ++x) pv_step(2 * d + x, cat(c0[2 * x], c0[2 * x + 1]), cat(c1[2 * x], c1[2 * x + 1]));
      }
    } else {  // INT2 values: codes 0..3, value = c * s + z (z added at the end)
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        h2 c0[8], c1[8];
        v_int2_pairs(R.vw[w], c0);
        v_int2_pairs(R.vw[CDW + w], c1);
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          pv_step(4 * w + kk, cat(c0[2 * kk], c0[2 * kk + 1]), cat(c1[2 * kk], c1[2 * kk + 1]));
      }
    }
  };

  // ---------------------------------------------------------------- one exactly recomputed chunk
  auto exact_chunk = [&](int ch) {
    const int tok0 = ch * TILE;
    const bool bf16 = a.in_bf16 != 0;
    const int tau = lane;
    const bool live = tok0 + tau < T;
    float lh[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    // Loads are issued in batches ahead of their use (the token's key row in two
    // halves, the value rows 16 at a time), a few memory round trips per chunk
    // rather than one per row.
    const uint4* kp = reinterpret_cast<const uint4*>(orig_rows(a.k_orig, a.k_win, ch) + (size_t)tau * D);
    const uint32_t* vp = reinterpret_cast<const uint32_t*>(orig_rows(a.v_orig, a.v_win, ch)) + lane;
    const float(*qo)[D] = sm.qo;
    float(*pb)[4] = sm.u.loop.pb[wv];
    uint4 kr[8];
    uint32_t vr[2][16];
#pragma unroll
    for (int i = 0; i < 8; ++i) kr[i] = kp[i];
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      if (i == 8) {
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int e = 0; e < 8; ++e) kr[e] = kp[8 + e];
#pragma unroll
        for (int k = 0; k < 16; ++k) vr[0][k] = vp[(size_t)k * (D / 2)];
        __builtin_amdgcn_sched_barrier(0);
      }
      const uint4 uq = kr[i & 7];
      const uint32_t ws[4] = {uq.x, uq.y, uq.z, uq.w};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int c = 8 * i + 2 * jj;
        const float k0 = widen((uint16_t)(ws[jj] & 0xFFFF), bf16), k1 = widen((uint16_t)(ws[jj] >> 16), bf16);
#pragma unroll
        for (int hh = 0; hh < 4; ++hh) lh[hh] = fmaf(qo[hh][c + 1], k1, fmaf(qo[hh][c], k0, lh[hh]));
      }
    }
    float cm[4];
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      if (!live) lh[hh] = NEG_INF;
      cm[hh] = wave_max(lh[hh]);
    }
    const float mine = (j == 0) ? cm[0] : (j == 1) ? cm[1] : (j == 2) ? cm[2] : cm[3];
    const float m_new = fmaxf(m, mine);
    const float alpha = (m_new == NEG_INF) ? 1.0f : fast_exp2(m - m_new);
    m = m_new;
    const float mh[4] = {quad_bcast<0>(m), quad_bcast<1>(m), quad_bcast<2>(m), quad_bcast<3>(m)};
    float sums[4];
#pragma unroll
    for (int hh = 0; hh < 4; ++hh) {
      const float ph = (mh[hh] == NEG_INF || !live) ? 0.0f : fast_exp2(lh[hh] - mh[hh]);
      sums[hh] = wave_sum(ph);
      pb[tau][hh] = ph;
    }
    const float mysum = (j == 0) ? sums[0] : (j == 1) ? sums[1] : (j == 2) ? sums[2] : sums[3];
    lsum = lsum * alpha + (lane < 4 ? mysum : 0.0f);
    eta = eta * alpha;
    const f4 av = {quad_bcast<0>(alpha), quad_bcast<1>(alpha), quad_bcast<2>(alpha), quad_bcast<3>(alpha)};
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      o[hf] *= av;
      oo[hf] *= av;
    }
    if constexpr (VF == KVQ_INT2) {
#pragma unroll
      for (int g = 0; g < 4; ++g) zacc[g] *= alpha;
    }
    lds_wait();
    pv_orig(ch, vp, vr);
  };

  // ---------------------------------------------------------------- software-pipelined walk
  // The loads of the next chunk are in flight while the current one is computed
  // (two register sets used alternately).
  auto visit = [&](const ChunkRegs<KF, VF, vmeta_words(VF, VG)>& R, int ch, const ChunkAux<CERT>& X) {
    float ev_c = 0.0f;
    bool fl = false, fv = false;  // exact keys and values; exact values only
    if constexpr (EXACT) fl = in_window(ch);
    if constexpr (CERT) {
      const uint32_t f = a.flags != nullptr ? __builtin_amdgcn_readfirstlane(X.flag) : 0u;
      fl = fl || (f & 1u) != 0;
      fv = !fl && (f & 2u) != 0;
      if (a.desc != nullptr) {
        ev_c = fv ? 0.0f : X.ev;
        vnmax = fmaxf(vnmax, X.vn);
        if (!fl) ekmax = fmaxf(ekmax, X.ek);
      }
    }
    if (fl) {
      if constexpr (EXACT) exact_chunk(ch);
    } else {
      quant_chunk(R, ch, ev_c, fv);
    }
  };
  // Every iteration issues the same claims and loads (a load past the range's last chunk
  // reloads the current, valid chunk), so the number of memory operations in flight at
  // the loop head is the same on entry and on every iteration; the wave leaves as soon
  // as a claimed index is past the end.  (Claims only grow, so once one is past the end
  // the next is too: the loop leaves at its head, its single exit.)  Each chunk is claimed
  // right after the visit before it, so a wave holds at most one chunk beyond the one it
  // visits and the waves of a workgroup end closer together; a wave issues its loads at raised
  // priority, so that they leave before the other wave of its SIMD takes the issue slots.
  while (cA < c1) {
    const int cB = c0 + __builtin_amdgcn_readfirstlane(pB);
    __builtin_amdgcn_s_setprio(3);
    load_chunk<KF, KG, VF, VG>(a, stream, cB < c1 ? cB : cA, lane, tok_a, RB);
    load_aux(cB < c1 ? cB : cA, XB);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    visit(RA, cA, XA);
    const int pC = claim();
    const int cC = c0 + __builtin_amdgcn_readfirstlane(pC);
    __builtin_amdgcn_s_setprio(3);
    load_chunk<KF, KG, VF, VG>(a, stream, cC < c1 ? cC : cA, lane, tok_a, RA);
    load_aux(cC < c1 ? cC : cA, XA);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
    if (cB < c1) visit(RB, cB, XB);
    pB = claim();
    cA = cC;
  }

  // ---------------- per-wave totals, then merge the waves in LDS
  const float lt = sum_same_head(lsum);
  const float et = CERT ? sum_same_head(eta) : 0.0f;
  if constexpr (VF == KVQ_INT2) {
    float ztl[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) ztl[g] = sum_same_head(zacc[g]);
    if (lane < 4)
#pragma unroll
      for (int g = 0; g < 4; ++g) sm.zt[wv][lane][g] = ztl[g];
    __builtin_amdgcn_wave_barrier();
    lds_wait();
  }
  __syncthreads();  // every wave has left its loop: the merge area aliases the loop buffers
  MergeArea<NWS>& mg = sm.u.mrg;
  if (lane < 4) {
    mg.m[wv][lane] = m;
    mg.l[wv][lane] = lt;
    mg.e[wv][lane] = et;
  }
  if (lane == 0) {
    mg.ek[wv] = ekmax;
    mg.vn[wv] = vnmax;
  }
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    float zb = 0.0f;
    if constexpr (VF == KVQ_INT2) zb = sm.zt[wv][hh][vgrp];
    mg.o[wv][hh][2 * lane] = o[0][hh] + zb;
    mg.o[wv][hh][2 * lane + 1] = o[1][hh] + zb;
    if constexpr (EXACT) {
      mg.oo[wv][hh][2 * lane] = oo[0][hh];
      mg.oo[wv][hh][2 * lane + 1] = oo[1][hh];
    }
  }
  __syncthreads();
  if (wv < 4) write_record<EXACT, NWS, true>(a, mg, sm.qo, 0, NWS, b, hq0, nh, split, wv, lane);

  // ---------------- the last workgroup of the unit to finish merges its splits
  // The records are agent-coherent atomic stores; every thread waits for its own
  // stores to complete before the barrier, so they are performed before the
  // arrival is counted.  The last arrival reads every split's record with
  // agent-coherent loads.  (No cache write-back or invalidate is needed: only
  // the records cross workgroups, and they never sit in a non-coherent cache.)
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (t == 0) {
    KVQ_DCHECK(u >= 0 && u < a.U, DBG_COUNTER, u, split);
    const int prev = __hip_atomic_fetch_add(a.ctr + u, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    sm.last = prev == S - 1;
  }
  __syncthreads();
  if (sm.last) {
    if (wv < nh) {
      if (S <= 2)
        combine_row<EXACT, true, 2>(a, b * a.Hq + hq0 + wv, sm.u.zsw[wv], sm.ctab);
      else
        combine_row<EXACT, true, 8>(a, b * a.Hq + hq0 + wv, sm.u.zsw[wv], sm.ctab);
    }
    if (t == 0) __hip_atomic_store(a.ctr + u, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// ------------------------------------------------------------------ dense fp16 decode
// Decode over uncompressed fp16/bf16 K/V (layout of k_orig/v_orig, original basis): one
// workgroup of 4 waves per (sequence, kv head, group of 4 query heads, split), wave w
// taking the split's chunks w, w + 4, ...  Per chunk a wave issues all its loads at once
// (lane t: the key row of token t; lane l: channels 2l, 2l+1 of the 64 value rows), so
// a whole chunk is in flight per wave.  QK^T on fp16 MFMA with the query split into an
// fp16 high part and the fp16 rounding of the remainder (two products, fp32
// accumulation: the logits carry the fp32 query to about 2^-22), softmax in the exp2
// domain, PV in fp32 on the vector ALUs from the probabilities in LDS.  FB: the dense
// fallback, which skips the units none of whose rows needs recomputing.
// One (sequence b, kv head and query-head group y, split) of the fp16/bf16 decode.
template <bool FB>
__device__ __forceinline__ void dense_unit(const DecodeArgs& a, DenseSmem& sm, int b, int y, int split) {
  const int HG = (a.G + 3) >> 2;
  const int hkv = y / HG, hg = y % HG;
  const int hq0 = hkv * a.G + hg * 4;
  const int nh = min(4, a.G - hg * 4);
  if constexpr (FB) {
    bool any = false;
    for (int hh = 0; hh < nh; ++hh) any = any || fallback_row(a, (size_t)b * a.Hq + hq0 + hh);
    if (!any) return;  // uniform over the workgroup
  }
  const int T = a.seq.v[b];
  const int nchunks = (T + TILE - 1) / TILE;
  const int c0 = split * a.chunks_per_split;
  const int c1 = min(nchunks, c0 + a.chunks_per_split);
  const int t = threadIdx.x, wv = t >> 6, lane = t & 63;
  const int j = lane & 3;
  const size_t stream = (size_t)b * a.H + hkv;
  const bool bf16 = a.in_bf16 != 0;
  {
    const int hh = t >> 6, l = t & 63;
    float x0 = 0.0f, x1 = 0.0f;
    if (hh < nh) {
      const uint16_t* qp = a.q + ((size_t)b * a.Hq + hq0 + hh) * D;
      x0 = widen(qp[2 * l], bf16);
      x1 = widen(qp[2 * l + 1], bf16);
    }
    x0 *= a.scale * LOG2E;
    x1 *= a.scale * LOG2E;
    sm.qo[hh][2 * l] = x0;
    sm.qo[hh][2 * l + 1] = x1;
    // query operand of step n (channels 4n..4n+3): lane l builds half of step l / 2
    const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
    const _Float16 r0 = (_Float16)(x0 - (float)h0), r1 = (_Float16)(x1 - (float)h1);
    uint32_t* qw = reinterpret_cast<uint32_t*>(&sm.qhl[hh][l >> 1]);
    qw[l & 1] = as_u(h2{h0, h1});
    qw[2 + (l & 1)] = as_u(h2{r0, r1});
  }
  __syncthreads();
  float m = NEG_INF, lsum = 0.0f;
  f4 o[2] = {f4{0, 0, 0, 0}, f4{0, 0, 0, 0}};
  for (int ch = c0 + wv; ch < c1; ch += 4) {
    const int tok0 = ch * TILE;
    const int nlive = T - tok0;  // rows below the sequence end (>= 1)
    KVQ_DCHECK(stream < (size_t)a.B * a.H, DBG_STREAM, stream, ch);
    KVQ_DCHECK(ch >= 0 && ch < a.nt, DBG_CHUNK, stream, ch);
    const uint4* kp = reinterpret_cast<const uint4*>(a.k_orig + (stream * a.Tmax + tok0 + lane) * D);
    const uint32_t* vp = reinterpret_cast<const uint32_t*>(a.v_orig + (stream * a.Tmax + tok0) * D) + lane;
    uint4 kr[16];
    uint32_t vr[TILE];
#pragma unroll
    for (int i = 0; i < 16; ++i) kr[i] = kp[i];
#pragma unroll
    for (int tt = 0; tt < TILE; ++tt) vr[tt] = vp[(size_t)tt * (D / 2)];
    f4 acc = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint4 u = kr[i];
      h4 k0, k1;
      if (bf16) {
        const uint32_t w[4] = {u.x, u.y, u.z, u.w};
        float f[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          f[2 * e] = __uint_as_float(w[e] << 16);
          f[2 * e + 1] = __uint_as_float(w[e] & 0xFFFF0000u);
        }
        k0 = h4{(_Float16)f[0], (_Float16)f[1], (_Float16)f[2], (_Float16)f[3]};
        k1 = h4{(_Float16)f[4], (_Float16)f[5], (_Float16)f[6], (_Float16)f[7]};
      } else {
        k0 = __builtin_bit_cast(h4, make_uint2(u.x, u.y));
        k1 = __builtin_bit_cast(h4, make_uint2(u.z, u.w));
      }
      const uint4 q0 = sm.qhl[j][2 * i], q1 = sm.qhl[j][2 * i + 1];
      acc = __builtin_amdgcn_mfma_f32_4x4x4f16(k0, __builtin_bit_cast(h4, make_uint2(q0.x, q0.y)), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_4x4x4f16(k0, __builtin_bit_cast(h4, make_uint2(q0.z, q0.w)), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_4x4x4f16(k1, __builtin_bit_cast(h4, make_uint2(q1.x, q1.y)), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_4x4x4f16(k1, __builtin_bit_cast(h4, make_uint2(q1.z, q1.w)), acc, 0, 0, 0);
    }
    float l[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) l[r] = (4 * (lane >> 2) + r < nlive) ? acc[r] : NEG_INF;
    float cmax = max_same_head(fmaxf(fmaxf(l[0], l[1]), fmaxf(l[2], l[3])));
    const float m_new = fmaxf(m, cmax);
    const float alpha = (m_new == NEG_INF) ? 1.0f : exp2f(m - m_new);
    float p[4], ps = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      p[r] = (m_new == NEG_INF) ? 0.0f : exp2f(l[r] - m_new);
      ps += p[r];
    }
    lsum = lsum * alpha + ps;
    m = m_new;
    const f4 av = {quad_bcast<0>(alpha), quad_bcast<1>(alpha), quad_bcast<2>(alpha), quad_bcast<3>(alpha)};
    o[0] *= av;
    o[1] *= av;
#pragma unroll
    for (int r = 0; r < 4; ++r) sm.pb[wv][4 * (lane >> 2) + r][j] = p[r];
    lds_wait();
#pragma unroll
    for (int tt = 0; tt < TILE; ++tt) {
      // rows at or past the sequence end count as zeros (weight 0, whatever bits they hold)
      const uint32_t vv = tt < nlive ? vr[tt] : 0u;
      const float v0 = widen((uint16_t)(vv & 0xFFFF), bf16), v1 = widen((uint16_t)(vv >> 16), bf16);
      const float4 pp = *reinterpret_cast<const float4*>(&sm.pb[wv][tt][0]);
      o[0] += f4{pp.x, pp.y, pp.z, pp.w} * v0;
      o[1] += f4{pp.x, pp.y, pp.z, pp.w} * v1;
    }
    lds_wait();
  }
  const float lt = sum_same_head(lsum);
  if (lane < 4) {
    sm.mrg.m[wv][lane] = m;
    sm.mrg.l[wv][lane] = lt;
    sm.mrg.e[wv][lane] = 0.0f;
  }
  if (lane == 0) {
    sm.mrg.ek[wv] = 0.0f;
    sm.mrg.vn[wv] = 0.0f;
  }
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    sm.mrg.o[wv][hh][2 * lane] = o[0][hh];
    sm.mrg.o[wv][hh][2 * lane + 1] = o[1][hh];
  }
  __syncthreads();
  write_record<false, 4, false>(a, sm.mrg, sm.qo, 0, 4, b, hq0, nh, split, wv, lane);
}

// The same-shape baseline: one workgroup per (split, kv head and query-head group,
// sequence).  The dense fallback (FB): a persistent grid over the (unit, split) pairs of
// the units with a row to recompute, listed by every workgroup in the same order from the
// rows' certificates and check results (units are few there, and workgroups of units
// without such a row would only be dispatched to leave); units beyond the list's room
// take the unlisted form, each workgroup walking all pairs and skipping the idle units.
template <bool FB>
__global__ __launch_bounds__(NT, 2) void decode_dense_split(DecodeArgs a) {
  __shared__ DenseSmem sm;
  if constexpr (!FB) {
    dense_unit<false>(a, sm, blockIdx.z, blockIdx.y, blockIdx.x);
  } else {
    const int HG = (a.G + 3) >> 2, S = a.n_splits;
    const int U = a.B * a.H * HG;
    constexpr int CAP = (int)(sizeof(sm.pad) / sizeof(int));
    static_assert(CAP / NT <= 64, "one 64-bit mask of active units per thread");
    int* list = reinterpret_cast<int*>(sm.pad);
    __shared__ int cnt[NT / 64];
    int nitems;
    if (U <= CAP) {
      // thread t takes units t, t + NT, ...: count, exclusive scan over the threads, write
      const int t = threadIdx.x;
      auto active = [&](int u) {
        const int b = u / (a.H * HG), y = u % (a.H * HG);
        const int hq0 = (y / HG) * a.G + (y % HG) * 4, nh = min(4, a.G - (y % HG) * 4);
        bool any = false;
        for (int hh = 0; hh < nh; ++hh) any = any || fallback_row(a, (size_t)b * a.Hq + hq0 + hh);
        return any;
      };
      uint64_t bits = 0;  // unit t + NT k active (k < CAP / NT = 52)
      for (int u = t, k = 0; u < U; u += NT, ++k)
        if (active(u)) bits |= 1ull << k;
      const int mine = __builtin_popcountll(bits);
      // exclusive scan of the counts: inclusive within each wave by shuffles, then the
      // totals of the waves before
      const int wl = t & 63, ww = t >> 6;
      int incl = mine;
      for (int o = 1; o < 64; o <<= 1) {
        const int v = __shfl_up(incl, o);
        if (wl >= o) incl += v;
      }
      if (wl == 63) cnt[ww] = incl;
      __syncthreads();
      int base = 0;
      for (int w = 0; w < ww; ++w) base += cnt[w];
      if (t == NT - 1) sm.nlist = base + incl;
      int pos = base + incl - mine;
      for (int u = t, k = 0; u < U; u += NT, ++k)
        if ((bits >> k) & 1ull) list[pos++] = u;
      __syncthreads();
      nitems = sm.nlist * S;
    } else {
      nitems = U * S;
    }
    for (int it = blockIdx.x; it < nitems; it += gridDim.x) {
      const int u = U <= CAP ? list[it / S] : it / S;
      dense_unit<true>(a, sm, u / (a.H * HG), u % (a.H * HG), it % S);
      __syncthreads();  // the next pair reuses the shared areas
    }
  }
}

// ------------------------------------------------------------------ allocation-free workspace
// A fixed device array that serves as the decode workspace of kvq_decode_attn_noalloc:
// arrival counters in its first SCRATCH_CTR_BYTES (only ever written as counters, so
// every completed call leaves all of them zero, whatever the shapes of the calls),
// split records after them.  Every device holds its own copy, at its own address.
static __device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

__global__ __launch_bounds__(256) void zero_words(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

}  // namespace

// Device address of this device's scratch array (the array's name is only a host-side
// stand-in).  Looked up once per device, with that device current; the first lookup also
// clears the counter region with a fill kernel on the caller's stream (no memset: the
// call may be under graph capture).
hipError_t decode_scratch(void** ptr, hipStream_t s) {
  static std::mutex mu;
  static void* addr[MAX_DEVICES] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    hipLaunchKernelGGL(zero_words, dim3(16), dim3(256), 0, s, static_cast<uint32_t*>(p),
                       (int)(SCRATCH_CTR_BYTES / sizeof(uint32_t)));
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_decode(const DecodeArgs& a, int k_fmt, int v_fmt, bool dense, hipStream_t s) {
  const int HG = (a.G + 3) / 4;
  const dim3 cgrid((a.B * a.Hq + 3) / 4);
  if (dense) {
    const dim3 dgrid(a.n_splits, a.H * HG, a.B);
    hipLaunchKernelGGL(decode_dense_split<false>, dgrid, dim3(NT), 0, s, a);
    hipLaunchKernelGGL(combine_kernel<false>, cgrid, dim3(NT), 0, s, a);
    return hipGetLastError();
  }
  // the exact-recompute instantiation serves the certified cache and the window
  // 2: certified cache; 1: full-precision window only; 0: codes only.  (With 8-bit
  // keys the window-only variant would need more than 256 registers per lane, so
  // those caches take the certified variant, whose flag and descriptor loads then
  // read a stand-in address and are ignored.)
  const int mode = a.desc != nullptr ? 2 : (a.k_win != nullptr ? (k_fmt == KVQ_INT8 ? 2 : 1) : 0);
  // one workgroup per (unit, split), the splits of a unit consecutive
  const dim3 grid(a.U * a.n_splits);
#define KVQ_LAUNCH(KF, KG, VF, VG)                                                            \
  if (k_fmt == KF && a.k_group == KG && v_fmt == VF && a.v_group == VG) {                     \
    if (mode == 2) {                                                                          \
      hipLaunchKernelGGL((decode_split<KF, KG, VF, VG, 2>), grid, dim3(NTS), 0, s, a);        \
    } else if (mode == 1) {                                                                   \
      if constexpr (KF != KVQ_INT8)                                                           \
        hipLaunchKernelGGL((decode_split<KF, KG, VF, VG, 1>), grid, dim3(NTS), 0, s, a);      \
    } else {                                                                                  \
      hipLaunchKernelGGL((decode_split<KF, KG, VF, VG, 0>), grid, dim3(NTS), 0, s, a);        \
    }                                                                                         \
    return hipGetLastError();                                                                 \
  }
  KVQ_LAUNCH(KVQ_INT4, 32, KVQ_INT4, 32)
  KVQ_LAUNCH(KVQ_INT4, 16, KVQ_INT4, 16)
  KVQ_LAUNCH(KVQ_INT4, 128, KVQ_INT4, 128)
  KVQ_LAUNCH(KVQ_INT4, 32, KVQ_INT4, 128)
  KVQ_LAUNCH(KVQ_INT4, 128, KVQ_INT4, 32)
  KVQ_LAUNCH(KVQ_INT8, 128, KVQ_INT4, 128)
  KVQ_LAUNCH(KVQ_INT8, 128, KVQ_INT4, 32)
  KVQ_LAUNCH(KVQ_INT8, 32, KVQ_INT4, 32)
  KVQ_LAUNCH(KVQ_INT8, 32, KVQ_INT4, 128)
  KVQ_LAUNCH(KVQ_INT2, 32, KVQ_INT2, 32)
  KVQ_LAUNCH(KVQ_FP4, 16, KVQ_FP4, 16)
#undef KVQ_LAUNCH
  return hipErrorNotSupported;
}


// The dense fallback: the fp16/bf16 decode over the cache's originals, restricted to the
// units holding a row to recompute (the others leave at once), then the combine of those
// rows only.
hipError_t launch_dense_fallback(const DecodeArgs& a, hipStream_t s) {
  const int HG = (a.G + 3) / 4;
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, decode_dense_split<true>, NT, 0) != hipSuccess || per_cu <= 0)
    per_cu = 1;
  const long pairs = (long)a.n_splits * a.H * HG * a.B;
  const int grid = (int)std::min<long>(pairs, (long)cus * per_cu);
  hipLaunchKernelGGL(decode_dense_split<true>, dim3(grid), dim3(NT), 0, s, a);
  hipLaunchKernelGGL(combine_kernel<true>, dim3((a.B * a.Hq + 3) / 4), dim3(NT), 0, s, a);
  return hipGetLastError();
}

#ifdef KVQ_DEBUG
KVQ_DBG_READER(dbg_read_decode)
#endif

}  // namespace kvq
