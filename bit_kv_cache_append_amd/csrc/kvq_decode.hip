// Read side: single-token decode attention over the packed cache.
//
// Split kernel: one workgroup (4 waves) per (context split, kv head, group of 4
// query heads, sequence).  Each wave walks 64-token chunks of its split (the
// chunk is also the V tile and the descriptor block).  Per chunk:
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
// Combine kernel: log-sum-exp merge of the splits, inverse rotation back to the
// original basis ("OSCAR", section 2.2B), certificate.

#include "kvq_common.h"

namespace kvq {

namespace {

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef _Float16 h4 __attribute__((ext_vector_type(4)));
typedef float f4 __attribute__((ext_vector_type(4)));
typedef int i4 __attribute__((ext_vector_type(4)));

constexpr int NT = 256;
constexpr float LOG2E = 1.4426950408889634f;
constexpr float NEG_INF = -__builtin_huge_valf();

__device__ __forceinline__ h2 as_h2(uint32_t u) { return __builtin_bit_cast(h2, u); }
__device__ __forceinline__ uint32_t as_u(h2 v) { return __builtin_bit_cast(uint32_t, v); }
__device__ __forceinline__ h4 cat(h2 a, h2 b) { return h4{a.x, a.y, b.x, b.y}; }

// ------------------------------------------------------------------ token order
// QK slice s (lanes 4s..4s+3) covers tokens pi(s, 0..3) of the chunk.
template <int VF>
__device__ __forceinline__ int tok_of(int s, int r) {
  if constexpr (VF == KVQ_INT2) return 16 * (s >> 2) + 2 * (s & 3) + ((r & 1) << 3) + (r >> 1);
  return 8 * (s >> 1) + 2 * (s & 1) + ((r & 1) << 2) + (r >> 1);
}
// inverse: token tau -> position 4s + r
template <int VF>
__device__ __forceinline__ int pos_of(int tau) {
  if constexpr (VF == KVQ_INT2) {
    const int w = tau >> 4, e = tau & 15, rem = e & 7;
    const int s = 4 * w + (rem >> 1), r = ((e >> 3) & 1) | ((rem & 1) << 1);
    return 4 * s + r;
  } else {
    const int d = tau >> 3, e = tau & 7;
    const int s = 2 * d + ((e >> 1) & 1), r = ((e >> 2) & 1) | ((e & 1) << 1);
    return 4 * s + r;
  }
}

// ------------------------------------------------------------------ K formats
template <int KF>
struct KFmt;
template <>
struct KFmt<KVQ_INT4> {
  static constexpr int DW = 16;  // dwords per row
  static constexpr int MDW = 2;  // metadata dwords per token (g32: 4 fp16); g128 uses 1 fp16
  __device__ static __forceinline__ int a_op(const uint32_t* row, int n) {
    uint32_t t = row[n >> 1] ^ 0x88888888u;
    return (int)((n & 1) ? ((t >> 4) & 0x0F0F0F0Fu) : (t & 0x0F0F0F0Fu));
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
__device__ __forceinline__ void v_int4_pairs(uint32_t w, h2 out[4]) {
  const uint32_t t = w ^ 0x88888888u;
  const uint32_t t8 = t >> 8;
  const h2 k1032 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const h2 k16 = {(_Float16)0.0625f, (_Float16)0.0625f};
  const h2 k72 = {(_Float16)-72.0f, (_Float16)-72.0f};
  out[0] = as_h2((t & 0x000F000Fu) | 0x64006400u) + k1032;                     // tokens 0, 4
  out[1] = as_h2((t & 0x00F000F0u) | 0x64006400u) * k16 + k72;                 // tokens 1, 5
  out[2] = as_h2((t8 & 0x000F000Fu) | 0x64006400u) + k1032;                    // tokens 2, 6
  out[3] = as_h2((t8 & 0x00F000F0u) | 0x64006400u) * k16 + k72;                // tokens 3, 7
}
// int2: element k and k+8 of a 16-token dword, codes 0..3
__device__ __forceinline__ void v_int2_pairs(uint32_t w, h2 out[8]) {
  const uint32_t magic = 0x64006400u;
  const uint32_t w10 = w >> 10;
  out[0] = as_h2((w & 0x00030003u) | magic) + h2{(_Float16)-1024.0f, (_Float16)-1024.0f};
  out[1] = as_h2((w & 0x000C000Cu) | magic) * h2{(_Float16)0.25f, (_Float16)0.25f} + h2{(_Float16)-256.0f, (_Float16)-256.0f};
  out[2] = as_h2((w & 0x00300030u) | magic) * h2{(_Float16)0.0625f, (_Float16)0.0625f} + h2{(_Float16)-64.0f, (_Float16)-64.0f};
  out[3] = as_h2((w & 0x00C000C0u) | magic) * h2{(_Float16)0.015625f, (_Float16)0.015625f} + h2{(_Float16)-16.0f, (_Float16)-16.0f};
  out[4] = as_h2((w & 0x03000300u) | magic) * h2{(_Float16)0.00390625f, (_Float16)0.00390625f} + h2{(_Float16)-4.0f, (_Float16)-4.0f};
  out[5] = as_h2((w10 & 0x00030003u) | magic) + h2{(_Float16)-1024.0f, (_Float16)-1024.0f};
  out[6] = as_h2((w10 & 0x000C000Cu) | magic) * h2{(_Float16)0.25f, (_Float16)0.25f} + h2{(_Float16)-256.0f, (_Float16)-256.0f};
  out[7] = as_h2((w10 & 0x00300030u) | magic) * h2{(_Float16)0.0625f, (_Float16)0.0625f} + h2{(_Float16)-64.0f, (_Float16)-64.0f};
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

// ------------------------------------------------------------------ reductions
__device__ __forceinline__ float max_same_head(float v) {  // over lanes with equal (lane & 3)
  v = fmaxf(v, __shfl_xor(v, 4));
  v = fmaxf(v, __shfl_xor(v, 8));
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}
__device__ __forceinline__ float sum_same_head(float v) {
  v += __shfl_xor(v, 4);
  v += __shfl_xor(v, 8);
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
  for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
  return v;
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

struct __align__(16) DecodeSmem {
  float qf[4][D];          // query (fp32), rotated in place
  float qr[4][D];          // dense rotation output
  float qo[4][D];          // original query * scale * log2e (certified recompute)
  uint32_t qh[4][32];      // high int8 halves, MFMA operand order
  uint32_t ql[4][32];      // low int8 halves
  float qs[4];             // per-head dequantization of the 16-bit query
  float qsum[4][4];        // per head, per group: sum of 16-bit query codes
  uint16_t vmeta[4][8][16][4];  // per wave: V metadata by (element, slice, r)
  float pb[4][TILE][4];    // per wave: probabilities by token (certified recompute)
  float mrg_m[4][4], mrg_l[4][4], mrg_e[4][4];
  float mrg_ek[4], mrg_vn[4];
  float mrg_o[4][4][D];    // per wave, head, channel
  float mrg_oo[4][4][D];
  int is_last;
};

// ------------------------------------------------------------------ prologue
// rotate the 4 query heads of this workgroup, prescale, quantize to 16 bits
template <int KF>
__device__ void query_prologue(const DecodeArgs& a, DecodeSmem& sm, int b, int hq0, int nh, int kgroup) {
  const int t = threadIdx.x, j = t >> 6, l = t & 63;
  const bool bf16 = a.in_bf16 != 0;
  float x0 = 0.0f, x1 = 0.0f;
  if (j < nh) {
    const uint16_t* qp = a.q + ((size_t)b * a.Hq + hq0 + j) * D;
    x0 = widen(qp[2 * l], bf16);
    x1 = widen(qp[2 * l + 1], bf16);
  }
  const float pre = a.scale * LOG2E;
  sm.qo[j][2 * l] = x0 * pre;
  sm.qo[j][2 * l + 1] = x1 * pre;
  if (a.rotation == KVQ_ROT_SIGN_FWHT) {
    x0 = a.signs[2 * l] < 0 ? -x0 : x0;
    x1 = a.signs[2 * l + 1] < 0 ? -x1 : x1;
  }
  sm.qf[j][2 * l] = x0;
  sm.qf[j][2 * l + 1] = x1;
  __syncthreads();
  if (a.rotation == KVQ_ROT_SIGN_FWHT) {
    for (int h = 1; h < D; h <<= 1) {
      const int i = (l / h) * 2 * h + (l % h);
      float u = sm.qf[j][i], v = sm.qf[j][i + h];
      __syncthreads();
      sm.qf[j][i] = u + v;
      sm.qf[j][i + h] = u - v;
      __syncthreads();
    }
  } else if (a.rotation == KVQ_ROT_DENSE) {
    for (int rr = 0; rr < 2; ++rr) {
      const int row = l + 64 * rr;
      const uint16_t* rp = a.rot + (size_t)row * D;
      float acc = 0.0f;
      for (int k = 0; k < D; ++k) acc = fmaf(f16_bits_to_f32(rp[k]), sm.qf[j][k], acc);
      sm.qr[j][row] = acc;
    }
    __syncthreads();
    sm.qf[j][2 * l] = sm.qr[j][2 * l];
    sm.qf[j][2 * l + 1] = sm.qr[j][2 * l + 1];
    __syncthreads();
  }
  const float norm = a.rotation == KVQ_ROT_SIGN_FWHT ? bits_to_f32(KVQ_INV_SQRT_D_BITS) : 1.0f;
  float y0 = sm.qf[j][2 * l] * norm * pre, y1 = sm.qf[j][2 * l + 1] * norm * pre;
  float mx = wave_max(fmaxf(fabsf(y0), fabsf(y1)));
  const float qs = mx > 0.0f ? mx / 32000.0f : 1.0f;
  const int q0 = (int)rintf(y0 / qs), q1 = (int)rintf(y1 / qs);
  // scatter int8 halves into MFMA operand order
  uint8_t* hb = reinterpret_cast<uint8_t*>(&sm.qh[j][0]);
  uint8_t* lb = reinterpret_cast<uint8_t*>(&sm.ql[j][0]);
  const int qv[2] = {q0, q1};
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int c = 2 * l + e;
    const int hi = (qv[e] + 128) >> 8;
    const int lo = qv[e] - 256 * hi;
    const int sl = KFmt<KF>::slot(c);
    hb[sl] = (uint8_t)(hi & 0xFF);
    lb[sl] = (uint8_t)(lo & 0xFF);
  }
  // per-group sums of the 16-bit codes (groups of 32 channels = 16 lanes)
  float gs = (float)(q0 + q1);
  gs += __shfl_xor(gs, 1);
  gs += __shfl_xor(gs, 2);
  gs += __shfl_xor(gs, 4);
  gs += __shfl_xor(gs, 8);
  if (kgroup == 128) {
    gs += __shfl_xor(gs, 16);
    gs += __shfl_xor(gs, 32);
  }
  if ((l & 15) == 0) sm.qsum[j][l >> 4] = gs;
  if (l == 0) sm.qs[j] = qs;
  __syncthreads();
}

// ------------------------------------------------------------------ split merge
// Writes this workgroup's record (per head: running max, sum, value-error mass,
// descriptor maxima, unnormalised accumulators); the last workgroup to arrive for
// its (sequence, kv head, head group) merges every split with log-sum-exp weights,
// rotates the result back to the original basis ("OSCAR", section 2.2B: inverse
// rotation) and writes the output and the certificate.  The arrival counters live
// in the caller's workspace and are reset to zero by that last workgroup.
template <bool CERT>
__device__ void finish(const DecodeArgs& a, DecodeSmem& sm, int b, int hq0, int nh, int split) {
  const int t = threadIdx.x, hh = t >> 6, l = t & 63, c = 2 * l;
  if (hh < nh) {
    float M = NEG_INF;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, sm.mrg_m[w][hh]);
    float wgt[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) wgt[w] = (M == NEG_INF) ? 0.0f : exp2f(sm.mrg_m[w][hh] - M);
    float* rec = a.part + (((size_t)b * a.Hq + hq0 + hh) * a.n_splits + split) * PART_FLOATS;
    float o0 = 0.0f, o1 = 0.0f, p0 = 0.0f, p1 = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      o0 += wgt[w] * sm.mrg_o[w][hh][c];
      o1 += wgt[w] * sm.mrg_o[w][hh][c + 1];
      if constexpr (CERT) {
        p0 += wgt[w] * sm.mrg_oo[w][hh][c];
        p1 += wgt[w] * sm.mrg_oo[w][hh][c + 1];
      }
    }
    rec[8 + c] = o0;
    rec[8 + c + 1] = o1;
    if constexpr (CERT) {
      rec[8 + D + c] = p0;
      rec[8 + D + c + 1] = p1;
    }
    if (l == 0) {
      float L = 0.0f, E = 0.0f, ek = 0.0f, vn = 0.0f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        L += wgt[w] * sm.mrg_l[w][hh];
        E += wgt[w] * sm.mrg_e[w][hh];
        ek = fmaxf(ek, sm.mrg_ek[w]);
        vn = fmaxf(vn, sm.mrg_vn[w]);
      }
      rec[0] = M;
      rec[1] = L;
      rec[2] = E;
      rec[3] = ek;
      rec[4] = vn;
    }
  }
  __threadfence();
  __syncthreads();
  if (t == 0) {
    unsigned int* ctr = a.counters + ((size_t)b * gridDim.y + blockIdx.y);
    const unsigned int old = atomicAdd(ctr, 1u);
    const bool last = old == (unsigned int)(a.n_splits - 1);
    if (last) *ctr = 0u;
    sm.is_last = last ? 1 : 0;
  }
  __syncthreads();
  if (!sm.is_last) return;
  __threadfence();
  if (hh >= nh) return;  // whole waves: no barrier below
  const int hq = hq0 + hh;
  const size_t row = (size_t)b * a.Hq + hq;
  float* out = a.out + row * D;
  if (a.seq.v[b] == 0) {
    out[c] = 0.0f;
    out[c + 1] = 0.0f;
    if (a.cert && l == 0) a.cert[row] = 0.0f;
    return;
  }
  const float* rec0 = a.part + row * a.n_splits * PART_FLOATS;
  float M = NEG_INF;
  for (int s = 0; s < a.n_splits; ++s) M = fmaxf(M, rec0[s * PART_FLOATS]);
  float L = 0.0f, E = 0.0f, ek = 0.0f, vn = 0.0f, o0 = 0.0f, o1 = 0.0f, p0 = 0.0f, p1 = 0.0f;
  for (int s = 0; s < a.n_splits; ++s) {
    const float* rec = rec0 + s * PART_FLOATS;
    const float w = (rec[0] == NEG_INF) ? 0.0f : exp2f(rec[0] - M);
    L += w * rec[1];
    E += w * rec[2];
    ek = fmaxf(ek, rec[3]);
    vn = fmaxf(vn, rec[4]);
    const float2 ov = *reinterpret_cast<const float2*>(rec + 8 + c);
    o0 += w * ov.x;
    o1 += w * ov.y;
    if constexpr (CERT) {
      const float2 pv = *reinterpret_cast<const float2*>(rec + 8 + D + c);
      p0 += w * pv.x;
      p1 += w * pv.y;
    }
  }
  const float inv = 1.0f / L;
  o0 *= inv;
  o1 *= inv;
  float r0 = o0, r1 = o1;
  if (a.rotation == KVQ_ROT_SIGN_FWHT) {
    // R^T o = diag(s) H o / sqrt(128): the butterflies over this head's 64 lanes
    r0 = o0 + o1;
    r1 = o0 - o1;
    for (int msk = 1; msk < 64; msk <<= 1) {
      const float q0 = __shfl_xor(r0, msk), q1 = __shfl_xor(r1, msk);
      const bool up = (l & msk) != 0;
      r0 = up ? q0 - r0 : r0 + q0;
      r1 = up ? q1 - r1 : r1 + q1;
    }
    const float cn = bits_to_f32(KVQ_INV_SQRT_D_BITS);
    r0 *= a.signs[c] < 0 ? -cn : cn;
    r1 *= a.signs[c + 1] < 0 ? -cn : cn;
  } else if (a.rotation == KVQ_ROT_DENSE) {
    sm.qr[hh][c] = o0;
    sm.qr[hh][c + 1] = o1;
    lds_wait();
    float acc0 = 0.0f, acc1 = 0.0f;
    for (int k = 0; k < D; ++k) {
      const float z = sm.qr[hh][k];
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
  if (CERT && a.cert) {
    // ||q||: the prologue kept q * scale * log2(e) in LDS
    const float q0 = sm.qo[hh][c], q1 = sm.qo[hh][c + 1];
    float sq = q0 * q0 + q1 * q1;
    for (int off = 32; off > 0; off >>= 1) sq += __shfl_xor(sq, off);
    if (l == 0) {
      const float qn = sqrtf(sq) / LOG2E;  // = ||q|| * scale
      const float dstar = qn * ek;
      a.cert[row] = 2.0f * (1.0f - expf(-2.0f * dstar)) * vn + E * inv;
    }
  }
}

// ------------------------------------------------------------------ split kernel
template <int KF, int KG, int VF, bool CERT>
__global__ __launch_bounds__(NT, 2) void decode_split(DecodeArgs a) {
  __shared__ DecodeSmem sm;
  const int b = blockIdx.z;
  const int HG = (a.G + 3) >> 2;
  const int hkv = blockIdx.y / HG, hg = blockIdx.y % HG;
  const int hq0 = hkv * a.G + hg * 4;
  const int nh = min(4, a.G - hg * 4);
  const int split = blockIdx.x;
  const int T = a.seq.v[b];
  const int nchunks = (T + TILE - 1) / TILE;
  const int c0 = split * a.chunks_per_split;
  const int c1 = min(nchunks, c0 + a.chunks_per_split);
  const int t = threadIdx.x, wv = t >> 6, lane = t & 63;
  const int j = lane & 3;       // head of this lane (QK output / softmax role)
  const int s_a = lane >> 2;    // QK slice of this lane (A role)
  const int r_a = lane & 3;
  const size_t stream = (size_t)b * a.H + hkv;
  constexpr int KDW = KFmt<KF>::DW;
  constexpr int KM = meta_bytes(KF, KG);
  const int vg = a.v_group;
  const int vgrp = (vg == 128) ? 0 : (lane >> 4);  // V group of channels 2*lane, 2*lane+1

  query_prologue<KF>(a, sm, b, hq0, nh, KG);

  uint32_t qh[32], ql[32];
#pragma unroll
  for (int n = 0; n < 32; ++n) {
    qh[n] = sm.qh[j][n];
    ql[n] = sm.ql[j][n];
  }
  const float qs = sm.qs[j];
  float qsum[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) qsum[g] = sm.qsum[j][g];

  float m = NEG_INF, lsum = 0.0f, eta = 0.0f, ekmax = 0.0f, vnmax = 0.0f;
  f4 o[2], oo[2], oz;
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    o[hf] = f4{0, 0, 0, 0};
    oo[hf] = f4{0, 0, 0, 0};
  }
  oz = f4{0, 0, 0, 0};

  for (int ch = c0 + wv; ch < c1; ch += 4) {
    const int tok0 = ch * TILE;
    bool flagged = false;
    float ev_c = 0.0f;
    if constexpr (CERT) {
      const float* dsc = a.desc + (stream * a.nt + ch) * 3;
      const float ek_c = dsc[0];
      ev_c = dsc[1];
      vnmax = fmaxf(vnmax, dsc[2]);
      flagged = a.flags != nullptr && a.flags[stream * a.nt + ch] != 0;
      if (!flagged) ekmax = fmaxf(ekmax, ek_c);
    }
    float p[4];
    float alpha;
    if (!flagged) {
      // ---------------- K: row of token pi(s_a, r_a) and its metadata
      const int tok_a = tok_of<VF>(s_a, r_a);
      uint32_t row[KDW];
      {
        const uint4* rp = reinterpret_cast<const uint4*>(a.k_codes + (stream * a.Tmax + tok0 + tok_a) * (KDW * 4));
#pragma unroll
        for (int i = 0; i < KDW / 4; ++i) {
          uint4 u = rp[i];
          row[4 * i] = u.x; row[4 * i + 1] = u.y; row[4 * i + 2] = u.z; row[4 * i + 3] = u.w;
        }
      }
      uint32_t mt[4] = {0, 0, 0, 0};
      {
        const uint8_t* mp = a.k_meta + (stream * a.Tmax + tok0 + tok_a) * KM;
        if constexpr (KM == 16) {
          uint4 u = *reinterpret_cast<const uint4*>(mp);
          mt[0] = u.x; mt[1] = u.y; mt[2] = u.z; mt[3] = u.w;
        } else if constexpr (KM == 8) {
          uint2 u = *reinterpret_cast<const uint2*>(mp);
          mt[0] = u.x; mt[1] = u.y;
        } else {
          mt[0] = *reinterpret_cast<const uint16_t*>(mp);
        }
      }
      // ---------------- V: channels 2*lane, 2*lane+1 of this tile
      constexpr int CDW = VFmt<VF>::CDW;
      uint32_t vw[2 * CDW];
      {
        const uint4* vp = reinterpret_cast<const uint4*>(a.v_codes + (stream * a.nt + ch) * (size_t)(D * CDW * 4) +
                                                         (size_t)(2 * lane) * CDW * 4);
#pragma unroll
        for (int i = 0; i < CDW / 2; ++i) {
          uint4 u = vp[i];
          vw[4 * i] = u.x; vw[4 * i + 1] = u.y; vw[4 * i + 2] = u.z; vw[4 * i + 3] = u.w;
        }
      }
      // V metadata tile -> LDS, ordered by (element, slice, r)
      {
        const int NM = meta_elems(VF, vg);
        const uint16_t* vm = reinterpret_cast<const uint16_t*>(a.v_meta + (stream * a.nt + ch) * (size_t)(NM * TILE * 2));
        for (int e = lane; e < NM * TILE; e += 64) {
          const int mm = e >> 6, tau = e & 63;
          const int ps = pos_of<VF>(tau);
          sm.vmeta[wv][mm][ps >> 2][ps & 3] = vm[e];
        }
      }
      // ---------------- QK^T: exact integer group dot products
      float l[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      constexpr int NG = (KG == 128) ? 1 : 4;
      constexpr int PER = 32 / NG;
#pragma unroll
      for (int g = 0; g < NG; ++g) {
        i4 acc = {0, 0, 0, 0};
#pragma unroll
        for (int n = g * PER; n < (g + 1) * PER; ++n)
          acc = __builtin_amdgcn_mfma_i32_4x4x4i8(KFmt<KF>::a_op(row, n), (int)qh[n], acc, 0, 0, 0);
        int corr = 0;
        if constexpr (KF == KVQ_INT4) corr = -8 * (int)qsum[g];
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[r] = acc[r] * 256 + corr;
#pragma unroll
        for (int n = g * PER; n < (g + 1) * PER; ++n)
          acc = __builtin_amdgcn_mfma_i32_4x4x4i8(KFmt<KF>::a_op(row, n), (int)ql[n], acc, 0, 0, 0);
        // scales of tokens pi(s, r): held by lanes 4s + r (A role); gather within the quad
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          uint32_t sw, zw = 0;
          const int widx = (KF == KVQ_INT2) ? (g >> 1) : (g >> 1);
          uint32_t src = mt[widx];
          uint32_t srcz = (KF == KVQ_INT2) ? mt[2 + (g >> 1)] : 0u;
          if (r == 0) { sw = quad_bcast_u<0>(src); if (KF == KVQ_INT2) zw = quad_bcast_u<0>(srcz); }
          else if (r == 1) { sw = quad_bcast_u<1>(src); if (KF == KVQ_INT2) zw = quad_bcast_u<1>(srcz); }
          else if (r == 2) { sw = quad_bcast_u<2>(src); if (KF == KVQ_INT2) zw = quad_bcast_u<2>(srcz); }
          else { sw = quad_bcast_u<3>(src); if (KF == KVQ_INT2) zw = quad_bcast_u<3>(srcz); }
          const uint16_t sb = (g & 1) ? (uint16_t)(sw >> 16) : (uint16_t)(sw & 0xFFFF);
          float v = (float)acc[r] * f16_bits_to_f32(sb);
          if constexpr (KF == KVQ_INT2) {
            const uint16_t zb = (g & 1) ? (uint16_t)(zw >> 16) : (uint16_t)(zw & 0xFFFF);
            v = fmaf(f16_bits_to_f32(zb), qsum[g], v);
          }
          l[r] += v;
        }
      }
      // mask tokens past the sequence end
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        l[r] *= qs;
        if (tok0 + tok_of<VF>(s_a, r) >= T) l[r] = NEG_INF;
      }
      // ---------------- online softmax
      float cmax = fmaxf(fmaxf(l[0], l[1]), fmaxf(l[2], l[3]));
      cmax = max_same_head(cmax);
      const float m_new = fmaxf(m, cmax);
      alpha = (m_new == NEG_INF) ? 1.0f : exp2f(m - m_new);
      float ps = 0.0f;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        p[r] = (m_new == NEG_INF) ? 0.0f : exp2f(l[r] - m_new);
        ps += p[r];
      }
      lsum = lsum * alpha + ps;
      if constexpr (CERT) eta = eta * alpha + ps * ev_c;
      m = m_new;
      // rescale accumulators (row h of the PV output needs head h's alpha)
      const float a0 = quad_bcast<0>(alpha), a1 = quad_bcast<1>(alpha), a2 = quad_bcast<2>(alpha),
                  a3 = quad_bcast<3>(alpha);
      const f4 av = {a0, a1, a2, a3};
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        o[hf] *= av;
        if constexpr (CERT) oo[hf] *= av;
      }
      if constexpr (VF == KVQ_INT2) oz *= av;
      // ---------------- PV
      lds_wait();
      const uint32_t P0 = as_u(h2{(_Float16)p[0], (_Float16)p[1]});
      const uint32_t P1 = as_u(h2{(_Float16)p[2], (_Float16)p[3]});
      if constexpr (VF == KVQ_INT4) {
#pragma unroll
        for (int d = 0; d < 8; ++d) {
          h2 c0[4], c1[4];
          v_int4_pairs(vw[d], c0);
          v_int4_pairs(vw[CDW + d], c1);
#pragma unroll
          for (int x = 0; x < 2; ++x) {
            const int s = 2 * d + x;
            const int src = (4 * s + j) << 2;
            const uint32_t A0 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)P0);
            const uint32_t A1 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)P1);
            const uint2 sc = *reinterpret_cast<const uint2*>(&sm.vmeta[wv][vgrp][s][0]);
            const h4 A = cat(as_h2(A0) * as_h2(sc.x), as_h2(A1) * as_h2(sc.y));
            o[0] = __builtin_amdgcn_mfma_f32_4x4x4f16(A, cat(c0[2 * x], c0[2 * x + 1]), o[0], 0, 0, 0);
            o[1] = __builtin_amdgcn_mfma_f32_4x4x4f16(A, cat(c1[2 * x], c1[2 * x + 1]), o[1], 0, 0, 0);
          }
        }
      } else {  // INT2 values: codes 0..3, value = c * s + z
        const h4 ones = {(_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f, (_Float16)1.0f};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          h2 c0[8], c1[8];
          v_int2_pairs(vw[w], c0);
          v_int2_pairs(vw[CDW + w], c1);
#pragma unroll
          for (int kk = 0; kk < 4; ++kk) {
            const int s = 4 * w + kk;
            const int src = (4 * s + j) << 2;
            const uint32_t A0 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)P0);
            const uint32_t A1 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)P1);
            const uint2 sc = *reinterpret_cast<const uint2*>(&sm.vmeta[wv][vgrp][s][0]);
            const uint2 zc = *reinterpret_cast<const uint2*>(&sm.vmeta[wv][4 + vgrp][s][0]);
            const h4 A = cat(as_h2(A0) * as_h2(sc.x), as_h2(A1) * as_h2(sc.y));
            const h4 Az = cat(as_h2(A0) * as_h2(zc.x), as_h2(A1) * as_h2(zc.y));
            o[0] = __builtin_amdgcn_mfma_f32_4x4x4f16(A, cat(c0[2 * kk], c0[2 * kk + 1]), o[0], 0, 0, 0);
            o[1] = __builtin_amdgcn_mfma_f32_4x4x4f16(A, cat(c1[2 * kk], c1[2 * kk + 1]), o[1], 0, 0, 0);
            oz = __builtin_amdgcn_mfma_f32_4x4x4f16(Az, ones, oz, 0, 0, 0);
          }
        }
      }
    } else if constexpr (CERT) {
      // ---------------- exact recompute from the fp16 originals (original basis)
      const bool bf16 = a.in_bf16 != 0;
      const int tau = lane;
      const bool live = tok0 + tau < T;
      float lh[4] = {0.0f, 0.0f, 0.0f, 0.0f};
      {
        const uint4* kp = reinterpret_cast<const uint4*>(a.k_orig + (stream * a.Tmax + tok0 + tau) * D);
        for (int i = 0; i < 16; ++i) {
          uint4 u = kp[i];
          uint32_t ws[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const int c = 8 * i + 2 * jj;
            const float k0 = widen((uint16_t)(ws[jj] & 0xFFFF), bf16), k1 = widen((uint16_t)(ws[jj] >> 16), bf16);
#pragma unroll
            for (int hh = 0; hh < 4; ++hh) lh[hh] = fmaf(sm.qo[hh][c + 1], k1, fmaf(sm.qo[hh][c], k0, lh[hh]));
          }
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
      alpha = (m_new == NEG_INF) ? 1.0f : exp2f(m - m_new);
      m = m_new;
      const float mh[4] = {quad_bcast<0>(m), quad_bcast<1>(m), quad_bcast<2>(m), quad_bcast<3>(m)};
      float ph[4], sums[4];
#pragma unroll
      for (int hh = 0; hh < 4; ++hh) {
        ph[hh] = (mh[hh] == NEG_INF || !live) ? 0.0f : exp2f(lh[hh] - mh[hh]);
        sums[hh] = wave_sum(ph[hh]);
        sm.pb[wv][tau][hh] = ph[hh];
      }
      const float mysum = (j == 0) ? sums[0] : (j == 1) ? sums[1] : (j == 2) ? sums[2] : sums[3];
      lsum = lsum * alpha + (lane < 4 ? mysum : 0.0f);
      eta = eta * alpha;
      const float a0 = quad_bcast<0>(alpha), a1 = quad_bcast<1>(alpha), a2 = quad_bcast<2>(alpha),
                  a3 = quad_bcast<3>(alpha);
      const f4 av = {a0, a1, a2, a3};
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        o[hf] *= av;
        oo[hf] *= av;
      }
      if constexpr (VF == KVQ_INT2) oz *= av;
      lds_wait();
      const uint32_t* vp = reinterpret_cast<const uint32_t*>(a.v_orig + (stream * a.Tmax + tok0) * D) + lane;
      for (int tt = 0; tt < TILE; ++tt) {
        const uint32_t vv = vp[(size_t)tt * (D / 2)];
        const float v0 = widen((uint16_t)(vv & 0xFFFF), bf16), v1 = widen((uint16_t)(vv >> 16), bf16);
        const float4 pp = *reinterpret_cast<const float4*>(&sm.pb[wv][tt][0]);
        oo[0] += f4{pp.x, pp.y, pp.z, pp.w} * v0;
        oo[1] += f4{pp.x, pp.y, pp.z, pp.w} * v1;
      }
      lds_wait();
      (void)p;
    }
  }

  // ---------------- per-wave totals, then merge the 4 waves in LDS
  const float lt = sum_same_head(lsum);
  const float et = CERT ? sum_same_head(eta) : 0.0f;
  if (lane < 4) {
    sm.mrg_m[wv][lane] = m;
    sm.mrg_l[wv][lane] = lt;
    sm.mrg_e[wv][lane] = et;
  }
  if (lane == 0) {
    sm.mrg_ek[wv] = ekmax;
    sm.mrg_vn[wv] = vnmax;
  }
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    float zb = 0.0f;
    if constexpr (VF == KVQ_INT2) zb = oz[hh];
    sm.mrg_o[wv][hh][2 * lane] = o[0][hh] + zb;
    sm.mrg_o[wv][hh][2 * lane + 1] = o[1][hh] + zb;
    if constexpr (CERT) {
      sm.mrg_oo[wv][hh][2 * lane] = oo[0][hh];
      sm.mrg_oo[wv][hh][2 * lane + 1] = oo[1][hh];
    }
  }
  __syncthreads();
  finish<CERT>(a, sm, b, hq0, nh, split);
}

// ------------------------------------------------------------------ dense fp16 baseline
// Same split structure over uncompressed [Tmax][128] fp16/bf16 K and V (no rotation).
// QK^T: 4x4x4 fp16 MFMA (lane 4s+r loads token 4s+r); PV: each lane owns channels
// 2l, 2l+1 and accumulates p * v with the probabilities broadcast through LDS.
__global__ __launch_bounds__(NT, 2) void decode_dense_split(DecodeArgs a) {
  __shared__ DecodeSmem sm;
  const int b = blockIdx.z;
  const int HG = (a.G + 3) >> 2;
  const int hkv = blockIdx.y / HG, hg = blockIdx.y % HG;
  const int hq0 = hkv * a.G + hg * 4;
  const int nh = min(4, a.G - hg * 4);
  const int split = blockIdx.x;
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
    sm.qo[hh][2 * l] = x0 * (a.scale * LOG2E);
    sm.qo[hh][2 * l + 1] = x1 * (a.scale * LOG2E);
  }
  __syncthreads();
  // query operand: fp16 of (q * scale * log2e) for head j, channels 4n..4n+3
  h4 qop[32];
#pragma unroll
  for (int n = 0; n < 32; ++n)
    qop[n] = h4{(_Float16)sm.qo[j][4 * n], (_Float16)sm.qo[j][4 * n + 1], (_Float16)sm.qo[j][4 * n + 2],
                (_Float16)sm.qo[j][4 * n + 3]};
  float m = NEG_INF, lsum = 0.0f;
  f4 o[2] = {f4{0, 0, 0, 0}, f4{0, 0, 0, 0}};
  for (int ch = c0 + wv; ch < c1; ch += 4) {
    const int tok0 = ch * TILE;
    f4 acc = {0, 0, 0, 0};
    const uint4* kp = reinterpret_cast<const uint4*>(a.k_orig + (stream * a.Tmax + tok0 + lane) * D);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint4 u = kp[i];
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
      acc = __builtin_amdgcn_mfma_f32_4x4x4f16(k0, qop[2 * i], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_4x4x4f16(k1, qop[2 * i + 1], acc, 0, 0, 0);
    }
    float l[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) l[r] = (tok0 + 4 * (lane >> 2) + r < T) ? acc[r] : NEG_INF;
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
    const uint32_t* vp = reinterpret_cast<const uint32_t*>(a.v_orig + (stream * a.Tmax + tok0) * D) + lane;
#pragma unroll 8
    for (int tt = 0; tt < TILE; ++tt) {
      const uint32_t vv = vp[(size_t)tt * (D / 2)];
      const float v0 = widen((uint16_t)(vv & 0xFFFF), bf16), v1 = widen((uint16_t)(vv >> 16), bf16);
      const float4 pp = *reinterpret_cast<const float4*>(&sm.pb[wv][tt][0]);
      o[0] += f4{pp.x, pp.y, pp.z, pp.w} * v0;
      o[1] += f4{pp.x, pp.y, pp.z, pp.w} * v1;
    }
    lds_wait();
  }
  const float lt = sum_same_head(lsum);
  if (lane < 4) {
    sm.mrg_m[wv][lane] = m;
    sm.mrg_l[wv][lane] = lt;
    sm.mrg_e[wv][lane] = 0.0f;
  }
  if (lane == 0) {
    sm.mrg_ek[wv] = 0.0f;
    sm.mrg_vn[wv] = 0.0f;
  }
#pragma unroll
  for (int hh = 0; hh < 4; ++hh) {
    sm.mrg_o[wv][hh][2 * lane] = o[0][hh];
    sm.mrg_o[wv][hh][2 * lane + 1] = o[1][hh];
  }
  __syncthreads();
  finish<false>(a, sm, b, hq0, nh, split);
}

}  // namespace

hipError_t launch_decode(const DecodeArgs& a, int k_fmt, int v_fmt, bool dense, hipStream_t s) {
  const int HG = (a.G + 3) / 4;
  dim3 grid(a.n_splits, a.H * HG, a.B);
  if (dense) {
    hipLaunchKernelGGL(decode_dense_split, grid, dim3(NT), 0, s, a);
    return hipGetLastError();
  }
  const bool cert = a.desc != nullptr;
#define KVQ_LAUNCH(KF, KG, VF)                                                        \
  if (k_fmt == KF && a.k_group == KG && v_fmt == VF) {                                \
    if (cert)                                                                         \
      hipLaunchKernelGGL((decode_split<KF, KG, VF, true>), grid, dim3(NT), 0, s, a);  \
    else                                                                              \
      hipLaunchKernelGGL((decode_split<KF, KG, VF, false>), grid, dim3(NT), 0, s, a); \
    return hipGetLastError();                                                         \
  }
  KVQ_LAUNCH(KVQ_INT4, 32, KVQ_INT4)
  KVQ_LAUNCH(KVQ_INT4, 128, KVQ_INT4)
  KVQ_LAUNCH(KVQ_INT8, 128, KVQ_INT4)
  KVQ_LAUNCH(KVQ_INT8, 32, KVQ_INT4)
  KVQ_LAUNCH(KVQ_INT2, 32, KVQ_INT2)
#undef KVQ_LAUNCH
  return hipErrorNotSupported;
}


}  // namespace kvq
