// Adaptive precision of "Runtime-Certified Bounded-Error Quantized Attention",
// Methodology section 3: a light scoring pass estimates every block's attention
// mass from the quantized keys, the top-K* blocks covering a fraction tau_cov of
// it are promoted to the full-precision originals (through the decode pass's
// exact-recompute flags), and a head whose certificate still exceeds a tolerance
// is recomputed with dense attention over the originals.
#include <algorithm>

#include "kvq_common.h"

namespace kvq {
namespace {

constexpr int NTA = 256;  // 4 waves
constexpr float NEG_INF_A = -__builtin_huge_valf();

__device__ __forceinline__ float wmax(float v) {
  for (int o = 1; o < 64; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wsum(float v) {
  for (int o = 1; o < 64; o <<= 1) v += __shfl_xor(v, o);
  return v;
}

// Forward 64-point complex FFT across the lanes of a wave (lane l holds point l),
// radix 2, decimation in frequency; the result is in bit-reversed order (lane p holds
// point rev6(p)).  ctab: cos(2 pi k / 128) (sin: index + 96).
__device__ __forceinline__ void wave_fft64(float& re, float& im, int l, const float* ctab) {
#pragma unroll
  for (int h = 32; h >= 1; h >>= 1) {
    const float pr = __shfl_xor(re, h), pi = __shfl_xor(im, h);
    const bool up = (l & h) != 0;
    const float sr = up ? pr - re : re + pr;
    const float si = up ? pi - im : im + pi;
    const int e2 = 2 * (l & (h - 1)) * (32 / h);  // W64^e = W128^(2e) = (c, -sn)
    const float c = ctab[e2 & 127], sn = ctab[(e2 + 96) & 127];
    re = up ? sr * c + si * sn : sr;
    im = up ? si * c - sr * sn : si;
  }
}
__device__ __forceinline__ int rev6(int l) { return (int)(__builtin_bitreverse32((uint32_t)l) >> 26); }

// The query of head hq rotated like the cache (y = R q) and multiplied by the
// softmax scale, into dst[128]; one wave, lane l computes channels 2l, 2l+1 (the
// dense rotation: rows l and l + 64).  tmp: 128 floats of LDS private to the wave.
__device__ __forceinline__ void rotated_query(const AdaptArgs& a, int b, int hq, float* dst, float* tmp,
                                              const float* ctab) {
  const int l = threadIdx.x & 63;
  const bool bf16 = a.in_bf16 != 0;
  const uint16_t* qp = a.q + ((size_t)b * a.Hq + hq) * D;
  float x0 = widen(qp[2 * l], bf16), x1 = widen(qp[2 * l + 1], bf16);
  if (a.rotation == KVQ_ROT_SRFT) {
    // y = R q, R the packed unitary DFT times diag(s): the 64-point FFT of
    // z_n = u_2n + i u_2n+1 across the wave, then X_l = E + W128^l O from Z_l and
    // conj Z_(64-l) (lane 0: X_0 and X_64)
    float re = a.signs[2 * l] < 0 ? -x0 : x0, im = a.signs[2 * l + 1] < 0 ? -x1 : x1;
    wave_fft64(re, im, l, ctab);
    const int ka = rev6(l), kb = rev6((64 - l) & 63);
    const float a_re = __shfl(re, ka), a_im = __shfl(im, ka);
    const float b_re = __shfl(re, kb), b_im = -__shfl(im, kb);
    const float e_re = 0.5f * (a_re + b_re), e_im = 0.5f * (a_im + b_im);
    const float o_re = 0.5f * (a_im - b_im), o_im = -0.5f * (a_re - b_re);
    const float c = ctab[l], sn = ctab[(l + 96) & 127];  // W128^l = (c, -sn)
    float y0 = (e_re + (o_re * c + o_im * sn)) * 0.125f;
    float y1 = (e_im + (o_im * c - o_re * sn)) * 0.125f;
    if (l == 0) {
      const float c0 = bits_to_f32(KVQ_INV_SQRT_D_BITS);
      y0 = (a_re + a_im) * c0;
      y1 = (a_re - a_im) * c0;
    }
    (void)tmp;
    dst[2 * l] = y0 * a.scale;
    dst[2 * l + 1] = y1 * a.scale;
    return;
  }
  if (a.rotation == KVQ_ROT_DENSE) {
    tmp[2 * l] = x0;
    tmp[2 * l + 1] = x1;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's LDS writes are visible
#pragma unroll
    for (int rr = 0; rr < 2; ++rr) {
      const int row = l + 64 * rr;
      const uint16_t* rp = a.rot + (size_t)row * D;
      float acc = 0.0f;
      for (int k = 0; k < D; ++k) acc = fmaf(f16_bits_to_f32(rp[k]), tmp[k], acc);
      dst[row] = acc * a.scale;
    }
    return;
  }
  float y0 = x0, y1 = x1;
  if (a.rotation == KVQ_ROT_SIGN_FWHT) {
    if (a.signs[2 * l] < 0) x0 = -x0;
    if (a.signs[2 * l + 1] < 0) x1 = -x1;
    y0 = x0 + x1;  // the pair inside the lane (h = 1), then h = 2..64 across lanes
    y1 = x0 - x1;
    for (int msk = 1; msk < 64; msk <<= 1) {
      const float p0 = __shfl_xor(y0, msk), p1 = __shfl_xor(y1, msk);
      const bool up = (l & msk) != 0;
      y0 = up ? p0 - y0 : y0 + p0;
      y1 = up ? p1 - y1 : y1 + p1;
    }
    const float cn = bits_to_f32(KVQ_INV_SQRT_D_BITS);
    y0 *= cn;
    y1 *= cn;
  }
  dst[2 * l] = y0 * a.scale;
  dst[2 * l + 1] = y1 * a.scale;
}

typedef int i4a __attribute__((ext_vector_type(4)));
typedef float f4a __attribute__((ext_vector_type(4)));
typedef _Float16 h2a __attribute__((ext_vector_type(2)));
typedef _Float16 h4a __attribute__((ext_vector_type(4)));

template <int H>
__device__ __forceinline__ uint32_t quad_bcast_a(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, H * 0x55, 0xF, 0xF, false);
}
__device__ __forceinline__ uint32_t quad_pick(uint32_t v, int r) {  // value of lane 4 (lane / 4) + r (r constant)
  return r == 0 ? quad_bcast_a<0>(v) : r == 1 ? quad_bcast_a<1>(v) : r == 2 ? quad_bcast_a<2>(v) : quad_bcast_a<3>(v);
}

// Key operand of 4-channel step n as four bytes (integer formats): INT8 channels
// 4n..4n+3; INT4 offset-binary nibbles (code + 8) of channels 8(n/2) + 2m + n%2;
// INT2 codes of channels 16(n/4) + 4m + n%4.  step_of(c) inverts it: (n, m).
template <int KF>
__device__ __forceinline__ int key_op(const uint32_t* row, int n) {
  if constexpr (KF == KVQ_INT8) return (int)row[n];
  if constexpr (KF == KVQ_INT4) {
    const uint32_t t = (n & 1) ? (row[n >> 1] >> 4) : row[n >> 1];
    return (int)((t & 0x0F0F0F0Fu) ^ 0x08080808u);
  }
  return (int)((row[n >> 2] >> (2 * (n & 3))) & 0x03030303u);
}
template <int KF>
__device__ __forceinline__ void step_of(int c, int& n, int& m) {
  if constexpr (KF == KVQ_INT8) {
    n = c >> 2;
    m = c & 3;
  } else if constexpr (KF == KVQ_INT4) {
    n = 2 * (c >> 3) + (c & 1);
    m = (c & 7) >> 1;
  } else if constexpr (KF == KVQ_INT2) {
    n = 4 * (c >> 4) + (c & 3);
    m = (c & 15) >> 2;
  } else {  // FP4: channels 4n..4n+3 in order
    n = c >> 2;
    m = c & 3;
  }
}
// FP4 keys: the fp16 values of channels 4n..4n+3 (E2M1 is exact in fp16)
__device__ __forceinline__ h4a fp4_op(const uint32_t* row, int n) {
  const uint32_t w = row[n >> 1];
  const h2a lo = (n & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) : __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0);
  const h2a hi = (n & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) : __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1);
  return h4a{lo.x, lo.y, hi.x, hi.y};
}

// One token's packed key row and its metadata (lane 4s + r holds token 4s + r of the block)
template <int KF, int KG>
struct KeyRegs {
  static constexpr int NW = D * fmt_bits(KF) / 32;
  static constexpr int NM = (meta_bytes(KF, fmt_group(KF, KG)) + 3) / 4;
  uint32_t w[NW];
  uint32_t m[NM];
};
template <int KF, int KG>
__device__ __forceinline__ void load_keys(const uint8_t* row, const uint8_t* meta, KeyRegs<KF, KG>& r) {
  const uint4* rp = reinterpret_cast<const uint4*>(row);
#pragma unroll
  for (int i = 0; i < KeyRegs<KF, KG>::NW / 4; ++i) {
    const uint4 u = rp[i];
    r.w[4 * i] = u.x; r.w[4 * i + 1] = u.y; r.w[4 * i + 2] = u.z; r.w[4 * i + 3] = u.w;
  }
  constexpr int KM = meta_bytes(KF, fmt_group(KF, KG));
  if constexpr (KM >= 16) {
    const uint4 u = *reinterpret_cast<const uint4*>(meta);
    r.m[0] = u.x; r.m[1] = u.y; r.m[2] = u.z; r.m[3] = u.w;
  } else if constexpr (KM == 8) {
    const uint2 u = *reinterpret_cast<const uint2*>(meta);
    r.m[0] = u.x; r.m[1] = u.y;
  } else {
    r.m[0] = *reinterpret_cast<const uint16_t*>(meta);
  }
}

// Scoring pass: log of the softmax numerator mass of every 64-token block,
// lse_b = log sum_{t in b} exp(scale * q_rot . k_hat_t), per query head, written into
// mass and normalised by mass_kernel.  One workgroup per (16 blocks, kv head, group of
// 4 query heads, sequence); wave w takes blocks w, w + 4, w + 8, w + 12 of its 16, the
// key rows of the next one in flight while one is scored.  (Measured on the certified
// workload: ≈265 µs for 1.09 GB, ≈4.1 TB/s, with the VALU nearly idle; neither two
// blocks in flight, eight blocks per wave nor staging coalesced loads through LDS
// changed that, so what limits it is still open.)  The products run on the matrix
// cores, 4 tokens x 4 heads x 4 channels per block of the 4x4x4 MFMA (lane 4s + r: token
// 4s + r as the key operand; head r as the query operand and output):
//  * integer keys: the rotated query is quantized to 24 bits (qs = max|q| / 8e6) and
//    split into three balanced int8 digits, so each group's dot product is three exact
//    integer sums (INT4 codes enter offset-binary, the offset removed through the digit
//    sums; INT2 offsets through the group's query sum);
//  * FP4 keys: exact fp16 codes against the query in two fp16 parts after a power-of-two
//    scaling, fp32 accumulation per 16-channel block.
// Each group's sum is scaled once by the token's group scale.
template <int KF, int KG>
__global__ __launch_bounds__(NTA) void score_kernel(AdaptArgs a) {
  constexpr int GS = fmt_group(KF, KG);  // channels per scale
  constexpr int NG = D / GS, SPG = GS / 4;
  constexpr int KB = row_bytes(KF);
  constexpr int KM = meta_bytes(KF, GS);
  constexpr int NBW = 4;  // blocks per wave
  constexpr int PF = 1;   // blocks in flight ahead of the one being scored
  __shared__ float qr[4][D];
  __shared__ float tmp[4][D];
  __shared__ float ctab[128];
  __shared__ uint4 qop[4][32];  // per head and step: INT: digits 0, 1, 2 of 4 channels; FP4: fp16 high, low pairs
  __shared__ float qsc[4];      // per head: the query's unit (INT: qs; FP4: the power-of-two scale)
  __shared__ int qds[4][8][4];  // per head, group, digit: digit sums (INT4 offset correction)
  __shared__ float qsf[4][4];   // per head, 32-channel group: sum of the rotated query (INT2 offsets)
  const int b = blockIdx.z;
  const int HG = (a.G + 3) >> 2;
  const int hkv = blockIdx.y / HG, hg = blockIdx.y % HG;
  const int hq0 = hkv * a.G + hg * 4;
  const int nh = min(4, a.G - hg * 4);
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int T = a.seq.v[b];
  const int nchunks = (T + TILE - 1) / TILE;
  const int cfirst = blockIdx.x * (4 * NBW);
  if (cfirst >= nchunks) return;  // uniform over the workgroup
  const size_t stream = (size_t)b * a.H + hkv;
  // the first block's keys are in flight during the query prologue
  auto key_ptrs = [&](int c, const uint8_t*& rp, const uint8_t*& mp) {
    const int cc = min(c, nchunks - 1);  // past the last block: reload a valid one (never scored)
    const size_t t = (size_t)cc * TILE + lane;
    rp = a.k_codes + (stream * a.Tmax + t) * KB;
    mp = a.k_meta + (stream * a.Tmax + t) * KM;
  };
  KeyRegs<KF, KG> R[PF + 1];
#pragma unroll
  for (int p = 0; p < PF; ++p) {
    const uint8_t *rp, *mp;
    key_ptrs(cfirst + wv + 4 * p, rp, mp);
    load_keys<KF, KG>(rp, mp, R[p]);
  }
  if (a.rotation == KVQ_ROT_SRFT) {
    if (threadIdx.x < 128) ctab[threadIdx.x] = a.cos128[threadIdx.x];
    __syncthreads();
  }
  // ---- prologue: wave w rotates query head w and stores its operands
  float y0 = 0.0f, y1 = 0.0f;
  if (wv < nh) {
    rotated_query(a, b, hq0 + wv, qr[wv], tmp[wv], ctab);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xc07f);
    y0 = qr[wv][2 * lane];
    y1 = qr[wv][2 * lane + 1];
    if (a.lam_k != nullptr) {  // keys were stored times lambda_k
      const float* lp = a.lam_k + (size_t)hkv * D;
      y0 = y0 / lp[2 * lane];
      y1 = y1 / lp[2 * lane + 1];
    }
  }
  {
    const float ys[2] = {y0, y1};
    const float mx = wmax(fmaxf(fabsf(y0), fabsf(y1)));
    if constexpr (KF == KVQ_FP4) {
      int ex = 0;
      frexpf(mx, &ex);
      const float qs = mx > 0.0f ? ldexpf(1.0f, ex - 14) : 1.0f, inv = mx > 0.0f ? ldexpf(1.0f, 14 - ex) : 1.0f;
      uint16_t* qh = reinterpret_cast<uint16_t*>(&qop[wv][0]);
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int c = 2 * lane + e, n = c >> 2, m = c & 3;
        const float v = ys[e] * inv;
        const _Float16 hh = (_Float16)v, ll = (_Float16)(v - (float)hh);
        qh[n * 8 + m] = __builtin_bit_cast(uint16_t, hh);
        qh[n * 8 + 4 + m] = __builtin_bit_cast(uint16_t, ll);
      }
      if (lane == 0) qsc[wv] = qs;
    } else {
      const float qs = mx > 0.0f ? mx / 8.0e6f : 1.0f;
      uint8_t* qb = reinterpret_cast<uint8_t*>(&qop[wv][0]);
      int dsum[2][3];
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int c = 2 * lane + e;
        const int qv = (int)rintf(ys[e] / qs);  // |qv| <= 8e6
        const int d0 = ((qv + 128) & 255) - 128, r1 = (qv - d0) >> 8;
        const int d1 = ((r1 + 128) & 255) - 128, d2 = (r1 - d1) >> 8;  // |d2| <= 123
        int n, m;
        step_of<KF>(c, n, m);
        qb[16 * n + m] = (uint8_t)(d0 & 0xFF);
        qb[16 * n + 4 + m] = (uint8_t)(d1 & 0xFF);
        qb[16 * n + 8 + m] = (uint8_t)(d2 & 0xFF);
        qb[16 * n + 12 + m] = 0;
        dsum[e][0] = d0;
        dsum[e][1] = d1;
        dsum[e][2] = d2;
      }
      if (lane == 0) qsc[wv] = qs;
      if constexpr (KF == KVQ_INT4) {  // digit sums per group: lanes (GS / 2) l' .. hold group l'
#pragma unroll
        for (int p = 0; p < 3; ++p) {
          int v = dsum[0][p] + dsum[1][p];
          for (int o = 1; o < GS / 2; o <<= 1) v += __shfl_xor(v, o);
          if ((lane & (GS / 2 - 1)) == 0) qds[wv][lane / (GS / 2)][p] = v;
        }
      }
      if constexpr (KF == KVQ_INT2) {  // query sums per 32-channel group: lanes 16g..16g+15
        float v = y0 + y1;
        for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o);
        if ((lane & 15) == 0) qsf[wv][lane >> 4] = v;
      }
    }
  }
  __syncthreads();
  const int j = lane & 3;  // head of this lane's outputs
  const float unit = qsc[j];
#pragma unroll
  for (int k = 0; k < NBW; ++k) {
    const int c = cfirst + wv + 4 * k;
    if (c >= nchunks) break;  // uniform over the wave; no barrier follows
    if (k + PF < NBW) {
      const uint8_t *rp, *mp;
      key_ptrs(c + 4 * PF, rp, mp);
      load_keys<KF, KG>(rp, mp, R[(k + PF) % (PF + 1)]);
    }
    // issue the next block's loads before this block's products (otherwise the
    // compiler gives both blocks the same registers and the loads wait for the products)
    __builtin_amdgcn_sched_barrier(0);
    const KeyRegs<KF, KG>& K = R[k % (PF + 1)];
    float sc[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // tokens 4s + r, head j
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      float part[4];
      if constexpr (KF == KVQ_FP4) {
        f4a acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int n = g * SPG; n < (g + 1) * SPG; ++n) {
          const uint4 qv = qop[j][n];
          const h4a av = fp4_op(K.w, n);
          acc = __builtin_amdgcn_mfma_f32_4x4x4f16(av, h4a{__builtin_bit_cast(h2a, qv.x).x, __builtin_bit_cast(h2a, qv.x).y,
                                                          __builtin_bit_cast(h2a, qv.y).x, __builtin_bit_cast(h2a, qv.y).y},
                                                   acc, 0, 0, 0);
          acc = __builtin_amdgcn_mfma_f32_4x4x4f16(av, h4a{__builtin_bit_cast(h2a, qv.z).x, __builtin_bit_cast(h2a, qv.z).y,
                                                          __builtin_bit_cast(h2a, qv.w).x, __builtin_bit_cast(h2a, qv.w).y},
                                                   acc, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) part[r] = acc[r];
      } else {
        int corr[3] = {0, 0, 0};
        if constexpr (KF == KVQ_INT4) {
          corr[0] = -8 * qds[j][g][0];
          corr[1] = -8 * qds[j][g][1];
          corr[2] = -8 * qds[j][g][2];
        }
        i4a a0 = {corr[0], corr[0], corr[0], corr[0]}, a1 = {corr[1], corr[1], corr[1], corr[1]},
            a2 = {corr[2], corr[2], corr[2], corr[2]};
#pragma unroll
        for (int n = g * SPG; n < (g + 1) * SPG; ++n) {
          const uint4 qv = qop[j][n];
          const int av = key_op<KF>(K.w, n);
          a0 = __builtin_amdgcn_mfma_i32_4x4x4i8(av, (int)qv.x, a0, 0, 0, 0);
          a1 = __builtin_amdgcn_mfma_i32_4x4x4i8(av, (int)qv.y, a1, 0, 0, 0);
          a2 = __builtin_amdgcn_mfma_i32_4x4x4i8(av, (int)qv.z, a2, 0, 0, 0);
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) part[r] = ((float)a2[r] * 65536.0f + (float)a1[r] * 256.0f) + (float)a0[r];
      }
      // the group scale (and INT2 offset) of token 4s + r: metadata of lane 4s + r
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if constexpr (KF == KVQ_FP4) {
          const uint32_t w = quad_pick(K.m[g >> 2], r);
          sc[r] = fmaf(part[r] * unit, e4m3_value((w >> (8 * (g & 3))) & 0xFFu), sc[r]);
        } else {
          const uint32_t w = quad_pick(K.m[g >> 1], r);
          const float sg = f16_bits_to_f32((uint16_t)(w >> (16 * (g & 1))));
          sc[r] = fmaf(part[r] * unit, sg, sc[r]);
          if constexpr (KF == KVQ_INT2) {
            const uint32_t zw = quad_pick(K.m[(NG + g) >> 1], r);
            sc[r] = fmaf(f16_bits_to_f32((uint16_t)(zw >> (16 * ((NG + g) & 1)))), qsf[j][g], sc[r]);
          }
        }
      }
      // one group at a time: overlapping groups would keep every group's operands live
      if constexpr (NG > 1) __builtin_amdgcn_sched_barrier(0);
    }
    // log-sum-exp of the block per head: 4 tokens per lane, then the 16 lanes of head j
    const int s4 = lane & ~3;
    float mx = NEG_INF_A;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if (c * TILE + s4 + r >= T) sc[r] = NEG_INF_A;
      mx = fmaxf(mx, sc[r]);
    }
    for (int o = 4; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    float se = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) se += sc[r] == NEG_INF_A ? 0.0f : expf(sc[r] - mx);
    for (int o = 4; o < 64; o <<= 1) se += __shfl_xor(se, o);
    if (lane < nh) a.mass[((size_t)b * a.Hq + hq0 + lane) * a.nt + c] = mx + logf(se);
  }
}

// Block masses of one (sequence, query head): P_b = exp(lse_b - LSE), zero past
// the sequence.  One workgroup per row, in place over the scoring pass's output.
__global__ __launch_bounds__(NTA) void mass_kernel(AdaptArgs a) {
  __shared__ float red[NTA / 64];
  const int row = blockIdx.x, b = row / a.Hq;
  const int nb = (a.seq.v[b] + TILE - 1) / TILE;
  float* m = a.mass + (size_t)row * a.nt;
  const int t = threadIdx.x, wv = t >> 6, lane = t & 63;
  float mx = NEG_INF_A;
  for (int j = t; j < nb; j += NTA) mx = fmaxf(mx, m[j]);
  mx = wmax(mx);
  if (lane == 0) red[wv] = mx;
  __syncthreads();
  mx = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  __syncthreads();
  float s = 0.0f;
  for (int j = t; j < nb; j += NTA) s += expf(m[j] - mx);
  s = wsum(s);
  if (lane == 0) red[wv] = s;
  __syncthreads();
  const float lse = mx + logf(red[0] + red[1] + red[2] + red[3]);
  for (int j = t; j < a.nt; j += NTA) m[j] = j < nb ? expf(m[j] - lse) : 0.0f;
}

// Promotion flags.  flags_init_kernel writes the given flags (or zeros); then one
// workgroup per (sequence, query head) sorts that head's blocks by decreasing mass
// (equal masses: lower index first) and marks the shortest prefix whose fp32
// running sum, taken in that order, reaches tau_cov.  The query heads of a kv head
// mark the same flag row; they only ever store 1, so their order does not matter.
// The running sum is one thread's sequential fp32 additions, so the choice is
// reproducible bit for bit.
__global__ __launch_bounds__(NTA) void flags_init_kernel(AdaptArgs a) {
  const size_t n = (size_t)a.B * a.H * a.nt;
  for (size_t j = (size_t)blockIdx.x * NTA + threadIdx.x; j < n; j += (size_t)gridDim.x * NTA)
    a.flags_out[j] = (a.flags_in != nullptr && a.flags_in[j] != 0) ? 1 : 0;
}

__global__ __launch_bounds__(NTA) void select_kernel(AdaptArgs a) {
  __shared__ unsigned long long key[MAX_SELECT_BLOCKS];
  __shared__ int kstar;
  const int row = blockIdx.x, b = row / a.Hq, h = (row % a.Hq) / a.G;
  const int t = threadIdx.x;
  const int nb = (a.seq.v[b] + TILE - 1) / TILE;
  if (nb == 0) return;  // uniform
  int npow = 2;
  while (npow < nb) npow <<= 1;
  const float* m = a.mass + (size_t)row * a.nt;
  for (int j = t; j < npow; j += NTA)
    key[j] = j < nb ? (((unsigned long long)__float_as_uint(m[j]) << 32) | (0xFFFFFFFFu - (uint32_t)j)) : 0ull;
  __syncthreads();
  for (int k = 2; k <= npow; k <<= 1) {
    for (int jj = k >> 1; jj > 0; jj >>= 1) {
      for (int i = t; i < npow; i += NTA) {
        const int ixj = i ^ jj;
        if (ixj > i) {
          const unsigned long long x = key[i], y = key[ixj];
          const bool desc = (i & k) == 0;
          if (desc ? (x < y) : (x > y)) {
            key[i] = y;
            key[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
  if (t == 0) {
    // the masses are read 16 at a time (the LDS loads overlap) and added one by one
    float run = 0.0f;
    int k = 0;
    bool done = false;
    for (int k0 = 0; k0 < nb && !done; k0 += 16) {
      float mk[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) mk[i] = k0 + i < npow ? __uint_as_float((uint32_t)(key[k0 + i] >> 32)) : 0.0f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (!done && k0 + i < nb) {
          run = run + mk[i];
          k = k0 + i + 1;
          done = run >= a.tau_cov;
        }
      }
    }
    kstar = k;
  }
  __syncthreads();
  uint8_t* fl = a.flags_out + ((size_t)b * a.H + h) * a.nt;
  for (int j = t; j < kstar; j += NTA) fl[0xFFFFFFFFu - (uint32_t)key[j]] = 1;
}

// Dense fallback of one (sequence, query head): if its certificate exceeds eps,
// exact attention over the originals (original basis, no rotation), and the
// certificate becomes 0.  One workgroup per row; wave w takes blocks w, w + 4, ...
// with a running max and sum, and the waves are merged at the end.
__global__ __launch_bounds__(NTA) void fallback_kernel(AdaptArgs a) {
  __shared__ float qs[D];
  __shared__ float pb[4][TILE];
  __shared__ float wm[4], wl[4];
  __shared__ float wo[4][D];
  const int row = blockIdx.x, b = row / a.Hq, hq = row % a.Hq, h = hq / a.G;
  if (!(a.cert[row] > a.eps)) return;  // uniform over the workgroup
  const int T = a.seq.v[b];
  const int t = threadIdx.x, wv = t >> 6, lane = t & 63;
  const bool bf16 = a.in_bf16 != 0;
  if (t < D) qs[t] = widen(a.q[(size_t)row * D + t], bf16) * a.scale;
  __syncthreads();
  const size_t stream = (size_t)b * a.H + h;
  const int nchunks = (T + TILE - 1) / TILE;
  float m = NEG_INF_A, l = 0.0f, o0 = 0.0f, o1 = 0.0f;
  for (int c = wv; c < nchunks; c += 4) {
    const int tok = c * TILE + lane;
    const uint4* kp = reinterpret_cast<const uint4*>(a.k_orig + (stream * a.Tmax + tok) * D);
    uint4 kr[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) kr[i] = kp[i];
    float lg = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t w4[4] = {kr[i].x, kr[i].y, kr[i].z, kr[i].w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int ch = 8 * i + 2 * e;
        lg = fmaf(qs[ch], widen((uint16_t)(w4[e] & 0xFFFF), bf16), lg);
        lg = fmaf(qs[ch + 1], widen((uint16_t)(w4[e] >> 16), bf16), lg);
      }
    }
    if (tok >= T) lg = NEG_INF_A;
    const float m_new = fmaxf(m, wmax(lg));
    const float alpha = m == NEG_INF_A ? 0.0f : expf(m - m_new);
    const float p = tok < T ? expf(lg - m_new) : 0.0f;
    l = l * alpha + wsum(p);
    o0 *= alpha;
    o1 *= alpha;
    m = m_new;
    pb[wv][lane] = p;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xc07f);
    const uint32_t* vp = reinterpret_cast<const uint32_t*>(a.v_orig + (stream * a.Tmax + (size_t)c * TILE) * D) + lane;
    for (int t0 = 0; t0 < TILE; t0 += 16) {
      uint32_t vr[16];
#pragma unroll
      for (int k = 0; k < 16; ++k) vr[k] = vp[(size_t)(t0 + k) * (D / 2)];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const float pk = pb[wv][t0 + k];
        o0 = fmaf(pk, widen((uint16_t)(vr[k] & 0xFFFF), bf16), o0);
        o1 = fmaf(pk, widen((uint16_t)(vr[k] >> 16), bf16), o1);
      }
    }
    __builtin_amdgcn_wave_barrier();
  }
  if (lane == 0) {
    wm[wv] = m;
    wl[wv] = l;
  }
  wo[wv][2 * lane] = o0;
  wo[wv][2 * lane + 1] = o1;
  __syncthreads();
  if (wv == 0) {
    float M = NEG_INF_A;
#pragma unroll
    for (int w = 0; w < 4; ++w) M = fmaxf(M, wm[w]);
    float L = 0.0f, r0 = 0.0f, r1 = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float e = wm[w] == NEG_INF_A ? 0.0f : expf(wm[w] - M);
      L += e * wl[w];
      r0 += e * wo[w][2 * lane];
      r1 += e * wo[w][2 * lane + 1];
    }
    const float inv = L > 0.0f ? 1.0f / L : 0.0f;
    *reinterpret_cast<float2*>(a.out + (size_t)row * D + 2 * lane) = make_float2(r0 * inv, r1 * inv);
    if (lane == 0) a.cert[row] = 0.0f;
  }
}

}  // namespace

hipError_t launch_block_mass(const AdaptArgs& a, hipStream_t s) {
  const int HG = (a.G + 3) / 4;
  int max_chunks = 0;
  for (int b = 0; b < a.B; ++b) max_chunks = max(max_chunks, (a.seq.v[b] + TILE - 1) / TILE);
  if (max_chunks > 0) {
    const dim3 grid((max_chunks + 15) / 16, a.H * HG, a.B);  // 16 blocks per workgroup
#define KVQ_SCORE(KF, KG)                                                          \
    if (a.k_fmt == KF && a.k_group == KG) {                                        \
      hipLaunchKernelGGL((score_kernel<KF, KG>), grid, dim3(NTA), 0, s, a);        \
    } else
    KVQ_SCORE(KVQ_INT4, 16) KVQ_SCORE(KVQ_INT4, 32) KVQ_SCORE(KVQ_INT4, 128) KVQ_SCORE(KVQ_INT8, 32) KVQ_SCORE(KVQ_INT8, 128)
    KVQ_SCORE(KVQ_INT2, 32) KVQ_SCORE(KVQ_FP4, 16) { return hipErrorNotSupported; }
#undef KVQ_SCORE
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(mass_kernel, dim3(a.B * a.Hq), dim3(NTA), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_select(const AdaptArgs& a, hipStream_t s) {
  const size_t n = (size_t)a.B * a.H * a.nt;
  hipLaunchKernelGGL(flags_init_kernel, dim3((unsigned)std::min<size_t>((n + NTA - 1) / NTA, 1024)), dim3(NTA), 0, s, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(select_kernel, dim3(a.B * a.Hq), dim3(NTA), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fallback(const AdaptArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(fallback_kernel, dim3(a.B * a.Hq), dim3(NTA), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvq
