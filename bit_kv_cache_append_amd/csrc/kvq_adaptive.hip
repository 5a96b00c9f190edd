// Adaptive precision of "Runtime-Certified Bounded-Error Quantized Attention",
// Methodology section 3: a light scoring pass estimates every block's attention
// mass from the quantized keys, the top-K* blocks covering a fraction tau_cov of
// it are promoted to the full-precision originals (through the decode pass's
// exact-recompute flags), blocks whose value error is large against their mass take
// exact values, and the ranking of each head's promoted blocks is checked against
// the originals.  (The dense recompute of a head is the fp16 decode's split kernel,
// restricted to the heads that need it.)
#include <algorithm>

#include "kvq_common.h"

namespace kvq {
namespace {

constexpr int NTA = 256;  // 4 waves
constexpr int NTW = 512;  // the scoring pass: 8 waves
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

// 8-bit keys with one scale per token, for the 16 x 16 x 64 integer product: tile t of
// the block (tokens 16t..16t+15), K half s (channels 64s..64s+63); lane l holds token
// 16t + (l & 15), channels 64s + 16 (l >> 4) .. + 15 (the product's row-operand layout),
// and the fp16 scales of tokens 16t + 4 (l >> 4) + 0..3 (its output rows).
struct WideKeys {
  i4a a[8];
  uint2 sc[4];
};

// Max (MAX) or sum over the 16 lanes of one head (the lanes with equal lane & 3): row
// rotations by 4 and 8 inside each row of 16 lanes (DPP), then the gfx950 row and
// half-wave swaps, which give every lane its own value and its partner's; no round trip
// through the LDS crossbar.
template <bool MAX>
__device__ __forceinline__ float head_reduce(float v) {
  auto op = [](float x, float y) { return MAX ? fmaxf(x, y) : x + y; };
  v = op(v, dpp_f<0x124>(v));  // row_ror:4
  v = op(v, dpp_f<0x128>(v));  // row_ror:8
  const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_int(v), __float_as_int(v), false, false);
  v = op(__int_as_float(p16[0]), __int_as_float(p16[1]));
  const auto p32 = __builtin_amdgcn_permlane32_swap(__float_as_int(v), __float_as_int(v), false, false);
  return op(__int_as_float(p32[0]), __int_as_float(p32[1]));
}

// Scoring pass: log of the softmax numerator mass of every 64-token block,
// lse_b = log sum_{t in b} exp(scale * q_rot . k_hat_t), per query head, written into
// mass and normalised by mass_kernel.  One workgroup of 8 waves per (unit, split): a
// unit is (sequence, kv head, group of 4 query heads), a split a range of its blocks.
// Waves 0..3 prepare the query heads once; then wave w starts with the range's block w
// and claims further blocks through a counter in LDS, one visit ahead, the next block's
// key rows in flight while one is scored (two register sets used alternately).  (The
// earlier form, short-lived 4-wave workgroups of 16 blocks each, spent a quarter of
// every wave's life on its own query prologue and ran at ~4.1 TB/s on the certified
// shape.)  The products run on the matrix
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
__global__ __launch_bounds__(NTW) void score_kernel(AdaptArgs a) {
  constexpr int GS = fmt_group(KF, KG);  // channels per scale
  constexpr int NG = D / GS, SPG = GS / 4;
  constexpr int KB = row_bytes(KF);
  constexpr int KM = meta_bytes(KF, GS);
  constexpr int NWV = NTW / 64;
  __shared__ float qr[4][D];
  __shared__ float tmp[4][D];
  __shared__ float ctab[128];
  __shared__ uint4 qop[4][32];  // per head and step: INT: digits 0, 1, 2 of 4 channels; FP4: fp16 high, low pairs
  __shared__ float qsc[4];      // per head: the query's unit (INT: qs; FP4: the power-of-two scale)
  __shared__ int qds[4][8][4];  // per head, group, digit: digit sums (INT4 offset correction)
  __shared__ float qsf[4][4];   // per head, 32-channel group: sum of the rotated query (INT2 offsets)
  __shared__ int qint[4][D];    // per head and channel: the 24-bit query (8-bit keys, one scale per token)
  __shared__ int next;          // next block (offset from the split's first) to claim
  const int S = a.score_splits;
  const int u = blockIdx.x / S, split = blockIdx.x % S;
  const int HG = (a.G + 3) >> 2;
  const int b = u / (a.H * HG), hkv = (u / HG) % a.H, hg = u % HG;
  const int hq0 = hkv * a.G + hg * 4;
  const int nh = min(4, a.G - hg * 4);
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int T = a.seq.v[b];
  const int nchunks = (T + TILE - 1) / TILE;
  const int c0 = split * a.score_cps, c1 = min(nchunks, c0 + a.score_cps);
  if (c0 >= c1) return;  // uniform over the workgroup
  const size_t stream = (size_t)b * a.H + hkv;
  auto key_ptrs = [&](int c, const uint8_t*& rp, const uint8_t*& mp) {
    const size_t t = (size_t)c * TILE + lane;
    KVQ_DCHECK(stream < (size_t)a.B * a.H && c >= 0 && c < a.nt, DBG_CHUNK, stream, c);
    rp = a.k_codes + (stream * a.Tmax + t) * KB;
    mp = a.k_meta + (stream * a.Tmax + t) * KM;
  };
  auto load_block = [&](int c, KeyRegs<KF, KG>& R) {
    const uint8_t *rp, *mp;
    key_ptrs(c, rp, mp);
    load_keys<KF, KG>(rp, mp, R);
  };
  // 8-bit keys with one scale per token (the certified workload's keys) take the
  // 16 x 16 x 64 integer product: 8 per block and wave instead of 96 of the 4 x 4 x 4 one
  constexpr bool WIDE = KF == KVQ_INT8 && GS == D;
  auto load_wide = [&](int c, WideKeys& R) {
    KVQ_DCHECK(stream < (size_t)a.B * a.H && c >= 0 && c < a.nt, DBG_CHUNK, stream, c);
    const uint8_t* kb = a.k_codes + (stream * a.Tmax + (size_t)c * TILE) * KB;
    const uint8_t* mb = a.k_meta + (stream * a.Tmax + (size_t)c * TILE) * KM;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint4 u = *reinterpret_cast<const uint4*>(kb + (size_t)(16 * t + (lane & 15)) * KB + 64 * h + 16 * (lane >> 4));
        R.a[2 * t + h] = i4a{(int)u.x, (int)u.y, (int)u.z, (int)u.w};
      }
      R.sc[t] = *reinterpret_cast<const uint2*>(mb + (size_t)(16 * t + 4 * (lane >> 4)) * KM);
    }
  };
  // the first block's keys are in flight during the query prologue
  KeyRegs<KF, KG> RA, RB;
  WideKeys WA, WB;
  int cA = c0 + wv;
  if constexpr (WIDE)
    load_wide(cA < c1 ? cA : c0, WA);
  else
    load_block(cA < c1 ? cA : c0, RA);
  __builtin_amdgcn_sched_barrier(0);
  if (threadIdx.x == 0) next = NWV;  // published by the prologue's barrier
  if (a.rotation == KVQ_ROT_SRFT) {
    if (threadIdx.x < 128) ctab[threadIdx.x] = a.cos128[threadIdx.x];
    __syncthreads();
  }
  // ---- prologue: wave w < 4 rotates query head w and stores its operands
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
  if (wv < 4) {
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
        if constexpr (WIDE) qint[wv][c] = qv;
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
  // wide products: the query operand of K half s for column l & 15 = 4 d + h is digit d
  // (0, 1, 2; column d = 3 is zero) of head h at channels 64s + 16 (l >> 4) .. + 15, the
  // digits split as in the prologue's 4 x 4 x 4 operands
  i4a qb[2] = {i4a{0, 0, 0, 0}, i4a{0, 0, 0, 0}};
  if constexpr (WIDE) {
    const int dg = (lane & 15) >> 2;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      int w4[4];
#pragma unroll
      for (int k4 = 0; k4 < 4; ++k4) {
        uint32_t word = 0;
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const int qv = qint[j][64 * h + 16 * (lane >> 4) + 4 * k4 + bb];
          const int d0 = ((qv + 128) & 255) - 128, r1 = (qv - d0) >> 8;
          const int d1 = ((r1 + 128) & 255) - 128, d2 = (r1 - d1) >> 8;
          const int dig = dg == 0 ? d0 : dg == 1 ? d1 : dg == 2 ? d2 : 0;
          word |= (uint32_t)(dig & 0xFF) << (8 * bb);
        }
        w4[k4] = (int)word;
      }
      qb[h] = i4a{w4[0], w4[1], w4[2], w4[3]};
    }
  }
  // one block by the wide products: lane l holds digit (l & 15) >> 2 of head l & 3 for
  // tokens 16t + 4 (l >> 4) + i; the lanes of digit 0 gather digits 1 and 2 from the
  // lanes 4 and 8 places on in their row of 16 (a rotation by 8 either way, and the sum
  // of the rotations by 4 and by 12, one of which reads the zero digit-3 lane) and form
  // the sum as the 4 x 4 x 4 path does; the other lanes take no part in the reductions
  auto score_wide = [&](const WideKeys& K, int c) {
    i4a acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      acc[t] = i4a{0, 0, 0, 0};
#pragma unroll
      for (int h = 0; h < 2; ++h) acc[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(K.a[2 * t + h], qb[h], acc[t], 0, 0, 0);
    }
    const bool lead = (lane & 12) == 0;  // digit 0
    const int tok = c * TILE + 4 * (lane >> 4);
    float mx = NEG_INF_A;
    float sc[16];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int a0 = acc[t][i];
        const int a1 = __builtin_amdgcn_mov_dpp(a0, 0x124, 0xF, 0xF, false) + __builtin_amdgcn_mov_dpp(a0, 0x12C, 0xF, 0xF, false);
        const int a2 = __builtin_amdgcn_mov_dpp(a0, 0x128, 0xF, 0xF, false);
        const float part = ((float)a2 * 65536.0f + (float)a1 * 256.0f) + (float)a0;
        const uint32_t sw = (i < 2) ? K.sc[t].x : K.sc[t].y;
        const float sg = f16_bits_to_f32((uint16_t)(sw >> (16 * (i & 1))));
        float v = fmaf(part * unit, sg, 0.0f);
        if (!lead || tok + 16 * t + i >= T) v = NEG_INF_A;
        sc[4 * t + i] = v;
        mx = fmaxf(mx, v);
      }
    }
    mx = head_reduce<true>(mx);
    float se = 0.0f;
#pragma unroll
    for (int k = 0; k < 16; ++k) se += sc[k] == NEG_INF_A ? 0.0f : expf(sc[k] - mx);
    se = head_reduce<false>(se);
    KVQ_DCHECK(lane >= nh || hq0 + lane < a.Hq, DBG_ROW, (size_t)b * a.Hq + hq0 + lane, c);
    if (lane < nh) a.mass[((size_t)b * a.Hq + hq0 + lane) * a.nt + c] = mx + logf(se);
  };
  auto claim = [&]() -> int {
    int v = 0;
    if (lane == 0) v = atomicAdd(&next, 1);
    return v;
  };
  // ---- one block: products, group scales, the block's log-sum-exp per head
  auto score = [&](const KeyRegs<KF, KG>& K, int c) {
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
    mx = head_reduce<true>(mx);
    float se = 0.0f;
#pragma unroll
    for (int r = 0; r < 4; ++r) se += sc[r] == NEG_INF_A ? 0.0f : expf(sc[r] - mx);
    se = head_reduce<false>(se);
    KVQ_DCHECK(lane >= nh || hq0 + lane < a.Hq, DBG_ROW, (size_t)b * a.Hq + hq0 + lane, c);
    if (lane < nh) a.mass[((size_t)b * a.Hq + hq0 + lane) * a.nt + c] = mx + logf(se);
  };
  // Blocks are claimed one visit ahead and their loads issued before the current block is
  // scored, alternating two register sets; a load past the range's end reloads the current,
  // valid block, so every iteration issues the same loads (claims only grow: once one is
  // past the end the next is too, and the wave leaves at the loop head).
  int pB = claim();
  if constexpr (WIDE) {
    while (cA < c1) {
      const int cB = c0 + __builtin_amdgcn_readfirstlane(pB);
      const int pC = claim();
      load_wide(cB < c1 ? cB : cA, WB);
      __builtin_amdgcn_sched_barrier(0);
      score_wide(WA, cA);
      int pCv = pC;
      asm volatile("" : "+v"(pCv));
      const int cC = c0 + __builtin_amdgcn_readfirstlane(pCv);
      pB = claim();
      load_wide(cC < c1 ? cC : cA, WA);
      __builtin_amdgcn_sched_barrier(0);
      if (cB < c1) score_wide(WB, cB);
      asm volatile("" : "+v"(pB));
      cA = cC;
    }
    return;
  }
  while (cA < c1) {
    const int cB = c0 + __builtin_amdgcn_readfirstlane(pB);
    const int pC = claim();
    load_block(cB < c1 ? cB : cA, RB);
    __builtin_amdgcn_sched_barrier(0);
    score(RA, cA);
    int pCv = pC;
    asm volatile("" : "+v"(pCv));
    const int cC = c0 + __builtin_amdgcn_readfirstlane(pCv);
    pB = claim();
    load_block(cC < c1 ? cC : cA, RA);
    __builtin_amdgcn_sched_barrier(0);
    if (cB < c1) score(RB, cB);
    asm volatile("" : "+v"(pB));
    cA = cC;
  }
}

// Block masses of one (sequence, query head): P_b = exp(lse_b - LSE), zero past
// the sequence.  One workgroup per row, in place over the scoring pass's output.
__global__ __launch_bounds__(NTA) void mass_kernel(AdaptArgs a) {
  __shared__ float red[NTA / 64];
  const int row = blockIdx.x, b = row / a.Hq;
  const int nb = (a.seq.v[b] + TILE - 1) / TILE;
  KVQ_DCHECK(row < a.B * a.Hq && nb <= a.nt, DBG_ROW, row, nb);
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

// Promotion flags.  flags_init_kernel copies the given flags (or writes zeros); then
// one workgroup per (sequence, query head) sets bit 0 on its top-K* blocks.  The query
// heads of a kv head mark the same flag row; each stores the byte's initial value with
// bit 0 set (no one changes another bit meanwhile), so their order does not matter.
__global__ __launch_bounds__(NTA) void flags_init_kernel(AdaptArgs a) {
  const size_t n = (size_t)a.B * a.H * a.nt;
  for (size_t j = (size_t)blockIdx.x * NTA + threadIdx.x; j < n; j += (size_t)gridDim.x * NTA)
    a.flags_out[j] = a.flags_in != nullptr ? a.flags_in[j] : 0;
}

// Sorts the blocks [0, nb) of row (sequence, query head) by decreasing mass (equal
// masses: lower index first) into key[] (the mass bits above the complemented block
// index) and returns K*, the length of the shortest prefix whose fp32 running sum
// reaches tau_cov (nb if none does).  Called by the whole workgroup, nb >= 1; the
// result is uniform.  The running sum is one thread's sequential fp32 additions, so
// the choice is reproducible bit for bit.
__device__ int sorted_top(const AdaptArgs& a, int row, int nb, unsigned long long* key, int* kstar) {
  const int t = threadIdx.x;
  {
    // Peaked heads first: up to FAST extractions of the largest remaining key (each thread
    // holds up to 16 keys of blocks t, t + 256, ...; a wave reduction, then the four waves'
    // best through LDS), the same additions in the same order as the walk over the sorted
    // keys below.  Heads that are still short of tau_cov after FAST blocks take the sort.
    constexpr int FAST = 32, PER = MAX_SELECT_BLOCKS / NTA;
    __shared__ unsigned long long wbest[NTA / 64];
    const float* mf = a.mass + (size_t)row * a.nt;
    unsigned long long mine[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int j = t + NTA * i;
      mine[i] = j < nb ? (((unsigned long long)__float_as_uint(mf[j]) << 32) | (0xFFFFFFFFu - (uint32_t)j)) : 0ull;
    }
    float run = 0.0f;
    int k = 0;
    bool done = false;
    while (!done && k < FAST && k < nb) {
      unsigned long long best = 0ull;
#pragma unroll
      for (int i = 0; i < PER; ++i) best = mine[i] > best ? mine[i] : best;
      for (int o = 1; o < 64; o <<= 1) {
        const unsigned long long other = __shfl_xor(best, o);
        best = other > best ? other : best;
      }
      if ((t & 63) == 0) wbest[t >> 6] = best;
      __syncthreads();
#pragma unroll
      for (int w = 0; w < NTA / 64; ++w) best = wbest[w] > best ? wbest[w] : best;
      __syncthreads();  // wbest is rewritten by the next round
#pragma unroll
      for (int i = 0; i < PER; ++i)
        if (mine[i] == best) mine[i] = 0ull;  // keys are distinct: only the owner matches
      if (t == 0) key[k] = best;
      run = run + __uint_as_float((uint32_t)(best >> 32));
      ++k;
      done = run >= a.tau_cov;
    }
    if (done || k == nb) {
      if (t == 0) *kstar = k;
      __syncthreads();
      return *kstar;
    }
  }
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
    *kstar = k;
  }
  __syncthreads();
  return *kstar;
}
__device__ __forceinline__ int block_of_key(unsigned long long k) { return (int)(0xFFFFFFFFu - (uint32_t)k); }

__global__ __launch_bounds__(NTA) void select_kernel(AdaptArgs a) {
  __shared__ unsigned long long key[MAX_SELECT_BLOCKS];
  __shared__ int kstar;
  const int row = blockIdx.x, b = row / a.Hq, h = (row % a.Hq) / a.G;
  const int nb = (a.seq.v[b] + TILE - 1) / TILE;
  if (nb == 0) return;  // uniform
  const int K = sorted_top(a, row, nb, key, &kstar);
  uint8_t* fl = a.flags_out + ((size_t)b * a.H + h) * a.nt;
  for (int j = threadIdx.x; j < K; j += NTA) {
    const int blk = block_of_key(key[j]);
    KVQ_DCHECK(blk >= 0 && blk < nb, DBG_CHUNK, row, blk);
    fl[blk] = (uint8_t)(fl[blk] | 1);
  }
}

// Value promotion (rung 2): a block without bit 0 gets bit 1 when mass * ev (fp32) of
// some query head of its kv head exceeds tau_v.  One thread per (sequence, kv head,
// block), in place.
__global__ __launch_bounds__(NTA) void promote_kernel(AdaptArgs a) {
  const size_t n = (size_t)a.B * a.H * a.nt;
  for (size_t idx = (size_t)blockIdx.x * NTA + threadIdx.x; idx < n; idx += (size_t)gridDim.x * NTA) {
    const int jb = (int)(idx % a.nt);
    const size_t bh = idx / a.nt;
    const int h = (int)(bh % a.H), b = (int)(bh / a.H);
    if (jb >= (a.seq.v[b] + TILE - 1) / TILE) continue;
    const uint8_t f = a.flags_out[idx];
    if (f & 1) continue;
    const float ev = a.desc[idx * 3 + 1];
    const float* m = a.mass + ((size_t)b * a.Hq + (size_t)h * a.G) * a.nt + jb;
    bool up = false;
    for (int g = 0; g < a.G; ++g) up = up || __fmul_rn(m[(size_t)g * a.nt], ev) > a.tau_v;
    if (up) a.flags_out[idx] = (uint8_t)(f | 2);
  }
}

// Ranking-consistency check of one (sequence, query head): its promoted blocks (the
// top-K* of its masses, in that order) are scored from the fp16 originals, score =
// log sum_t exp(scale q . k_t) over the block's positions (fp32), and the pairs (i, j),
// i ranked before j, with score_j > score_i + margin are counted; the head fails when
// the count exceeds max_inv.  Wave w scores ranks w, w + 4, ... (lane = token); the
// pairs are counted by thread in columns j.
__global__ __launch_bounds__(NTA) void rank_kernel(AdaptArgs a) {
  __shared__ unsigned long long key[MAX_SELECT_BLOCKS];
  __shared__ float sc[MAX_SELECT_BLOCKS];
  __shared__ float qs[D];
  __shared__ int kstar, count;
  const int row = blockIdx.x, b = row / a.Hq, hq = row % a.Hq, h = hq / a.G;
  const int t = threadIdx.x, wv = t >> 6, lane = t & 63;
  const int T = a.seq.v[b];
  const int nb = (T + TILE - 1) / TILE;
  if (nb == 0) {  // uniform: no promoted blocks
    if (t == 0) {
      a.inv[row] = 0;
      a.fail[row] = 0;
    }
    return;
  }
  const bool bf16 = a.in_bf16 != 0;
  if (t < D) qs[t] = widen(a.q[(size_t)row * D + t], bf16) * a.scale;
  if (t == 0) count = 0;
  const int K = sorted_top(a, row, nb, key, &kstar);  // (its barriers publish qs and count)
  const size_t stream = (size_t)b * a.H + h;
  for (int i = wv; i < K; i += NTA / 64) {
    const int tok = block_of_key(key[i]) * TILE + lane;
    KVQ_DCHECK(stream < (size_t)a.B * a.H && tok >= 0 && tok < nb * TILE && nb <= a.nt, DBG_CHUNK, stream, tok);
    float lg = NEG_INF_A;
    if (tok < T) {
      const uint4* kp = reinterpret_cast<const uint4*>(a.k_orig + (stream * a.Tmax + tok) * D);
      uint4 kr[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) kr[e] = kp[e];
      lg = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const uint32_t w4[4] = {kr[e].x, kr[e].y, kr[e].z, kr[e].w};
#pragma unroll
        for (int x = 0; x < 4; ++x) {
          const int ch = 8 * e + 2 * x;
          lg = fmaf(qs[ch], widen((uint16_t)(w4[x] & 0xFFFF), bf16), lg);
          lg = fmaf(qs[ch + 1], widen((uint16_t)(w4[x] >> 16), bf16), lg);
        }
      }
    }
    const float mx = wmax(lg);  // a promoted block holds at least one position below T
    const float se = wsum(tok < T ? expf(lg - mx) : 0.0f);
    if (lane == 0) sc[i] = mx + logf(se);
  }
  __syncthreads();
  int n = 0;
  for (int jj = t; jj < K; jj += NTA) {
    const float sj = sc[jj];
    for (int i = 0; i < jj; ++i) n += sj > sc[i] + a.margin ? 1 : 0;
  }
  for (int o = 1; o < 64; o <<= 1) n += __shfl_xor(n, o);
  if (lane == 0) atomicAdd(&count, n);
  __syncthreads();
  if (t == 0) {
    a.inv[row] = count;
    a.fail[row] = count > a.max_inv ? 1 : 0;
  }
}

}  // namespace

hipError_t launch_block_mass(const AdaptArgs& a, hipStream_t s) {
  const int HG = (a.G + 3) / 4;
  int max_chunks = 0;
  for (int b = 0; b < a.B; ++b) max_chunks = max(max_chunks, (a.seq.v[b] + TILE - 1) / TILE);
  if (max_chunks > 0) {
    // one workgroup per (unit, split): enough splits for ~512 workgroups (two per CU),
    // >= 32 blocks each
    AdaptArgs b = a;
    const int units = a.B * a.H * HG;
    int S = (512 + units - 1) / units;
    S = std::max(1, std::min(S, max_chunks / 32));
    b.score_splits = S;
    b.score_cps = (max_chunks + S - 1) / S;
    const dim3 grid(units * S);
#define KVQ_SCORE(KF, KG)                                                          \
    if (a.k_fmt == KF && a.k_group == KG) {                                        \
      hipLaunchKernelGGL((score_kernel<KF, KG>), grid, dim3(NTW), 0, s, b);        \
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

hipError_t launch_promote_values(const AdaptArgs& a, hipStream_t s) {
  const size_t n = (size_t)a.B * a.H * a.nt;
  hipLaunchKernelGGL(promote_kernel, dim3((unsigned)std::min<size_t>((n + NTA - 1) / NTA, 4096)), dim3(NTA), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_ranking_check(const AdaptArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(rank_kernel, dim3(a.B * a.Hq), dim3(NTA), 0, s, a);
  return hipGetLastError();
}

#ifdef KVQ_DEBUG
KVQ_DBG_READER(dbg_read_adaptive)
#endif

}  // namespace kvq
