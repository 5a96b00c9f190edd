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
    // y = R q, R the packed unitary DFT times diag(s): lane l forms X_l (lane 0: X_0, X_64)
    tmp[2 * l] = a.signs[2 * l] < 0 ? -x0 : x0;
    tmp[2 * l + 1] = a.signs[2 * l + 1] < 0 ? -x1 : x1;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xc07f);
    float re = 0.0f, im = 0.0f, y0, y1;
    if (l == 0) {
      for (int n = 0; n < D; n += 2) {
        re += tmp[n] + tmp[n + 1];
        im += tmp[n] - tmp[n + 1];
      }
      const float c0 = bits_to_f32(KVQ_INV_SQRT_D_BITS);
      y0 = re * c0;
      y1 = im * c0;
    } else {
      for (int n = 0; n < D; ++n) {
        const int ix = (l * n) & 127;
        re = fmaf(tmp[n], ctab[ix], re);
        im = fmaf(tmp[n], ctab[(ix + 96) & 127], im);
      }
      y0 = re * 0.125f;
      y1 = -im * 0.125f;
    }
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

typedef float v2f __attribute__((ext_vector_type(2)));

// the two E2M1 codes of byte s of w as floats (the selector must be a constant)
__device__ __forceinline__ v2f fp4_byte(uint32_t w, int s) {
  switch (s) {
    case 0: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    case 1: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    case 2: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    default: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
  }
}

// Dequantized key channel values times the rotated query, summed per head:
// acc[h] += sum_c qr[h][c] * k_hat[c] for the token's packed row.  Codes enter as
// exact small floats; each group's sum is scaled once (INT2: plus offset times the
// group's query sum, qsum[h][g]).  All four heads are computed (rows past the
// group's last query head are zero).
// One token's packed key row and its metadata, in registers.
template <int KF, int KG>
struct KeyRow {
  static constexpr int NW = D * fmt_bits(KF) / 32;                   // 32-bit words of codes
  static constexpr int NM = (meta_bytes(KF, fmt_group(KF, KG)) + 3) / 4;  // 32-bit words of metadata
  uint32_t w[NW];
  uint32_t m[NM];
};

template <int KF, int KG>
__device__ __forceinline__ void load_key_row(const uint8_t* row, const uint8_t* meta, KeyRow<KF, KG>& r) {
  const uint4* rp = reinterpret_cast<const uint4*>(row);
#pragma unroll
  for (int i = 0; i < KeyRow<KF, KG>::NW / 4; ++i) {
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

// Dequantized key channel values times the rotated query, summed per head:
// acc[h] = sum_c qr[h][c] * k_hat[c].  Codes enter as exact small floats; each
// group's sum is scaled once (INT2: plus offset times the group's query sum,
// qsum[h][g]).  All four heads are computed (rows past the group's last query
// head are zero).
template <int KF, int KG>
__device__ __forceinline__ void key_dot(const KeyRow<KF, KG>& r, const float (*qr)[D], const float (*qsum)[4],
                                        float acc[4]) {
  constexpr int GS = fmt_group(KF, KG);  // channels per scale
  constexpr int NG = D / GS;
  float sc[NG], z[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    if constexpr (KF == KVQ_FP4) {
      sc[g] = e4m3_value((r.m[g >> 2] >> (8 * (g & 3))) & 0xFFu);
    } else {
      sc[g] = f16_bits_to_f32((uint16_t)(r.m[g >> 1] >> (16 * (g & 1))));
      if constexpr (KF == KVQ_INT2) z[g] = f16_bits_to_f32((uint16_t)(r.m[(NG + g) >> 1] >> (16 * ((NG + g) & 1))));
    }
  }
  constexpr int CPW = 32 / fmt_bits(KF);  // channels per 32-bit word
#pragma unroll
  for (int h = 0; h < 4; ++h) acc[h] = 0.0f;
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    float ag[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int c = g * GS; c < (g + 1) * GS; ++c) {
      const uint32_t ww = r.w[c / CPW];
      const int n = c % CPW;
      float v;
      if constexpr (KF == KVQ_INT4) {
        v = (float)(((int)(ww << (28 - 4 * n))) >> 28);
      } else if constexpr (KF == KVQ_INT8) {
        v = (float)(((int)(ww << (24 - 8 * n))) >> 24);
      } else if constexpr (KF == KVQ_INT2) {
        v = (float)((ww >> (2 * n)) & 3u);
      } else {  // FP4: the gfx950 conversion of the two E2M1 codes of one byte (exact, scale 1)
        if ((n & 1) != 0) continue;  // both channels of the byte are taken at the even one
        const v2f p = fp4_byte(ww, n >> 1);
#pragma unroll
        for (int h = 0; h < 4; ++h) ag[h] = fmaf(qr[h][c + 1], p.y, fmaf(qr[h][c], p.x, ag[h]));
        continue;
      }
#pragma unroll
      for (int h = 0; h < 4; ++h) ag[h] = fmaf(qr[h][c], v, ag[h]);
    }
#pragma unroll
    for (int h = 0; h < 4; ++h) {
      acc[h] = fmaf(ag[h], sc[g], acc[h]);
      if constexpr (KF == KVQ_INT2) acc[h] = fmaf(qsum[h][g], z[g], acc[h]);
    }
  }
}

// Scoring pass: log of the softmax numerator mass of every 64-token block,
// lse_b = log sum_{t in b} exp(scale * q_rot . k_hat_t), per query head.  One
// workgroup per (4 blocks, kv head, group of 4 query heads, sequence), one wave
// per block, one lane per token.  Written into mass, normalised by mass_kernel.
// (VALU-bound: about 1000 vector instructions per block and wave, most of them the
// 512 fma of four heads times 128 channels.)
template <int KF, int KG>
__global__ __launch_bounds__(NTA) void score_kernel(AdaptArgs a) {
  __shared__ float qr[4][D];
  __shared__ float tmp[4][D];
  __shared__ float qsum[4][4];  // per head, per 32-channel group (INT2 offsets)
  __shared__ float ctab[128];   // cos(2 pi k / 128) (SRFT)
  const int b = blockIdx.z;
  const int HG = (a.G + 3) >> 2;
  const int hkv = blockIdx.y / HG, hg = blockIdx.y % HG;
  const int hq0 = hkv * a.G + hg * 4;
  const int nh = min(4, a.G - hg * 4);
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int T = a.seq.v[b];
  const int nchunks = (T + TILE - 1) / TILE;
  if ((int)blockIdx.x * 4 >= nchunks) return;  // uniform over the workgroup
  if (a.rotation == KVQ_ROT_SRFT) {
    if (threadIdx.x < 128) ctab[threadIdx.x] = a.cos128[threadIdx.x];
    __syncthreads();
  }
  if (wv < nh) {
    rotated_query(a, b, hq0 + wv, qr[wv], tmp[wv], ctab);
    if (a.lam_k != nullptr) {  // keys were stored times lambda_k
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_s_waitcnt(0xc07f);
      const float* lp = a.lam_k + (size_t)hkv * D;
      qr[wv][2 * lane] = qr[wv][2 * lane] / lp[2 * lane];
      qr[wv][2 * lane + 1] = qr[wv][2 * lane + 1] / lp[2 * lane + 1];
    }
  } else {
    qr[wv][2 * lane] = 0.0f;
    qr[wv][2 * lane + 1] = 0.0f;
  }
  if constexpr (KF == KVQ_INT2) {
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0xc07f);
    float v = qr[wv][2 * lane] + qr[wv][2 * lane + 1];  // lanes 16g..16g+15 hold group g
    for (int o = 1; o < 16; o <<= 1) v += __shfl_xor(v, o);
    if ((lane & 15) == 0) qsum[wv][lane >> 4] = v;
  }
  __syncthreads();
  const int c = blockIdx.x * 4 + wv;
  if (c >= nchunks) return;  // no barrier follows
  constexpr int KB = row_bytes(KF);
  constexpr int KM = meta_bytes(KF, fmt_group(KF, KG));
  const size_t stream = (size_t)b * a.H + hkv;
  const int t = c * TILE + lane;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (t < T) {
    KeyRow<KF, KG> R;
    load_key_row<KF, KG>(a.k_codes + (stream * a.Tmax + t) * KB, a.k_meta + (stream * a.Tmax + t) * KM, R);
    key_dot<KF, KG>(R, qr, qsum, acc);
  }
#pragma unroll
  for (int h = 0; h < 4; ++h) {
    if (h >= nh) break;
    const float l = t < T ? acc[h] : NEG_INF_A;
    const float m = wmax(l);
    const float s = wsum(t < T ? expf(l - m) : 0.0f);
    if (lane == 0) a.mass[((size_t)b * a.Hq + hq0 + h) * a.nt + c] = m + logf(s);
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
    const dim3 grid((max_chunks + 3) / 4, a.H * HG, a.B);
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
