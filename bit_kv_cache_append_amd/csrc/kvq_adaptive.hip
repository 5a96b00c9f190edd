// Adaptive precision of "Runtime-Certified Bounded-Error Quantized Attention",
// Methodology section 3: a light scoring pass estimates every block's attention
// mass from the quantized keys, the top-K* blocks covering a fraction tau_cov of
// it are promoted to the full-precision originals (through the decode pass's
// exact-recompute flags), and a head whose certificate still exceeds a tolerance
// is recomputed with dense attention over the originals.
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
__device__ __forceinline__ void rotated_query(const AdaptArgs& a, int b, int hq, float* dst, float* tmp) {
  const int l = threadIdx.x & 63;
  const bool bf16 = a.in_bf16 != 0;
  const uint16_t* qp = a.q + ((size_t)b * a.Hq + hq) * D;
  float x0 = widen(qp[2 * l], bf16), x1 = widen(qp[2 * l + 1], bf16);
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

// Dequantized key channel values times the rotated query, summed per head:
// acc[h] += sum_c qr[h][c] * k_hat[c] for the token's packed row.
template <int KF, int KG>
__device__ __forceinline__ void key_dot(const uint8_t* row, const uint8_t* meta, const float (*qr)[D], int nh,
                                        float acc[4]) {
  auto add = [&](int c, float v) {
#pragma unroll
    for (int h = 0; h < 4; ++h)
      if (h < nh) acc[h] = fmaf(qr[h][c], v, acc[h]);
  };
  if constexpr (KF == KVQ_INT4 || KF == KVQ_INT8) {
    constexpr int NG = D / KG;
    const uint16_t* mp = reinterpret_cast<const uint16_t*>(meta);
    float sc[NG];
#pragma unroll
    for (int g = 0; g < NG; ++g) sc[g] = f16_bits_to_f32(mp[g]);
    constexpr int NW = KF == KVQ_INT4 ? 16 : 32;  // 32-bit words per row
    const uint4* rp = reinterpret_cast<const uint4*>(row);
#pragma unroll
    for (int i = 0; i < NW / 4; ++i) {
      const uint4 u = rp[i];
      const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = w4[e];
        if constexpr (KF == KVQ_INT4) {
#pragma unroll
          for (int n = 0; n < 8; ++n) {
            const int c = (4 * i + e) * 8 + n;
            const int code = ((int)(w << (28 - 4 * n))) >> 28;
            add(c, (float)code * sc[c / KG]);
          }
        } else {
#pragma unroll
          for (int n = 0; n < 4; ++n) {
            const int c = (4 * i + e) * 4 + n;
            const int code = ((int)(w << (24 - 8 * n))) >> 24;
            add(c, (float)code * sc[c / KG]);
          }
        }
      }
    }
  } else if constexpr (KF == KVQ_INT2) {
    const uint16_t* mp = reinterpret_cast<const uint16_t*>(meta);
    float sc[4], z[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      sc[g] = f16_bits_to_f32(mp[g]);
      z[g] = f16_bits_to_f32(mp[4 + g]);
    }
    const uint4* rp = reinterpret_cast<const uint4*>(row);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const uint4 u = rp[i];
      const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e)
#pragma unroll
        for (int n = 0; n < 16; ++n) {
          const int c = (4 * i + e) * 16 + n;
          const float code = (float)((w4[e] >> (2 * n)) & 3u);
          add(c, fmaf(code, sc[c / 32], z[c / 32]));
        }
    }
  } else {  // FP4: E2M1 nibbles (even channel in the low nibble), one E4M3 scale per 16 channels
    float sc[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) sc[g] = e4m3_value(meta[g]);
    const uint4* rp = reinterpret_cast<const uint4*>(row);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 u = rp[i];
      const uint32_t w4[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int c0 = (4 * i + e) * 8;
        const float s = sc[c0 / 16];
        // the gfx950 conversion of the two E2M1 codes of one byte (exact, scale 1)
        const v2f r0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w4[e], 1.0f, 0);
        const v2f r1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w4[e], 1.0f, 1);
        const v2f r2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w4[e], 1.0f, 2);
        const v2f r3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w4[e], 1.0f, 3);
        add(c0 + 0, r0.x * s); add(c0 + 1, r0.y * s);
        add(c0 + 2, r1.x * s); add(c0 + 3, r1.y * s);
        add(c0 + 4, r2.x * s); add(c0 + 5, r2.y * s);
        add(c0 + 6, r3.x * s); add(c0 + 7, r3.y * s);
      }
    }
  }
}

// Scoring pass: log of the softmax numerator mass of every 64-token block,
// lse_b = log sum_{t in b} exp(scale * q_rot . k_hat_t), per query head.  One
// workgroup per (4 blocks, kv head, group of 4 query heads, sequence); one wave
// per block, one lane per token.  Written into mass, normalised by mass_kernel.
template <int KF, int KG>
__global__ __launch_bounds__(NTA) void score_kernel(AdaptArgs a) {
  __shared__ float qr[4][D];
  __shared__ float tmp[4][D];
  const int b = blockIdx.z;
  const int HG = (a.G + 3) >> 2;
  const int hkv = blockIdx.y / HG, hg = blockIdx.y % HG;
  const int hq0 = hkv * a.G + hg * 4;
  const int nh = min(4, a.G - hg * 4);
  const int wv = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int T = a.seq.v[b];
  const int nchunks = (T + TILE - 1) / TILE;
  if ((int)blockIdx.x * 4 >= nchunks) return;  // uniform over the workgroup
  if (wv < nh) rotated_query(a, b, hq0 + wv, qr[wv], tmp[wv]);
  __syncthreads();
  const int c = blockIdx.x * 4 + wv;
  if (c >= nchunks) return;  // no barrier follows
  constexpr int KB = row_bytes(KF);
  constexpr int KM = meta_bytes(KF, KG);
  const size_t stream = (size_t)b * a.H + hkv;
  const int t = c * TILE + lane;
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  if (t < T) key_dot<KF, KG>(a.k_codes + (stream * a.Tmax + t) * KB, a.k_meta + (stream * a.Tmax + t) * KM, qr, nh, acc);
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

// Promotion flags of one (sequence, kv head): for each of its query heads, the
// blocks sorted by decreasing mass (equal masses: lower index first) and the
// shortest prefix whose fp32 running sum, taken in that order, reaches tau_cov;
// the union over the query heads, OR the flags given.  The running sum is one
// thread's sequential fp32 additions, so the choice is reproducible bit for bit.
__global__ __launch_bounds__(NTA) void select_kernel(AdaptArgs a) {
  __shared__ unsigned long long key[MAX_SELECT_BLOCKS];
  __shared__ uint8_t fl[MAX_SELECT_BLOCKS];
  __shared__ int kstar;
  const int b = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int t = threadIdx.x;
  const int nb = (a.seq.v[b] + TILE - 1) / TILE;
  const size_t base = ((size_t)b * a.H + h) * a.nt;
  for (int j = t; j < a.nt; j += NTA) fl[j] = (a.flags_in != nullptr && a.flags_in[base + j] != 0) ? 1 : 0;
  int npow = 2;
  while (npow < nb) npow <<= 1;
  for (int g = 0; g < a.G && nb > 0; ++g) {
    const float* m = a.mass + ((size_t)b * a.Hq + h * a.G + g) * a.nt;
    __syncthreads();
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
      float run = 0.0f;
      int k = 0;
      while (k < nb) {
        run = run + __uint_as_float((uint32_t)(key[k] >> 32));
        ++k;
        if (run >= a.tau_cov) break;
      }
      kstar = k;
    }
    __syncthreads();
    for (int j = t; j < kstar; j += NTA) fl[0xFFFFFFFFu - (uint32_t)key[j]] = 1;
  }
  __syncthreads();
  for (int j = t; j < a.nt; j += NTA) a.flags_out[base + j] = fl[j];
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
    KVQ_SCORE(KVQ_INT4, 32) KVQ_SCORE(KVQ_INT4, 128) KVQ_SCORE(KVQ_INT8, 32) KVQ_SCORE(KVQ_INT8, 128)
    KVQ_SCORE(KVQ_INT2, 32) KVQ_SCORE(KVQ_FP4, 16) { return hipErrorNotSupported; }
#undef KVQ_SCORE
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(mass_kernel, dim3(a.B * a.Hq), dim3(NTA), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_select(const AdaptArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(select_kernel, dim3(a.B * a.H), dim3(NTA), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_fallback(const AdaptArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(fallback_kernel, dim3(a.B * a.Hq), dim3(NTA), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvq
