// Write side: rotate, scale, quantize and pack new K/V head vectors into the cache.
//
// One workgroup (256 threads) handles the tokens of one 64-token tile of one
// (sequence, kv head) for one tensor (K or V).  Thread t owns token tau = t / 4
// and the 32 channels [32q, 32q + 32), q = t % 4, so a quad of lanes holds one
// vector.  The rotation follows "When Quantization Is Free", Methodology
// sections 1-2 (sign flip then a fast orthogonal transform, in registers): the
// Walsh-Hadamard butterflies with stride 1..16 are in-lane, strides 32 and 64
// are lane exchanges inside the quad (DPP).  The dense rotation ("OSCAR",
// section 2.2A) is a fixed-order fp32 multiply-add chain per output, with each
// lane owning two matrix rows in registers and the inputs broadcast from LDS.
//
// Bit-exactness: this file is compiled with -ffp-contract=off; every rounding
// is an explicit fp32 add/sub/mul (or fma where the product is exact), in the
// order the oracle uses.  Codes are the round-half-to-even of the exact
// quotient by the stored scale (residual check with an exact fma).
//
// K rows are written straight from registers.  V codes go through LDS and are
// transposed into the channel-major 64-token tile; bytes of the tile shared with
// tokens outside this call are read, merged and written back.

#include "kvq_common.h"

#include <algorithm>
#include <type_traits>

namespace kvq {

namespace {

constexpr int NT = 256;

// ---------------------------------------------------------------- load / rotate
__device__ __forceinline__ void load32(const uint16_t* src, bool bf16, float v[32]) {
  const uint4* p = reinterpret_cast<const uint4*>(src);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint4 w = p[i];
    uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[8 * i + 2 * j] = widen((uint16_t)(ws[j] & 0xFFFF), bf16);
      v[8 * i + 2 * j + 1] = widen((uint16_t)(ws[j] >> 16), bf16);
    }
  }
}

// sign flip + Walsh-Hadamard, stages h = 1..64 in order, then * fl32(1/sqrt(128))
__device__ __forceinline__ void sign_fwht(float v[32], const int8_t* signs, int q) {
  const int8_t* s = signs + 32 * q;
#pragma unroll
  for (int j = 0; j < 32; ++j) v[j] = s[j] < 0 ? -v[j] : v[j];
#pragma unroll
  for (int h = 1; h < 32; h *= 2) {
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if ((j & h) == 0) {
        float a = v[j], b = v[j + h];
        v[j] = a + b;
        v[j + h] = a - b;
      }
    }
  }
  // stride 32: partner lane q^1 ; stride 64: partner lane q^2
  {
    bool up = (q & 1) != 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      float p = dpp_f<KVQ_DPP_XOR1>(v[j]);
      v[j] = up ? (p - v[j]) : (v[j] + p);
    }
  }
  {
    bool up = (q & 2) != 0;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      float p = dpp_f<KVQ_DPP_XOR2>(v[j]);
      v[j] = up ? (p - v[j]) : (v[j] + p);
    }
  }
  const float c = bits_to_f32(KVQ_INV_SQRT_D_BITS);
#pragma unroll
  for (int j = 0; j < 32; ++j) v[j] = v[j] * c;
}

// ---------------------------------------------------------------- exact rounding
// round-half-to-even of the exact quotient y / sf, sf > 0 an fp16 value, r = fl32(1/sf)
__device__ __forceinline__ float rne_quot(float y, float sf, float r) {
  float c = rintf(y * r);             // within +-1 of the answer
  float e = __builtin_fmaf(-c, sf, y);  // exact residual y - c*sf where it matters
  float h = 0.5f * sf;
  if (e > h) {
    c += 1.0f;
  } else if (e < -h) {
    c -= 1.0f;
  } else if (e == h || e == -h) {  // y/sf is exactly c +- 1/2: keep the even neighbour
    if (__builtin_fmodf(c, 2.0f) != 0.0f) c += (e > 0.0f ? 1.0f : -1.0f);
  }
  return c;
}

// ---------------------------------------------------------------- quantizers
// Each returns packed code dwords for the lane's 32 channels, writes metadata
// elements (fp16 bits or E4M3 codes) and the squared-residual partial sum (each
// residual times il[j] when il is given: with per-channel factors lambda, il = 1 /
// lambda takes the residual back to the unscaled basis).

// symmetric int4/int8; group 16 (two per lane), 32 (in-lane) or 128 (quad).
// meta0/meta1: the scales of channels 0..15 and 16..31 of the lane (equal unless group 16)
__device__ __forceinline__ void quant_sym(const float y[32], int qmax, int group, int codes[32],
                                          uint16_t& meta0, uint16_t& meta1, float& res2, const float* il) {
  float a[2] = {0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < 32; ++j) a[j >> 4] = fmaxf(a[j >> 4], fabsf(y[j]));
  if (group != 16) {
    a[0] = fmaxf(a[0], a[1]);  // max is exact: any order gives the group's absmax
    if (group == 128) {
      a[0] = fmaxf(a[0], dpp_f<KVQ_DPP_XOR1>(a[0]));
      a[0] = fmaxf(a[0], dpp_f<KVQ_DPP_XOR2>(a[0]));
    }
    a[1] = a[0];
  }
  uint16_t sb[2];
  float sf[2], r[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    sb[i] = f16_sat_bits(a[i] / (float)qmax);  // correctly rounded fp32 divide
    sf[i] = f16_bits_to_f32(sb[i]);
    r[i] = __builtin_amdgcn_rcpf(sf[i]);
  }
  meta0 = sb[0];
  meta1 = sb[1];
  float qm = (float)qmax;
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    const float s = sf[j >> 4];
    float c = 0.0f;
    if (s != 0.0f) c = fminf(fmaxf(rne_quot(y[j], s, r[j >> 4]), -qm), qm);
    codes[j] = (int)c;
    float d = y[j] - c * s;
    if (il) d = d * il[j];
    acc = acc + d * d;
  }
  res2 = acc;
}

// asymmetric int2, group 32, optional clamp to [-t_c, t_c] first
__device__ __forceinline__ void quant_asym2(const float y[32], const float* clip, int codes[32], uint16_t& ms,
                                            uint16_t& mz, float& res2, const float* il) {
  float yc[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    float v = y[j];
    if (clip) {
      float t = clip[j];
      v = fminf(fmaxf(v, -t), t);
    }
    yc[j] = v;
  }
  float lo = yc[0], hi = yc[0];
#pragma unroll
  for (int j = 1; j < 32; ++j) {
    lo = fminf(lo, yc[j]);
    hi = fmaxf(hi, yc[j]);
  }
  float rng = hi - lo;
  uint16_t sb = f16_sat_bits(rng / 3.0f);
  uint16_t zb = f16_sat_bits(lo);
  float sf = f16_bits_to_f32(sb), zf = f16_bits_to_f32(zb);
  ms = sb;
  mz = zb;
  float r = __builtin_amdgcn_rcpf(sf);
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    float c = 0.0f;
    if (sf != 0.0f) {
      float rr = yc[j] - zf;
      c = fminf(fmaxf(rne_quot(rr, sf, r), 0.0f), 3.0f);
    }
    codes[j] = (int)c;
    float d = y[j] - (c * sf + zf);  // residual against the unclipped value
    if (il) d = d * il[j];
    acc = acc + d * d;
  }
  res2 = acc;
}

// E2M1 magnitude of index 0..7: 0, 0.5, 1, 1.5, 2, 3, 4, 6 (selects, no table)
__device__ __forceinline__ float e2m1_mag(int idx) {
  float v = 0.5f * (float)(idx < 4 ? idx : 4);
  v = idx >= 5 ? v + 1.0f : v;
  v = idx >= 6 ? v + 1.0f : v;
  v = idx >= 7 ? v + 2.0f : v;
  return v;
}

// FP4 E2M1 codes for one block of 16 with scale S (> 0): nibble codes, value*S and err
__device__ __forceinline__ float fp4_block(const float* y, float S, int* codes, bool want_codes) {
  // thresholds between E2M1 magnitudes, times S (exact products)
  const float t0 = 0.25f * S, t1 = 0.75f * S, t2 = 1.25f * S, t3 = 1.75f * S, t4 = 2.5f * S, t5 = 3.5f * S,
              t6 = 5.0f * S;
  float lo = 0.0f, hi = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    float ay = fabsf(y[j]);
    // ties go to the even code: strict '>' above an even code, '>=' above an odd one
    int idx = (ay > t0) + (ay >= t1) + (ay > t2) + (ay >= t3) + (ay > t4) + (ay >= t5) + (ay > t6);
    float q = e2m1_mag(idx) * S;  // exact
    float d = ay - q;
    float sq = d * d;
    if (j < 8)
      lo = lo + sq;
    else
      hi = hi + sq;
    if (want_codes) codes[j] = ((__float_as_uint(y[j]) >> 31) << 3) | idx;
  }
  return lo + hi;
}

__device__ __forceinline__ float fp4_zero_err(const float* y) {
  float lo = 0.0f, hi = 0.0f;
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    float sq = y[j] * y[j];
    if (j < 8)
      lo = lo + sq;
    else
      hi = hi + sq;
  }
  return lo + hi;
}

// FP4 with E4M3 block scales (two blocks of 16 per lane).  Candidates: E4M3(t * m_k) for the
// multiplicative search, the bit patterns c0 - 2 .. c0 + 6 of c0 = E4M3(t) (kept inside
// 0x00..0x7E) for the offset search, c0 alone for absmax.
__device__ __forceinline__ void quant_fp4(const float y[32], int mode, int codes[32], uint8_t sc[2],
                                          float& res2, const float* il) {
  const float mults[9] = {0.9f, 0.925f, 0.95f, 0.975f, 1.0f, 1.025f, 1.05f, 1.075f, 1.1f};
  float acc = 0.0f;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const float* yb = y + 16 * blk;
    float a = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) a = fmaxf(a, fabsf(yb[j]));
    float t = a / 6.0f;
    uint32_t best_c = 0;
    float best_e = 0.0f;
    bool have = false;
    uint32_t prev_c = 0xFFFFFFFFu;
    const int c0 = (int)e4m3_encode_nonneg(t);
#pragma unroll
    for (int k = 0; k < 9; ++k) {
      if (mode == KVQ_SCALE_ABSMAX && k != 4) continue;
      uint32_t c = mode == KVQ_SCALE_SEARCH_OFFSETS ? (uint32_t)min(max(c0 + k - 2, 0), 0x7E)
                                                    : e4m3_encode_nonneg(t * mults[k]);
      if (c == prev_c) continue;  // same stored scale as the previous candidate: same error
      prev_c = c;
      float S = e4m3_value(c);
      float err = (S == 0.0f) ? fp4_zero_err(yb) : fp4_block(yb, S, nullptr, false);
      if (!have || err < best_e) {
        best_e = err;
        best_c = c;
        have = true;
      }
    }
    sc[blk] = (uint8_t)best_c;
    float S = e4m3_value(best_c);
    if (S == 0.0f) {
#pragma unroll
      for (int j = 0; j < 16; ++j) codes[16 * blk + j] = 0;
    } else {
      fp4_block(yb, S, codes + 16 * blk, true);
    }
    // residual for the descriptors
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      int cd = codes[16 * blk + j];
      float v = e2m1_mag(cd & 7) * S;
      float d = fabsf(yb[j]) - v;
      if (il) d = d * il[16 * blk + j];
      acc = acc + d * d;
    }
  }
  res2 = acc;
}

// ---------------------------------------------------------------- packing
__device__ __forceinline__ void pack_row(const int codes[32], int fmt, uint32_t out[8], int& ndw) {
  if (fmt == KVQ_INT8) {
    ndw = 8;
#pragma unroll
    for (int w = 0; w < 8; ++w)
      out[w] = (codes[4 * w] & 0xFF) | ((codes[4 * w + 1] & 0xFF) << 8) | ((codes[4 * w + 2] & 0xFF) << 16) |
               ((uint32_t)(codes[4 * w + 3] & 0xFF) << 24);
  } else if (fmt == KVQ_INT2) {
    ndw = 2;
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      uint32_t x = 0;
#pragma unroll
      for (int e = 0; e < 16; ++e) x |= (uint32_t)(codes[16 * w + e] & 3) << (2 * e);
      out[w] = x;
    }
  } else {
    ndw = 4;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t x = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) x |= (uint32_t)(codes[8 * w + e] & 0xF) << (4 * e);
      out[w] = x;
    }
  }
}

// max over the 16 quads of a wave (value held by every lane of the quad)
__device__ __forceinline__ float wave_quad_max(float v) {
  v = fmaxf(v, __shfl_xor(v, 4));
  v = fmaxf(v, __shfl_xor(v, 8));
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

__device__ __forceinline__ float quad_sum(float v) {
  v = v + dpp_f<KVQ_DPP_XOR1>(v);
  v = v + dpp_f<KVQ_DPP_XOR2>(v);
  return v;
}

struct __align__(16) StageSmem {
  uint8_t codes[TILE][D + 16];  // V codes staged token-major (one code per byte)
  uint16_t meta[TILE][8];       // V metadata elements per token
};
struct __align__(16) DenseSmem {
  uint16_t xs[TILE][D];  // input vectors (fp16/bf16 bits)
  float ys[TILE][D + 4];  // rotated vectors
};
struct __align__(16) SrftSmem {
  float zre[TILE][65], zim[TILE][65];  // the 64 complex points of each vector
  float twr[65], twi[65];              // W128^k
};

// SRFT ("When Quantization Is Free", Methodology sections 1-2) of the vector held by
// a quad (lane q: channels 32q..32q+31), returned in the same layout: the sign flip,
// z_n = u_2n + i u_2n+1 into LDS, six radix-2 Stockham passes of the 64-point FFT
// (lane q computes butterflies 8q..8q+7 of each pass), the Hermitian unpack of
// X_0..X_64 and the orthonormal packing.  All fp32 operations in the stated order
// (this unit is compiled without contraction), so the result is bit-exact.
// Every thread of the workgroup must call it (barriers); sm.twr/twi must be set
// before the call.
__device__ void srft_quad(float v[32], const int8_t* signs, int q, int vec, SrftSmem& sm) {
  const int8_t* s = signs + 32 * q;
#pragma unroll
  for (int j = 0; j < 32; ++j) v[j] = s[j] < 0 ? -v[j] : v[j];
  float* zre = sm.zre[vec];
  float* zim = sm.zim[vec];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    zre[16 * q + e] = v[2 * e];
    zim[16 * q + e] = v[2 * e + 1];
  }
  __syncthreads();
  int lm = 0;  // log2 of the stride m
#pragma unroll
  for (int pass = 0; pass < 6; ++pass, ++lm) {
    const int m = 1 << lm, half = 32 >> lm;  // sub-length L = 64 >> pass, half = L / 2
    float ar[8], ai[8], br[8], bi[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int bf = 8 * q + e, j = bf >> lm, k = bf & (m - 1);
      ar[e] = zre[j * m + k];
      ai[e] = zim[j * m + k];
      br[e] = zre[(j + half) * m + k];
      bi[e] = zim[(j + half) * m + k];
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int bf = 8 * q + e, j = bf >> lm, k = bf & (m - 1);
      const float wr = sm.twr[2 * j * m], wi = sm.twi[2 * j * m];  // W64^(j m) = W128^(2 j m)
      zre[2 * j * m + k] = ar[e] + br[e];
      zim[2 * j * m + k] = ai[e] + bi[e];
      const float dr = ar[e] - br[e], di = ai[e] - bi[e];
      zre[(2 * j + 1) * m + k] = dr * wr - di * wi;
      zim[(2 * j + 1) * m + k] = dr * wi + di * wr;
    }
    __syncthreads();
  }
  // X_k = E + W128^k O with A = Z_k, B = conj(Z_(64-k)), E = (A + B) / 2, O = (A - B) / 2i
  auto unpack = [&](int k, float& xr, float& xi) {
    const int ia = k & 63, ib = (64 - k) & 63;
    const float a_re = zre[ia], a_im = zim[ia];
    const float b_re = zre[ib], b_im = -zim[ib];
    const float e_re = 0.5f * (a_re + b_re), e_im = 0.5f * (a_im + b_im);
    const float o_re = 0.5f * (a_im - b_im), o_im = -(0.5f * (a_re - b_re));
    const float wr = sm.twr[k], wi = sm.twi[k];
    const float t_re = o_re * wr - o_im * wi, t_im = o_re * wi + o_im * wr;
    xr = e_re + t_re;
    xi = e_im + t_im;
  };
  const float c0 = bits_to_f32(KVQ_INV_SQRT_D_BITS);
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int k = 16 * q + e;
    float xr, xi;
    if (k == 0) {
      float nr, ni;
      unpack(0, xr, xi);
      unpack(64, nr, ni);
      v[0] = xr * c0;
      v[1] = nr * c0;
    } else {
      unpack(k, xr, xi);
      v[2 * e] = xr * 0.125f;
      v[2 * e + 1] = xi * 0.125f;
    }
  }
  __syncthreads();  // the rows may be reused
}


// Rows lane and lane + 64 of the dense rotation for the 16 vectors of wave wv, NV
// vectors at a time (2 NV independent fma chains per lane)
template <bool BF16>
__device__ __forceinline__ void dense_rows(const uint16_t (*xs)[D], float (*ys)[D + 4], const uint32_t r0[64],
                                           const uint32_t r1[64], int wv, int lane, int tile0, int lo, int hi) {
  typedef _Float16 hh2 __attribute__((ext_vector_type(2)));
  constexpr int NV = 1;
  for (int v0 = 0; v0 < 16; v0 += NV) {
    const int vec0 = wv * 16 + v0;
    if (tile0 + vec0 + NV <= lo || tile0 + vec0 >= hi) continue;  // uniform over the wave
    float acc0[NV], acc1[NV];
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      acc0[e] = 0.0f;
      acc1[e] = 0.0f;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      uint32_t xw[NV][4];
#pragma unroll
      for (int e = 0; e < NV; ++e) {
        const uint4 u = reinterpret_cast<const uint4*>(&xs[vec0 + e][0])[i];
        xw[e][0] = u.x; xw[e][1] = u.y; xw[e][2] = u.z; xw[e][3] = u.w;
      }
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        const int kp = 4 * i + jj;  // channels 2kp, 2kp+1
        const hh2 ra = __builtin_bit_cast(hh2, r0[kp]), rb = __builtin_bit_cast(hh2, r1[kp]);
#pragma unroll
        for (int e = 0; e < NV; ++e) {
          float x0, x1;
          if constexpr (BF16) {
            x0 = __uint_as_float(xw[e][jj] << 16);
            x1 = __uint_as_float(xw[e][jj] & 0xFFFF0000u);
          } else {
            const hh2 xv = __builtin_bit_cast(hh2, xw[e][jj]);
            x0 = (float)xv.x;
            x1 = (float)xv.y;
          }
          acc0[e] = __builtin_fmaf((float)ra.x, x0, acc0[e]);
          acc1[e] = __builtin_fmaf((float)rb.x, x0, acc1[e]);
          acc0[e] = __builtin_fmaf((float)ra.y, x1, acc0[e]);
          acc1[e] = __builtin_fmaf((float)rb.y, x1, acc1[e]);
        }
      }
    }
#pragma unroll
    for (int e = 0; e < NV; ++e) {
      ys[vec0 + e][lane] = acc0[e];
      ys[vec0 + e][lane + 64] = acc1[e];
    }
  }
}

}  // namespace

template <bool DENSE, bool SRFT>
__global__ __launch_bounds__(NT) void append_kernel(AppendArgs a) {
  __shared__ StageSmem sm;
  const int b = blockIdx.z >> 1, h = blockIdx.y;
  const int tensor = blockIdx.z & 1;  // 0 = K, 1 = V
  const int start = a.start.v[b];
  const int tile = start / TILE + (int)blockIdx.x;
  const int lo = max(start, tile * TILE), hi = min(start + a.n_new, tile * TILE + TILE);
  if (lo >= hi) return;  // uniform over the workgroup
  const int t = threadIdx.x, tau = t >> 2, q = t & 3;
  const int pos = tile * TILE + tau;
  const bool valid = pos >= lo && pos < hi;
  const bool bf16 = a.in_bf16 != 0;
  const int fmt = tensor ? a.v_fmt : a.k_fmt;
  const int group = tensor ? a.v_group : a.k_group;
  const size_t stream_idx = (size_t)b * a.H + h;
  if (valid) KVQ_DCHECK_APPEND(a, stream_idx, pos, start);
  const uint16_t* src_base = tensor ? a.v_new : a.k_new;
  const uint16_t* src = src_base + ((stream_idx * a.n_new + (valid ? pos - start : 0)) * D + 32 * q);

  float x[32];
  if (valid) {
    load32(src, bf16, x);
  } else {
#pragma unroll
    for (int j = 0; j < 32; ++j) x[j] = 0.0f;
  }
  float xnorm2 = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) xnorm2 = xnorm2 + x[j] * x[j];

  float y[32];
  if constexpr (SRFT) {
    __shared__ SrftSmem ss;
    if (t < 65) {
      ss.twr[t] = a.tw_re[t];
      ss.twi[t] = a.tw_im[t];
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) y[j] = x[j];
    srft_quad(y, a.signs, q, tau, ss);
  } else if (a.rotation == KVQ_ROT_SIGN_FWHT) {
#pragma unroll
    for (int j = 0; j < 32; ++j) y[j] = x[j];
    sign_fwht(y, a.signs, q);
  } else if constexpr (DENSE) {
    // stage inputs, then every wave rotates 16 vectors: lane l owns rows l and l+64
    __shared__ DenseSmem sm;
    {
      const uint4* s4 = reinterpret_cast<const uint4*>(src);
      uint4* d4 = reinterpret_cast<uint4*>(&sm.xs[tau][32 * q]);
#pragma unroll
      for (int i = 0; i < 4; ++i) d4[i] = valid ? s4[i] : make_uint4(0, 0, 0, 0);
    }
    __syncthreads();
    const int lane = t & 63, wv = t >> 6;
    uint32_t r0[64], r1[64];  // rows lane and lane+64 as fp16 pairs
    {
      const uint4* ra = reinterpret_cast<const uint4*>(a.rot + (size_t)lane * D);
      const uint4* rb = reinterpret_cast<const uint4*>(a.rot + (size_t)(lane + 64) * D);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        uint4 u = ra[i], w = rb[i];
        r0[4 * i] = u.x; r0[4 * i + 1] = u.y; r0[4 * i + 2] = u.z; r0[4 * i + 3] = u.w;
        r1[4 * i] = w.x; r1[4 * i + 1] = w.y; r1[4 * i + 2] = w.z; r1[4 * i + 3] = w.w;
      }
    }
    // y_j = fma chain over k = 0..127 in order (the oracle's chain); with fp16 inputs
    // both operands go straight into a mixed-precision fma (exact conversions)
    if (bf16)
      dense_rows<true>(sm.xs, sm.ys, r0, r1, wv, lane, tile * TILE, lo, hi);
    else
      dense_rows<false>(sm.xs, sm.ys, r0, r1, wv, lane, tile * TILE, lo, hi);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 32; ++j) y[j] = sm.ys[tau][32 * q + j];
  } else {
#pragma unroll
    for (int j = 0; j < 32; ++j) y[j] = x[j];
  }

  // norm of the rotated vector (descriptor slack), before any rescale
  float ynorm2 = 0.0f;
  if (a.desc) {
#pragma unroll
    for (int j = 0; j < 32; ++j) ynorm2 = ynorm2 + y[j] * y[j];
  }
  // per-channel rescale ("When Quantization Is Free", Methodology sections 2-3), fp32;
  // with descriptors the residuals are taken back to the unscaled basis (times 1 / lambda)
  float ilam[32];
  const float* il = nullptr;
  if (const float* lam = tensor ? a.lam_v : a.lam_k) {
    const float* lp = lam + (size_t)h * D + 32 * q;
#pragma unroll
    for (int j = 0; j < 32; ++j) y[j] = y[j] * lp[j];
    if (a.desc) {
#pragma unroll
      for (int j = 0; j < 32; ++j) ilam[j] = 1.0f / lp[j];
      il = ilam;
    }
  }

  // quantize
  int codes[32];
  uint16_t m0 = 0, m1 = 0;  // metadata elements of this lane
  float res2 = 0.0f;
  if (fmt == KVQ_INT4 || fmt == KVQ_INT8) {
    quant_sym(y, fmt == KVQ_INT4 ? 7 : 127, group, codes, m0, m1, res2, il);
  } else if (fmt == KVQ_INT2) {
    const float* clip = tensor ? a.clip_v : a.clip_k;
    quant_asym2(y, clip ? clip + (size_t)h * D + 32 * q : nullptr, codes, m0, m1, res2, il);
  } else {
    uint8_t sc[2];
    quant_fp4(y, a.scale_mode, codes, sc, res2, il);
    m0 = (uint16_t)(sc[0] | (sc[1] << 8));
  }

  // originals and descriptors
  if (a.desc) {
    uint16_t* orig = tensor ? a.v_orig : a.k_orig;
    if (valid) {
      const uint4* s4 = reinterpret_cast<const uint4*>(src);
      uint4* d4 = reinterpret_cast<uint4*>(orig + ((stream_idx * a.Tmax + pos) * D + 32 * q));
#pragma unroll
      for (int i = 0; i < 4; ++i) d4[i] = s4[i];
    }
    // outward-rounded norms: fp32 sum/sqrt error and the rotation's own rounding
    // (SRFT: six butterfly passes and the unpack, each a few fp32 roundings of values no
    // larger than the vector norm, twiddles within half an ulp: far below 4e-6 relative);
    // with factors, also the rounding of y * lambda (|fl(y l) - y l| / l <= |y| 2^-24)
    const float slack = (a.rotation == KVQ_ROT_DENSE ? 2.44140625e-4f
                         : a.rotation == KVQ_ROT_SIGN_FWHT ? 9.5367431640625e-7f
                         : a.rotation == KVQ_ROT_SRFT ? 4.0e-6f : 0.0f) + (il ? 1.1920928955078125e-7f : 0.0f);
    float rn = sqrtf(quad_sum(res2)) * 1.0009765625f + sqrtf(quad_sum(ynorm2)) * slack;
    float vn = sqrtf(quad_sum(xnorm2)) * 1.0009765625f;
    if (!valid) {
      rn = 0.0f;
      vn = 0.0f;
    }
    rn = wave_quad_max(rn);
    vn = wave_quad_max(vn);
    if ((t & 63) == 0) {
      unsigned int* dsc = reinterpret_cast<unsigned int*>(a.desc + (stream_idx * (a.Tmax / TILE) + tile) * 3);
      atomicMax(dsc + (tensor ? 1 : 0), __float_as_uint(rn));
      if (tensor) atomicMax(dsc + 2, __float_as_uint(vn));
    }
  }

  uint32_t packed[8];
  int ndw = 0;
  const int KB = row_bytes(fmt);
  if (tensor == 0) {
    // K row: this lane's quarter of the codes, then its metadata
    if (valid) {
      pack_row(codes, fmt, packed, ndw);
      uint8_t* row = a.k_codes + (stream_idx * a.Tmax + pos) * KB + q * (KB / 4);
      if (ndw == 8) {
        uint4* r4 = reinterpret_cast<uint4*>(row);
        r4[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
        r4[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
      } else if (ndw == 4) {
        *reinterpret_cast<uint4*>(row) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
      } else {
        *reinterpret_cast<uint2*>(row) = make_uint2(packed[0], packed[1]);
      }
      uint8_t* mrow = a.k_meta + (stream_idx * a.Tmax + pos) * meta_bytes(fmt, group);
      uint16_t* m16 = reinterpret_cast<uint16_t*>(mrow);
      if (fmt == KVQ_INT2) {
        m16[q] = m0;
        m16[4 + q] = m1;
      } else if (fmt == KVQ_FP4) {
        m16[q] = m0;  // two E4M3 bytes: blocks 2q and 2q+1
      } else if (group == 16) {
        m16[2 * q] = m0;
        m16[2 * q + 1] = m1;
      } else if (group == 32) {
        m16[q] = m0;
      } else if (q == 0) {
        m16[0] = m0;
      }
    }
    return;
  }

  // V: stage token-major codes and metadata in LDS
#pragma unroll
  for (int j = 0; j < 32; ++j) sm.codes[tau][32 * q + j] = (uint8_t)(codes[j] & 0xFF);
  if (fmt == KVQ_INT2) {
    sm.meta[tau][q] = m0;
    sm.meta[tau][4 + q] = m1;
  } else if (fmt == KVQ_FP4) {
    sm.meta[tau][2 * q] = m0 & 0xFF;
    sm.meta[tau][2 * q + 1] = m0 >> 8;
  } else if (group == 16) {
    sm.meta[tau][2 * q] = m0;
    sm.meta[tau][2 * q + 1] = m1;
  } else if (group == 32) {
    sm.meta[tau][q] = m0;
  } else if (q == 0) {
    sm.meta[tau][0] = m0;
  }
  __syncthreads();

  const int bits = fmt_bits(fmt);
  const int per_dw = 32 / bits;            // tokens per dword
  const int dw_per_chan = TILE / per_dw;   // dwords per channel in a tile
  const int CB = chan_bytes(fmt);
  const int tlo = lo - tile * TILE, thi = hi - tile * TILE;
  uint8_t* vtile = a.v_codes + (stream_idx * (a.Tmax / TILE) + tile) * (size_t)(D * CB);
  const uint32_t emask = (1u << bits) - 1u;
  for (int item = t; item < D * dw_per_chan; item += NT) {
    const int c = item / dw_per_chan, d = item % dw_per_chan;
    const int t0 = d * per_dw;
    if (t0 + per_dw <= tlo || t0 >= thi) continue;
    uint32_t val = 0, mask = 0;
    for (int e = 0; e < per_dw; ++e) {
      const int tt = t0 + e;
      if (tt >= tlo && tt < thi) {
        val |= ((uint32_t)sm.codes[tt][c] & emask) << (bits * e);
        mask |= emask << (bits * e);
      }
    }
    uint32_t* dst = reinterpret_cast<uint32_t*>(vtile + (size_t)c * CB) + d;
    if (mask != 0xFFFFFFFFu) val = (*dst & ~mask) | val;
    *dst = val;
  }
  const int NM = meta_elems(fmt, group);
  const int ES = meta_esize(fmt);
  uint8_t* mtile = a.v_meta + (stream_idx * (a.Tmax / TILE) + tile) * (size_t)(NM * TILE * ES);
  for (int item = t; item < NM * TILE; item += NT) {
    const int m = item / TILE, tt = item % TILE;
    if (tt < tlo || tt >= thi) continue;
    if (ES == 2)
      reinterpret_cast<uint16_t*>(mtile)[m * TILE + tt] = sm.meta[tt][m];
    else
      mtile[m * TILE + tt] = (uint8_t)sm.meta[tt][m];
  }
}

// ================================================================ fast path
// Symmetric int4/int8 codes with the sign + Walsh-Hadamard rotation (or none).
// Same thread layout and the same fp32 operations in the same order as the
// generic kernel above, with the work per element cut down:
//  * sign flips are xors of the fp16/bf16 sign bits before widening (exact);
//  * the cross-lane butterflies negate the own value and add the partner's
//    (fl32(p + (-v)) is fl32(p - v));
//  * the quotient y / s is rounded with one refinement of y * (1/s) by its exact
//    residual, then a magic-number add that rounds half to even (see
//    quot_magic);
//  * codes are packed with byte permutes, and V codes reach the channel-major
//    tile through an 8x8 nibble transpose of LDS words.
namespace {

constexpr float MAGIC = 8388608.0f;  // 2^23

// RNE(y / sf) + offset, as the low mantissa bits of 2^23 + offset + RNE(y / sf),
// clamped to [offset - qmax, offset + qmax].  r = rcp(sf) (<= 1 ulp).  t = y r
// is within |q| 2^-22 of q = y / sf; one step with the exact residual brings
// the error below |q| 2^-43, and a quotient that is not a midpoint k + 1/2 lies
// at least one fp32 ulp of q away from every midpoint (y has 24 significant
// bits, sf 11), so rounding the refined value is rounding q.
template <int OFF, int QMAX>
__device__ __forceinline__ float quot_magic(float y, float sf, float r) {
  const float t = y * r;
  const float e = __builtin_fmaf(-t, sf, y);
  const float tq = __builtin_fmaf(e, r, t);
  const float m = tq + (MAGIC + (float)OFF);  // ulp 1: round half to even
  return __builtin_amdgcn_fmed3f(m, MAGIC + (float)(OFF - QMAX), MAGIC + (float)(OFF + QMAX));
}

// y[j] = fma(partner's y[j], s, y[j]) for j = 0..15, the partner given by a DPP quad
// permutation: v_fmac_f32 with its first source read through DPP, one instruction per
// value (for an fma the compiler keeps a separate DPP move).  A DPP read of a register
// written by the VALU instruction just before it needs two wait states, hence the s_nop
// at the head of the block; inside it each instruction writes a register the next ones
// do not read.
#define KVQ_FMAC_DPP16(QP)                                                                \
  asm volatile("s_nop 1\n\t"                                                              \
      "v_fmac_f32_dpp %0, %0, %16 " QP " row_mask:0xf bank_mask:0xf\n\t"  \
      "v_fmac_f32_dpp %1, %1, %16 " QP " row_mask:0xf bank_mask:0xf\n\t"  \
      "v_fmac_f32_dpp %2, %2, %16 " QP " row_mask:0xf bank_mask:0xf\n\t"  \
      "v_fmac_f32_dpp %3, %3, %16 " QP " row_mask:0xf bank_mask:0xf\n\t"  \
      "v_fmac_f32_dpp %4, %4, %16 " QP " row_mask:0xf bank_mask:0xf\n\t"  \
      "v_fmac_f32_dpp %5, %5, %16 " QP " row_mask:0xf bank_mask:0xf\n\t"  \
      "v_fmac_f32_dpp %6, %6, %16 " QP " row_mask:0xf bank_mask:0xf\n\t"  \
      "v_fmac_f32_dpp %7, %7, %16 " QP " row_mask:0xf bank_mask:0xf\n\t"  \
      "v_fmac_f32_dpp %8, %8, %16 " QP " row_mask:0xf bank_mask:0xf\n\t"  \
      "v_fmac_f32_dpp %9, %9, %16 " QP " row_mask:0xf bank_mask:0xf\n\t"  \
      "v_fmac_f32_dpp %10, %10, %16 " QP " row_mask:0xf bank_mask:0xf\n\t"  \
      "v_fmac_f32_dpp %11, %11, %16 " QP " row_mask:0xf bank_mask:0xf\n\t"  \
      "v_fmac_f32_dpp %12, %12, %16 " QP " row_mask:0xf bank_mask:0xf\n\t"  \
      "v_fmac_f32_dpp %13, %13, %16 " QP " row_mask:0xf bank_mask:0xf\n\t"  \
      "v_fmac_f32_dpp %14, %14, %16 " QP " row_mask:0xf bank_mask:0xf\n\t"  \
      "v_fmac_f32_dpp %15, %15, %16 " QP " row_mask:0xf bank_mask:0xf\n\t"  \
               : "+v"(y[0]), "+v"(y[1]), "+v"(y[2]), "+v"(y[3]), "+v"(y[4]), "+v"(y[5]), "+v"(y[6]), "+v"(y[7]), "+v"(y[8]), "+v"(y[9]), "+v"(y[10]), "+v"(y[11]), "+v"(y[12]), "+v"(y[13]), "+v"(y[14]), "+v"(y[15]) \
               : "v"(s))
__device__ __forceinline__ void fmac_dpp16_xor1(float* y, float s) { KVQ_FMAC_DPP16("quad_perm:[1,0,3,2]"); }
__device__ __forceinline__ void fmac_dpp16_xor2(float* y, float s) { KVQ_FMAC_DPP16("quad_perm:[2,3,0,1]"); }

// gather the low bytes of 4 floats into one dword (byte i = x[i] low byte)
__device__ __forceinline__ uint32_t low_bytes4(float x0, float x1, float x2, float x3) {
  const uint32_t a = __builtin_amdgcn_perm(__float_as_uint(x1), __float_as_uint(x0), 0x0C0C0400u);
  const uint32_t b = __builtin_amdgcn_perm(__float_as_uint(x3), __float_as_uint(x2), 0x0C0C0400u);
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}

struct __align__(16) FastSmem {
  uint32_t smask[4][16];     // per quarter: sign masks of 16 fp16 pairs
  uint32_t vt[TILE][17];     // V: per token 16 nibble words (8 channels each), padded
};

// SRFT in registers (the fast path).  Twiddles W128^k, k = 0..64, and one
// 128-float row per vector of the tile for the final reorder.
struct __align__(16) SrftRegSmem {
  float twr[65], twi[65];
  float rows[TILE][D + 4];
};

__device__ __forceinline__ constexpr int rev4(int i) {
  return ((i & 1) << 3) | ((i & 2) << 1) | ((i & 4) >> 1) | ((i & 8) >> 3);
}

// The same fp32 operations as the LDS version above (srft_quad), on values that
// stay in place.  Lane q of the quad holds the complex points z_n, n = 16q + i, in
// register i.  Every Stockham pass combines the points whose current index differs
// in its top bit (32 apart); computed in place, the passes leave the labels moving
// instead of the data: the pair bit is lane bit 1 in pass 0 and lane bit 0 in pass 1
// (DPP partners), then register bits 3, 2, 1, 0, and the index of the twiddle
// W64^(jm) follows from the label of the upper element.  Afterwards register i of
// lane q holds Z_k, k = 4 rev4(i) + r with r = (q >> 1) + 2 (q & 1); the partner
// Z_(64-k) of the Hermitian unpack is in the same lane (r = 0, 2) or in lane q ^ 1
// (r = 1, 3), at register 15 - i (lane 0: rev4(16 - rev4(i))).  The packed output
// goes through one LDS row per vector back to the natural channel order.  y holds
// the sign-flipped input on entry and the rotated vector on return.
// NEG (integer codes): passes 0 and 1 form own + s * partner in one DPP-sourced fma, so
// the upper lane of each pair holds the negated butterfly output (as in the Hadamard fast
// path); the twiddle of the lower lane is W^0 = 1, so no select is needed.  After both
// passes lane q holds its values times sigma_q = (-1)^(q0 + q1); everything after is
// linear, the Hermitian partner taken from lane q ^ 1 carries -sigma_q and is negated, and
// sigma_q goes into the output factor.  Only signs of zeros can differ from the exact form,
// which integer codes do not see.
template <bool NEG>
__device__ __forceinline__ void srft_regs(float y[32], int q, int vec, SrftRegSmem& sm) {
  float zr[16], zi[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    zr[i] = y[2 * i];
    zi[i] = y[2 * i + 1];
  }
  const int q0 = q & 1, q1 = q >> 1;
  if constexpr (NEG) {
    fmac_dpp16_xor2(zr, q1 ? -1.0f : 1.0f);
    fmac_dpp16_xor2(zi, q1 ? -1.0f : 1.0f);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = q1 ? 32 * q0 + 2 * i : 0;
      const float wr = sm.twr[e], wi = sm.twi[e], vr = zr[i], vi = zi[i];
      zr[i] = vr * wr - vi * wi;
      zi[i] = vr * wi + vi * wr;
    }
    fmac_dpp16_xor1(zr, q0 ? -1.0f : 1.0f);
    fmac_dpp16_xor1(zi, q0 ? -1.0f : 1.0f);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int e = q0 ? 4 * i : 0;
      const float wr = sm.twr[e], wi = sm.twi[e], vr = zr[i], vi = zi[i];
      zr[i] = vr * wr - vi * wi;
      zi[i] = vr * wi + vi * wr;
    }
  } else {
  // passes 0 and 1: the lower element takes own + partner, the upper one
  // (partner - own) W, with W64^(jm) = W128^(2jm): 32 q0 + 2i in pass 0, 4i in pass 1
  {
    const float sg = q1 ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float vr = __builtin_fmaf(zr[i], sg, dpp_f<KVQ_DPP_XOR2>(zr[i]));
      const float vi = __builtin_fmaf(zi[i], sg, dpp_f<KVQ_DPP_XOR2>(zi[i]));
      const int e = 32 * q0 + 2 * i;
      const float wr = sm.twr[e], wi = sm.twi[e];
      const float tr = vr * wr - vi * wi, ti = vr * wi + vi * wr;
      zr[i] = q1 ? tr : vr;
      zi[i] = q1 ? ti : vi;
    }
  }
  {
    const float sg = q0 ? -1.0f : 1.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float vr = __builtin_fmaf(zr[i], sg, dpp_f<KVQ_DPP_XOR1>(zr[i]));
      const float vi = __builtin_fmaf(zi[i], sg, dpp_f<KVQ_DPP_XOR1>(zi[i]));
      const float wr = sm.twr[4 * i], wi = sm.twi[4 * i];
      const float tr = vr * wr - vi * wi, ti = vr * wi + vi * wr;
      zr[i] = q0 ? tr : vr;
      zi[i] = q0 ? ti : vi;
    }
  }
  }
  // passes 2..5 inside the lane: pairs (i, i + h), h = 8, 4, 2, 1
  auto bfly = [&](int ia, int ib, int e) {
    const float ar = zr[ia], ai = zi[ia], br = zr[ib], bi = zi[ib];
    zr[ia] = ar + br;
    zi[ia] = ai + bi;
    const float dr = ar - br, di = ai - bi;
    const float wr = sm.twr[e], wi = sm.twi[e];
    zr[ib] = dr * wr - di * wi;
    zi[ib] = dr * wi + di * wr;
  };
#pragma unroll
  for (int i = 0; i < 8; ++i) bfly(i, i + 8, 8 * i);
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if ((i & 4) == 0) bfly(i, i + 4, 16 * (i & 3));
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if ((i & 2) == 0) bfly(i, i + 2, 32 * (i & 1));
#pragma unroll
  for (int i = 0; i < 16; i += 2) bfly(i, i + 1, 0);
  // Hermitian unpack: X_k = E + W128^k O, A = Z_k, B = conj(Z_(64-k)),
  // E = (A + B) / 2, O = (A - B) / 2i
  const int r = q1 + 2 * q0;
  float* row = sm.rows[vec];
  const float c0 = bits_to_f32(KVQ_INV_SQRT_D_BITS);
  auto unpack = [&](float a_re, float a_im, float p_re, float p_im, int k, float& xr, float& xi) {
    const float b_re = p_re, b_im = -p_im;
    const float e_re = 0.5f * (a_re + b_re), e_im = 0.5f * (a_im + b_im);
    const float o_re = 0.5f * (a_im - b_im), o_im = -(0.5f * (a_re - b_re));
    const float wr = sm.twr[k], wi = sm.twi[k];
    const float t_re = o_re * wr - o_im * wi, t_im = o_re * wi + o_im * wr;
    xr = e_re + t_re;
    xi = e_im + t_im;
  };
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int i1 = 15 - i, i0 = rev4((16 - rev4(i)) & 15);
    float pr = zr[i1], pi = zi[i1];
    const float dr = dpp_f<KVQ_DPP_XOR1>(zr[i1]), di = dpp_f<KVQ_DPP_XOR1>(zi[i1]);
    if (q1) {
      pr = NEG ? -dr : dr;  // (the partner lane carries the opposite sign)
      pi = NEG ? -di : di;
    } else if (q == 0) {
      pr = zr[i0];
      pi = zi[i0];
    }
    const int k = 4 * rev4(i) + r;
    float xr, xi;
    unpack(zr[i], zi[i], pr, pi, k, xr, xi);
    const float sc = NEG && (q0 ^ q1) ? -0.125f : 0.125f;  // 0.125 sigma_q
    float v0 = xr * sc, v1 = xi * sc;
    if (i == 0 && q == 0) {  // X_0 and X_64 (both from Z_0) are the two real channels
      float nr, ni;
      unpack(zr[0], zi[0], zr[0], zi[0], 64, nr, ni);
      v0 = xr * c0;
      v1 = nr * c0;
    }
    row[2 * k] = v0;
    row[2 * k + 1] = v1;
  }
  __syncthreads();
  const float4* rp = reinterpret_cast<const float4*>(row + 32 * q);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float4 u = rp[i];
    y[4 * i] = u.x;
    y[4 * i + 1] = u.y;
    y[4 * i + 2] = u.z;
    y[4 * i + 3] = u.w;
  }
}

// 8x8 transpose of nibbles: w[e] nibble j -> w[j] nibble e
__device__ __forceinline__ void transpose8x8_nibbles(uint32_t w[8]) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {  // 4-nibble blocks
    const uint32_t a = w[e], b = w[e + 4];
    w[e] = __builtin_amdgcn_perm(b, a, 0x05040100u);
    w[e + 4] = __builtin_amdgcn_perm(b, a, 0x07060302u);
  }
#pragma unroll
  for (int e0 = 0; e0 < 8; e0 += 4)
#pragma unroll
    for (int e = e0; e < e0 + 2; ++e) {  // 2-nibble blocks (bytes)
      const uint32_t a = w[e], b = w[e + 2];
      w[e] = __builtin_amdgcn_perm(b, a, 0x06020400u);
      w[e + 2] = __builtin_amdgcn_perm(b, a, 0x07030501u);
    }
#pragma unroll
  for (int e = 0; e < 8; e += 2) {  // single nibbles
    const uint32_t a = w[e], b = w[e + 1];
    w[e] = (a & 0x0F0F0F0Fu) | ((b << 4) & 0xF0F0F0F0u);
    w[e + 1] = ((a >> 4) & 0x0F0F0F0Fu) | (b & 0xF0F0F0F0u);
  }
}

}  // namespace

// One workgroup per (tensor, tile, kv head, sequence) unit; the tensor is the
// fastest-varying index so that the K and V workgroups of a tile are adjacent.
struct FastUnit {
  int b, h, tensor, tile, lo, hi, pos;
  bool valid;
  size_t stream_idx;
  const uint16_t* src;
};

__device__ __forceinline__ FastUnit fast_unit(const AppendArgs& a, int u, int ntiles) {
  FastUnit U;
  const int tau = threadIdx.x >> 2, q = threadIdx.x & 3;
  U.tensor = u & 1;
  const int r = u >> 1;
  const int ti = r % ntiles, r2 = r / ntiles;
  U.h = r2 % a.H;
  U.b = r2 / a.H;
  const int start = a.start.v[U.b];
  U.tile = start / TILE + ti;
  U.lo = max(start, U.tile * TILE);
  U.hi = min(start + a.n_new, U.tile * TILE + TILE);
  U.pos = U.tile * TILE + tau;
  U.valid = U.pos >= U.lo && U.pos < U.hi;
  U.stream_idx = (size_t)U.b * a.H + U.h;
  if (U.valid) KVQ_DCHECK_APPEND(a, U.stream_idx, U.pos, start);
  U.src = (U.tensor ? a.v_new : a.k_new) + ((U.stream_idx * a.n_new + (U.valid ? U.pos - start : 0)) * D + 32 * q);
  return U;
}

__device__ __forceinline__ void fast_load(const uint16_t* src, uint32_t w[16]) {
  const uint4* p4 = reinterpret_cast<const uint4*>(src);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint4 u = p4[i];
    w[4 * i] = u.x; w[4 * i + 1] = u.y; w[4 * i + 2] = u.z; w[4 * i + 3] = u.w;
  }
}

// quantize 32 rotated values of one lane (its group of 32, its two groups of 16,
// or a quarter of a group of 128) into packed code dwords; optional residual and
// norm sums.  meta: the lane's scale (groups of 16: of channels 0..15; meta1 of 16..31)
template <int FMT, int GROUP>
__device__ __forceinline__ void fast_quantize(const float y[32], bool want_sums, uint32_t packed[8], uint16_t& meta,
                                              uint16_t& meta1, float& res2, float& ynorm2) {
  constexpr int QMAX = FMT == KVQ_INT4 ? 7 : 127;
  constexpr int OFF = FMT == KVQ_INT4 ? 8 : 128;
  constexpr int NH = GROUP == 16 ? 2 : 1;  // scales per lane
  float am[NH];
#pragma unroll
  for (int i = 0; i < NH; ++i) am[i] = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) am[j * NH / 32] = fmaxf(am[j * NH / 32], fabsf(y[j]));
  if constexpr (GROUP == 128) {
    am[0] = fmaxf(am[0], dpp_f<KVQ_DPP_XOR1>(am[0]));
    am[0] = fmaxf(am[0], dpp_f<KVQ_DPP_XOR2>(am[0]));
  }
  uint16_t sb[NH];
  float sf[NH], sq[NH], r[NH];
#pragma unroll
  for (int i = 0; i < NH; ++i) {
    sb[i] = f16_sat_bits(am[i] / (float)QMAX);  // correctly rounded fp32 divide
    sf[i] = f16_bits_to_f32(sb[i]);
    // a zero scale gives code 0 for every element: divisor 1 and reciprocal 0 do that
    sq[i] = sf[i] != 0.0f ? sf[i] : 1.0f;
    r[i] = sf[i] != 0.0f ? __builtin_amdgcn_rcpf(sf[i]) : 0.0f;
  }
  meta = sb[0];
  meta1 = sb[NH - 1];
  float acc = 0.0f, yn = 0.0f;
#pragma unroll
  for (int k = 0; k < 4; ++k) {  // 8 elements at a time (one scale: groups of 16 are k = 0, 1 and 2, 3)
    const int hs = k * NH / 4;
    float m[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) m[e] = quot_magic<OFF, QMAX>(y[8 * k + e], sq[hs], r[hs]);
    if (want_sums) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float cj = m[e] - (MAGIC + (float)OFF);  // exact
        const float d = y[8 * k + e] - cj * sf[hs];
        acc = acc + d * d;
        yn = yn + y[8 * k + e] * y[8 * k + e];
      }
    }
    if constexpr (FMT == KVQ_INT4) {
      // offset-binary nibbles: bytes of even / odd elements, then nibble-merged; ^8 -> two's complement
      const uint32_t ev = low_bytes4(m[0], m[2], m[4], m[6]);
      const uint32_t od = low_bytes4(m[1], m[3], m[5], m[7]);
      packed[k] = ((od << 4) | (ev & 0x0F0F0F0Fu)) ^ 0x88888888u;
    } else {
      packed[2 * k] = low_bytes4(m[0], m[1], m[2], m[3]) ^ 0x80808080u;
      packed[2 * k + 1] = low_bytes4(m[4], m[5], m[6], m[7]) ^ 0x80808080u;
    }
  }
  res2 = acc;
  ynorm2 = yn;
}

// FP4 E2M1 codes with E4M3 scales, two blocks of 16 per lane.  The scale search
// visits the distinct E4M3 codes of fl32(t * m), m = 0.900, 0.925, ..., 1.100 in
// that order; those codes are consecutive (a step of m moves t by at most 2.8%,
// while every E4M3 rounding interval is at least 6.4% wide), so the candidates
// are the codes c_lo .. c_hi of m = 0.9 and m = 1.1, in increasing order, and
// the first strictly smallest error wins as in a skip-duplicates scan.  The
// bit-offset search scans the patterns c0 - 2 .. c0 + 6 of c0 = E4M3(t) the
// same way (clamped to 0x00..0x7E, which only drops repeats).  Errors
// use the same fp32 operations as the generic quantizer: per element
// d = |y| - Q(|y|), squared, summed over elements 0..7 and 8..15, then added.
//
// Q(x) for a scale S is S times the E2M1 value nearest to x / S, ties to the even code
// (the definition's threshold chain).  Here the quotient is formed as in quot_magic (x
// times rcp(S), one step with the exact residual: within |q| 2^-43 of q = x / S, while a
// quotient that is not a midpoint m of the E2M1 grid lies at least 2^-24 m from it, since
// m S has at most 7 significant bits; a midpoint quotient comes out exact) and rounded by
// the gfx950 fp32 -> E2M1 conversion with scale 1, which rounds to nearest, ties to the
// even code, and saturates at 6 (checked against the chain on every midpoint, its
// neighbours, zeros, subnormals and values past 6); the reverse conversion gives the
// grid value exactly.  xs: the magnitudes with infinities replaced by 1e30 and NaN by 0
// (their codes under the chain: 7 and 0), so that no quotient is a NaN.
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ void e2m1_quot16(const float xs[16], float S, float u[16]) {
  const float r = S != 0.0f ? __builtin_amdgcn_rcpf(S) : 0.0f;  // S = 0: every quotient 0
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const float t = xs[j] * r;
    const float e = __builtin_fmaf(-t, S, xs[j]);
    u[j] = __builtin_fmaf(e, r, t);
  }
}
__device__ __forceinline__ float fp4_err16(const float* y, const float xs[16], float S) {
  float u[16];
  e2m1_quot16(xs, S, u);
  float lo = 0.0f, hi = 0.0f;
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t c = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, u[2 * k], u[2 * k + 1], 1.0f, 0);
    const f32x2 g = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
    // |y| - grid value times S: the product is exact (at most 6 significant bits), so one
    // fma gives the rounded difference of the definition
    const float d0 = __builtin_fmaf(-g.x, S, fabsf(y[2 * k])), d1 = __builtin_fmaf(-g.y, S, fabsf(y[2 * k + 1]));
    const float s0 = d0 * d0, s1 = d1 * d1;
    if (k < 4) {
      lo = lo + s0;
      lo = lo + s1;
    } else {
      hi = hi + s0;
      hi = hi + s1;
    }
  }
  return lo + hi;
}

__device__ __forceinline__ void fast_quantize_fp4(const float y[32], int mode, bool want_sums, uint32_t packed[4],
                                                  uint16_t& meta, float& res2, float& ynorm2) {
  float acc = 0.0f;
  uint32_t sc[2];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const float* yb = y + 16 * blk;
    float xs[16];
    float am = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float ay = fabsf(yb[j]);
      am = fmaxf(am, ay);
      xs[j] = ay <= 1e30f ? ay : (ay > 1e30f ? 1e30f : 0.0f);
    }
    const float t = am / 6.0f;  // correctly rounded fp32 divide
    uint32_t best, chi;
    if (mode == KVQ_SCALE_SEARCH9) {
      best = e4m3_encode_nonneg(t * 0.9f);
      chi = e4m3_encode_nonneg(t * 1.1f);
    } else {
      const uint32_t c0 = e4m3_encode_nonneg(t);
      best = mode == KVQ_SCALE_SEARCH_OFFSETS ? (c0 > 2u ? c0 - 2u : 0u) : c0;
      chi = mode == KVQ_SCALE_SEARCH_OFFSETS ? min(c0 + 6u, 0x7Eu) : c0;
    }
    if (chi > best) {
      float best_e = fp4_err16(yb, xs, e4m3_value(best));
      for (uint32_t c = best + 1; c <= chi; ++c) {
        const float e = fp4_err16(yb, xs, e4m3_value(c));
        if (e < best_e) {
          best_e = e;
          best = c;
        }
      }
    }
    sc[blk] = best;
    const float S = e4m3_value(best);
    // codes with their signs: the quotient takes the sign bit of y, and the conversion
    // carries it (-0 included) into bit 3; a zero scale gives code 0 for every element
    float u[16];
    e2m1_quot16(xs, S, u);
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      const uint32_t sg0 = __float_as_uint(y[16 * blk + 2 * k]) & 0x80000000u;
      const uint32_t sg1 = __float_as_uint(y[16 * blk + 2 * k + 1]) & 0x80000000u;
      const float v0 = __uint_as_float(__float_as_uint(u[2 * k]) | sg0);
      const float v1 = __uint_as_float(__float_as_uint(u[2 * k + 1]) | sg1);
      const uint32_t c = S != 0.0f ? __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v0, v1, 1.0f, 0) & 0xFFu : 0u;
      w[k >> 2] |= c << (8 * (k & 3));
      if (want_sums) {
        const f32x2 g = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
        const float d0 = __builtin_fmaf(-fabsf(g.x), S, fabsf(yb[2 * k]));
        const float d1 = __builtin_fmaf(-fabsf(g.y), S, fabsf(yb[2 * k + 1]));
        acc = acc + d0 * d0;
        acc = acc + d1 * d1;
      }
    }
    packed[2 * blk] = w[0];
    packed[2 * blk + 1] = w[1];
  }
  meta = (uint16_t)(sc[0] | (sc[1] << 8));
  res2 = acc;
  float yn = 0.0f;
  if (want_sums) {
#pragma unroll
    for (int j = 0; j < 32; ++j) yn = yn + y[j] * y[j];
  }
  ynorm2 = yn;
}

template <int KF, int KG, int VF, int VG, bool BF16, bool SRFT>
__device__ __forceinline__ void fast_process(const AppendArgs& a, FastSmem& sm, SrftRegSmem* ss, const FastUnit& U,
                                             const uint32_t w[16]) {
  const int t = threadIdx.x, tau = t >> 2, q = t & 3;
  const int tensor = U.tensor, tile = U.tile, pos = U.pos;
  const bool valid = U.valid;
  const size_t stream_idx = U.stream_idx;
  const bool fwht = a.rotation == KVQ_ROT_SIGN_FWHT;
  const bool desc = a.desc != nullptr;

  // originals and the input norm first, so the raw words are dead after the rotation
  float xnorm2 = 0.0f;
  if (desc) {
    if (valid) {
      uint16_t* orig = tensor ? a.v_orig : a.k_orig;
      uint4* d4 = reinterpret_cast<uint4*>(orig + ((stream_idx * a.Tmax + pos) * D + 32 * q));
#pragma unroll
      for (int i = 0; i < 4; ++i) d4[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
    }
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const float x0 = widen((uint16_t)(w[k] & 0xFFFF), BF16), x1 = widen((uint16_t)(w[k] >> 16), BF16);
      xnorm2 = xnorm2 + x0 * x0;
      xnorm2 = xnorm2 + x1 * x1;
    }
  }

  float y[32];
  if constexpr (SRFT) {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      const uint32_t ws = w[k] ^ sm.smask[q][k];
      y[2 * k] = widen((uint16_t)(ws & 0xFFFF), BF16);
      y[2 * k + 1] = widen((uint16_t)(ws >> 16), BF16);
    }
    srft_regs<KF != KVQ_FP4 && VF != KVQ_FP4>(y, q, tau, *ss);
  } else if (fwht) {
    if constexpr (BF16) {
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const uint32_t ws = w[k] ^ sm.smask[q][k];
        y[2 * k] = widen((uint16_t)(ws & 0xFFFF), BF16);
        y[2 * k + 1] = widen((uint16_t)(ws >> 16), BF16);
      }
    } else {
      // stage h = 1 straight from the fp16 pair: fma(a, +-1, b) with fp16 operands and an
      // fp32 result is the exactly rounded a +- b of the widened values (mixed-precision
      // fma), so widening and the first butterfly take one instruction per element
      float one = 1.0f;
      asm volatile("" : "+v"(one));  // kept opaque, so that the fma is not turned into an add
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        const uint32_t ws = w[k] ^ sm.smask[q][k];
        const float u = (float)__builtin_bit_cast(_Float16, (uint16_t)(ws & 0xFFFF));
        const float v = (float)__builtin_bit_cast(_Float16, (uint16_t)(ws >> 16));
        y[2 * k] = __builtin_fmaf(v, one, u);
        y[2 * k + 1] = __builtin_fmaf(v, -one, u);
      }
    }
#pragma unroll
    for (int hh = BF16 ? 1 : 2; hh < 32; hh *= 2)
#pragma unroll
      for (int j = 0; j < 32; ++j)
        if ((j & hh) == 0) {
          const float u = y[j], v = y[j + hh];
          y[j] = u + v;
          y[j + hh] = u - v;
        }
    const float s1 = (q & 1) ? -1.0f : 1.0f, s2 = (q & 2) ? -1.0f : 1.0f;
    float c = bits_to_f32(KVQ_INV_SQRT_D_BITS);
    if constexpr (KF != KVQ_FP4 && VF != KVQ_FP4) {
      // h = 32, 64 across the quad: each lane forms own + s * partner (s = -1 in the upper
      // lane of the pair), one fma with the partner as its DPP operand.  The lower lane gets
      // own + partner; the upper lane gets own - partner, the negation of the butterfly's
      // partner - own (rounding to nearest is symmetric), save that an exact cancellation
      // gives +0 either way.  Stage 64 pairs lanes with the same sign, so it runs on the
      // negated values alike, and the lane's two signs go into its normalising factor
      // (multiplying by -c negates multiplying by c).  Only zeros can come out with the
      // other sign, and an integer code does not see the sign of a zero (FP4 codes do: they
      // take the exact form below).
      fmac_dpp16_xor1(y, s1);
      fmac_dpp16_xor1(y + 16, s1);
      fmac_dpp16_xor2(y, s2);
      fmac_dpp16_xor2(y + 16, s2);
      c = c * (s1 * s2);
    } else {
      // lower index: own + partner; upper index: partner - own = fma(own, -1, partner)
#pragma unroll
      for (int j = 0; j < 32; ++j) y[j] = __builtin_fmaf(y[j], s1, dpp_f<KVQ_DPP_XOR1>(y[j]));
#pragma unroll
      for (int j = 0; j < 32; ++j) y[j] = __builtin_fmaf(y[j], s2, dpp_f<KVQ_DPP_XOR2>(y[j]));
    }
#pragma unroll
    for (int j = 0; j < 32; ++j) y[j] = y[j] * c;
  } else {
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      y[2 * k] = widen((uint16_t)(w[k] & 0xFFFF), BF16);
      y[2 * k + 1] = widen((uint16_t)(w[k] >> 16), BF16);
    }
  }

  uint32_t packed[8];
  uint16_t meta = 0, meta1 = 0;
  float res2 = 0.0f, ynorm2 = 0.0f;
  const int smode = a.scale_mode;
  if (tensor == 0) {
    if constexpr (KF == KVQ_FP4)
      fast_quantize_fp4(y, smode, desc, packed, meta, res2, ynorm2);
    else
      fast_quantize<KF, KG>(y, desc, packed, meta, meta1, res2, ynorm2);
  } else {
    if constexpr (VF == KVQ_FP4)
      fast_quantize_fp4(y, smode, desc, packed, meta, res2, ynorm2);
    else
      fast_quantize<VF, VG>(y, desc, packed, meta, meta1, res2, ynorm2);
  }

  if (desc) {  // outward-rounded norms, as in the generic kernel
    const float slack = SRFT ? 4.0e-6f : fwht ? 9.5367431640625e-7f : 0.0f;
    float rn = sqrtf(quad_sum(res2)) * 1.0009765625f + sqrtf(quad_sum(ynorm2)) * slack;
    float vn = sqrtf(quad_sum(xnorm2)) * 1.0009765625f;
    if (!valid) {
      rn = 0.0f;
      vn = 0.0f;
    }
    rn = wave_quad_max(rn);
    vn = wave_quad_max(vn);
    if ((t & 63) == 0) {
      unsigned int* dsc = reinterpret_cast<unsigned int*>(a.desc + (stream_idx * (a.Tmax / TILE) + tile) * 3);
      atomicMax(dsc + (tensor ? 1 : 0), __float_as_uint(rn));
      if (tensor) atomicMax(dsc + 2, __float_as_uint(vn));
    }
  }

  if (tensor == 0) {
    if (valid) {
      constexpr int KB = row_bytes(KF);
      uint8_t* row = a.k_codes + (stream_idx * a.Tmax + pos) * KB + q * (KB / 4);
      if constexpr (KF == KVQ_INT8) {
        uint4* r4 = reinterpret_cast<uint4*>(row);
        r4[0] = make_uint4(packed[0], packed[1], packed[2], packed[3]);
        r4[1] = make_uint4(packed[4], packed[5], packed[6], packed[7]);
      } else {
        *reinterpret_cast<uint4*>(row) = make_uint4(packed[0], packed[1], packed[2], packed[3]);
      }
      uint16_t* m16 = reinterpret_cast<uint16_t*>(a.k_meta + (stream_idx * a.Tmax + pos) * meta_bytes(KF, KG));
      if constexpr (KF == KVQ_FP4 || KG == 32) m16[q] = meta;  // FP4: E4M3 bytes of blocks 2q, 2q + 1
      else if constexpr (KG == 16) reinterpret_cast<uint32_t*>(m16)[q] = (uint32_t)meta | ((uint32_t)meta1 << 16);
      else if (q == 0) m16[0] = meta;
    }
    return;
  }

  // V: metadata straight to the tile ([element][64 tokens] fp16), codes via LDS
  {
    constexpr int NM = meta_elems(VF, VG);
    uint8_t* mbase = a.v_meta + (stream_idx * (a.Tmax / TILE) + tile) * (size_t)(NM * TILE * meta_esize(VF));
    if (valid) {
      if constexpr (VF == KVQ_FP4) {
        mbase[(2 * q) * TILE + tau] = (uint8_t)(meta & 0xFF);
        mbase[(2 * q + 1) * TILE + tau] = (uint8_t)(meta >> 8);
      } else {
        uint16_t* mtile = reinterpret_cast<uint16_t*>(mbase);
        if constexpr (VG == 32) {
          mtile[q * TILE + tau] = meta;
        } else if constexpr (VG == 16) {
          mtile[(2 * q) * TILE + tau] = meta;
          mtile[(2 * q + 1) * TILE + tau] = meta1;
        } else if (q == 0) {
          mtile[tau] = meta;
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < 4; ++k) sm.vt[tau][4 * q + k] = packed[k];
  __syncthreads();
  if (t < 128) {
    const int k = t >> 3, d = t & 7;  // channels 8k..8k+7, tokens 8d..8d+7
    const int tlo = U.lo - tile * TILE, thi = U.hi - tile * TILE;
    if (8 * d + 8 > tlo && 8 * d < thi) {
      uint32_t wv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) wv[e] = sm.vt[8 * d + e][k];
      transpose8x8_nibbles(wv);
      uint32_t mask = 0xFFFFFFFFu;
      if (8 * d < tlo || 8 * d + 8 > thi) {
        mask = 0u;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (8 * d + e >= tlo && 8 * d + e < thi) mask |= 0xFu << (4 * e);
      }
      uint32_t* vtile = reinterpret_cast<uint32_t*>(a.v_codes + (stream_idx * (a.Tmax / TILE) + tile) * (size_t)(D * chan_bytes(VF)));
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        uint32_t* dst = vtile + (8 * k + j) * (TILE / 8) + d;
        *dst = mask == 0xFFFFFFFFu ? wv[j] : ((*dst & ~mask) | (wv[j] & mask));
      }
    }
  }
}

// Two units per workgroup (the K and the V tile of one position range): both
// units' input rows are loaded first, so twice the bytes are in flight per thread.
template <int KF, int KG, int VF, int VG, bool BF16, bool SRFT = false>
__global__ __launch_bounds__(NT) void append_fast_kernel(AppendArgs a, int ntiles) {
  static_assert(VF == KVQ_INT4 || VF == KVQ_FP4, "V codes of the fast path are nibbles");
  __shared__ FastSmem sm;
  const int t = threadIdx.x;
  const int nunits = ntiles * a.H * 2 * a.B;
  const int u0 = 2 * (int)blockIdx.x, u1 = min(u0 + 1, nunits - 1);
  const FastUnit U0 = fast_unit(a, u0, ntiles), U1 = fast_unit(a, u1, ntiles);
  const bool run0 = U0.lo < U0.hi, run1 = u1 != u0 && U1.lo < U1.hi;  // uniform over the workgroup
  if (!run0 && !run1) return;
  uint32_t w0[16], w1[16];
  fast_load(U0.src, w0);  // rows of an empty unit still lie inside the input (row 0 of its stream)
  fast_load(U1.src, w1);
  __builtin_amdgcn_sched_barrier(0);
  // sign masks: bit 15 / bit 31 of pair k of quarter q set where the sign is negative
  if ((SRFT || a.rotation == KVQ_ROT_SIGN_FWHT) && t < 64) {
    const int qq = t >> 4, k = t & 15;
    const uint16_t sp = *reinterpret_cast<const uint16_t*>(a.signs + 32 * qq + 2 * k);
    sm.smask[qq][k] = ((uint32_t)(sp & 0x80u) << 8) | ((uint32_t)(sp & 0x8000u) << 16);
  }
  SrftRegSmem* ssp = nullptr;
  if constexpr (SRFT) {
    __shared__ SrftRegSmem ss;
    if (t < 65) {
      ss.twr[t] = a.tw_re[t];
      ss.twi[t] = a.tw_im[t];
    }
    ssp = &ss;
  }
  __syncthreads();
  if (run0) fast_process<KF, KG, VF, VG, BF16, SRFT>(a, sm, ssp, U0, w0);
  __syncthreads();  // the shared staging areas are reused by the second unit
  if (run1) fast_process<KF, KG, VF, VG, BF16, SRFT>(a, sm, ssp, U1, w1);
}

// ================================================================ dense rotation on matrix cores
// The dense rotation y_j = chain over k = 0..127 of fma(R[j][k], x_k, acc) runs
// as 128 rank-1 steps of the fp32 MFMA with K = 1: each step adds one exact-input
// product to every accumulator with a single rounding, which is the same fused
// multiply-add, in the same k order, as the scalar chain.  A workgroup rotates a
// 64-token tile: wave w owns output channels [32w, 32w + 32) (the quantization
// group w), the rotation rows it needs stay in registers for the whole
// (persistent) launch, and the tile's inputs are read from LDS.  The product
// lands in the MFMA's own layout: lane l holds tokens l % 32 and 32 + l % 32
// for 16 channels of the group, so a group's min/max needs one exchange between
// lanes l and l ^ 32; K rows are merged from the two halves with byte permutes
// and V tiles come out of a 16 x 16 transpose of 2-bit fields inside each row of
// 16 lanes.  Asymmetric int2 with groups of 32 (the 2-bit workload); other
// formats with the dense rotation use the generic kernel.
namespace {

typedef float f32x32 __attribute__((ext_vector_type(32)));

struct __align__(16) DenseMfmaSmem {
  uint32_t xs[TILE][68];  // input vectors as fp16/bf16 pairs; rows padded to 272 bytes
  uint32_t rs[D][68];     // the rotation as fp16 pairs, same padding
  float clip[2][D];       // clipping thresholds of the unit, double-buffered by parity
};

template <bool BF16>
__device__ __forceinline__ float half_lo(uint32_t w) {
  if constexpr (BF16) return __uint_as_float(w << 16);
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
}
template <bool BF16>
__device__ __forceinline__ float half_hi(uint32_t w) {
  if constexpr (BF16) return __uint_as_float(w & 0xFFFF0000u);
  return (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
}

// channel (within the group) of accumulator v, v = 0..15, for lanes of half hf
__device__ __forceinline__ int mfma_row(int v, int hf) { return 8 * (v >> 2) + 4 * hf + (v & 3); }

// RNE(y / sf) clamped to [0, 3], as 2^23 + code (see quot_magic)
__device__ __forceinline__ float quot_magic_u2(float y, float sf, float r) {
  const float t = y * r;
  const float e = __builtin_fmaf(-t, sf, y);
  const float tq = __builtin_fmaf(e, r, t);
  return __builtin_amdgcn_fmed3f(tq + MAGIC, MAGIC, MAGIC + 3.0f);
}

// 16 codes held as 2^23 + c (c < 4) -> c_v at bits 2v
__device__ __forceinline__ uint32_t pack16_u2(const float m[16]) {
  uint32_t p2[8], p4[4], p8[2];
#pragma unroll
  for (int i = 0; i < 8; ++i) p2[i] = (__float_as_uint(m[2 * i + 1]) << 2) | __float_as_uint(m[2 * i]);
#pragma unroll
  for (int i = 0; i < 4; ++i) p4[i] = (p2[2 * i + 1] << 4) | p2[2 * i];
#pragma unroll
  for (int i = 0; i < 2; ++i) p8[i] = (p4[2 * i + 1] << 8) | p4[2 * i];
  return __builtin_amdgcn_perm(p8[1], p8[0], 0x05040100u);  // bits 0..15 of each
}

// one stage of the 16 x 16 transpose of 2-bit fields across a row of 16 lanes:
// fields whose index bit S differs from the lane's bit S swap with lane ^ S
template <int S>
__device__ __forceinline__ uint32_t t16_stage(uint32_t w, int lane) {
  constexpr uint32_t ML = S == 1 ? 0x33333333u : S == 2 ? 0x0F0F0F0Fu : S == 4 ? 0x00FF00FFu : 0x0000FFFFu;
  uint32_t p;
  if constexpr (S == 1)
    p = (uint32_t)__builtin_amdgcn_mov_dpp((int)w, KVQ_DPP_XOR1, 0xF, 0xF, false);
  else if constexpr (S == 2)
    p = (uint32_t)__builtin_amdgcn_mov_dpp((int)w, KVQ_DPP_XOR2, 0xF, 0xF, false);
  else
    p = (uint32_t)__builtin_amdgcn_ds_swizzle((int)w, (S << 10) | 0x1F);  // lane ^ S within 32
  if (lane & S) return (w & ~ML) | ((p >> (2 * S)) & ML);
  return (w & ML) | ((p << (2 * S)) & ~ML);
}

__device__ __forceinline__ uint32_t transpose16_u2(uint32_t w, int lane) {
  w = t16_stage<8>(w, lane);
  w = t16_stage<4>(w, lane);
  w = t16_stage<2>(w, lane);
  return t16_stage<1>(w, lane);
}

// next unit at or after u (stride gridDim.x) that has tokens in this call; nunits if none
__device__ __forceinline__ int next_dense_unit(const AppendArgs& a, int u, int ntiles, int nunits, FastUnit& U) {
  for (; u < nunits; u += gridDim.x) {
    U = fast_unit(a, u, ntiles);
    if (U.lo < U.hi) break;
  }
  return u;
}

template <bool BF16>
__device__ __forceinline__ void dense_int2_store(const AppendArgs& a, const FastUnit& C, const f32x32& acc, int wv,
                                                 int lane, const float* sclip) {
  const int hf = lane >> 5, col = lane & 31;
  const int tensor = C.tensor;
  const bool clip = (tensor ? a.clip_v : a.clip_k) != nullptr;
  float tc[16];
  if (clip) {
    const float* cp = sclip + 32 * wv + 4 * hf;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float4 c4 = *reinterpret_cast<const float4*>(cp + 8 * g);
      tc[4 * g] = c4.x; tc[4 * g + 1] = c4.y; tc[4 * g + 2] = c4.z; tc[4 * g + 3] = c4.w;
    }
  }
  uint32_t P[2];
  uint16_t sbits[2], zbits[2];
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {  // token col (blk 0) and 32 + col (blk 1)
    float yc[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const float y = acc[16 * blk + v];
      yc[v] = clip ? fminf(fmaxf(y, -tc[v]), tc[v]) : y;
    }
    float lo = yc[0], hi = yc[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) {
      lo = fminf(lo, yc[v]);
      hi = fmaxf(hi, yc[v]);
    }
    lo = fminf(lo, __shfl_xor(lo, 32));
    hi = fmaxf(hi, __shfl_xor(hi, 32));
    const uint16_t sb = f16_sat_bits((hi - lo) / 3.0f);  // correctly rounded fp32 divide
    const uint16_t zb = f16_sat_bits(lo);
    const float sf = f16_bits_to_f32(sb), zf = f16_bits_to_f32(zb);
    const float sq = sf != 0.0f ? sf : 1.0f;
    const float r = sf != 0.0f ? __builtin_amdgcn_rcpf(sf) : 0.0f;
    float m[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) m[v] = quot_magic_u2(yc[v] - zf, sq, r);
    P[blk] = pack16_u2(m);
    sbits[blk] = sb;
    zbits[blk] = zb;
  }
  // this lane stores token `kt` (col for the lower half, 32 + col for the upper)
  const int kt = 32 * hf + col;
  const int pos = C.tile * TILE + kt;
  const bool valid = pos >= C.lo && pos < C.hi;
  if (valid) KVQ_DCHECK_APPEND(a, C.stream_idx, pos, a.start.v[C.b]);
  const uint16_t sk = hf ? sbits[1] : sbits[0], zk = hf ? zbits[1] : zbits[0];
  if (tensor == 0) {
    const uint32_t give = hf ? P[0] : P[1], keep = hf ? P[1] : P[0];
    const uint32_t recv = (uint32_t)__shfl_xor((int)give, 32);
    const uint32_t p0 = hf ? recv : keep, p1 = hf ? keep : recv;  // halves 0 and 1 of the kept token
    const uint32_t d0 = __builtin_amdgcn_perm(p1, p0, 0x05010400u);
    const uint32_t d1 = __builtin_amdgcn_perm(p1, p0, 0x07030602u);
    if (valid) {
      const size_t row = C.stream_idx * a.Tmax + pos;
      *reinterpret_cast<uint2*>(a.k_codes + row * row_bytes(KVQ_INT2) + 8 * wv) = make_uint2(d0, d1);
      uint16_t* m16 = reinterpret_cast<uint16_t*>(a.k_meta + row * meta_bytes(KVQ_INT2, 32));
      m16[wv] = sk;
      m16[4 + wv] = zk;
    }
    return;
  }
  // V: metadata [element][64 tokens]; codes channel-major, 16 tokens per dword
  const size_t tile_idx = C.stream_idx * (a.Tmax / TILE) + C.tile;
  if (valid) {
    uint16_t* mtile = reinterpret_cast<uint16_t*>(a.v_meta + tile_idx * (size_t)(meta_elems(KVQ_INT2, 32) * TILE * 2));
    mtile[wv * TILE + kt] = sk;
    mtile[(4 + wv) * TILE + kt] = zk;
  }
  const int x = lane & 15, r16 = (lane >> 4) & 1;
  const int c = 32 * wv + mfma_row(x, hf);
  uint32_t* vt = reinterpret_cast<uint32_t*>(a.v_codes + tile_idx * (size_t)(D * chan_bytes(KVQ_INT2))) + 4 * c;
  const int tlo = C.lo - C.tile * TILE, thi = C.hi - C.tile * TILE;
#pragma unroll
  for (int blk = 0; blk < 2; ++blk) {
    const uint32_t wt = transpose16_u2(P[blk], lane);
    const int d = 2 * blk + r16;  // tokens 16d .. 16d + 15
    if (16 * d + 16 <= tlo || 16 * d >= thi) continue;
    if (16 * d >= tlo && 16 * d + 16 <= thi) {
      vt[d] = wt;
    } else {
      uint32_t mask = 0u;
#pragma unroll
      for (int e = 0; e < 16; ++e)
        if (16 * d + e >= tlo && 16 * d + e < thi) mask |= 3u << (2 * e);
      vt[d] = (vt[d] & ~mask) | (wt & mask);
    }
  }
}

}  // namespace

template <bool BF16>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(3, 3))) void append_dense_int2_kernel(AppendArgs a, int ntiles,
                                                                                                   int nunits) {
  __shared__ DenseMfmaSmem sm;
  const int t = threadIdx.x, lane = t & 63;
  const int wv = __builtin_amdgcn_readfirstlane(t >> 6);
  const int tau = t >> 2, q = t & 3;
  // the rotation to LDS once (made visible by the first barrier of the loop)
  {
    const uint4* r4 = reinterpret_cast<const uint4*>(a.rot);
#pragma unroll
    for (int i = 0; i < D * 16 / NT; ++i) {
      const int c = t + NT * i;  // 16-byte chunk: row c / 16, column chunk c % 16
      *reinterpret_cast<uint4*>(&sm.rs[c >> 4][4 * (c & 15)]) = r4[c];
    }
  }
  const int rrow = 32 * wv + (lane & 31);  // the rotation row this lane feeds
  FastUnit U;
  int u = next_dense_unit(a, blockIdx.x, ntiles, nunits, U);
  uint32_t w[16];
  float4 cl = make_float4(0.0f, 0.0f, 0.0f, 0.0f);  // lanes t < 32: 4 clipping thresholds
  auto load_unit = [&]() {
    fast_load(U.src, w);
    const float* clip = U.tensor ? a.clip_v : a.clip_k;
    if (clip && t < D / 4) cl = *reinterpret_cast<const float4*>(clip + (size_t)U.h * D + 4 * t);
  };
  if (u < nunits) load_unit();
  int par = 0;
  while (u < nunits) {
    const FastUnit C = U;
    {
      uint4* d4 = reinterpret_cast<uint4*>(&sm.xs[tau][16 * q]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
        d4[i] = C.valid ? make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]) : make_uint4(0, 0, 0, 0);
      if (t < D / 4) *reinterpret_cast<float4*>(&sm.clip[par][4 * t]) = cl;
    }
    __syncthreads();
    u = next_dense_unit(a, u + gridDim.x, ntiles, nunits, U);
    if (u < nunits) load_unit();  // the next tile's inputs, in flight during the products
    f32x32 acc;
#pragma unroll
    for (int v = 0; v < 32; ++v) acc[v] = 0.0f;
    // eight channels per LDS read, the next reads in flight during the current eight steps
    uint4 xv = *reinterpret_cast<const uint4*>(&sm.xs[lane][0]);
    uint4 rv = *reinterpret_cast<const uint4*>(&sm.rs[rrow][0]);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint4 xn = *reinterpret_cast<const uint4*>(&sm.xs[lane][4 * ((i + 1) & 15)]);
      const uint4 rn = *reinterpret_cast<const uint4*>(&sm.rs[rrow][4 * ((i + 1) & 15)]);
      __builtin_amdgcn_sched_barrier(0);  // keep the reads ahead of this step's products
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
      const uint32_t rw[4] = {rv.x, rv.y, rv.z, rv.w};
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) {
        acc = __builtin_amdgcn_mfma_f32_32x32x1f32(half_lo<false>(rw[jj]), half_lo<BF16>(xw[jj]), acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x1f32(half_hi<false>(rw[jj]), half_hi<BF16>(xw[jj]), acc, 0, 0, 0);
      }
      xv = xn;
      rv = rn;
    }
    __syncthreads();  // every wave is done with the staged tile
    dense_int2_store<BF16>(a, C, acc, wv, lane, sm.clip[par]);
    par ^= 1;
  }
}

// resident workgroups of the persistent dense kernel on the current device
// Resident workgroups of the persistent dense int2 kernel on the current device (asked
// on every call: no state is kept between calls).
static int dense_grid_limit(bool bf16) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  hipError_t e = bf16 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, append_dense_int2_kernel<true>, NT, 0)
                      : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, append_dense_int2_kernel<false>, NT, 0);
  if (e != hipSuccess || per_cu <= 0) per_cu = 1;
  return cus * per_cu;
}

hipError_t launch_append(const AppendArgs& a, int grid_x, hipStream_t s) {
  dim3 grid(grid_x, a.H, 2 * a.B);  // K and V of every sequence in one launch
  const bool rescale = a.lam_k != nullptr || a.lam_v != nullptr;  // the generic kernel applies it
  if (a.rotation == KVQ_ROT_SRFT && !rescale) {  // SRFT in registers for the common pairs
    const dim3 fgrid((grid_x * a.H * 2 * a.B + 1) / 2);  // two units per workgroup
#define KVQ_FAST_SRFT(KF, KG, VF, VG)                                                  \
    if (a.k_fmt == KF && (KF == KVQ_FP4 || a.k_group == KG) && a.v_fmt == VF &&          \
        (VF == KVQ_FP4 || a.v_group == VG)) {                                            \
      if (a.in_bf16)                                                                    \
        hipLaunchKernelGGL((append_fast_kernel<KF, KG, VF, VG, true, true>), fgrid, dim3(NT), 0, s, a, grid_x); \
      else                                                                              \
        hipLaunchKernelGGL((append_fast_kernel<KF, KG, VF, VG, false, true>), fgrid, dim3(NT), 0, s, a, grid_x); \
      return hipGetLastError();                                                         \
    }
    KVQ_FAST_SRFT(KVQ_INT4, 32, KVQ_INT4, 32)
    KVQ_FAST_SRFT(KVQ_INT4, 16, KVQ_INT4, 16)
    KVQ_FAST_SRFT(KVQ_INT4, 128, KVQ_INT4, 128)
    KVQ_FAST_SRFT(KVQ_INT8, 128, KVQ_INT4, 128)
    KVQ_FAST_SRFT(KVQ_INT8, 32, KVQ_INT4, 32)
    KVQ_FAST_SRFT(KVQ_FP4, 16, KVQ_FP4, 16)
#undef KVQ_FAST_SRFT
  }
  if ((a.rotation == KVQ_ROT_NONE || a.rotation == KVQ_ROT_SIGN_FWHT) && !rescale) {
    const dim3 fgrid((grid_x * a.H * 2 * a.B + 1) / 2);  // two units per workgroup
#define KVQ_FAST(KF, KG, VF, VG)                                                       \
    if (a.k_fmt == KF && a.k_group == KG && a.v_fmt == VF && a.v_group == VG) {         \
      if (a.in_bf16)                                                                    \
        hipLaunchKernelGGL((append_fast_kernel<KF, KG, VF, VG, true>), fgrid, dim3(NT), 0, s, a, grid_x); \
      else                                                                              \
        hipLaunchKernelGGL((append_fast_kernel<KF, KG, VF, VG, false>), fgrid, dim3(NT), 0, s, a, grid_x); \
      return hipGetLastError();                                                         \
    }
    KVQ_FAST(KVQ_INT4, 32, KVQ_INT4, 32)
    KVQ_FAST(KVQ_INT4, 16, KVQ_INT4, 16)
    KVQ_FAST(KVQ_INT4, 128, KVQ_INT4, 128)
    KVQ_FAST(KVQ_INT8, 128, KVQ_INT4, 128)
    KVQ_FAST(KVQ_INT8, 32, KVQ_INT4, 32)
    KVQ_FAST(KVQ_INT4, 32, KVQ_INT4, 128)
    KVQ_FAST(KVQ_INT4, 128, KVQ_INT4, 32)
    KVQ_FAST(KVQ_INT8, 128, KVQ_INT4, 32)
    KVQ_FAST(KVQ_INT8, 32, KVQ_INT4, 128)
#undef KVQ_FAST
    if (a.k_fmt == KVQ_FP4 && a.v_fmt == KVQ_FP4) {  // group fields are not used by FP4
      if (a.in_bf16)
        hipLaunchKernelGGL((append_fast_kernel<KVQ_FP4, 16, KVQ_FP4, 16, true>), fgrid, dim3(NT), 0, s, a, grid_x);
      else
        hipLaunchKernelGGL((append_fast_kernel<KVQ_FP4, 16, KVQ_FP4, 16, false>), fgrid, dim3(NT), 0, s, a, grid_x);
      return hipGetLastError();
    }
  }
  if (a.rotation == KVQ_ROT_DENSE && a.desc == nullptr && !rescale && a.k_fmt == KVQ_INT2 && a.v_fmt == KVQ_INT2 &&
      a.k_group == 32 && a.v_group == 32) {
    const int nunits = grid_x * a.H * 2 * a.B;
    const int g = std::min(nunits, dense_grid_limit(a.in_bf16 != 0));
    if (a.in_bf16)
      hipLaunchKernelGGL(append_dense_int2_kernel<true>, dim3(g), dim3(NT), 0, s, a, grid_x, nunits);
    else
      hipLaunchKernelGGL(append_dense_int2_kernel<false>, dim3(g), dim3(NT), 0, s, a, grid_x, nunits);
    return hipGetLastError();
  }
  if (a.rotation == KVQ_ROT_DENSE)
    hipLaunchKernelGGL((append_kernel<true, false>), grid, dim3(NT), 0, s, a);
  else if (a.rotation == KVQ_ROT_SRFT)
    hipLaunchKernelGGL((append_kernel<false, true>), grid, dim3(NT), 0, s, a);
  else
    hipLaunchKernelGGL((append_kernel<false, false>), grid, dim3(NT), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- full-precision window
// Copies the originals of the window blocks this append reaches ("OSCAR", section
// 2.2B, mixed-precision layout: sink and recent tokens kept at full precision).
// Workgroup w < n_sink takes sink block w; workgroup n_sink + i takes block
// jlast - i, the i-th newest block of the call (skipped if it is a sink block), so
// the ring slots written by one call are distinct.  Rows are 256-byte copies.
__global__ __launch_bounds__(NT) void window_copy_kernel(AppendArgs a) {
  const int b = blockIdx.z >> 1, h = blockIdx.y, tensor = blockIdx.z & 1;
  const int start = a.start.v[b], end = start + a.n_new;
  const int w = blockIdx.x;
  const int jlast = (end - 1) / TILE;
  int j = w;
  if (w >= a.n_sink) {
    j = jlast - (w - a.n_sink);
    if (j < a.n_sink) return;  // a sink block, or before position 0
  }
  const int lo = max(start, j * TILE), hi = min(end, j * TILE + TILE);
  if (lo >= hi) return;  // uniform over the workgroup
  const int slot = j < a.n_sink ? j : a.n_sink + j % a.n_recent;
  const size_t stream = (size_t)b * a.H + h;
  KVQ_DCHECK(slot >= 0 && slot < a.n_sink + a.n_recent && lo >= j * TILE && hi <= j * TILE + TILE, DBG_WINDOW,
             stream, j);
  KVQ_DCHECK(stream < (size_t)a.B * a.H && lo >= start && hi <= end && hi <= a.Tmax, DBG_POS, stream, hi);
  const uint4* src = reinterpret_cast<const uint4*>((tensor ? a.v_new : a.k_new) + (stream * a.n_new + (lo - start)) * D);
  uint4* dst = reinterpret_cast<uint4*>((tensor ? a.v_win : a.k_win) +
                                        ((stream * (a.n_sink + a.n_recent) + slot) * TILE + (lo - j * TILE)) * D);
  const int n16 = (hi - lo) * (D * 2 / 16);
  for (int i = threadIdx.x; i < n16; i += NT) dst[i] = src[i];
}

hipError_t launch_window_copy(const AppendArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(window_copy_kernel, dim3(a.n_sink + a.n_recent, a.H, 2 * a.B), dim3(NT), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- clip calibration
// t[h][c] = fl32(ratio * max_t |y_t,c|): one workgroup per kv head, 64 tokens per step.
__global__ __launch_bounds__(NT) void calibrate_kernel(CalibArgs a) {
  __shared__ DenseSmem sm;
  __shared__ unsigned int amax[D];
  static_assert(sizeof(SrftSmem) <= sizeof(DenseSmem), "the SRFT rows share the dense staging area");
  SrftSmem& ss = *reinterpret_cast<SrftSmem*>(&sm);  // used only by the SRFT rotation
  const int h = blockIdx.x;
  const int t = threadIdx.x, tau = t >> 2, q = t & 3;
  const bool bf16 = a.in_bf16 != 0;
  if (t < D) amax[t] = 0u;
  if (a.rotation == KVQ_ROT_SRFT && t < 65) {
    ss.twr[t] = a.tw_re[t];
    ss.twi[t] = a.tw_im[t];
  }
  float run[32];
#pragma unroll
  for (int j = 0; j < 32; ++j) run[j] = 0.0f;
  for (int base = 0; base < a.n; base += TILE) {
    const int tok = base + tau;
    const bool valid = tok < a.n;
    const uint16_t* src = a.x + (((size_t)h * a.n + (valid ? tok : 0)) * D + 32 * q);
    float y[32];
    if (a.rotation == KVQ_ROT_DENSE) {
      __syncthreads();
      {
        const uint4* s4 = reinterpret_cast<const uint4*>(src);
        uint4* d4 = reinterpret_cast<uint4*>(&sm.xs[tau][32 * q]);
#pragma unroll
        for (int i = 0; i < 4; ++i) d4[i] = valid ? s4[i] : make_uint4(0, 0, 0, 0);
      }
      __syncthreads();
      const int lane = t & 63, wv = t >> 6;
      for (int vv = 0; vv < 16; ++vv) {
        const int vec = wv * 16 + vv;
        float acc0 = 0.0f, acc1 = 0.0f;
        const uint16_t* r0 = a.rot + (size_t)lane * D;
        const uint16_t* r1 = a.rot + (size_t)(lane + 64) * D;
        for (int k = 0; k < D; ++k) {
          float xk = widen(sm.xs[vec][k], bf16);
          acc0 = __builtin_fmaf(f16_bits_to_f32(r0[k]), xk, acc0);
          acc1 = __builtin_fmaf(f16_bits_to_f32(r1[k]), xk, acc1);
        }
        sm.ys[vec][lane] = acc0;
        sm.ys[vec][lane + 64] = acc1;
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < 32; ++j) y[j] = sm.ys[tau][32 * q + j];
    } else {
      if (valid) {
        load32(src, bf16, y);
      } else {
#pragma unroll
        for (int j = 0; j < 32; ++j) y[j] = 0.0f;
      }
      if (a.rotation == KVQ_ROT_SIGN_FWHT) sign_fwht(y, a.signs, q);
      if (a.rotation == KVQ_ROT_SRFT) srft_quad(y, a.signs, q, t >> 2, ss);  // uniform: every thread
    }
    if (a.lam != nullptr && a.mode == 0) {  // thresholds of the rescaled vectors
      const float* lp = a.lam + (size_t)h * D + 32 * q;
#pragma unroll
      for (int j = 0; j < 32; ++j) y[j] = y[j] * lp[j];
    }
    if (valid) {
#pragma unroll
      for (int j = 0; j < 32; ++j) run[j] = fmaxf(run[j], fabsf(y[j]));
    }
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 32; ++j) atomicMax(&amax[32 * q + j], __float_as_uint(run[j]));
  __syncthreads();
  if (t < D) {
    const float m = __uint_as_float(amax[t]);
    a.out[(size_t)h * D + t] = a.mode == 0 ? a.ratio * m : (m > 0.0f ? 1.0f / m : 1.0f);
  }
}

hipError_t launch_calibrate(const CalibArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(calibrate_kernel, dim3(a.H), dim3(NT), 0, s, a);
  return hipGetLastError();
}

#ifdef KVQ_DEBUG
KVQ_DBG_READER(dbg_read_append)
#endif

}  // namespace kvq
