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
// elements (fp16 bits or E4M3 codes) and the squared-residual partial sum.

// symmetric int4/int8; group 32 (in-lane) or 128 (quad)
__device__ __forceinline__ void quant_sym(const float y[32], int qmax, int group, int codes[32],
                                          uint16_t& meta, float& res2) {
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) a = fmaxf(a, fabsf(y[j]));
  if (group == 128) {
    a = fmaxf(a, dpp_f<KVQ_DPP_XOR1>(a));
    a = fmaxf(a, dpp_f<KVQ_DPP_XOR2>(a));
  }
  uint16_t sb = f16_sat_bits(a / (float)qmax);  // correctly rounded fp32 divide
  float sf = f16_bits_to_f32(sb);
  meta = sb;
  float r = __builtin_amdgcn_rcpf(sf);
  float qm = (float)qmax;
  float acc = 0.0f;
#pragma unroll
  for (int j = 0; j < 32; ++j) {
    float c = 0.0f;
    if (sf != 0.0f) c = fminf(fmaxf(rne_quot(y[j], sf, r), -qm), qm);
    codes[j] = (int)c;
    float d = y[j] - c * sf;
    acc = acc + d * d;
  }
  res2 = acc;
}

// asymmetric int2, group 32, optional clamp to [-t_c, t_c] first
__device__ __forceinline__ void quant_asym2(const float y[32], const float* clip, int codes[32], uint16_t& ms,
                                            uint16_t& mz, float& res2) {
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

// FP4 with E4M3 block scales (two blocks of 16 per lane)
__device__ __forceinline__ void quant_fp4(const float y[32], int search, int codes[32], uint8_t sc[2],
                                          float& res2) {
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
#pragma unroll
    for (int k = 0; k < 9; ++k) {
      if (!search && k != 4) continue;
      uint32_t c = e4m3_encode_nonneg(t * mults[k]);
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

}  // namespace

template <bool DENSE>
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
  if (a.rotation == KVQ_ROT_SIGN_FWHT) {
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
    for (int vv = 0; vv < 16; ++vv) {
      const int vec = wv * 16 + vv;
      const int vpos = tile * TILE + vec;
      if (vpos < lo || vpos >= hi) continue;  // uniform over the wave
      float acc0 = 0.0f, acc1 = 0.0f;
      const uint4* xr = reinterpret_cast<const uint4*>(&sm.xs[vec][0]);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        uint4 u = xr[i];
        uint32_t xw[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          const int k = 8 * i + 2 * jj;
          float x0 = widen((uint16_t)(xw[jj] & 0xFFFF), bf16), x1 = widen((uint16_t)(xw[jj] >> 16), bf16);
          uint32_t p0 = r0[k / 2], p1 = r1[k / 2];
          acc0 = __builtin_fmaf(f16_bits_to_f32((uint16_t)(p0 & 0xFFFF)), x0, acc0);
          acc0 = __builtin_fmaf(f16_bits_to_f32((uint16_t)(p0 >> 16)), x1, acc0);
          acc1 = __builtin_fmaf(f16_bits_to_f32((uint16_t)(p1 & 0xFFFF)), x0, acc1);
          acc1 = __builtin_fmaf(f16_bits_to_f32((uint16_t)(p1 >> 16)), x1, acc1);
        }
      }
      sm.ys[vec][lane] = acc0;
      sm.ys[vec][lane + 64] = acc1;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 32; ++j) y[j] = sm.ys[tau][32 * q + j];
  } else {
#pragma unroll
    for (int j = 0; j < 32; ++j) y[j] = x[j];
  }

  // quantize
  int codes[32];
  uint16_t m0 = 0, m1 = 0;  // metadata elements of this lane
  float res2 = 0.0f;
  if (fmt == KVQ_INT4 || fmt == KVQ_INT8) {
    quant_sym(y, fmt == KVQ_INT4 ? 7 : 127, group, codes, m0, res2);
  } else if (fmt == KVQ_INT2) {
    const float* clip = tensor ? a.clip_v : a.clip_k;
    quant_asym2(y, clip ? clip + (size_t)h * D + 32 * q : nullptr, codes, m0, m1, res2);
  } else {
    uint8_t sc[2];
    quant_fp4(y, a.scale_mode == KVQ_SCALE_SEARCH9, codes, sc, res2);
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
    float ynorm2 = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; ++j) ynorm2 = ynorm2 + y[j] * y[j];
    // outward-rounded norms: fp32 sum/sqrt error and the rotation's own rounding
    const float slack = a.rotation == KVQ_ROT_DENSE ? 2.44140625e-4f : (a.rotation == KVQ_ROT_SIGN_FWHT ? 9.5367431640625e-7f : 0.0f);
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

hipError_t launch_append(const AppendArgs& a, int grid_x, hipStream_t s) {
  dim3 grid(grid_x, a.H, 2 * a.B);  // K and V of every sequence in one launch
  if (a.rotation == KVQ_ROT_DENSE)
    hipLaunchKernelGGL(append_kernel<true>, grid, dim3(NT), 0, s, a);
  else
    hipLaunchKernelGGL(append_kernel<false>, grid, dim3(NT), 0, s, a);
  return hipGetLastError();
}

// ---------------------------------------------------------------- clip calibration
// t[h][c] = fl32(ratio * max_t |y_t,c|): one workgroup per kv head, 64 tokens per step.
__global__ __launch_bounds__(NT) void calibrate_kernel(CalibArgs a) {
  __shared__ DenseSmem sm;
  __shared__ unsigned int amax[D];
  const int h = blockIdx.x;
  const int t = threadIdx.x, tau = t >> 2, q = t & 3;
  const bool bf16 = a.in_bf16 != 0;
  if (t < D) amax[t] = 0u;
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
  if (t < D) a.out[(size_t)h * D + t] = a.ratio * __uint_as_float(amax[t]);
}

hipError_t launch_calibrate(const CalibArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(calibrate_kernel, dim3(a.H), dim3(NT), 0, s, a);
  return hipGetLastError();
}

}  // namespace kvq
