// Per-block certified error bound ("Runtime-Certified Bounded-Error Quantized
// Attention", Methodology section 2): the key term is the largest logit change
// any token of the block can see, max ||q|| * scale * ek (Cauchy-Schwarz over the
// GQA group sharing the kv head), the value term is ev; a block whose sum
// exceeds tau is flagged for exact recompute.  Only tracked quantities are read
// (descriptors and the query), never the fp16 originals.
#include "kvq_common.h"

namespace kvq {

__global__ __launch_bounds__(256) void bound_kernel(BoundArgs a) {
  const int b = blockIdx.x / a.H, h = blockIdx.x % a.H;
  const int G = a.Hq / a.H;
  const bool bf16 = a.in_bf16 != 0;
  __shared__ float qn_s;
  // largest query norm of the group: one wave, lanes over channels
  if (threadIdx.x < 64) {
    float best = 0.0f;
    for (int g = 0; g < G; ++g) {
      const uint16_t* qp = a.q + ((size_t)b * a.Hq + h * G + g) * D;
      float x0 = widen(qp[2 * threadIdx.x], bf16), x1 = widen(qp[2 * threadIdx.x + 1], bf16);
      float s = x0 * x0 + x1 * x1;
      for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
      best = fmaxf(best, sqrtf(s));
    }
    if (threadIdx.x == 0) qn_s = best;
  }
  __syncthreads();
  const float coef = qn_s * a.scale;
  const int nb = (a.seq.v[b] + TILE - 1) / TILE;
  const size_t base = ((size_t)b * a.H + h) * a.nt;
  KVQ_DCHECK(b < a.B && nb >= 0 && nb <= a.nt, DBG_CHUNK, (size_t)b * a.H + h, nb);
  for (int j = threadIdx.x; j < a.nt; j += blockDim.x) {
    float bd = 0.0f;
    if (j < nb) {
      const float* d = a.desc + (base + j) * 3;
      bd = coef * d[0] + d[1];
    }
    a.bound[base + j] = bd;
    a.flags[base + j] = bd > a.tau ? 1 : 0;
  }
}

hipError_t launch_bound(const BoundArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(bound_kernel, dim3(a.B * a.H), dim3(256), 0, s, a);
  return hipGetLastError();
}

#ifdef KVQ_DEBUG
KVQ_DBG_READER(dbg_read_bound)
#endif

}  // namespace kvq
