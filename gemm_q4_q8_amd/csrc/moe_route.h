// Top-k routing of one token by one wave, shared by the routing kernels and
// the routed decode kernel: the token's topk largest logits (ties to the
// lower expert id, NaN as -inf) and their softmax over the selected logits
// ("BaseRT: Advancing Best-in-Class LLM Inference with Apple M5 Neural
// Accelerators", review, "Method": mixture-of-experts routing).
#pragma once

#include "q4q8_dev.h"

#include <math.h>

namespace q4q8 {

// (v, i) ranks before (bv, bi): larger value, then lower expert id.
__device__ __forceinline__ bool route_before(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// Top-k of token t by one wave.  NS: 64-expert slots per lane (E <= 64 NS).
// Branch-free: out-of-range and taken experts compare as never better.
template <int NS>
__device__ __forceinline__ void topk_token(const float* __restrict__ logits, int t, int E, int topk, int lane,
                                           int32_t* __restrict__ ids, float* __restrict__ gates) {
  // Lane holds experts lane + 64 i.  NaN ranks as -inf.
  const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(logits + (int64_t)t * E, E * 4);
  float v[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) {
    const float x = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (lane + 64 * i) * 4, 0, 0));
    v[i] = (lane + 64 * i < E && x == x) ? x : -INFINITY;
  }
  uint32_t live = 0;   // bit i: expert lane + 64 i exists and is not taken yet
#pragma unroll
  for (int i = 0; i < NS; ++i) live |= (lane + 64 * i < E ? 1u : 0u) << i;
  float v0 = 0.0f, my_exp = 0.0f, sum = 0.0f;
  for (int j = 0; j < topk; ++j) {
    float bv = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const bool better = ((live >> i) & 1u) && route_before(v[i], lane + 64 * i, bv, bi);
      bv = better ? v[i] : bv;
      bi = better ? lane + 64 * i : bi;
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
      const float ov = __shfl_xor(bv, off);
      const int oi = __shfl_xor(bi, off);
      const bool better = route_before(ov, oi, bv, bi);
      bv = better ? ov : bv;
      bi = better ? oi : bi;
    }
    // Every lane now holds the winner; its owner marks it taken.
    live &= ~(((bi & 63) == lane ? 1u : 0u) << (bi >> 6));
    v0 = j == 0 ? bv : v0;
    const float ex = expf(bv - v0);
    sum += ex;
    my_exp = lane == j ? ex : my_exp;
    if (lane == 0) ids[(int64_t)t * topk + j] = bi;
  }
  if (lane < topk) gates[(int64_t)t * topk + lane] = my_exp / sum;
}

}  // namespace q4q8
