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

// One step of the wave's arg-max: each lane takes the better of its own
// (value, id) and the one DPP pattern C brings from another lane of its row.
template <int C>
__device__ __forceinline__ void route_dpp_step(float& bv, int& bi) {
  const float ov = __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, bv), C, 0xF, 0xF,
                                                                         false));
  const int oi = __builtin_amdgcn_update_dpp(0, bi, C, 0xF, 0xF, false);
  const bool better = route_before(ov, oi, bv, bi);
  bv = better ? ov : bv;
  bi = better ? oi : bi;
}

// Token t's logits for the top-k below: lane holds experts lane + 64 i
// (raw; the selection reads NaN as -inf).  A separate step so that a caller
// can issue these loads before other memory work and select afterwards.
template <int NS>
__device__ __forceinline__ void topk_load(const float* __restrict__ logits, int t, int E, int lane, float (&v)[NS]) {
  const __amdgpu_buffer_rsrc_t rs = uniform_rsrc(logits + (int64_t)t * E, E * 4);
#pragma unroll
  for (int i = 0; i < NS; ++i)
    v[i] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(rs, (lane + 64 * i) * 4, 0, 0));
}

// Top-k of token t by one wave from its loaded logits.  NS: 64-expert slots
// per lane (E <= 64 NS).  Branch-free: out-of-range and taken experts compare
// as never better.
template <int NS>
__device__ __forceinline__ void topk_select(const float (&raw)[NS], int t, int E, int topk, int lane,
                                            int32_t* __restrict__ ids, float* __restrict__ gates) {
  // NaN ranks as -inf.
  float v[NS];
#pragma unroll
  for (int i = 0; i < NS; ++i) v[i] = (lane + 64 * i < E && raw[i] == raw[i]) ? raw[i] : -INFINITY;
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
    // Arg-max over the wave under the strict order route_before (unique, so
    // the order of combination does not matter): within each 16-lane row by
    // DPP (swap neighbours, swap pairs, mirror each half-row, mirror the row;
    // a few cycles each, where a general lane shuffle is a round trip
    // through the LDS crossbar), then over the four rows' lane 0.
    route_dpp_step<0xB1>(bv, bi);    // quad_perm [1, 0, 3, 2]
    route_dpp_step<0x4E>(bv, bi);    // quad_perm [2, 3, 0, 1]
    route_dpp_step<0x141>(bv, bi);   // row_half_mirror
    route_dpp_step<0x140>(bv, bi);   // row_mirror
    {
      float rv = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bv), 0));
      int ri = __builtin_amdgcn_readlane(bi, 0);
#pragma unroll
      for (int row = 1; row < 4; ++row) {
        const float ov = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, bv), 16 * row));
        const int oi = __builtin_amdgcn_readlane(bi, 16 * row);
        const bool better = route_before(ov, oi, rv, ri);
        rv = better ? ov : rv;
        ri = better ? oi : ri;
      }
      bv = rv;
      bi = ri;
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

template <int NS>
__device__ __forceinline__ void topk_token(const float* __restrict__ logits, int t, int E, int topk, int lane,
                                           int32_t* __restrict__ ids, float* __restrict__ gates) {
  float v[NS];
  topk_load<NS>(logits, t, E, lane, v);
  topk_select<NS>(v, t, E, topk, lane, ids, gates);
}

}  // namespace q4q8
