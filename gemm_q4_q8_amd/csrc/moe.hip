// Mixture-of-experts layer over Q4_0 / Q8_0 expert weights: route, sort,
// grouped gate+up GEMM with SwiGLU, grouped down GEMM, weighted combine.
//
// The pages run MoE layers with expert GEMMs and fused expert projections on
// the matrix units ("BaseRT" M5 follow-up review, "Method"); routing and the
// permutation are not on the pages and follow the plainest reading: top-k of
// the router logits (descending, equal logits to the lower expert id),
// softmax over the k selected logits, pairs p = t k + j sorted stably by
// expert.
//
//   moe_topk_kernel   one wave per token: k rounds of a wave-wide argmax.
//   moe_sort_kernel   one workgroup: per-wave histograms, scan, then each
//                     wave places its pairs in order (ranks from ballots), so
//                     the order is stable and bit-exact.
//   moe_gateup_kernel tile engine with two weight matrices (gate, up) over
//                     the expert's rows gathered from X by token; epilogue
//                     h = silu(z_gate) * z_up, rounded to bf16 (h's storage
//                     precision) and kept as fp16 for the down GEMM (exact).
//   moe_down_kernel   tile engine over the contiguous h rows of the expert;
//                     y_p stored as fp16 at its pair index p.
//   moe_combine_kernel out[t] = sum_j g[t, j] y_{t k + j} in fp32, j in order:
//                     deterministic (no atomics).
#include "q4q8_dev.h"
#include "q4q8_internal.h"
#include "qgemm_core.h"

#include <math.h>

namespace q4q8 {

constexpr int kRouteMaxE = 1024;
constexpr int kRouteMaxK = 16;
constexpr int kSortWaves = 16;

// ---------------------------------------------------------------------------
// Route: ids[t, j], gates[t, j]
// ---------------------------------------------------------------------------

// (v, i) ranks before (bv, bi): larger value, then lower expert id.
__device__ __forceinline__ bool route_before(float v, int i, float bv, int bi) {
  return v > bv || (v == bv && i < bi);
}

// NS: 64-expert slots per lane (E <= 64 NS).  Branch-free: out-of-range and
// taken experts compare as never better.
template <int NS>
__global__ __launch_bounds__(256) void moe_topk_kernel(const float* __restrict__ logits, int T, int E, int topk,
                                                       int32_t* __restrict__ ids, float* __restrict__ gates) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;   // whole wave
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

// ---------------------------------------------------------------------------
// Sort: counts, offsets, sorted_pairs (stable counting sort, one workgroup)
// ---------------------------------------------------------------------------

__global__ __launch_bounds__(1024) void moe_sort_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                        int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ sorted_pairs) {
  __shared__ int hist_s[kSortWaves * kRouteMaxE];   // [wave][expert]: counts, then bases
  int* hist = hist_s;
  __shared__ int wave_sum[kSortWaves];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int chunk = ((P + kSortWaves - 1) / kSortWaves + 63) / 64 * 64;
  const int p0 = w * chunk, p1 = min(P, p0 + chunk);

  for (int i = tid; i < kSortWaves * E; i += 1024) hist[i] = 0;
  __syncthreads();
  for (int p = p0 + lane; p < p1; p += 64) {
    const int e = min(max(ids[p], 0), E - 1);
    atomicAdd(&hist[w * E + e], 1);
  }
  __syncthreads();

  // Thread e: total count, exclusive scan over experts, per-wave bases.
  int tot = 0;
  if (tid < E)
    for (int k = 0; k < kSortWaves; ++k) tot += hist[k * E + tid];
  int incl = tot;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) wave_sum[w] = incl;
  __syncthreads();
  int before = 0;
  for (int k = 0; k < w; ++k) before += wave_sum[k];
  const int excl = before + incl - tot;
  if (tid < E) {
    counts[tid] = tot;
    offsets[tid] = excl;
    int run = excl;
    for (int k = 0; k < kSortWaves; ++k) {
      const int c = hist[k * E + tid];
      hist[k * E + tid] = run;
      run += c;
    }
  }
  if (tid == 0) offsets[E] = P;
  __syncthreads();

  // Each wave places its own range in order.  Lanes with equal expert find
  // each other with one ballot per bit of the expert id.
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int base = p0; base < p1; base += 64) {
    const int p = base + lane;
    const bool active = p < p1;
    const int e = active ? min(max(ids[p], 0), E - 1) : 0;
    uint64_t match = __ballot(active);
#pragma unroll
    for (int b = 0; b < 10; ++b) {
      const uint64_t ones = __ballot(active && ((e >> b) & 1));
      match &= ((e >> b) & 1) ? ones : ~ones;
    }
    const int rank = __popcll(match & below);
    const int pos = hist[w * E + e] + rank;
    if (active) sorted_pairs[pos] = p;
    const int last = 63 - __clzll(match);
    if (active && lane == last) hist[w * E + e] = pos + 1;
  }
}

hipError_t launch_moe_route(const float* logits, int T, int E, int topk, int32_t* ids, float* gates,
                            int32_t* counts, int32_t* offsets, int32_t* sorted_pairs, hipStream_t stream) {
  const dim3 grid((unsigned)((T + 3) / 4)), block(256);
  if (E <= 64) moe_topk_kernel<1><<<grid, block, 0, stream>>>(logits, T, E, topk, ids, gates);
  else if (E <= 128) moe_topk_kernel<2><<<grid, block, 0, stream>>>(logits, T, E, topk, ids, gates);
  else if (E <= 256) moe_topk_kernel<4><<<grid, block, 0, stream>>>(logits, T, E, topk, ids, gates);
  else if (E <= 512) moe_topk_kernel<8><<<grid, block, 0, stream>>>(logits, T, E, topk, ids, gates);
  else moe_topk_kernel<16><<<grid, block, 0, stream>>>(logits, T, E, topk, ids, gates);
  moe_sort_kernel<<<dim3(1), dim3(1024), 0, stream>>>(ids, T * topk, E, counts, offsets, sorted_pairs);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Expert GEMMs
// ---------------------------------------------------------------------------

// Workgroup row index idx -> (expert e, first row r0 of the expert's segment)
// over the experts' ceil(count / BM) row tiles in expert order.  Every wave
// computes it (no barrier).  False when idx is past the last tile.
__device__ __forceinline__ bool find_row_tile(const int32_t* __restrict__ offsets, int E, int BM, int idx, int& e_out,
                                              int& r0_out) {
  const int lane = threadIdx.x & 63;
  int cum = 0;
  for (int base = 0; base < E; base += 64) {
    const int e = base + lane;
    const int c = e < E ? offsets[e + 1] - offsets[e] : 0;
    const int nt = (max(c, 0) + BM - 1) / BM;
    int incl = nt;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off);
      if (lane >= off) incl += o;
    }
    const int lo = cum + incl - nt;
    const uint64_t hit = __ballot(nt > 0 && idx >= lo && idx < cum + incl);
    if (hit) {
      const int src = __ffsll((unsigned long long)hit) - 1;
      e_out = __shfl(e, src);
      r0_out = (idx - __shfl(lo, src)) * BM;
      return true;
    }
    cum += __shfl(incl, 63);
  }
  return false;
}

// silu(z) = z / (1 + exp(-z)), fp32.
__device__ __forceinline__ float silu_f32(float z) { return z / (1.0f + expf(-z)); }

// Gate+up for one row tile of one expert and 64 NT h columns (per wave
// 16 NT).  x16: fp16 [T, H]; h16: fp16 [P, F] and h_out: bf16 [P, F] (may be
// null), both in sorted-pair order.
template <int FMT, int MT, int NT, int S>
__global__ __launch_bounds__(512) void moe_gateup_kernel(const uint8_t* __restrict__ Wg, const uint8_t* __restrict__ Wu,
                                                         int64_t wstride, int E, int H, int F,
                                                         const uint16_t* __restrict__ x16, int T, int topk,
                                                         const int32_t* __restrict__ offsets,
                                                         const int32_t* __restrict__ sorted_pairs,
                                                         uint16_t* __restrict__ h16, uint16_t* __restrict__ h_out) {
  using C = TileCfg<FMT, MT, NT, 2, S>;
  __shared__ __attribute__((aligned(1024))) uint16_t xs[C::LDS_HALFS];
  int e, r0;
  if (!find_row_tile(offsets, E, C::BM, blockIdx.y, e, r0)) return;   // uniform over the workgroup

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nw = wave & 3;
  const int r = lane & 15, g = lane >> 4;
  const int seg = offsets[e];
  const int valid = min(C::BM, offsets[e + 1] - seg - r0);
  const int nchunks = H / kChunkK;
  const int tiles = F / kTileRows;

  const int t0 = (blockIdx.x * 4 + nw) * NT;
  const int tv = tiles - t0 < NT ? (tiles - t0 > 0 ? tiles - t0 : 0) : NT;
  const int64_t woff = e * wstride + (int64_t)(t0 < tiles ? t0 : 0) * nchunks * C::REC;
  const __amdgpu_buffer_rsrc_t wres[2] = {uniform_rsrc(Wg + woff, tv * nchunks * C::REC),
                                          uniform_rsrc(Wu + woff, tv * nchunks * C::REC)};
  // Rows gathered by token: row i of the tile is pair sorted_pairs[seg + r0 + i].
  const __amdgpu_buffer_rsrc_t xres = uniform_rsrc(x16, (int)((int64_t)T * H * 2));
  uint32_t xv[C::XLOADS];
#pragma unroll
  for (int p = 0; p < C::XLOADS; ++p) {
    int row, cg;
    x_slot(p, tid, row, cg);
    uint32_t v = kOOB;
    if (row < valid) {
      const int tok = min(sorted_pairs[seg + r0 + row] / topk, T - 1);
      v = (uint32_t)(((int64_t)tok * H + cg * 8) * 2);
    }
    xv[p] = v;
  }

  float4_t acc[2 * MT * NT];
  tile_mainloop<FMT, MT, NT, 2, S, false>(wres, tv, H, nchunks, xres, xv, xs, acc);
  float4_t kept[2 * (MT / 2) * NT];
  khalf_reduce<MT, NT, 2>(acc, (float4_t*)xs, kept);

  const int rk = (wave >> 2) * (MT / 2) * 16 + 4 * g;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = (t0 + t) * kTileRows + r;
    if (n < F) {
#pragma unroll
      for (int i = 0; i < MT / 2; ++i)
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const int row = rk + i * 16 + k;
          if (row < valid) {
            const float zg = kept[i * NT + t][k], zu = kept[((MT / 2) + i) * NT + t][k];
            const __bf16 hb = (__bf16)(silu_f32(zg) * zu);
            const int64_t idx = (int64_t)(seg + r0 + row) * F + n;
            h16[idx] = __builtin_bit_cast(uint16_t, (_Float16)(float)hb);
            if (h_out) h_out[idx] = __builtin_bit_cast(uint16_t, hb);
          }
        }
    }
  }
}

// Down projection for one row tile of one expert and 64 NT output columns:
// y16[p] (fp16 [P, H], pair order) = h16 rows (contiguous per expert) W_d^T.
template <int FMT, int MT, int NT, int S>
__global__ __launch_bounds__(512) void moe_down_kernel(const uint8_t* __restrict__ Wd, int64_t wstride, int E, int H,
                                                       int F, const uint16_t* __restrict__ h16, int P,
                                                       const int32_t* __restrict__ offsets,
                                                       const int32_t* __restrict__ sorted_pairs,
                                                       uint16_t* __restrict__ y16) {
  using C = TileCfg<FMT, MT, NT, 1, S>;
  __shared__ __attribute__((aligned(1024))) uint16_t xs[C::LDS_HALFS];
  int e, r0;
  if (!find_row_tile(offsets, E, C::BM, blockIdx.y, e, r0)) return;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nw = wave & 3;
  const int r = lane & 15, g = lane >> 4;
  const int seg = offsets[e];
  const int valid = min(C::BM, offsets[e + 1] - seg - r0);
  const int nchunks = F / kChunkK;
  const int tiles = H / kTileRows;

  const int t0 = (blockIdx.x * 4 + nw) * NT;
  const int tv = tiles - t0 < NT ? (tiles - t0 > 0 ? tiles - t0 : 0) : NT;
  const __amdgpu_buffer_rsrc_t wres[1] = {
      uniform_rsrc(Wd + e * wstride + (int64_t)(t0 < tiles ? t0 : 0) * nchunks * C::REC, tv * nchunks * C::REC)};
  const __amdgpu_buffer_rsrc_t xres = uniform_rsrc(h16, (int)((int64_t)P * F * 2));
  uint32_t xv[C::XLOADS];
#pragma unroll
  for (int p = 0; p < C::XLOADS; ++p) {
    int row, cg;
    x_slot(p, tid, row, cg);
    xv[p] = row < valid ? (uint32_t)(((int64_t)(seg + r0 + row) * F + cg * 8) * 2) : kOOB;
  }

  float4_t acc[MT * NT];
  tile_mainloop<FMT, MT, NT, 1, S, false>(wres, tv, F, nchunks, xres, xv, xs, acc);
  float4_t kept[(MT / 2) * NT];
  khalf_reduce<MT, NT, 1>(acc, (float4_t*)xs, kept);

  const int rk = (wave >> 2) * (MT / 2) * 16 + 4 * g;
#pragma unroll
  for (int i = 0; i < MT / 2; ++i)
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const int row = rk + i * 16 + k;
      if (row < valid) {
        const int64_t pair = min(max(sorted_pairs[seg + r0 + row], 0), P - 1);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          const int n = (t0 + t) * kTileRows + r;
          if (n < H) y16[pair * H + n] = __builtin_bit_cast(uint16_t, (_Float16)kept[i * NT + t][k]);
        }
      }
    }
}

// out[t, n] = sum_j gates[t, j] y16[t k + j, n]; 8 columns per thread.
__global__ __launch_bounds__(256) void moe_combine_kernel(const uint16_t* __restrict__ y16,
                                                          const float* __restrict__ gates, int T, int topk, int H,
                                                          float* __restrict__ out) {
  const int c8 = blockIdx.x * 256 + threadIdx.x;
  const int t = blockIdx.y;
  if (c8 * 8 >= H) return;
  float s[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int j = 0; j < topk; ++j) {
    const float gj = gates[(int64_t)t * topk + j];
    const u32x4_t v = *(const u32x4_t*)(y16 + ((int64_t)t * topk + j) * H + c8 * 8);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint32_t w = v[q];
      const half2_t h = __builtin_bit_cast(half2_t, w);
      s[2 * q] += gj * (float)h[0];
      s[2 * q + 1] += gj * (float)h[1];
    }
  }
  float4_t* o = (float4_t*)(out + (int64_t)t * H + c8 * 8);
  o[0] = float4_t{s[0], s[1], s[2], s[3]};
  o[1] = float4_t{s[4], s[5], s[6], s[7]};
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

namespace {
constexpr int kMoeMT = 4;   // 64-row tiles: about one per expert at 32 pairs per expert
constexpr int kMoeNT = 2;   // 128 columns per workgroup
constexpr int kMoeS = 4;
constexpr int kMoeBM = 16 * kMoeMT;

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

struct MoeWs {
  uint16_t* x16;
  uint16_t* h16;
  uint16_t* y16;
};

MoeWs moe_ws_layout(void* ws, int T, int topk, int H, int F) {
  const size_t P = (size_t)T * topk;
  uint8_t* b = (uint8_t*)ws;
  MoeWs w;
  w.x16 = (uint16_t*)b;
  b += round256((size_t)T * H * 2);
  w.h16 = (uint16_t*)b;
  b += round256(P * F * 2);
  w.y16 = (uint16_t*)b;
  return w;
}

template <int FMT>
void launch_experts(const void* Wg, const void* Wu, const void* Wd, int E, int H, int F, const uint16_t* x16, int T,
                    int topk, const float* gates, const int32_t* offsets, const int32_t* sorted_pairs, float* out,
                    void* h_out, const MoeWs& w, hipStream_t s) {
  const int P = T * topk;
  const int max_rtiles = (P + kMoeBM - 1) / kMoeBM + E;
  const int64_t sg = (int64_t)(F / kTileRows) * (H / kChunkK) * Fmt<FMT>::kRecBytes;   // repacked [F, H]
  const int64_t sd = (int64_t)(H / kTileRows) * (F / kChunkK) * Fmt<FMT>::kRecBytes;   // repacked [H, F]
  moe_gateup_kernel<FMT, kMoeMT, kMoeNT, kMoeS>
      <<<dim3((unsigned)((F + 64 * kMoeNT - 1) / (64 * kMoeNT)), (unsigned)max_rtiles), dim3(512), 0, s>>>(
          (const uint8_t*)Wg, (const uint8_t*)Wu, sg, E, H, F, x16, T, topk, offsets, sorted_pairs, w.h16,
          (uint16_t*)h_out);
  moe_down_kernel<FMT, kMoeMT, kMoeNT, kMoeS>
      <<<dim3((unsigned)((H + 64 * kMoeNT - 1) / (64 * kMoeNT)), (unsigned)max_rtiles), dim3(512), 0, s>>>(
          (const uint8_t*)Wd, sd, E, H, F, w.h16, P, offsets, sorted_pairs, w.y16);
  moe_combine_kernel<<<dim3((unsigned)((H / 8 + 255) / 256), (unsigned)T), dim3(256), 0, s>>>(w.y16, gates, T, topk,
                                                                                              H, out);
}
}  // namespace

size_t moe_workspace_bytes(int fmt, int T, int E, int topk, int H, int F) {
  (void)fmt;
  (void)E;
  const size_t P = (size_t)T * topk;
  return round256((size_t)T * H * 2) + round256(P * F * 2) + round256(P * H * 2);
}

hipError_t launch_moe_qgemm(int fmt, int xdt, const void* Wg, const void* Wu, const void* Wd, int E, int H, int F,
                            const void* X, int T, int topk, const float* gates, const int32_t* offsets,
                            const int32_t* sorted_pairs, float* out, void* h_out, void* ws, hipStream_t stream) {
  const MoeWs w = moe_ws_layout(ws, T, topk, H, F);
  const uint16_t* x16 = (const uint16_t*)X;
  if (xdt == kBF16) {
    const hipError_t e = launch_bf16_to_f16(X, H, w.x16, H, T, H, H, stream, LaunchEvents());
    if (e != hipSuccess) return e;
    x16 = w.x16;
  }
  if (fmt == kQ4_0)
    launch_experts<kQ4_0>(Wg, Wu, Wd, E, H, F, x16, T, topk, gates, offsets, sorted_pairs, out, h_out, w, stream);
  else
    launch_experts<kQ8_0>(Wg, Wu, Wd, E, H, F, x16, T, topk, gates, offsets, sorted_pairs, out, h_out, w, stream);
  return hipGetLastError();
}

}  // namespace q4q8
