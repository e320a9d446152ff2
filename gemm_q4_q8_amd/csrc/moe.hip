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
//   moe_route_small_kernel  both in one workgroup for up to 16 tokens.
//   moe_stream_kernel gate+up: the expert's rows gathered from X by token
//                     into LDS, gate and up weights streamed per wave;
//                     epilogue h = silu(z_gate) * z_up, rounded to bf16 (h's
//                     storage precision) and kept as fp16 for the down GEMM
//                     (exact).  down: the expert's contiguous h rows in LDS,
//                     y_p stored as fp16 at its pair index p.
//   moe_combine_kernel out[t] = sum_j g[t, j] y_{t k + j} in fp32, j in order:
//                     deterministic (no atomics).
#include "q4q8_dev.h"
#include "q4q8_internal.h"
#include "moe_route.h"
#include "qgemm_core.h"   // static_for, x_slot, kOOB

#include <math.h>

#include <algorithm>

namespace q4q8 {

constexpr int kRouteMaxE = 1024;
constexpr int kRouteMaxK = 16;
constexpr int kSortWaves = 16;
constexpr int kRankSortMaxPairs = 32;

// ---------------------------------------------------------------------------
// Route: ids[t, j], gates[t, j]
// ---------------------------------------------------------------------------

template <int NS>
__global__ __launch_bounds__(256) void moe_topk_kernel(const float* __restrict__ logits, int T, int E, int topk,
                                                       int32_t* __restrict__ ids, float* __restrict__ gates) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t < T) topk_token<NS>(logits, t, E, topk, threadIdx.x & 63, ids, gates);   // whole wave
}

// Top-k of token t and its row scaling (as the row-scaling pre-pass: the
// row times 2^-xexp[t] as fp16, its largest magnitude in [4, 8)): the
// routing and the activation pre-pass of the one-call MoE in one launch.
// Workgroup of 8 waves for 4 tokens: wave w < 4 routes token 4 b + w, wave
// 4 + w scales its row, so the two latency chains run side by side.  H is a
// multiple of 8.
template <int NS, int SRC>
__global__ __launch_bounds__(512) void moe_prep_kernel(const float* __restrict__ logits, int T, int E, int topk,
                                                       int32_t* __restrict__ ids, float* __restrict__ gates,
                                                       const uint16_t* __restrict__ X, int H,
                                                       uint16_t* __restrict__ x16, int32_t* __restrict__ xexp) {
  const int w = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + (w & 3);
  if (t >= T) return;   // whole wave
  const int lane = threadIdx.x & 63;
  if (w < 4) {
    topk_token<NS>(logits, t, E, topk, lane, ids, gates);
    return;
  }
  const uint16_t* xr = X + (int64_t)t * H;
  uint32_t m = 0;
  for (int c8 = lane; c8 < H / 8; c8 += 64) m = max(m, max_mag_bits8(*(const u32x4_t*)(xr + c8 * 8)));
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  const int ex = row_exponent<SRC>(m);
  if (lane == 0) xexp[t] = ex;
  for (int c8 = lane; c8 < H / 8; c8 += 64)
    *(u32x4_t*)(x16 + (int64_t)t * H + c8 * 8) = f16x8_scaled<SRC>(*(const u32x4_t*)(xr + c8 * 8), -ex);
}

// ---------------------------------------------------------------------------
// Sort: counts, offsets, sorted_pairs (stable counting sort, one workgroup)
// ---------------------------------------------------------------------------

// The sort body, run by one workgroup of kSortWaves waves.
__device__ __forceinline__ void sort_pairs(const int32_t* __restrict__ ids, int P, int E,
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

__global__ __launch_bounds__(1024) void moe_sort_kernel(const int32_t* __restrict__ ids, int P, int E,
                                                        int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ sorted_pairs) {
  sort_pairs(ids, P, E, counts, offsets, sorted_pairs);
}

// A few tokens (T <= kSortWaves): top-k and sort in one workgroup, one
// launch.  Wave t takes token t.
template <int NS>
__global__ __launch_bounds__(1024) void moe_route_small_kernel(const float* __restrict__ logits, int T, int E,
                                                               int topk, int32_t* __restrict__ ids,
                                                               float* __restrict__ gates, int32_t* __restrict__ counts,
                                                               int32_t* __restrict__ offsets,
                                                               int32_t* __restrict__ sorted_pairs) {
  const int tid = threadIdx.x, w = tid >> 6;
  const int P = T * topk;
  if (P > kRankSortMaxPairs) {   // uniform
    if (w < T) topk_token<NS>(logits, w, E, topk, tid & 63, ids, gates);
    __syncthreads();
    sort_pairs(ids, P, E, counts, offsets, sorted_pairs);
    return;
  }
  // Up to 32 pairs the routing stays in LDS: top-k per wave, then each
  // pair's rank in the stable order by (expert, pair id) and each expert's
  // count and offset by direct counting (no histogram passes; measured on
  // MI355X, E 128 top-8: 1.0-1.3 us less per step at T = 1, 2, 1 us more at
  // T = 8, where the counting loops grow with the pairs).
  __shared__ int32_t s_ids[kRankSortMaxPairs];
  __shared__ float s_gates[kRankSortMaxPairs];
  if (w < T) topk_token<NS>(logits, w, E, topk, tid & 63, s_ids, s_gates);
  __syncthreads();
  if (tid < P) {
    const int ep = s_ids[tid];
    int rank = 0;
    for (int q = 0; q < P; ++q) rank += (s_ids[q] < ep || (s_ids[q] == ep && q < tid)) ? 1 : 0;
    ids[tid] = ep;
    gates[tid] = s_gates[tid];
    sorted_pairs[rank] = tid;
  }
  for (int x = tid; x <= E; x += 1024) {
    int below = 0, same = 0;
    for (int q = 0; q < P; ++q) {
      below += s_ids[q] < x ? 1 : 0;
      same += s_ids[q] == x ? 1 : 0;
    }
    offsets[x] = below;
    if (x < E) counts[x] = same;
  }
}

hipError_t launch_moe_route(const float* logits, int T, int E, int topk, int32_t* ids, float* gates,
                            int32_t* counts, int32_t* offsets, int32_t* sorted_pairs, hipStream_t stream) {
  if (T <= kSortWaves) {
    const dim3 g1(1), b1(1024);
    if (E <= 64) moe_route_small_kernel<1><<<g1, b1, 0, stream>>>(logits, T, E, topk, ids, gates, counts, offsets,
                                                                  sorted_pairs);
    else if (E <= 128) moe_route_small_kernel<2><<<g1, b1, 0, stream>>>(logits, T, E, topk, ids, gates, counts,
                                                                        offsets, sorted_pairs);
    else if (E <= 256) moe_route_small_kernel<4><<<g1, b1, 0, stream>>>(logits, T, E, topk, ids, gates, counts,
                                                                        offsets, sorted_pairs);
    else if (E <= 512) moe_route_small_kernel<8><<<g1, b1, 0, stream>>>(logits, T, E, topk, ids, gates, counts,
                                                                        offsets, sorted_pairs);
    else moe_route_small_kernel<16><<<g1, b1, 0, stream>>>(logits, T, E, topk, ids, gates, counts, offsets,
                                                           sorted_pairs);
    return hipGetLastError();
  }
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
// Expert GEMMs, streaming form (few rows per expert)
//
// At a few dozen rows per expert the expert GEMMs are weight streams, and a
// barrier per 128-wide chunk leaves them latency-bound.  Here a workgroup
// takes one expert and a range of its output tiles:
//   * the expert's rows (64 at a time) are copied once into LDS through the
//     buffer loads' LDS path -- all of K when it fits in 128 KB, else in
//     phases of 1024 columns -- in the same XOR-swizzled chunk layout as the
//     tile engine;
//   * each wave then streams its own weight tiles (NT at a time, both gate
//     and up for the gate+up pass) through a P-stage register ring that runs
//     across tile groups, K phases and row tiles, with no barrier except
//     around the LDS reloads;
//   * at the end of each tile group the epilogue stores h = silu(g) * u
//     (gate+up) or y at its pair row (down).
// Every step issues the same weight loads (past the last step with an
// out-of-range offset, which reads zero and moves no memory), so the
// compiler's wait counts stay exact.
// ---------------------------------------------------------------------------
enum { kGateUp = 0, kDown = 1 };
constexpr int kStreamBM = 64;   // rows per row tile (48 measured the same on MI355X at the MoE shape)

// Routing outputs the gate+up kernel forms itself (ROUTE): from the pairs'
// experts (ids, pair order) each expert's workgroups find its rows; the
// expert's first workgroup stores its count, offset and slice of the sorted
// pairs, the same values the sort kernel gives.
struct MoeRouteArgs {
  const int32_t* ids;   // [Ptot]
  int32_t* counts;      // [E]
  int32_t* offsets;     // [E + 1]
  int32_t* sorted;      // [Ptot]
  int32_t E;
};

// WAVES waves per workgroup; KP columns per LDS phase (64 rows x KP fp16).
template <int FMT, int MODE, int NT, int P, int WAVES, int KP, bool ROUTE = false>
__global__ __launch_bounds__(WAVES * 64) void moe_stream_kernel(
    const uint8_t* __restrict__ W0, const uint8_t* __restrict__ W1, int64_t wstride, int N, int K,
    const uint16_t* __restrict__ src, int src_rows, int T, int topk, int Ptot,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ sorted_pairs, const int32_t* __restrict__ xexp,
    uint16_t* __restrict__ out16, uint16_t* __restrict__ h_out, int tiles_per_wave, int groups, MoeRouteArgs ra) {
  static_assert(!ROUTE || MODE == kGateUp, "the routed form is the gate+up pass");
  constexpr int NW = MODE == kGateUp ? 2 : 1;
  constexpr int MT = kStreamBM / 16, BM = kStreamBM;
  constexpr int REC = Fmt<FMT>::kRecBytes;
  constexpr int CODE = Fmt<FMT>::kCodeBytes;
  constexpr int NV = FMT == kQ4_0 ? 1 : 2;
  constexpr int THREADS = WAVES * 64;
  __shared__ __attribute__((aligned(1024))) uint16_t xs[BM * KP];
  __shared__ int s_rowbase[BM];   // source row of each of the row tile's BM rows (-1: none)
  // Per row of the row tile, what its epilogue needs: the token's exponent
  // (gate+up) or the pair id (down).  Staged with the rows, so the epilogue
  // issues no global load (whose wait would also drain the weight ring).
  __shared__ int s_rowaux[BM];

  const int e = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // ROUTE: block-wide exclusive scan of two per-thread counts (pairs of this
  // expert, pairs of lower experts) over one round of THREADS x 8 pairs.
  __shared__ int s_wsum[2][WAVES];
  auto scan2 = [&](int v0, int v1, int& ex0, int& tot0, int& tot1) __attribute__((always_inline)) {
    int i0 = v0, i1 = v1;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o0 = __shfl_up(i0, off), o1 = __shfl_up(i1, off);
      if (lane >= off) {
        i0 += o0;
        i1 += o1;
      }
    }
    if (lane == 63) {
      s_wsum[0][wave] = i0;
      s_wsum[1][wave] = i1;
    }
    __syncthreads();
    int before = 0;
    tot0 = 0;
    tot1 = 0;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) {
      before += w < wave ? s_wsum[0][w] : 0;
      tot0 += s_wsum[0][w];
      tot1 += s_wsum[1][w];
    }
    ex0 = before + i0 - v0;
    __syncthreads();   // s_wsum is reused by the next round
  };
  // Thread tid's 8 pair experts of the round starting at r0 (-1 past Ptot):
  // two 16-byte buffer loads (4-byte alignment suffices for buffer loads).
  const __amdgpu_buffer_rsrc_t ids_res = uniform_rsrc(ra.ids, ROUTE ? Ptot * 4 : 0);
  auto load_ids8 = [&](int r0, int (&id)[8]) __attribute__((always_inline)) {
    const u32x4_t a0 = __builtin_amdgcn_raw_buffer_load_b128(ids_res, (uint32_t)(r0 + tid * 8) * 4, 0, 0);
    const u32x4_t a1 = __builtin_amdgcn_raw_buffer_load_b128(ids_res, (uint32_t)(r0 + tid * 8 + 4) * 4, 0, 0);
    const uint32_t v[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
#pragma unroll
    for (int q = 0; q < 8; ++q) id[q] = r0 + tid * 8 + q < Ptot ? (int)v[q] : -1;
  };

  int seg, cnt;
  bool rows0_done = false;   // ROUTE, one round: row tile 0 and the sorted pairs are stored already
  if constexpr (ROUTE) {
    seg = 0;
    cnt = 0;
    if (Ptot <= THREADS * 8) {
      // One round: the scan gives the ranks, seg and cnt together.
      int id[8];
      load_ids8(0, id);
      int cs = 0, cb = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        cs += id[q] == e ? 1 : 0;
        cb += (id[q] >= 0 && id[q] < e) ? 1 : 0;
      }
      if (tid < BM) s_rowbase[tid] = -1;
      int ex;
      scan2(cs, cb, ex, cnt, seg);   // (its barriers order the s_rowbase reset before the fills)
      int rank = ex;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (id[q] == e) {
          const int pr = tid * 8 + q;
          if (rank < BM) s_rowbase[rank] = min(pr / topk, T - 1);
          ra.sorted[seg + rank] = pr;
          ++rank;
        }
      }
      rows0_done = true;
    }
    // Otherwise pass 1: seg = pairs routed to lower experts, cnt = pairs
    // routed to e (pass 2, the ranks, follows in the prologue).
    for (int r0 = 0; !rows0_done && r0 < Ptot; r0 += THREADS * 8) {
      int id[8];
      load_ids8(r0, id);
      int cs = 0, cb = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        cs += id[q] == e ? 1 : 0;
        cb += (id[q] >= 0 && id[q] < e) ? 1 : 0;
      }
      int ex, ts, tb;
      scan2(cs, cb, ex, ts, tb);
      cnt += ts;
      seg += tb;
    }
    if (blockIdx.x == 0 && tid == 0) {
      ra.counts[e] = cnt;
      ra.offsets[e] = seg;
      if (e == ra.E - 1) ra.offsets[ra.E] = Ptot;
    }
  } else {
    // Clamped to the Ptot pairs, so malformed offsets cannot send the row
    // stores past h / y (the decode path clamps the same way).
    seg = min(max(offsets[e], 0), Ptot);
    cnt = min(offsets[e + 1], Ptot) - seg;
  }
  if (cnt <= 0) return;   // uniform over the workgroup
  const int r = lane & 15, g = lane >> 4;
  const int nchunks = K / kChunkK;
  const int tiles = N / kTileRows;
  const int kpc = K < KP ? K : KP;                    // columns per LDS phase
  const int cpp = kpc / kChunkK;                      // chunks per phase
  const int n_rt = (cnt + BM - 1) / BM;
  const int total = n_rt * groups * nchunks;

  // This wave's tiles: t_w0 .. t_w0 + tv - 1 of the expert's matrix.
  const int t_w0 = (blockIdx.x * WAVES + wave) * tiles_per_wave;
  const int tv = min(max(tiles - t_w0, 0), tiles_per_wave);
  const int64_t woff = e * wstride + (int64_t)(tv > 0 ? t_w0 : 0) * nchunks * REC;
  __amdgpu_buffer_rsrc_t wres[NW];
  wres[0] = uniform_rsrc(W0 + woff, tv * nchunks * REC);
  if constexpr (NW == 2) wres[1] = uniform_rsrc(W1 + woff, tv * nchunks * REC);

  struct WStage {
    u32x4_t codes[NW][NT][NV];
    u32x2_t sc[NW][NT];
  };
  // Load cursor: (group lg, chunk lc); it advances one chunk per step and
  // wraps over groups (and, implicitly, row tiles: the weights do not depend
  // on the row tile).
  // Steps past the last one (the ring's final P) issue the same loads with
  // an out-of-range offset: they read zero and move no memory, and the
  // compiler's wait counts stay exact.
  int lg = 0, lc = 0, ln = 0;
  auto load_next = [&](WStage& s) __attribute__((always_inline)) {
    const bool live = ln++ < total;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int lt = lg * NT + t;
      const int so = (lt * nchunks + lc) * REC;
      const bool ok = live && lt < tv;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
#pragma unroll
        for (int v = 0; v < NV; ++v)
          s.codes[w][t][v] =
              __builtin_amdgcn_raw_buffer_load_b128(wres[w], ok ? (uint32_t)(v * 1024 + lane * 16) : kOOB, so, 0);
        s.sc[w][t] = __builtin_amdgcn_raw_buffer_load_b64(wres[w], ok ? (uint32_t)(CODE + r * 8) : kOOB, so, 0);
      }
    }
    if (++lc == nchunks) {
      lc = 0;
      if (++lg == groups) lg = 0;
    }
  };

  // Activation rows of row tile rt, LDS phase kph -> xs.  Copy p of this
  // thread fills slot THREADS p + tid of the phase: chunk slot / (BM 16),
  // then row / column group as in the tile engine.
  const __amdgpu_buffer_rsrc_t xres = uniform_rsrc(src, (int)((int64_t)src_rows * K * 2));
  // Source rows of row tile rt into s_rowbase; the caller orders it with a
  // barrier before load_x reads it.
  // (ROUTE: the rows of every row tile but the first are read back from the
  // sorted pairs this workgroup stored in its prologue.)
  const int32_t* sp_rows = ROUTE ? ra.sorted : sorted_pairs;
  auto set_rows = [&](int rt) __attribute__((always_inline)) {
    if (tid < BM) {
      const int i = rt * BM + tid;
      int base = -1, aux = 0;
      if (i < cnt) {
        if constexpr (MODE == kGateUp) {
          base = min(max(sp_rows[seg + i], 0) / topk, T - 1);
          aux = xexp[base];
        } else {
          base = seg + i;
          aux = min(max(sorted_pairs[seg + i], 0), Ptot - 1);
        }
      }
      s_rowbase[tid] = base;
      s_rowaux[tid] = aux;
    }
  };
  // ROUTE prologue, pass 2: each of the expert's pairs gets its rank in pair
  // order (the stable sort); ranks below BM give row tile 0's rows.  Every
  // workgroup of the expert stores the same sorted pairs (equal values), so
  // each can read its later row tiles back.
  auto route_rows0 = [&]() __attribute__((always_inline)) {
    if (tid < BM) s_rowbase[tid] = -1;
    __syncthreads();
    int run = 0;
    for (int r0 = 0; r0 < Ptot; r0 += THREADS * 8) {
      int id[8];
      load_ids8(r0, id);
      int cs = 0;
#pragma unroll
      for (int q = 0; q < 8; ++q) cs += id[q] == e ? 1 : 0;
      int ex, ts, tb;
      scan2(cs, 0, ex, ts, tb);
      int rank = run + ex;
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (id[q] == e) {
          const int pr = r0 + tid * 8 + q;
          if (rank < BM) s_rowbase[rank] = min(pr / topk, T - 1);
          ra.sorted[seg + rank] = pr;
          ++rank;
        }
      }
      run += ts;
    }
  };
  auto load_x = [&](int kph) __attribute__((always_inline)) {
    const int col0 = kph * kpc;
    const int ncols = min(kpc, K - col0);
    const int nslots = BM * ncols / 8;
    // nslots is a multiple of 1024 (ncols of 128), so a wave's 64 slots are
    // all in or all past the phase: the copy is skipped per wave, and no LDS
    // write lands past xs whatever THREADS is.
    for (int p = 0; p * THREADS < nslots; ++p) {
      const int slot = p * THREADS + tid;
      if (p * THREADS + wave * 64 >= nslots) break;   // wave-uniform
      const int cc = slot / (BM * 16), q = slot % (BM * 16);
      const int row = q >> 4, cg = (q & 15) ^ (row & 15);
      const int base = s_rowbase[row];
      const uint32_t v = base >= 0 ? (uint32_t)(((int64_t)base * K + col0 + cc * kChunkK + cg * 8) * 2) : kOOB;
      uint16_t* dst = xs + (p * THREADS + wave * 64) * 8;   // wave-uniform
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xres, (__attribute__((address_space(3))) void*)dst, 16, v, 0, 0, 0);
    }
  };

  float4_t acc[NW * NT * MT];
#pragma unroll
  for (int i = 0; i < NW * NT * MT; ++i) acc[i] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // Products of chunk lcl of the loaded phase with one weight stage.
  auto compute = [&](const WStage& s, int lcl, int mtn) __attribute__((always_inline)) {
    const uint16_t* xb = xs + lcl * BM * kChunkK;
#pragma unroll
    for (int j = 0; j < kBlocksPerChunk; ++j) {
      half8_t b[NW][NT];
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          u32x4_t q;
          if constexpr (FMT == kQ4_0) {
            const uint32_t wd = s.codes[w][t][0][j];
            q = deq_q4_f16(wd);
          } else {
            const uint32_t d0 = s.codes[w][t][j >> 1][2 * (j & 1)], d1 = s.codes[w][t][j >> 1][2 * (j & 1) + 1];
            q = deq_q8<kF16>(d0, d1);
          }
          const uint32_t sbits = (j & 1) ? (s.sc[w][t][j >> 1] >> 16) : (s.sc[w][t][j >> 1] & 0xFFFFu);
          const _Float16 sh = __builtin_bit_cast(_Float16, (uint16_t)sbits);
          const half2_t s2 = {sh, sh};
          b[w][t] = __builtin_bit_cast(half8_t, scale_f16x8(q, s2));
        }
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        if (i >= mtn) break;   // uniform: 16-row tiles past the expert's rows
        const int row = i * 16 + r;
        const half8_t a = *(const half8_t*)(xb + (row * 16 + ((4 * j + g) ^ r)) * 8);
#pragma unroll
        for (int w = 0; w < NW; ++w)
#pragma unroll
          for (int t = 0; t < NT; ++t)
            acc[(w * NT + t) * MT + i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(b[w][t], a, acc[(w * NT + t) * MT + i], 0, 0, 0);
      }
    }
  };

  // The weights are the MFMA's A operand and the activation rows its B
  // operand, so the product comes out transposed: lane (r, g), register k of
  // tile (w, t, i) holds row 16 i + r, column 16 (t_w0 + gi NT + t) + 4 g + k.
  // Each lane thus stores its four adjacent columns as one 8-byte write.
  auto epilogue = [&](int rt, int gi) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int lt = gi * NT + t;
      const int n0 = (t_w0 + lt) * kTileRows + 4 * g;
      if (lt < tv) {
#pragma unroll
        for (int i = 0; i < MT; ++i) {
          const int row = rt * BM + i * 16 + r;
          if (row < cnt) {
            if constexpr (MODE == kGateUp) {
              // The token's row was scaled by 2^-ex: z = 2^ex acc exactly.  h
              // is formed at its true scale and rounded to bf16 (its storage
              // precision); the down product's fp16 copy carries 2^-2ex
              // (|h| <= |z_gate| |z_up|), undone by the combine.
              const int ex = s_rowaux[i * 16 + r];   // the row's token's exponent (row < cnt)
              const float4_t zg = acc[(0 * NT + t) * MT + i], zu = acc[(1 * NT + t) * MT + i];
              uint32_t hf[2], hb[2];
#pragma unroll
              for (int k2 = 0; k2 < 2; ++k2) {
                const __bf16 b0 = (__bf16)(silu_f32(__builtin_ldexpf(zg[2 * k2], ex)) *
                                           __builtin_ldexpf(zu[2 * k2], ex));
                const __bf16 b1 = (__bf16)(silu_f32(__builtin_ldexpf(zg[2 * k2 + 1], ex)) *
                                           __builtin_ldexpf(zu[2 * k2 + 1], ex));
                hf[k2] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)__builtin_ldexpf((float)b0, -2 * ex)) |
                         ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)__builtin_ldexpf((float)b1, -2 * ex))
                          << 16);
                hb[k2] = (uint32_t)__builtin_bit_cast(uint16_t, b0) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
              }
              const int64_t idx = (int64_t)(seg + row) * N + n0;
              *(u32x2_t*)(out16 + idx) = u32x2_t{hf[0], hf[1]};
              if (h_out) *(u32x2_t*)(h_out + idx) = u32x2_t{hb[0], hb[1]};
            } else {
              const int64_t pair = s_rowaux[i * 16 + r];
              const float4_t v = acc[t * MT + i];
              const uint32_t lo = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[0]) |
                                  ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[1]) << 16);
              const uint32_t hi = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[2]) |
                                  ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v[3]) << 16);
              *(u32x2_t*)(out16 + pair * N + n0) = u32x2_t{lo, hi};
            }
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < NW * NT * MT; ++i) acc[i] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  };

  // Prologue: the first phase of X, then P steps of weights in flight; the
  // barrier waits for the X copies only (they were issued first: the ring's
  // loads may still be in flight).
  WStage ws[P];
  if constexpr (ROUTE) {
    if (!rows0_done) route_rows0();
  } else {
    set_rows(0);
  }
  __syncthreads();
  if constexpr (ROUTE) {   // row tile 0's exponents (its rows were ranked above)
    if (tid < BM) s_rowaux[tid] = s_rowbase[tid] >= 0 ? xexp[s_rowbase[tid]] : 0;
  }
  load_x(0);
  static_for<0, P>([&](auto jc) __attribute__((always_inline)) { load_next(ws[decltype(jc)::value]); });
  constexpr int kRingLoads = P * NT * NW * (NV + 1);   // vector loads per load_next, P of them
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(kRingLoads) : "memory");
  __builtin_amdgcn_sched_barrier(0);
  int cur_rt = 0, cur_kph = 0;

  // Compute cursor: row tile rt, group gi, chunk c.
  int rt = 0, gi = 0, c = 0;
  for (int s0 = 0; s0 < total; s0 += P) {
    static_for<0, P>([&](auto jc) __attribute__((always_inline)) {
      constexpr int J = decltype(jc)::value;
      if (s0 + J < total) {
        const int kph = c / cpp;
        if (kph != cur_kph || rt != cur_rt) {   // uniform: reload the LDS phase
          // Every wave is done reading the phase (and its rows): LDS reads
          // only, the weight ring stays in flight.
          __builtin_amdgcn_sched_barrier(0);
          asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
          __builtin_amdgcn_sched_barrier(0);
          if (rt != cur_rt) {
            set_rows(rt);
            __syncthreads();
          }
          load_x(kph);
          __syncthreads();
          cur_rt = rt;
          cur_kph = kph;
        }
        compute(ws[J], c - kph * cpp, __builtin_amdgcn_readfirstlane(min(MT, (cnt - rt * BM + 15) / 16)));
        if (c == nchunks - 1) epilogue(rt, gi);
        if (++c == nchunks) {
          c = 0;
          if (++gi == groups) {
            gi = 0;
            ++rt;
          }
        }
      }
      load_next(ws[J]);
    });
  }
}

// out[t, n] = 2^(2 xexp[t]) sum_j gates[t, j] y16[t k + j, n] (y16 carries
// the token's 2^-2xexp scale); 8 columns per thread.
__global__ __launch_bounds__(256) void moe_combine_kernel(const uint16_t* __restrict__ y16,
                                                          const float* __restrict__ gates,
                                                          const int32_t* __restrict__ xexp, int T, int topk, int H,
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
  const int ex2 = 2 * xexp[t];
#pragma unroll
  for (int q = 0; q < 8; ++q) s[q] = __builtin_ldexpf(s[q], ex2);
  float4_t* o = (float4_t*)(out + (int64_t)t * H + c8 * 8);
  o[0] = float4_t{s[0], s[1], s[2], s[3]};
  o[1] = float4_t{s[4], s[5], s[6], s[7]};
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------

namespace {

// Streaming-kernel configuration (measured on MI355X).
// Streaming-kernel configuration (measured on MI355X, T 512, E 128, top-8,
// H 2048, F 768): 12 gate+up waves (3 a SIMD) with 2 Q4_0 tile pairs (1
// for Q8_0, whose codes take twice the registers) and 16 down waves (4 a
// SIMD) with 2 tiles, within the register budgets of those occupancies;
// 8 waves with 3 / 4 tiles (2 a SIMD) measured 63.6 / 39.0 us (Q4_0) and
// 108 / 56 us (Q8_0) against 61.4 / 37.0 and 98 / 55.
#ifndef Q4Q8_MOE_WAVES_G
#define Q4Q8_MOE_WAVES_G 12
#endif
#ifndef Q4Q8_MOE_WAVES_D
#define Q4Q8_MOE_WAVES_D 16
#endif
#ifndef Q4Q8_MOE_NTG4
#define Q4Q8_MOE_NTG4 2
#endif
#ifndef Q4Q8_MOE_NTG8
#define Q4Q8_MOE_NTG8 1
#endif
#ifndef Q4Q8_MOE_PG4
#define Q4Q8_MOE_PG4 2
#endif
#ifndef Q4Q8_MOE_PG8
#define Q4Q8_MOE_PG8 3
#endif
#ifndef Q4Q8_MOE_NTD
#define Q4Q8_MOE_NTD 2
#endif
#ifndef Q4Q8_MOE_PD4
#define Q4Q8_MOE_PD4 4
#endif
#ifndef Q4Q8_MOE_PD8
#define Q4Q8_MOE_PD8 3
#endif
constexpr int kMoeWavesG = Q4Q8_MOE_WAVES_G;   // waves per workgroup, gate+up
constexpr int kMoeWavesD = Q4Q8_MOE_WAVES_D;   // waves per workgroup, down
constexpr int kMoeKP = 1024;     // LDS phase columns (64 rows x kMoeKP fp16)
constexpr int kMoeSlots = 1;     // workgroups per CU the split aims at

size_t round256(size_t b) { return (b + 255) / 256 * 256; }

struct MoeWs {
  uint16_t* x16;
  uint16_t* h16;
  uint16_t* y16;
  int32_t* xexp;   // per token: its row was scaled by 2^-xexp
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
  b += round256(P * H * 2);
  w.xexp = (int32_t*)b;
  return w;
}

// ra: null, or the routed form (the gate+up kernel derives offsets and the
// sorted pairs from ra->ids and stores them in ra's arrays, which the down
// kernel then reads).
template <int FMT>
void launch_experts(const void* Wg, const void* Wu, const void* Wd, int E, int H, int F, const uint16_t* x16, int T,
                    int topk, const float* gates, const int32_t* offsets, const int32_t* sorted_pairs, float* out,
                    void* h_out, const MoeWs& w, hipStream_t s, const MoeRouteArgs* ra = nullptr) {
  const int P = T * topk;
  const int64_t sg = (int64_t)(F / kTileRows) * (H / kChunkK) * Fmt<FMT>::kRecBytes;   // repacked [F, H]
  const int64_t sd = (int64_t)(H / kTileRows) * (F / kChunkK) * Fmt<FMT>::kRecBytes;   // repacked [H, F]
  // Workgroups per expert: about kMoeSlots per CU over all experts.
  auto split = [&](int tiles, int nt, int waves, int& nwe, int& tpw, int& groups) {
    nwe = std::max(1, std::min(tiles, 256 * kMoeSlots / std::max(E, 1)));
    const int per_wg = (tiles + nwe - 1) / nwe;
    tpw = (per_wg + waves - 1) / waves;
    nwe = (tiles + waves * tpw - 1) / (waves * tpw);
    groups = (tpw + nt - 1) / nt;
  };
  // gate+up: tile pairs per group (Q8_0 codes are twice as large), stages.
  constexpr int NTG = FMT == kQ4_0 ? Q4Q8_MOE_NTG4 : Q4Q8_MOE_NTG8;
  constexpr int PG = FMT == kQ4_0 ? Q4Q8_MOE_PG4 : Q4Q8_MOE_PG8;
  constexpr int NTD = Q4Q8_MOE_NTD;                                    // down: tiles per group
  constexpr int PD = FMT == kQ4_0 ? Q4Q8_MOE_PD4 : Q4Q8_MOE_PD8;      // down: stages
  int nwe, tpw, groups;
  split(F / kTileRows, NTG, kMoeWavesG, nwe, tpw, groups);
  const dim3 ggrid((unsigned)nwe, (unsigned)E), gblock(kMoeWavesG * 64);
  if (ra) {
    moe_stream_kernel<FMT, kGateUp, NTG, PG, kMoeWavesG, kMoeKP, true><<<ggrid, gblock, 0, s>>>(
        (const uint8_t*)Wg, (const uint8_t*)Wu, sg, F, H, x16, T, T, topk, P, nullptr, nullptr, w.xexp, w.h16,
        (uint16_t*)h_out, tpw, groups, *ra);
    offsets = ra->offsets;
    sorted_pairs = ra->sorted;
  } else {
    moe_stream_kernel<FMT, kGateUp, NTG, PG, kMoeWavesG, kMoeKP><<<ggrid, gblock, 0, s>>>(
        (const uint8_t*)Wg, (const uint8_t*)Wu, sg, F, H, x16, T, T, topk, P, offsets, sorted_pairs, w.xexp, w.h16,
        (uint16_t*)h_out, tpw, groups, MoeRouteArgs{});
  }
  split(H / kTileRows, NTD, kMoeWavesD, nwe, tpw, groups);
  moe_stream_kernel<FMT, kDown, NTD, PD, kMoeWavesD, kMoeKP><<<dim3((unsigned)nwe, (unsigned)E),
                                                               dim3(kMoeWavesD * 64), 0, s>>>(
      (const uint8_t*)Wd, nullptr, sd, H, F, w.h16, P, T, topk, P, offsets, sorted_pairs, w.xexp, w.y16, nullptr,
      tpw, groups, MoeRouteArgs{});
  moe_combine_kernel<<<dim3((unsigned)((H / 8 + 255) / 256), (unsigned)T), dim3(256), 0, s>>>(w.y16, gates, w.xexp,
                                                                                              T, topk, H, out);
}
}  // namespace

size_t moe_workspace_bytes(int fmt, int T, int E, int topk, int H, int F) {
  (void)fmt;
  (void)E;
  const size_t P = (size_t)T * topk;
  return round256((size_t)T * H * 2) + round256(P * F * 2) + round256(P * H * 2) + round256((size_t)T * 4);
}

constexpr int kMoeRoutedMaxTokens = 4;

hipError_t launch_moe_decode_call(int fmt, int xdt, const void* Wg, const void* Wu, const void* Wd, int E, int H,
                                  int F, const void* X, int T, int topk, const MoeRouteOut& ro, float* out,
                                  void* h_out, void* ws, hipStream_t stream) {
  const MoeWs w = moe_ws_layout(ws, T, topk, H, F);
  uint16_t* h = h_out ? (uint16_t*)h_out : w.h16;
  if (T > kMoeRoutedMaxTokens) {
    // Past 4 tokens the in-kernel routing (one wave per token, in every
    // workgroup) costs more than the routing kernel's launch: route first
    // (measured on MI355X, E 128 top-8 H 2048 F 768, T = 8: 43.1 us per step
    // routed in-kernel against 42.0).  Same kernels as q4q8_moe_route +
    // q4q8_moe_qgemm, so the same results.
    const hipError_t e = launch_moe_route(ro.logits, T, E, topk, ro.ids, ro.gates, ro.counts, ro.offsets,
                                          ro.sorted_pairs, stream);
    if (e != hipSuccess) return e;
    if (!launch_moe_decode(fmt, xdt, Wg, Wu, Wd, E, H, F, X, T, topk, ro.gates, ro.offsets, ro.sorted_pairs, h,
                           w.y16, w.xexp, out, stream))
      moe_combine_kernel<<<dim3((unsigned)((H / 8 + 255) / 256), (unsigned)T), dim3(256), 0, stream>>>(
          w.y16, ro.gates, w.xexp, T, topk, H, out);
    return hipGetLastError();
  }
  if (!launch_moe_decode_routed(fmt, xdt, Wg, Wu, Wd, E, H, F, X, T, topk, ro, h, w.y16, w.xexp, out, stream))
    moe_combine_kernel<<<dim3((unsigned)((H / 8 + 255) / 256), (unsigned)T), dim3(256), 0, stream>>>(
        w.y16, ro.gates, w.xexp, T, topk, H, out);
  return hipGetLastError();
}

template <int NS>
static void launch_prep(int xdt, const float* logits, int T, int E, int topk, int32_t* ids, float* gates,
                        const void* X, int H, uint16_t* x16, int32_t* xexp, hipStream_t s) {
  const dim3 grid((unsigned)((T + 3) / 4)), block(512);
  if (xdt == kBF16)
    moe_prep_kernel<NS, kBF16><<<grid, block, 0, s>>>(logits, T, E, topk, ids, gates, (const uint16_t*)X, H, x16,
                                                      xexp);
  else
    moe_prep_kernel<NS, kF16><<<grid, block, 0, s>>>(logits, T, E, topk, ids, gates, (const uint16_t*)X, H, x16,
                                                     xexp);
}

hipError_t launch_moe_forward(int fmt, int xdt, const void* Wg, const void* Wu, const void* Wd, int E, int H, int F,
                              const void* X, int T, int topk, const MoeRouteOut& ro, float* out, void* h_out,
                              void* ws, hipStream_t stream) {
  if (moe_decode_fits(T, H, F))
    return launch_moe_decode_call(fmt, xdt, Wg, Wu, Wd, E, H, F, X, T, topk, ro, out, h_out, ws, stream);
  // Three launches before the combine: top-k and the row scaling of every
  // token; gate+up, whose workgroups find their expert's rows from the ids
  // (the stable sort, without a sort launch) and store counts, offsets and
  // the sorted pairs; down.
  const MoeWs w = moe_ws_layout(ws, T, topk, H, F);
  if (E <= 64) launch_prep<1>(xdt, ro.logits, T, E, topk, ro.ids, ro.gates, X, H, w.x16, w.xexp, stream);
  else if (E <= 128) launch_prep<2>(xdt, ro.logits, T, E, topk, ro.ids, ro.gates, X, H, w.x16, w.xexp, stream);
  else if (E <= 256) launch_prep<4>(xdt, ro.logits, T, E, topk, ro.ids, ro.gates, X, H, w.x16, w.xexp, stream);
  else if (E <= 512) launch_prep<8>(xdt, ro.logits, T, E, topk, ro.ids, ro.gates, X, H, w.x16, w.xexp, stream);
  else launch_prep<16>(xdt, ro.logits, T, E, topk, ro.ids, ro.gates, X, H, w.x16, w.xexp, stream);
  const MoeRouteArgs ra = {ro.ids, ro.counts, ro.offsets, ro.sorted_pairs, E};
  if (fmt == kQ4_0)
    launch_experts<kQ4_0>(Wg, Wu, Wd, E, H, F, w.x16, T, topk, ro.gates, nullptr, nullptr, out, h_out, w, stream,
                          &ra);
  else
    launch_experts<kQ8_0>(Wg, Wu, Wd, E, H, F, w.x16, T, topk, ro.gates, nullptr, nullptr, out, h_out, w, stream,
                          &ra);
  return hipGetLastError();
}

hipError_t launch_moe_qgemm(int fmt, int xdt, const void* Wg, const void* Wu, const void* Wd, int E, int H, int F,
                            const void* X, int T, int topk, const float* gates, const int32_t* offsets,
                            const int32_t* sorted_pairs, float* out, void* h_out, void* ws, hipStream_t stream) {
  const MoeWs w = moe_ws_layout(ws, T, topk, H, F);
  if (moe_decode_fits(T, H, F)) {
    // A few tokens: every expert product is a GEMV over the expert's weights.
    uint16_t* h = h_out ? (uint16_t*)h_out : w.h16;
    if (!launch_moe_decode(fmt, xdt, Wg, Wu, Wd, E, H, F, X, T, topk, gates, offsets, sorted_pairs, h, w.y16,
                           w.xexp, out, stream))
      moe_combine_kernel<<<dim3((unsigned)((H / 8 + 255) / 256), (unsigned)T), dim3(256), 0, stream>>>(
          w.y16, gates, w.xexp, T, topk, H, out);
    return hipGetLastError();
  }
  // Both dtypes: each token row scaled by a power of two (its exponent in
  // w.xexp), which also keeps h and y in the fp16 range.
  const hipError_t e = launch_rowscale_f16(xdt, X, H, w.x16, H, T, H, H, w.xexp, stream, LaunchEvents());
  if (e != hipSuccess) return e;
  const uint16_t* x16 = w.x16;
  if (fmt == kQ4_0)
    launch_experts<kQ4_0>(Wg, Wu, Wd, E, H, F, x16, T, topk, gates, offsets, sorted_pairs, out, h_out, w, stream);
  else
    launch_experts<kQ8_0>(Wg, Wu, Wd, E, H, F, x16, T, topk, gates, offsets, sorted_pairs, out, h_out, w, stream);
  return hipGetLastError();
}

}  // namespace q4q8
