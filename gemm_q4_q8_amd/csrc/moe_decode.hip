// Mixture-of-experts decode: T <= 8 tokens, each routed to its top-k experts.
//
// "BaseRT: Advancing Best-in-Class LLM Inference with Apple M5 Neural
// Accelerators" (review, "Method") keeps memory-bound decode on the GEMV
// kernels and sends only compute-bound work (prefill GEMM, MoE expert GEMM)
// to the matrix-unit tile path.  With a handful of tokens an expert sees at
// most T rows, so its products are GEMVs over its weights: this path runs
// them on the GEMV machinery (gemv_core.h) instead of 64-row MFMA tiles.
//
// Work split.  Pairs (token t, slot j) arrive sorted by expert (offsets,
// sorted_pairs from the routing step).  Workgroup (position p, group g) loads
// offsets into LDS and finds the expert e that owns sorted position p (binary
// search there: one memory round trip instead of a chain of them); only
// the expert's first position works, with the expert's M = offsets[e+1] -
// offsets[e] <= T rows as the GEMV's activation rows, so each selected
// expert's weights stream exactly once per call.  The other positions' groups
// exit at once.
//   * gate/up: a SwiGLU pair per 16-row tile (half of the tile's waves on
//     the gate rows, half on the up rows, K split in ksh shares each), x rows
//     gathered from the tokens into LDS; h = silu(gate) * up rounded to bf16,
//     stored in sorted-pair order;
//   * down: x = the expert's h rows (contiguous in sorted order), y rounded
//     to fp16 per pair id, then the weighted combine kernel of the prefill
//     path.
// The rows are staged in LDS as fp16, each token row scaled by a power of
// two as the prefill path's pre-pass does (its largest magnitude in [4, 8);
// h rows by the square of the token's factor, undone after the combine):
// the fp16 operands take the Q4_0 unpack's two-instruction fp16 form, where a bf16 operand would need a per-value integer conversion
// (measured at T = 8: gate/up 36.5 -> 19 us, down 20 -> 12 us).
// K-shares are reduced in a fixed order through LDS: results are bitwise
// reproducible.
// Routed form (q4q8_moe_decode): the gate/up kernel derives the routing
// itself from the logits (every workgroup: one wave per token's top-k, then
// the pairs' stable order in LDS), so no routing kernel runs before it;
// workgroup 0 stores the routing arrays the later kernels read.
#include "gemv_core.h"
#include "moe_route.h"
#include "q4q8_internal.h"

#include <algorithm>

namespace q4q8 {

enum { kDecGateUp = 0, kDecDown = 1 };

struct MoeDecArgs {
  const uint8_t* W;          // gate (gate/up pass) or down weights of expert 0
  const uint8_t* W2;         // up weights of expert 0 (gate/up pass)
  int64_t mat_bytes;         // repacked bytes of one expert's matrix
  const uint16_t* X;         // gate/up: tokens [T, ldx]; down: h [positions, ldx], sorted
  int64_t ldx;
  uint16_t* out;             // gate/up: h bf16 [positions, N], sorted; down: y fp16 [pair id, N]
  const int32_t* offsets;    // [E + 1]
  const int32_t* sorted_pairs;
  int32_t N, K;              // output rows per expert, reduction length (multiples of 128)
  int32_t topk, E, npos;     // npos = T * topk sorted positions
  int32_t T;
  int32_t groups;            // workgroups per sorted position
  int32_t ksh;               // K-shares per matrix, a power of 2
  // Per token: gate/up stores, down reads the power of two its row was
  // scaled by (2^-xexp; h carries 2^-2 xexp into the down product).
  int32_t* xexp;
  // Routed gate/up only: the router logits [T, E], and where workgroup 0
  // stores the routing it derives (the routing step's five outputs).
  const float* logits;
  int32_t* r_ids;
  float* r_gates;
  int32_t* r_counts;
  int32_t* r_offsets;
  int32_t* r_sorted;
};

constexpr int kDecXSlack = 512;
constexpr int kDecXP = 3;        // activation pieces per thread loaded before the first store (routed form)
constexpr int kDecMaxExperts = 1024;
constexpr int kDecMaxTopk = 16;            // the route's top-k limit

// SRC: dtype of the rows in memory (kF16 or kBF16); the operands are fp16.
// RNS > 0 (gate/up only): the routing is derived in the kernel from the
// logits instead of read from the routing step's outputs, RNS 64-expert slots
// per lane (E <= 64 RNS).  Every workgroup derives it (T <= 8 tokens: one
// wave per token, then the pairs' stable order by (expert, pair id));
// workgroup 0 also stores it.
template <int FMT, int SRC, int MODE, int NI, int WAVES, int P, int RNS>
__global__ __launch_bounds__(WAVES * 64) void moe_gemv_kernel(const MoeDecArgs a) {
  typedef typename Op<kF16>::vec vec;
  typedef GemvStage<FMT> Stage;
  constexpr int REC = Fmt<FMT>::kRecBytes;
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
  constexpr bool ROUTED = RNS > 0;
  static_assert(!ROUTED || (MODE == kDecGateUp && WAVES >= kMoeDecodeMaxTokens && WAVES * 64 >= 128),
                "routed form: gate/up, a wave per token, a thread per pair");

  const int pos = blockIdx.x / a.groups;
  const int grp = blockIdx.x - pos * a.groups;
  const int tid = threadIdx.x;
  __shared__ int32_t s_pair[kMoeDecodeMaxTokens];
  __shared__ uint32_t s_rmax[kMoeDecodeMaxTokens];   // gate/up: magnitude bits of each row's largest |x|
  __shared__ int32_t s_ex[kMoeDecodeMaxTokens];      // each row's exponent
  if (tid < kMoeDecodeMaxTokens) s_rmax[tid] = 0;    // ordered by a barrier before the first atomicMax
  int e, r0, M;
  if constexpr (ROUTED) {
    __shared__ int32_t s_ids[kMoeDecodeMaxTokens * kDecMaxTopk];
    __shared__ float s_gates[kMoeDecodeMaxTokens * kDecMaxTopk];
    __shared__ int32_t s_sorted[kMoeDecodeMaxTokens * kDecMaxTopk];
    const int npos = a.npos;
    // Every token's row (T <= 4), staged raw while the routing runs: row t
    // at xs + t (K + 8), its largest magnitude into s_rmax[t].  The expert's
    // rows are then a subset, read through their token index.
    __syncthreads();   // s_rmax cleared before any atomicMax
    // The routing waves' logits are loaded first, so their latency overlaps
    // the row staging below.
    float lg[ROUTED ? RNS : 1];
    if ((tid >> 6) < a.T) topk_load<ROUTED ? RNS : 1>(a.logits, tid >> 6, a.E, tid & 63, lg);
    {
      const int per_row = a.K / 8 + 1;
      const int pieces = a.T * per_row + kDecXSlack / 16;
      // The first kDecXP pieces of every thread are loaded before any is
      // stored (straight-line code: one wait covers them and the logits).
      u32x4_t xv[kDecXP];
#pragma unroll
      for (int u = 0; u < kDecXP; ++u) {
        const int i = tid + u * WAVES * 64;
        const int t = i / per_row, k8 = i - t * per_row;
        xv[u] = (i < pieces && t < a.T && k8 < a.K / 8) ? *(const u32x4_t*)(a.X + (int64_t)t * a.ldx + k8 * 8)
                                                        : u32x4_t{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < kDecXP; ++u) {
        const int i = tid + u * WAVES * 64;
        const int t = i / per_row;
        if (i < pieces) {
          if (t < a.T) atomicMax(&s_rmax[t], max_mag_bits8(xv[u]));
          *(u32x4_t*)(xs + i * 8) = xv[u];
        }
      }
      for (int i = tid + kDecXP * WAVES * 64; i < pieces; i += WAVES * 64) {
        const int t = i / per_row, k8 = i - t * per_row;
        u32x4_t v = u32x4_t{0, 0, 0, 0};
        if (t < a.T && k8 < a.K / 8) {
          v = *(const u32x4_t*)(a.X + (int64_t)t * a.ldx + k8 * 8);
          atomicMax(&s_rmax[t], max_mag_bits8(v));
        }
        *(u32x4_t*)(xs + i * 8) = v;
      }
    }
    if ((tid >> 6) < a.T) topk_select<ROUTED ? RNS : 1>(lg, tid >> 6, a.E, a.topk, tid & 63, s_ids, s_gates);
    __syncthreads();
    if (tid < npos) {   // rank of pair tid in the stable order by (expert, pair id)
      const int ep = s_ids[tid];
      int rank = 0;
      for (int q = 0; q < npos; ++q) rank += (s_ids[q] < ep || (s_ids[q] == ep && q < tid)) ? 1 : 0;
      s_sorted[rank] = tid;
    }
    __syncthreads();
    if (blockIdx.x == 0) {
      for (int p = tid; p < npos; p += WAVES * 64) {
        a.r_ids[p] = s_ids[p];
        a.r_gates[p] = s_gates[p];
        a.r_sorted[p] = s_sorted[p];
      }
      for (int x = tid; x <= a.E; x += WAVES * 64) {
        int below = 0, same = 0;
        for (int q = 0; q < npos; ++q) {
          below += s_ids[q] < x ? 1 : 0;
          same += s_ids[q] == x ? 1 : 0;
        }
        a.r_offsets[x] = below;
        if (x < a.E) a.r_counts[x] = same;
      }
    }
    e = s_ids[s_sorted[pos]];
    int below = 0, same = 0;
    for (int q = 0; q < npos; ++q) {
      below += s_ids[q] < e ? 1 : 0;
      same += s_ids[q] == e ? 1 : 0;
    }
    r0 = below;
    if (r0 != pos) return;                    // not the expert's first position (uniform)
    M = min(same, a.T);                       // a token picks an expert at most once
    if (tid < kMoeDecodeMaxTokens && pos + tid < npos) s_pair[tid] = s_sorted[pos + tid];
    __syncthreads();
  } else {
    // One round trip for the routing data: offsets into LDS, and the pair ids
    // of positions pos .. pos + 7 (this workgroup's rows if it leads).
    __shared__ int32_t s_off[kDecMaxExperts + 1];
    for (int i = tid; i <= a.E; i += WAVES * 64) s_off[i] = a.offsets[i];
    if (tid < kMoeDecodeMaxTokens && pos + tid < a.npos)
      s_pair[tid] = min(max(a.sorted_pairs[pos + tid], 0), a.npos - 1);   // clamped like the prefill path
    __syncthreads();
    // Expert owning sorted position pos: the largest e with offsets[e] <= pos.
    int lo = 0, hi = a.E;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (s_off[mid] <= pos) lo = mid;
      else hi = mid;
    }
    e = lo;
    r0 = s_off[e];
    if (r0 != pos) return;                    // not the expert's first position
    // The expert's rows: 1..T for routing from q4q8_moe_route (a token picks
    // an expert at most once); clamped so malformed routing stays in bounds.
    M = max(1, min(min(s_off[e + 1] - r0, a.T), a.npos - r0));
  }

  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  constexpr int MATS = MODE == kDecGateUp ? 2 : 1;
  const int KSH = a.ksh;
  const int KS = KSH * MATS;                  // waves per tile
  const int TPW = WAVES / KS;
  const int slot = wave / KS, kw = wave & (KS - 1);
  const bool up = MODE == kDecGateUp && kw >= KSH;
  const int ks = up ? kw - KSH : kw;
  const int N = a.N, K = a.K;
  const int nchunks = K / kChunkK;
  const int tiles = N / kTileRows;
  const int tile = grp * TPW + slot;
  const bool tile_ok = tile < tiles;
  const int r = lane & 15, g = lane >> 4;
  const int m = 4 * (r & 3) + (r >> 2);       // activation row fed by this lane
  const bool mvalid = m < M;

  const uint8_t* wbase = (up ? a.W2 : a.W) + (int64_t)e * a.mat_bytes;
  const __amdgpu_buffer_rsrc_t wres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(wbase + (int64_t)(tile_ok ? tile : 0) * nchunks * REC), (short)0, tile_ok ? nchunks * REC : 0,
      kGemvBufFlags);

  // Weight prefetch first (it does not depend on x), then the x rows into
  // LDS as fp16: rows of K + 8 halfs, then kDecXSlack zero bytes.  Each row
  // is scaled by a power of two, as the prefill path's pre-pass does: gate/up
  // finds each token row's largest magnitude while staging it raw, then
  // converts its own pieces in place; down takes the h rows' 2^-2 xexp.
  Stage st[P];
#pragma unroll
  for (int p = 0; p < P; ++p) gemv_load<FMT>(st[p], wres, ks + p * KSH, lane, r);
  const int per_row = K / 8 + 1;
  // ROUTED: every token's row is in LDS already (row t = token t); its
  // exponent, then the scaled fp16 copy in place.
  const int pieces = ROUTED ? 0 : M * per_row + kDecXSlack / 16;
  if constexpr (ROUTED) {
    if (tid < kMoeDecodeMaxTokens) {
      const int ex = row_exponent<SRC>(s_rmax[tid]);
      s_ex[tid] = ex;
      if (blockIdx.x == 0 && tid < a.T) a.xexp[tid] = ex;   // the down kernel's and combine's copy
    }
    __syncthreads();
    for (int i = tid; i < a.T * per_row; i += WAVES * 64) {   // the pieces this thread staged
      const int t = i / per_row;
      if (i - t * per_row < K / 8) *(u32x4_t*)(xs + i * 8) = f16x8_scaled<SRC>(*(const u32x4_t*)(xs + i * 8),
                                                                              -s_ex[t]);
    }
  }
  for (int i = tid; i < pieces; i += WAVES * 64) {
    const int mm = i / per_row, k8 = i - mm * per_row;
    u32x4_t v = u32x4_t{0, 0, 0, 0};
    if (mm < M && k8 < K / 8) {
      if constexpr (MODE == kDecGateUp) {
        v = *(const u32x4_t*)(a.X + (int64_t)(s_pair[mm] / a.topk) * a.ldx + k8 * 8);
        atomicMax(&s_rmax[mm], max_mag_bits8(v));
      } else {
        v = *(const u32x4_t*)(a.X + (int64_t)(r0 + mm) * a.ldx + k8 * 8);
        v = f16x8_scaled<SRC>(v, -2 * a.xexp[s_pair[mm] / a.topk]);
      }
    }
    *(u32x4_t*)(xs + i * 8) = v;
  }
  if constexpr (MODE == kDecGateUp && !ROUTED) {
    __syncthreads();
    if (tid < kMoeDecodeMaxTokens) {
      const int ex = row_exponent<SRC>(s_rmax[tid]);
      s_ex[tid] = ex;
      if (grp == 0 && tid < M) a.xexp[s_pair[tid] / a.topk] = ex;   // the down kernel's and combine's copy
    }
    __syncthreads();
    for (int i = tid; i < M * per_row; i += WAVES * 64) {   // the pieces this thread staged
      const int mm = i / per_row;
      if (i - mm * per_row < K / 8) *(u32x4_t*)(xs + i * 8) = f16x8_scaled<SRC>(*(const u32x4_t*)(xs + i * 8),
                                                                               -s_ex[mm]);
    }
  }
  __syncthreads();
  // The lane's activation row in LDS: row m, or (ROUTED) its token's row.
  const int xr = ROUTED ? (mvalid ? s_pair[m] / a.topk : 0) : (mvalid ? m : 0);
  const uint16_t* xrow = xs + xr * (K + 8) + 8 * g;

  float acc[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) acc[i] = 0.0f;
  auto compute = [&](const Stage& s, int c) {
    vec av[kBlocksPerChunk];
#pragma unroll
    for (int j = 0; j < kBlocksPerChunk; ++j) av[j] = *(const vec*)(xrow + c * kChunkK + j * 32);
    gemv_mma<FMT, kF16, NI>(s, av, acc);
  };
  // Chunks of this wave: ks + i KSH, i < nw; full groups of P prefetch the
  // next group, the last (possibly partial) group issues no loads.
  const int nw = (nchunks - ks + KSH - 1) / KSH;
  int i0 = 0;
  for (; i0 + P < nw; i0 += P) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int c = ks + (i0 + p) * KSH;
      compute(st[p], c);
      __builtin_amdgcn_sched_barrier(0);
      gemv_load<FMT>(st[p], wres, c + P * KSH, lane, r);
    }
  }
#pragma unroll
  for (int p = 0; p < P; ++p)
    if (i0 + p < nw) compute(st[p], ks + (i0 + p) * KSH);

  __shared__ float red[WAVES][NI][64];
  if (KS > 1) {   // uniform over the workgroup
#pragma unroll
    for (int i = 0; i < NI; ++i) red[wave][i][lane] = acc[i];
    __syncthreads();
    if (kw != 0) return;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float v = red[wave][i][lane];
      for (int w = 1; w < KSH; ++w) v += red[wave + w][i][lane];
      if (MODE == kDecGateUp) {   // z = 2^ex acc: h at its true scale
        float u = red[wave + KSH][i][lane];
        for (int w = 1; w < KSH; ++w) u += red[wave + KSH + w][i][lane];
        const int mo = min(4 * i + g, kMoeDecodeMaxTokens - 1);
        const int ex = ROUTED ? s_ex[s_pair[min(mo, M - 1)] / a.topk] : s_ex[mo];   // exponents by token (ROUTED) or row
        v = silu_f32(__builtin_ldexpf(v, ex)) * __builtin_ldexpf(u, ex);
      }
      acc[i] = v;
    }
  }
  if (!tile_ok) return;
  // Lane (r, g), register i holds row m = 4 i + g, output n = 16 tile + r.
  const int n = tile * kTileRows + r;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int mo = 4 * i + g;
    if (mo < M) {
      if (MODE == kDecGateUp) {
        a.out[(int64_t)(r0 + mo) * N + n] = __builtin_bit_cast(uint16_t, (__bf16)acc[i]);
      } else {
        const int pair = s_pair[mo];
        a.out[(int64_t)pair * N + n] = __builtin_bit_cast(uint16_t, (_Float16)acc[i]);
      }
    }
  }
}

// Down projection fused with the weighted combine.  Workgroup (token t,
// 16-row tile of H), WAVES waves: wave w < topk KQ takes the token's slot
// j = w / KQ (expert e_j,
// found from the pair's sorted position) and K-share w % KQ of the tile's
// F-long rows, with the pair's h row (bf16, converted to fp16 in LDS) as its
// activation row.  The reduction sums each slot's K-shares in order, rounds
// y to fp16 as the unfused path stores it, and accumulates
// out[t, n] = sum_j gates[t, j] y_j[n] over j = 0 .. topk-1 in the combine
// kernel's order: the same values, one launch and no y round trip fewer.
constexpr int kDcMaxTokens = 4;   // tokens up to which the fused form is used (measured below)
struct MoeDcArgs {
  const uint8_t* W;          // down weights of expert 0
  int64_t mat_bytes;         // repacked bytes of one expert's [H, F] matrix
  const uint16_t* h;         // bf16 [positions, F], sorted-pair order
  const float* gates;        // [T, topk]
  const int32_t* offsets;    // [E + 1]
  const int32_t* sorted_pairs;
  const int32_t* xexp;       // [T]: token t's h rows carry 2^-2 xexp[t]
  float* out;                // [T, H]
  int32_t H, F, topk, E, npos, kq;   // kq: K-shares per slot (topk kq <= WAVES)
};

template <int FMT, int WAVES, int P>
__global__ __launch_bounds__(WAVES * 64) void moe_down_combine_kernel(const MoeDcArgs a) {
  typedef typename Op<kF16>::vec vec;
  typedef GemvStage<FMT> Stage;
  constexpr int REC = Fmt<FMT>::kRecBytes;
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];
  __shared__ int32_t s_off[kDecMaxExperts + 1];
  __shared__ int32_t s_pos[kDecMaxTopk];     // sorted position of each of token t's pairs
  __shared__ float red[WAVES][64];

  const int tiles = a.H / kTileRows;
  const int t = blockIdx.x / tiles;
  const int tile = blockIdx.x - t * tiles;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int topk = a.topk, KQ = a.kq;
  // Both routing loads in one round trip: the offsets (two a thread) and
  // this thread's sorted pair (the fused path takes at most kDcMaxTokens
  // tokens, so every pair has a thread).
  constexpr int THREADS = WAVES * 64;
  static_assert(2 * THREADS > kDecMaxExperts && kDcMaxTokens * kDecMaxTopk <= THREADS, "one pass of loads");
  int offv[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int i = tid + u * THREADS;
    offv[u] = i <= a.E ? a.offsets[i] : 0;
  }
  const int spv = tid < a.npos ? a.sorted_pairs[tid] : -1;
  if (tid < kDecMaxTopk) s_pos[tid] = 0;   // stays in bounds for malformed routing
  __syncthreads();
#pragma unroll
  for (int u = 0; u < 2; ++u)
    if (tid + u * THREADS <= a.E) s_off[tid + u * THREADS] = offv[u];
  // Inverse of the sort for this token's pairs t topk .. t topk + topk - 1.
  if (tid < a.npos) {
    const int p = spv - t * topk;
    if (p >= 0 && p < topk) s_pos[p] = tid;
  }
  __syncthreads();
  const int j = wave / KQ, kw = wave - j * KQ;
  const bool active = j < topk;                 // uniform per wave
  const int pos = active ? s_pos[j] : 0;
  // Expert owning sorted position pos: the largest e with offsets[e] <= pos.
  int lo = 0, hi = a.E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (s_off[mid] <= pos) lo = mid;
    else hi = mid;
  }
  const int e = lo;

  const int F = a.F, nchunks = F / kChunkK;
  const int r = lane & 15, g = lane >> 4;
  const uint8_t* wbase = a.W + (int64_t)e * a.mat_bytes + (int64_t)tile * nchunks * REC;
  const __amdgpu_buffer_rsrc_t wres =
      __builtin_amdgcn_make_buffer_rsrc((void*)wbase, (short)0, active ? nchunks * REC : 0, kGemvBufFlags);
  Stage st[P];
#pragma unroll
  for (int p = 0; p < P; ++p) gemv_load<FMT>(st[p], wres, kw + p * KQ, lane, r);
  // The token's h rows (slot order) into LDS as fp16, rows of F + 8 halfs,
  // then kDecXSlack zero bytes.
  const int per_row = F / 8 + 1;
  const int pieces = topk * per_row + kDecXSlack / 16;
  const int ex = a.xexp[t];
  for (int i = tid; i < pieces; i += WAVES * 64) {
    const int jj = i / per_row, k8 = i - jj * per_row;
    u32x4_t v = u32x4_t{0, 0, 0, 0};
    if (jj < topk && k8 < F / 8) v = f16x8_scaled<kBF16>(*(const u32x4_t*)(a.h + (int64_t)s_pos[jj] * F + k8 * 8),
                                                          -2 * ex);
    *(u32x4_t*)(xs + i * 8) = v;
  }
  __syncthreads();
  // One activation row per wave: every lane reads the slot's row (rows of the
  // MFMA tile other than 0 are not used).
  const uint16_t* xrow = xs + (active ? j : 0) * (F + 8) + 8 * g;
  float acc[1] = {0.0f};
  auto compute = [&](const Stage& s, int c) {
    vec av[kBlocksPerChunk];
#pragma unroll
    for (int q = 0; q < kBlocksPerChunk; ++q) av[q] = *(const vec*)(xrow + c * kChunkK + q * 32);
    gemv_mma<FMT, kF16, 1>(s, av, acc);
  };
  const int nw = active ? (nchunks - kw + KQ - 1) / KQ : 0;
  int i0 = 0;
  for (; i0 + P < nw; i0 += P) {
#pragma unroll
    for (int p = 0; p < P; ++p) {
      const int c = kw + (i0 + p) * KQ;
      compute(st[p], c);
      __builtin_amdgcn_sched_barrier(0);
      gemv_load<FMT>(st[p], wres, c + P * KQ, lane, r);
    }
  }
#pragma unroll
  for (int p = 0; p < P; ++p)
    if (i0 + p < nw) compute(st[p], kw + (i0 + p) * KQ);

  red[wave][lane] = acc[0];
  __syncthreads();
  if (wave != 0 || g != 0) return;
  // Lane (r, 0) holds row 0, output n = 16 tile + r.
  float sum = 0.0f;
  for (int jj = 0; jj < topk; ++jj) {
    float v = red[jj * KQ][lane];
    for (int w = 1; w < KQ; ++w) v += red[jj * KQ + w][lane];
    const float y = (float)(_Float16)v;               // y as the unfused path stores it
    sum += a.gates[(int64_t)t * topk + jj] * y;       // the combine kernel's order
  }
  a.out[(int64_t)t * a.H + tile * kTileRows + r] = __builtin_ldexpf(sum, 2 * ex);
}

namespace {

constexpr int kDecWaves = 8;
constexpr int kDecRing = 4;

// K-shares per matrix: split K while the busiest case (every pair on its
// own expert) stays below about 4096 waves, each wave keeps >= 3 chunks and
// the tile's waves fit the workgroup.
int dec_ksh(int nchunks, int mats, int64_t tile_waves) {
  int ksh = 1;
  while (ksh * 2 * mats <= kDecWaves && nchunks >= 3 * ksh * 2 && tile_waves * ksh * 2 <= 4096) ksh *= 2;
  return ksh;
}

template <int FMT, int SRC, int MODE, int RNS = 0>
void launch_dec(MoeDecArgs a, int T, int npos, hipStream_t s) {
  const int mats = MODE == kDecGateUp ? 2 : 1;
  const int64_t experts = std::min(npos, a.E);
  a.ksh = dec_ksh(a.K / kChunkK, mats, experts * (a.N / kTileRows) * mats);
  const int tpw = kDecWaves / (a.ksh * mats);
  a.groups = (a.N / kTileRows + tpw - 1) / tpw;
  const dim3 grid((unsigned)(npos * a.groups)), block(kDecWaves * 64);
  const size_t lds = (size_t)T * (a.K + 8) * 2 + kDecXSlack;
  if (T > 4)
    moe_gemv_kernel<FMT, SRC, MODE, 2, kDecWaves, kDecRing, RNS><<<grid, block, lds, s>>>(a);
  else
    moe_gemv_kernel<FMT, SRC, MODE, 1, kDecWaves, kDecRing, RNS><<<grid, block, lds, s>>>(a);
}

// The fused down + combine kernel: topk K-share groups of KQ waves in at most
// kDcWaves waves, and the token's topk h rows in a 52 KB activation buffer.
constexpr int kDcWaves = 16;
// Past 4 tokens the unfused down (one pass over each expert's weights for all
// of its tokens) plus the combine is faster (measured on MI355X, E 128 top-8
// H 2048 F 768: fused 21.7/24.5/31.1/44.7 us per step at T = 1/2/4/8 against
// 23.1/26.5/32.3/42.8 unfused): kDcMaxTokens.
bool down_combine_fits(int topk, int F) {
  return topk >= 1 && topk <= kDecMaxTopk && (int64_t)topk * (F + 8) * 2 + kDecXSlack <= 52 * 1024;
}

// ro: null, or the routed form (the gate/up kernel derives the routing from
// ro->logits and stores it in ro's arrays, which the later kernels read).
template <int FMT>
bool launch_dec_fmt(int xdt, const void* Wg, const void* Wu, const void* Wd, int E, int H, int F, const void* X,
                    int T, int topk, const float* gates, const int32_t* offsets, const int32_t* sorted_pairs,
                    uint16_t* h, uint16_t* y16, int32_t* xexp, float* out, hipStream_t s, const MoeRouteOut* ro) {
  const int npos = T * topk;
  MoeDecArgs a = {};
  a.xexp = xexp;
  if (ro) {
    a.logits = ro->logits;
    a.r_ids = ro->ids;
    a.r_gates = ro->gates;
    a.r_counts = ro->counts;
    a.r_offsets = ro->offsets;
    a.r_sorted = ro->sorted_pairs;
    gates = ro->gates;
    offsets = ro->offsets;
    sorted_pairs = ro->sorted_pairs;
  }
  a.offsets = offsets;
  a.sorted_pairs = sorted_pairs;
  a.topk = topk;
  a.E = E;
  a.npos = npos;
  a.T = T;
  // gate/up: [F, H] per expert, x = the tokens.
  a.W = (const uint8_t*)Wg;
  a.W2 = (const uint8_t*)Wu;
  a.mat_bytes = (int64_t)(F / kTileRows) * (H / kChunkK) * Fmt<FMT>::kRecBytes;
  a.X = (const uint16_t*)X;
  a.ldx = H;
  a.out = h;
  a.N = F;
  a.K = H;
  if (ro) {   // 2 expert slots a lane up to 128 experts, else 16 (up to 1024)
    if (xdt == kF16) {
      if (E <= 128) launch_dec<FMT, kF16, kDecGateUp, 2>(a, T, npos, s);
      else launch_dec<FMT, kF16, kDecGateUp, 16>(a, T, npos, s);
    } else {
      if (E <= 128) launch_dec<FMT, kBF16, kDecGateUp, 2>(a, T, npos, s);
      else launch_dec<FMT, kBF16, kDecGateUp, 16>(a, T, npos, s);
    }
  } else {
    if (xdt == kF16) launch_dec<FMT, kF16, kDecGateUp>(a, T, npos, s);
    else launch_dec<FMT, kBF16, kDecGateUp>(a, T, npos, s);
  }
  // down: [H, F] per expert, x = the h rows.
  const int64_t dbytes = (int64_t)(H / kTileRows) * (F / kChunkK) * Fmt<FMT>::kRecBytes;
  if (T <= kDcMaxTokens && down_combine_fits(topk, F)) {
    // Fused with the combine: one workgroup per (token, 16-row tile), the
    // same K split per slot as the unfused down kernel would take.
    MoeDcArgs d;
    d.W = (const uint8_t*)Wd;
    d.mat_bytes = dbytes;
    d.h = h;
    d.gates = gates;
    d.offsets = offsets;
    d.sorted_pairs = sorted_pairs;
    d.xexp = xexp;
    d.out = out;
    d.H = H;
    d.F = F;
    d.topk = topk;
    d.E = E;
    d.npos = npos;
    const int64_t experts = std::min(npos, E);
    d.kq = dec_ksh(F / kChunkK, 1, experts * (H / kTileRows));
    while (d.kq > 1 && topk * d.kq > kDcWaves) d.kq /= 2;
    // Always kDcWaves waves (the kernel's strides assume it); waves past
    // topk kq stay idle.
    const dim3 grid((unsigned)(T * (H / kTileRows))), block(kDcWaves * 64);
    const size_t lds = (size_t)topk * (F + 8) * 2 + kDecXSlack;
    moe_down_combine_kernel<FMT, kDcWaves, kDecRing><<<grid, block, lds, s>>>(d);
    return true;
  }
  a.W = (const uint8_t*)Wd;
  a.W2 = nullptr;
  a.mat_bytes = dbytes;
  a.X = h;
  a.ldx = F;
  a.out = y16;
  a.N = H;
  a.K = F;
  launch_dec<FMT, kBF16, kDecDown>(a, T, npos, s);
  return false;
}

}  // namespace

bool moe_decode_fits(int T, int H, int F) {
  const int64_t k = H > F ? H : F;
  // Dynamic LDS plus the static buffers (reduction, offsets) stay within 64 KB.
  return T >= 1 && T <= kMoeDecodeMaxTokens && (int64_t)T * (k + 8) * 2 + kDecXSlack <= 52 * 1024;
}

bool launch_moe_decode(int fmt, int xdt, const void* Wg, const void* Wu, const void* Wd, int E, int H, int F,
                       const void* X, int T, int topk, const float* gates, const int32_t* offsets,
                       const int32_t* sorted_pairs, uint16_t* h, uint16_t* y16, int32_t* xexp, float* out,
                       hipStream_t s) {
  if (fmt == kQ4_0)
    return launch_dec_fmt<kQ4_0>(xdt, Wg, Wu, Wd, E, H, F, X, T, topk, gates, offsets, sorted_pairs, h, y16, xexp,
                                 out, s, nullptr);
  return launch_dec_fmt<kQ8_0>(xdt, Wg, Wu, Wd, E, H, F, X, T, topk, gates, offsets, sorted_pairs, h, y16, xexp, out,
                               s, nullptr);
}

bool launch_moe_decode_routed(int fmt, int xdt, const void* Wg, const void* Wu, const void* Wd, int E, int H, int F,
                              const void* X, int T, int topk, const MoeRouteOut& ro, uint16_t* h, uint16_t* y16,
                              int32_t* xexp, float* out, hipStream_t s) {
  if (fmt == kQ4_0)
    return launch_dec_fmt<kQ4_0>(xdt, Wg, Wu, Wd, E, H, F, X, T, topk, nullptr, nullptr, nullptr, h, y16, xexp, out,
                                 s, &ro);
  return launch_dec_fmt<kQ8_0>(xdt, Wg, Wu, Wd, E, H, F, X, T, topk, nullptr, nullptr, nullptr, h, y16, xexp, out, s,
                               &ro);
}

}  // namespace q4q8
