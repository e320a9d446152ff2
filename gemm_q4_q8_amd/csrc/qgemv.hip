// Decode GEMV over repacked Q4_0 / Q8_0 weights, M = 1..8 activation rows.
//
// The pages ("BaseRT: Best-in-Class LLM Inference on Apple Silicon via Native
// Metal", gist.science technical summary, "Methodologie", kernel
// specialisation) run decode on a GEMV per quantisation format that
// dequantises inside its inner loop.  On gfx950 the inner product of each
// 32-weight block is one v_mfma_f32_16x16x32 instruction instead of lane FMAs
// plus a cross-lane reduction (gemv_core.h):
//   * a wavefront owns a tile of 16 weight rows and a share of K; a workgroup
//     of WAVES waves holds WAVES / KS tiles x KS K-shares, KS chosen per
//     problem of a grouped launch so that every wave streams about as many
//     chunks; K-shares of one tile are reduced through LDS in a fixed order
//     at the end (split-K without atomics or workspace);
//   * the activation rows are staged once per workgroup in LDS; each lane
//     reads its 16-byte A fragment from there;
//   * weights stream through buffer loads into a ring of P chunks in flight.
//     The buffer range is the tile itself, so loads past its end return zero
//     (scale 0) and tails need no branches;
//   * a SwiGLU pair (gate and up rows of one FFN, same x) spends half of a
//     tile's waves on each matrix and forms h = silu(gate) * up in the
//     reduction, so neither product reaches memory (technical summary,
//     "Methodologie", fusion of feed-forward operator sequences).
#include "gemv_core.h"
#include "q4q8_internal.h"


#include <algorithm>
#include <mutex>
#include <type_traits>

namespace q4q8 {

constexpr int kXSlack = 512;            // zeroed LDS bytes after the activation rows
constexpr int XP = 4;                   // x pieces per thread staged before the prefetch
constexpr int64_t kLdsTotal = 160 * 1024;          // LDS per workgroup on gfx950
constexpr int64_t kLdsCap = kLdsTotal - 8 * 1024;  // dynamic LDS for the activations

// Where the activation rows come from: global memory, LDS, or LDS for the
// problems with K <= args.xk and global memory for the rest.
enum { kXGlobal = 0, kXLds = 1, kXMixed = 2 };

// The mixed form holds both paths; for Q4_0 at M > 4 it is held to 64
// registers like the other forms (no spills there), so that two 16-wave
// workgroups still share a CU.
template <int FMT, int XDT, int NI, int WAVES, int P, int XM>
__global__ __launch_bounds__(WAVES * 64)
__attribute__((amdgpu_waves_per_eu(XM == kXMixed && NI == 2 && FMT == kQ4_0 ? 8 : 1)))
void qgemv_kernel(const GemvArgs args) {
  constexpr int REC = Fmt<FMT>::kRecBytes;
  typedef typename Op<XDT>::vec vec;
  typedef GemvStage<FMT> Stage;
  extern __shared__ __attribute__((aligned(16))) uint16_t xs[];

  // Problem of the group that owns this workgroup.  Problem 0's fields are
  // loaded together with the boundaries; only later problems pay a second
  // kernel-argument round trip.
  const int bid = blockIdx.x;
  int pi = 0;
#pragma unroll
  for (int i = 1; i < kMaxGroup; ++i) pi += (i < args.count && bid >= args.wg0[i]) ? 1 : 0;
  GemvProb prob = args.p[0];
  if (pi != 0) prob = args.p[pi];
  const int N = prob.N, K = prob.K;
  const int nchunks = (K + kChunkK - 1) / kChunkK;
  const int nblocks = K / 32;
  const int tiles = (N + kTileRows - 1) / kTileRows;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int KS = __builtin_amdgcn_readfirstlane(args.ks[pi]);   // waves per tile, a power of 2 dividing WAVES
  const int TPW = WAVES / KS;
  const int slot = wave / KS, kw = wave & (KS - 1);
  // A SwiGLU pair spends the first half of a tile's waves on the gate rows
  // and the second half on the same rows of the up matrix.
  const bool pair = prob.W2 != nullptr;
  const int KSH = pair ? KS >> 1 : KS;           // K-shares per matrix
  const bool up = pair && kw >= KSH;
  const int ks = up ? kw - KSH : kw;             // this wave's K-share
  const int tile = (bid - args.wg0[pi]) * TPW + slot;
  const bool tile_ok = tile < tiles;
  const int r = lane & 15, g = lane >> 4;
  const int m = 4 * (r & 3) + (r >> 2);          // activation row fed by this lane
  const bool mvalid = m < args.M;

  // Buffer over this tile's records only: past the end reads return zero.
  const uint8_t* tbase = (up ? prob.W2 : prob.W) + (int64_t)(tile_ok ? tile : 0) * nchunks * REC;
  const __amdgpu_buffer_rsrc_t wres =
      __builtin_amdgcn_make_buffer_rsrc((void*)tbase, (short)0, tile_ok ? nchunks * REC : 0, kGemvBufFlags);
  auto load = [&](Stage& st, int c) { gemv_load<FMT>(st, wres, c, lane, r); };

  // Activations: LDS rows of K + 8 halfs (the pad staggers rows over banks),
  // plus kXSlack zeroed bytes after the last row.  x is loaded first, then
  // the weight prefetch is issued, so the wait before the LDS writes covers
  // only the x loads.  Reads of blocks past K (chunk tails, scale 0) land in
  // the zeroed pad, the next row or the slack: always finite.
  const int ldsx = K + 8;
  const int M = args.M;
  const uint16_t* __restrict__ xg = prob.x;
  __shared__ float red[WAVES][NI][64];   // split-K partial sums

  // The rest of the kernel, with x read from LDS (xl) or global memory.
  auto run = [&](auto xlc) __attribute__((always_inline)) {
    constexpr bool xl = decltype(xlc)::value;
    Stage st[P];
    if constexpr (xl) {
      const int per_row = K / 8 + 1;                 // 16-byte pieces incl. the pad
      const int pieces = M * per_row + kXSlack / 16;
      u32x4_t xv[XP];
#pragma unroll
      for (int u = 0; u < XP; ++u) {
        const int i = tid + u * WAVES * 64;
        const int mm = i / per_row, k8 = i - mm * per_row;
        xv[u] = (mm < M && k8 < K / 8) ? *(const u32x4_t*)(xg + (int64_t)mm * prob.ldx + k8 * 8) : u32x4_t{0, 0, 0, 0};
      }
#pragma unroll
      for (int p = 0; p < P; ++p) load(st[p], ks + p * KSH);   // past the tile: zero, no memory traffic
#pragma unroll
      for (int u = 0; u < XP; ++u) {
        const int i = tid + u * WAVES * 64;
        if (i < pieces) *(u32x4_t*)(xs + i * 8) = xv[u];
      }
      for (int i = tid + XP * WAVES * 64; i < pieces; i += WAVES * 64) {
        const int mm = i / per_row, k8 = i - mm * per_row;
        const u32x4_t v =
            (mm < M && k8 < K / 8) ? *(const u32x4_t*)(xg + (int64_t)mm * prob.ldx + k8 * 8) : u32x4_t{0, 0, 0, 0};
        *(u32x4_t*)(xs + i * 8) = v;
      }
      __syncthreads();
    } else {
#pragma unroll
      for (int p = 0; p < P; ++p) load(st[p], ks + p * KSH);
    }
    const int xrow_lds = (mvalid ? m : 0) * ldsx + 8 * g;
    const uint16_t* __restrict__ xrow_g = xg + (mvalid ? (int64_t)m * prob.ldx : 0) + 8 * g;

    float acc[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) acc[i] = 0.0f;

    auto compute = [&](const Stage& s, int c) {
      vec a[kBlocksPerChunk];
      if constexpr (xl) {
        const int cx = c < nchunks ? c : nchunks - 1;   // chunks past the tile are all zero-scale
        const uint16_t* xa = xs + xrow_lds + cx * kChunkK;
#pragma unroll
        for (int j = 0; j < kBlocksPerChunk; ++j) a[j] = *(const vec*)(xa + j * 32);
      } else {
#pragma unroll
        for (int j = 0; j < kBlocksPerChunk; ++j) {
          int blk = c * kBlocksPerChunk + j;
          blk = blk < nblocks ? blk : nblocks - 1;     // past-K blocks have scale 0
          a[j] = *(const vec*)(xrow_g + blk * 32);
        }
      }
      if constexpr (FMT == kFP16W) {
        half8_t ah[kBlocksPerChunk];
#pragma unroll
        for (int j = 0; j < kBlocksPerChunk; ++j) {
          if constexpr (XDT == kBF16) ah[j] = bf16x8_to_half8(a[j]);
          else ah[j] = a[j];
        }
        gemv_mma_fp16w<NI>(s, ah, acc);
      } else {
        gemv_mma<FMT, XDT, NI>(s, a, acc);
      }
    };

    // Chunks of this wave: ks + i KSH for i < nw.  Stage p holds chunk i with
    // i % P == p; full groups of P prefetch the next group, the last group
    // (possibly partial) issues no loads, so no load runs past the wave's share.
    const int nw = (nchunks - ks + KSH - 1) / KSH;
    int i0 = 0;
    for (; i0 + P < nw; i0 += P) {
#pragma unroll
      for (int p = 0; p < P; ++p) {
        const int c = ks + (i0 + p) * KSH;
        compute(st[p], c);
        __builtin_amdgcn_sched_barrier(0);
        load(st[p], c + P * KSH);
      }
    }
#pragma unroll
    for (int p = 0; p < P; ++p)
      if (i0 + p < nw) compute(st[p], ks + (i0 + p) * KSH);

    if (KS > 1) {   // uniform over the workgroup
#pragma unroll
      for (int i = 0; i < NI; ++i) red[wave][i][lane] = acc[i];
      __syncthreads();
      if (kw != 0) return;
      // Fixed order: K-shares 0..KSH-1 of the gate (or plain) rows, then of the
      // up rows; SwiGLU in fp32.
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        float v = red[wave][i][lane];
        for (int w = 1; w < KSH; ++w) v += red[wave + w][i][lane];
        if (pair) {
          float u = red[wave + KSH][i][lane];
          for (int w = 1; w < KSH; ++w) u += red[wave + KSH + w][i][lane];
          v = silu_f32(v) * u;
        }
        acc[i] = v;
      }
    }
    if (!tile_ok) return;
    // Lane (r, g), register i holds y[m = 4 i + g][n = 16 tile + r].
    const int n = tile * kTileRows + r;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int mo = 4 * i + g;
      if (mo < args.M && n < N) {
        const int64_t o = (int64_t)mo * prob.ldy + n;
        if (!pair || prob.ydt == kF32)
          ((float*)prob.y)[o] = acc[i];
        else if (prob.ydt == kBF16)
          ((__bf16*)prob.y)[o] = (__bf16)acc[i];
        else if (prob.ydt == kYF16ViaBF16)
          ((_Float16*)prob.y)[o] = (_Float16)(float)(__bf16)acc[i];
        else
          ((_Float16*)prob.y)[o] = (_Float16)acc[i];
      }
    }
  };

  // Problems up to K = args.xk stage x in LDS; a longer one in the same
  // launch (the LDS would not hold its rows) reads x from global memory.
  // Uniform over the workgroup, so the barriers inside are safe.
  if constexpr (XM == kXMixed) {
    if (K <= args.xk) run(std::integral_constant<bool, true>{});
    else run(std::integral_constant<bool, false>{});
  } else {
    run(std::integral_constant<bool, XM == kXLds>{});
  }
}

// ---------------------------------------------------------------------------
// Launch configuration
// ---------------------------------------------------------------------------
struct GemvShape {
  int ks, tpw, p;
  int xmode;
};

template <int FMT, int XDT, int NI, int WAVES, int P, int XM>
static void launch_mode(const GemvArgs& args, int wgs, size_t lds, hipStream_t s, const LaunchEvents& ev) {
  const dim3 grid((unsigned)wgs), block(WAVES * 64);
  auto k = qgemv_kernel<FMT, XDT, NI, WAVES, P, XM>;
  if (XM != kXGlobal && lds > 64 * 1024) {
    // Opt in once to dynamic LDS beyond 64 KB: the device's 160 KB per
    // workgroup minus this kernel's static LDS (the split-K buffer).
    static std::once_flag once;
    static size_t dyn_max = 64 * 1024;
    std::call_once(once, [&] {
      hipFuncAttributes fa;
      if (hipFuncGetAttributes(&fa, (const void*)k) == hipSuccess) {
        const size_t avail = kLdsTotal - fa.sharedSizeBytes;
        if (hipFuncSetAttribute((const void*)k, hipFuncAttributeMaxDynamicSharedMemorySize, (int)avail) ==
            hipSuccess)
          dyn_max = avail;
      }
    });
    if (lds > dyn_max) {   // does not fit: read x from global memory instead
      launch(qgemv_kernel<FMT, XDT, NI, WAVES, P, kXGlobal>, grid, block, 0, s, ev, args);
      return;
    }
  }
  launch(k, grid, block, XM == kXGlobal ? 0u : (uint32_t)lds, s, ev, args);
}

template <int FMT, int XDT, int NI, int WAVES, int P>
static void launch_cfg(int xmode, const GemvArgs& args, int wgs, size_t lds, hipStream_t s, const LaunchEvents& ev) {
  switch (xmode) {
    case kXLds: launch_mode<FMT, XDT, NI, WAVES, P, kXLds>(args, wgs, lds, s, ev); break;
    case kXMixed: launch_mode<FMT, XDT, NI, WAVES, P, kXMixed>(args, wgs, lds, s, ev); break;
    default: launch_mode<FMT, XDT, NI, WAVES, P, kXGlobal>(args, wgs, lds, s, ev); break;
  }
}

template <int FMT, int XDT, int NI, int P>
static void launch_p(int waves, int xmode, const GemvArgs& args, int wgs, size_t lds, hipStream_t s,
                     const LaunchEvents& ev) {
  switch (waves) {
    case 4: launch_cfg<FMT, XDT, NI, 4, P>(xmode, args, wgs, lds, s, ev); break;
    case 8: launch_cfg<FMT, XDT, NI, 8, P>(xmode, args, wgs, lds, s, ev); break;
    default: launch_cfg<FMT, XDT, NI, 16, P>(xmode, args, wgs, lds, s, ev); break;
  }
}

template <int FMT, int XDT, int NI>
static void launch_ni(int waves, const GemvShape& c, const GemvArgs& args, int wgs, size_t lds, hipStream_t s,
                      const LaunchEvents& ev) {
  launch_p<FMT, XDT, NI, 4>(waves, c.xmode, args, wgs, lds, s, ev);
}

// K-shares per tile: about 2048 waves over the chip (8 per CU) with at least
// 8 chunks each; a ring of 4 chunks in flight per wave.  (Measured on MI355X:
// more waves or a ring of 8 both lose, as does a split below 8 chunks.)
// The activation block goes to LDS when it fits in 160 KB; above 32 KB the
// workgroups get 8 or 16 waves since few of them then share a CU.
static GemvShape pick_shape(int tiles, int max_chunks, int M, int max_k) {
  GemvShape c;
  const int64_t lds = (int64_t)M * (max_k + 8) * 2 + kXSlack;
  int ks = 1;
  while (ks < 16 && tiles * ks < 2048 && max_chunks >= 16 * ks) ks *= 2;
  if (lds > 80 * 1024 && ks < 8) ks = 8;
  c.ks = ks;
  c.tpw = ks >= 4 ? 1 : 4 / ks;
  // A large activation block in LDS (M >= 4) caps the workgroups per CU, so
  // each workgroup gets more waves: 16 for big launches, 8 for small ones
  // (measured: M = 8 gate+up 23.3 -> 15.4 us, q/k/v 12.0 -> 8.9 us).
  if (lds > 32 * 1024 && lds <= kLdsCap) c.tpw = std::max(1, (tiles >= 1024 ? 16 : 8) / ks);
  c.p = 4;
  c.xmode = lds <= kLdsCap ? kXLds : kXGlobal;
  return c;
}

hipError_t launch_qgemv(int fmt, int xdt, GemvArgs args, int max_chunks, int max_k, hipStream_t s,
                        const LaunchEvents& ev) {
  // x goes to LDS for every problem whose rows fit there; the LDS is sized
  // for the longest of those, and a problem with a longer K reads x from
  // global memory (M = 8 with K = 12288 next to K = 4096 problems).
  // A launch of problems with different K stages only the problems whose
  // rows take <= 40 KB (at most 3 activation rows) or <= 76 KB (5 or more
  // rows, so that two workgroups share a CU); the deeper ones read x from
  // global memory, so the LDS no longer caps the workgroups a CU holds
  // (measured on MI355X, one grouped launch: 8B layer M = 2 22.5 -> 21.9 us,
  // M = 3 22.7 -> 22.5 us; Q8_0 3B matrices M = 8 19.9 -> 16.8 us, the
  // 8192-deep down projection's 131 KB of rows had held one workgroup a CU.
  // At M = 1 all rows fit anyway; at M = 4 the global reads of four rows cost
  // more: 25.0 -> 28.9 us).
  int64_t target = kLdsCap;
  {
    bool mk = false;
    for (int i = 1; i < args.count; ++i) mk |= args.p[i].K != args.p[0].K;
    if (mk && args.M <= 3) target = 40 * 1024;
    if (mk && args.M >= 5) target = 76 * 1024;   // two workgroups a CU
  }
  int xk = 0;
  for (int pass = 0; pass < 2 && xk == 0; ++pass)   // no problem under the target: the usual LDS cap
    for (int i = 0; i < args.count; ++i) {
      const int k = args.p[i].K;
      if ((int64_t)args.M * (k + 8) * 2 + kXSlack <= (pass ? kLdsCap : target) && k > xk) xk = k;
    }
  args.xk = xk;
  GemvShape c = pick_shape(args.total_tiles, max_chunks, args.M, xk > 0 ? xk : max_k);
  if (c.xmode == kXLds && xk < max_k) c.xmode = kXMixed;
  // Problems of one K share the launch-wide split.  When K differs, the
  // workgroup is 8 waves and each problem takes the finest power-of-2 split
  // that keeps at least 8 chunks a wave (up to the workgroup), so the long-K
  // problems do not trail the launch.
  // A SwiGLU pair takes twice its K-shares in waves (gate and up halves).
  bool mixed = false, pairs = false;
  for (int i = 1; i < args.count; ++i) mixed |= args.p[i].K != args.p[0].K;
  for (int i = 0; i < args.count; ++i) pairs |= args.p[i].W2 != nullptr;
  int waves = c.ks * c.tpw;
  if (mixed) {
    waves = c.ks * c.tpw > 8 ? c.ks * c.tpw : 8;
    for (int i = 0; i < args.count; ++i) {
      const int nch = (args.p[i].K + kChunkK - 1) / kChunkK;
      const int mats = args.p[i].W2 ? 2 : 1;
      int ks = 1;
      while (ks * mats < waves && nch >= 16 * ks) ks *= 2;   // >= 8 chunks a wave (measured: 24 -> 16 gave -4%)
      args.ks[i] = ks * mats;
    }
  } else {
    if (pairs && waves < 2 * c.ks) waves = 2 * c.ks > 16 ? 16 : 2 * c.ks;
    for (int i = 0; i < args.count; ++i) {
      const int ks = args.p[i].W2 ? (2 * c.ks > waves ? waves : 2 * c.ks) : c.ks;
      args.ks[i] = ks;
    }
  }
  // Problems with the longest chain of chunks per wave first in the grid, so
  // that their workgroups start in the first round and the launch's tail
  // holds short ones.  (Each problem writes its own y; the order is free.)
  {
    int cpw[kMaxGroup], order[kMaxGroup];
    for (int i = 0; i < args.count; ++i) {
      const int nch = (args.p[i].K + kChunkK - 1) / kChunkK;
      const int shares = args.p[i].W2 ? args.ks[i] / 2 : args.ks[i];
      cpw[i] = (nch + shares - 1) / shares;
      order[i] = i;
    }
    std::stable_sort(order, order + args.count, [&](int a, int b) { return cpw[a] > cpw[b]; });
    GemvProb p[kMaxGroup];
    int ks[kMaxGroup];
    for (int i = 0; i < args.count; ++i) {
      p[i] = args.p[order[i]];
      ks[i] = args.ks[order[i]];
    }
    for (int i = 0; i < args.count; ++i) {
      args.p[i] = p[i];
      args.ks[i] = ks[i];
    }
  }
  // Workgroup ranges per problem.
  int wgs = 0;
  for (int i = 0; i < args.count; ++i) {
    const int tpw = waves / args.ks[i];
    args.wg0[i] = wgs;
    wgs += (args.p[i].N + kTileRows * tpw - 1) / (kTileRows * tpw);
  }
  for (int i = args.count; i < kMaxGroup; ++i) {
    args.wg0[i] = wgs;
    args.ks[i] = 1;
  }
  const size_t lds = c.xmode != kXGlobal ? (size_t)args.M * (xk + 8) * 2 + kXSlack : 0;
  if (fmt == kQ4_0) {
    if (xdt == kF16) {
      if (args.M > 4) launch_ni<kQ4_0, kF16, 2>(waves, c, args, wgs, lds, s, ev);
      else launch_ni<kQ4_0, kF16, 1>(waves, c, args, wgs, lds, s, ev);
    } else {
      if (args.M > 4) launch_ni<kQ4_0, kBF16, 2>(waves, c, args, wgs, lds, s, ev);
      else launch_ni<kQ4_0, kBF16, 1>(waves, c, args, wgs, lds, s, ev);
    }
  } else if (fmt == kFP16W) {
    if (xdt == kF16) {
      if (args.M > 4) launch_ni<kFP16W, kF16, 2>(waves, c, args, wgs, lds, s, ev);
      else launch_ni<kFP16W, kF16, 1>(waves, c, args, wgs, lds, s, ev);
    } else {
      if (args.M > 4) launch_ni<kFP16W, kBF16, 2>(waves, c, args, wgs, lds, s, ev);
      else launch_ni<kFP16W, kBF16, 1>(waves, c, args, wgs, lds, s, ev);
    }
  } else {
    if (xdt == kF16) {
      if (args.M > 4) launch_ni<kQ8_0, kF16, 2>(waves, c, args, wgs, lds, s, ev);
      else launch_ni<kQ8_0, kF16, 1>(waves, c, args, wgs, lds, s, ev);
    } else {
      if (args.M > 4) launch_ni<kQ8_0, kBF16, 2>(waves, c, args, wgs, lds, s, ev);
      else launch_ni<kQ8_0, kBF16, 1>(waves, c, args, wgs, lds, s, ev);
    }
  }
  return hipGetLastError();
}

}  // namespace q4q8
