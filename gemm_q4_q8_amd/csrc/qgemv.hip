// Decode GEMV over repacked Q4_0 / Q8_0 weights, M = 1..8 activation rows.
//
// The pages ("BaseRT: Best-in-Class LLM Inference on Apple Silicon via Native
// Metal", gist.science technical summary, "Methodologie", kernel
// specialisation) run decode on a GEMV per quantisation format that
// dequantises inside its inner loop.  Here the inner product of each 32-weight
// block is done by one v_mfma_f32_16x16x32 instruction instead of lane FMAs
// plus a cross-lane reduction:
//   * a wavefront owns a tile of 16 weight rows; the waves of a workgroup
//     split K (chunk c goes to wave c % WAVES) and reduce through LDS in a
//     fixed order at the end (split-K without atomics or workspace);
//   * per chunk a lane loads 16 (Q4_0) or 32 (Q8_0) contiguous bytes of codes
//     -- the wave reads 1 or 2 KB contiguous -- plus its row's 4 scales, and
//     unpacks the codes in registers straight into the MFMA B operand;
//   * the A operand holds the activation rows: row m sits in A row
//     4 (m % 4) + m / 4, so the MFMA result for every m < 4 lands in the
//     first accumulator register of each lane (m < 8: the first two) and the
//     fp32 block scale costs one FMA per lane per block for M <= 4;
//   * codes are exact in the operand type (fp16 or bf16) and the block scale
//     is applied in fp32, so every product is exact and only the fp32
//     accumulation rounds.
#include "q4q8_dev.h"
#include "q4q8_internal.h"

#include <stdlib.h>

namespace q4q8 {

template <int FMT, int XDT, int NI, int WAVES>
__global__ __launch_bounds__(WAVES * 64) void qgemv_kernel(const GemvArgs args) {
  constexpr int REC = Fmt<FMT>::kRecBytes;
  constexpr int CODE = Fmt<FMT>::kCodeBytes;
  constexpr int NV = FMT == kQ4_0 ? 1 : 2;
  typedef typename Op<XDT>::vec vec;

  // Which problem of the group this workgroup serves (uniform selects).
  const int bid = blockIdx.x;
  const uint8_t* Wp = args.p[0].W;
  const uint16_t* xp = args.p[0].x;
  float* yp = args.p[0].y;
  int64_t ldx = args.p[0].ldx, ldy = args.p[0].ldy;
  int N = args.p[0].N, K = args.p[0].K, tile0 = args.p[0].tile0;
#pragma unroll
  for (int i = 1; i < kMaxGroup; ++i) {
    if (i < args.count && bid >= args.p[i].tile0) {
      Wp = args.p[i].W; xp = args.p[i].x; yp = args.p[i].y;
      ldx = args.p[i].ldx; ldy = args.p[i].ldy;
      N = args.p[i].N; K = args.p[i].K; tile0 = args.p[i].tile0;
    }
  }
  const int tile = bid - tile0;
  const int nchunks = (K + kChunkK - 1) / kChunkK;
  const int nblocks = K / 32;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int m = 4 * (r & 3) + (r >> 2);          // activation row fed by this lane
  const bool mvalid = m < args.M;
  // Lanes whose A row has no activation row (m >= M) read row 0: MFMA rows
  // are independent and those result rows are never stored.  Blocks past K
  // (padding, scale 0) read the last real block so every operand is finite.
  const uint16_t* __restrict__ xrow = xp + (mvalid ? (int64_t)m * ldx : 0) + 8 * g;
  const uint8_t* __restrict__ wt = Wp + (int64_t)tile * nchunks * REC;

  float acc[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) acc[i] = 0.0f;

  struct Stage {
    u32x4_t codes[NV];
    u32x2_t sc;
    vec a[kBlocksPerChunk];
  };
  auto load = [&](Stage& st, int c) {
    c = c < nchunks ? c : nchunks - 1;
    const uint8_t* __restrict__ rec = wt + (int64_t)c * REC;
#pragma unroll
    for (int v = 0; v < NV; ++v) st.codes[v] = *(const u32x4_t*)(rec + v * 1024 + lane * 16);
    st.sc = *(const u32x2_t*)(rec + CODE + r * 8);
#pragma unroll
    for (int j = 0; j < kBlocksPerChunk; ++j) {
      int blk = c * kBlocksPerChunk + j;
      blk = blk < nblocks ? blk : nblocks - 1;
      st.a[j] = *(const vec*)(xrow + blk * 32);
    }
  };
  auto compute = [&](const Stage& st) {
    // All four block products first (independent MFMAs), then the scales.
    float4_t d[kBlocksPerChunk];
#pragma unroll
    for (int j = 0; j < kBlocksPerChunk; ++j) {
      const u32x4_t b = deq_block<FMT, XDT>(st.codes, j);
      d[j] = Op<XDT>::mfma(st.a[j], __builtin_bit_cast(vec, b), float4_t{0.0f, 0.0f, 0.0f, 0.0f});
    }
#pragma unroll
    for (int j = 0; j < kBlocksPerChunk; ++j) {
      const uint32_t sbits = (j & 1) ? (st.sc[j >> 1] >> 16) : (st.sc[j >> 1] & 0xFFFFu);
      const float s = half_bits_to_float(sbits);
#pragma unroll
      for (int i = 0; i < NI; ++i) acc[i] = __builtin_fmaf(s, d[j][i], acc[i]);
    }
  };

  // Two-stage pipeline: the next chunk of this wave is in flight while the
  // current one is unpacked and multiplied.
  Stage s0, s1;
  int c = wave;
  if (c < nchunks) {
    load(s0, c);
    // The scheduling barriers keep the compiler from sinking the prefetch
    // next to its use, which would serialise memory latency per chunk.
    while (true) {
      load(s1, c + WAVES);
      __builtin_amdgcn_sched_barrier(0);
      compute(s0);
      c += WAVES;
      if (c >= nchunks) break;
      load(s0, c + WAVES);
      __builtin_amdgcn_sched_barrier(0);
      compute(s1);
      c += WAVES;
      if (c >= nchunks) break;
    }
  }

  if constexpr (WAVES > 1) {
    __shared__ float red[WAVES][NI][64];
#pragma unroll
    for (int i = 0; i < NI; ++i) red[wave][i][lane] = acc[i];
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float v = red[0][i][lane];
#pragma unroll
      for (int w = 1; w < WAVES; ++w) v += red[w][i][lane];
      acc[i] = v;
    }
  }
  // Lane (r, g), register i holds y[m = 4 i + g][n = 16 tile + r].
  const int n = tile * kTileRows + r;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int mo = 4 * i + g;
    if (mo < args.M && n < N) yp[(int64_t)mo * ldy + n] = acc[i];
  }
}

template <int FMT, int XDT, int NI>
static void launch_waves(int waves, const GemvArgs& args, hipStream_t s) {
  const dim3 grid((unsigned)args.total_tiles);
  switch (waves) {
    case 4: qgemv_kernel<FMT, XDT, NI, 4><<<grid, dim3(256), 0, s>>>(args); break;
    case 8: qgemv_kernel<FMT, XDT, NI, 8><<<grid, dim3(512), 0, s>>>(args); break;
    default: qgemv_kernel<FMT, XDT, NI, 16><<<grid, dim3(1024), 0, s>>>(args); break;
  }
}

template <int FMT, int XDT>
static void launch_ni(int waves, const GemvArgs& args, hipStream_t s) {
  if (args.M > 4)
    launch_waves<FMT, XDT, 2>(waves, args, s);
  else
    launch_waves<FMT, XDT, 1>(waves, args, s);
}

// Waves per workgroup: enough workgroups x waves to fill 256 CUs with a few
// waves each, but at least two chunks per wave.
static int pick_waves(int tiles, int max_chunks) {
  int waves = 4;
  while (waves < 16 && tiles * waves < 4096 && max_chunks >= 4 * waves) waves *= 2;
  return waves;
}

// Q4Q8_GEMV_WAVES=4|8|16 overrides the choice (tuning experiments only).
static int waves_override() {
  static const int v = [] {
    const char* e = getenv("Q4Q8_GEMV_WAVES");
    const int w = e ? atoi(e) : 0;
    return (w == 4 || w == 8 || w == 16) ? w : 0;
  }();
  return v;
}

hipError_t launch_qgemv(int fmt, int xdt, const GemvArgs& args, int max_chunks, hipStream_t s) {
  const int waves = waves_override() ? waves_override() : pick_waves(args.total_tiles, max_chunks);
  if (fmt == kQ4_0) {
    if (xdt == kF16) launch_ni<kQ4_0, kF16>(waves, args, s);
    else launch_ni<kQ4_0, kBF16>(waves, args, s);
  } else {
    if (xdt == kF16) launch_ni<kQ8_0, kF16>(waves, args, s);
    else launch_ni<kQ8_0, kBF16>(waves, args, s);
  }
  return hipGetLastError();
}

}  // namespace q4q8
