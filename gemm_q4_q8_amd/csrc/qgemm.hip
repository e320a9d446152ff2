// Prefill GEMM over repacked Q4_0 / Q8_0 weights: Y[M, N] = X[M, K] W[N, K]^T.
//
// The pages run prefill on tiled GEMM kernels on matrix intrinsics, one per
// quantisation format, dequantising in the inner loop ("BaseRT:
// Best-in-Class LLM Inference on Apple Silicon via Native Metal", technical
// summary, "Methodologie", prefill optimisation and kernel specialisation;
// the M5 follow-up review, "Method", routes the prefill GEMM to the matrix
// units).  On gfx950:
//   * matrix cores: v_mfma_f32_16x16x32_f16, fp32 accumulation.  Weights are
//     unpacked in registers and scaled to fp16 (one rounding, relative error
//     <= 2^-11); activations are converted to fp16 (exact for
//     2^-14 <= |x| < 65520).  Applying the block scale in fp32 after each
//     MFMA would cost one VALU FMA per output per block -- as much issue time
//     as the MFMAs themselves -- so the scale goes into the operand;
//   * a workgroup computes a BM x BN tile with 4 waves side by side along N:
//     each wave owns NT 16-row weight tiles, loads their records straight
//     from HBM into registers (buffer loads, one chunk ahead) and unpacks them
//     once per chunk for all BM rows; the BM x 128 activation chunk goes
//     through double-buffered LDS, shared by the 4 waves;
//   * workgroup ids are remapped so each XCD (ids i % 8) works through a
//     contiguous range of weight slabs for all M tiles: a slab is read from
//     HBM once per XCD and then served by that XCD's L2.
#include "q4q8_dev.h"
#include "q4q8_internal.h"

#include <type_traits>

namespace q4q8 {

constexpr int kGemmBufFlags = 0x00020000;
constexpr int kXPad = 8;                        // halfs of padding per LDS row
constexpr int kXRow = kChunkK + kXPad;          // LDS row stride (halfs)
constexpr uint32_t kOOB = 0x80000000u;          // buffer offset past any range: reads 0

// bf16 pair -> fp16 pair (exact for fp16-normal magnitudes; RTZ otherwise).
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t u) {
  const float lo = __builtin_bit_cast(float, u << 16);
  const float hi = __builtin_bit_cast(float, u & 0xFFFF0000u);
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
}

template <int XDT>
__device__ __forceinline__ u32x4_t to_f16(const u32x4_t v) {
  if constexpr (XDT == kBF16) {
    const uint32_t v0 = v[0], v1 = v[1], v2 = v[2], v3 = v[3];   // scalars first (see scale_f16x8)
    u32x4_t o;
    o[0] = bf16x2_to_f16x2(v0);
    o[1] = bf16x2_to_f16x2(v1);
    o[2] = bf16x2_to_f16x2(v2);
    o[3] = bf16x2_to_f16x2(v3);
    return o;
  }
  return v;
}

template <int YDT>
__device__ __forceinline__ void store_y(void* Y, int64_t idx, float v) {
  if constexpr (YDT == kF32) {
    ((float*)Y)[idx] = v;
  } else if constexpr (YDT == kF16) {
    ((_Float16*)Y)[idx] = (_Float16)v;
  } else {
    ((__bf16*)Y)[idx] = (__bf16)v;
  }
}

// MT m-tiles of 16 rows (BM = 16 MT), NT weight tiles per wave (BN = 64 NT).
template <int FMT, int XDT, int YDT, int MT, int NT>
__global__ __launch_bounds__(256) void qgemm_kernel(const uint8_t* __restrict__ W, int N, int K,
                                                    const uint16_t* __restrict__ X, int64_t ldx, int M,
                                                    void* __restrict__ Y, int64_t ldy, int m_tiles, int n_tiles) {
  constexpr int BM = 16 * MT;
  constexpr int REC = Fmt<FMT>::kRecBytes;
  constexpr int CODE = Fmt<FMT>::kCodeBytes;
  constexpr int NV = FMT == kQ4_0 ? 1 : 2;
  constexpr int XPIECES = BM * (kChunkK / 8) / 256;   // 16-byte X pieces per thread per chunk
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][BM * kXRow];

  // XCD-aware tile order.
  const int nwg = m_tiles * n_tiles;
  int wg = blockIdx.x;
  if (nwg % 8 == 0) wg = (wg % 8) * (nwg / 8) + wg / 8;
  const int nt_id = wg / m_tiles, mt_id = wg % m_tiles;
  const int m0 = mt_id * BM;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  const int nchunks = (K + kChunkK - 1) / kChunkK;
  const int tiles = (N + kTileRows - 1) / kTileRows;

  // This wave's weight tiles: t0 .. t0 + NT - 1 (past the last tile: zero).
  const int t0 = (nt_id * 4 + wave) * NT;
  const int tv = tiles - t0 < NT ? (tiles - t0 > 0 ? tiles - t0 : 0) : NT;
  const uint8_t* wbase = W + (int64_t)(t0 < tiles ? t0 : 0) * nchunks * REC;
  const __amdgpu_buffer_rsrc_t wres =
      __builtin_amdgcn_make_buffer_rsrc((void*)wbase, (short)0, tv * nchunks * REC, kGemmBufFlags);
  // Activations: rows m0.. of X; rows >= M and columns >= K read as zero.
  const __amdgpu_buffer_rsrc_t xres = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(X + (int64_t)m0 * ldx), (short)0, (int)((int64_t)(M - m0 < BM ? M - m0 : BM) * ldx * 2),
      kGemmBufFlags);

  struct WStage {
    u32x4_t codes[NT][NV];
    u32x2_t sc[NT];
  };
  auto load_w = [&](WStage& s, int c) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int off = (t * nchunks + c) * REC;
#pragma unroll
      for (int v = 0; v < NV; ++v)
        s.codes[t][v] = __builtin_amdgcn_raw_buffer_load_b128(wres, off + v * 1024 + lane * 16, 0, 0);
      s.sc[t] = __builtin_amdgcn_raw_buffer_load_b64(wres, off + CODE + r * 8, 0, 0);
    }
  };
  // X piece p of this thread: row pr = idx / 16, 8 columns at pc = (idx % 16) * 8.
  auto load_x = [&](u32x4_t (&xv)[XPIECES], int c) {
#pragma unroll
    for (int p = 0; p < XPIECES; ++p) {
      const int idx = tid + p * 256;
      const int pr = idx >> 4, pc = (idx & 15) * 8;
      const int k = c * kChunkK + pc;
      const uint32_t off = k < K ? (uint32_t)((pr * ldx + k) * 2) : kOOB;
      xv[p] = __builtin_amdgcn_raw_buffer_load_b128(xres, off, 0, 0);
    }
  };
  auto store_x = [&](const u32x4_t (&xv)[XPIECES], int buf) {
#pragma unroll
    for (int p = 0; p < XPIECES; ++p) {
      const int idx = tid + p * 256;
      const int pr = idx >> 4, pc = (idx & 15) * 8;
      *(u32x4_t*)(&xs[buf][pr * kXRow + pc]) = to_f16<XDT>(xv[p]);
    }
  };

  float4_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[i][t] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  WStage ws[2];
  u32x4_t xv[XPIECES];
  load_x(xv, 0);
  load_w(ws[0], 0);
  store_x(xv, 0);
  __syncthreads();

  auto compute = [&](const WStage& s, int buf) {
#pragma unroll
    for (int j = 0; j < kBlocksPerChunk; ++j) {
      half8_t b[NT];
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x4_t q = deq_block<FMT, kF16>(s.codes[t], j);
        const uint32_t sbits = (j & 1) ? (s.sc[t][j >> 1] >> 16) : (s.sc[t][j >> 1] & 0xFFFFu);
        const _Float16 sh = __builtin_bit_cast(_Float16, (uint16_t)sbits);
        const half2_t s2 = {sh, sh};
        b[t] = __builtin_bit_cast(half8_t, scale_f16x8(q, s2));
      }
#pragma unroll
      for (int i = 0; i < MT; ++i) {
        const half8_t a = *(const half8_t*)(&xs[buf][(i * 16 + r) * kXRow + j * 32 + 8 * g]);
#pragma unroll
        for (int t = 0; t < NT; ++t) acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[t], acc[i][t], 0, 0, 0);
      }
    }
  };

  // One chunk: prefetch chunk c + 1 (X into registers, W into the other
  // register stage), multiply chunk c, then publish X(c + 1) in the other LDS
  // buffer.  Stage / buffer indices are compile-time (the loop is unrolled by
  // two) so the register stages never go to scratch.
  auto step = [&](int c, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const bool more = c + 1 < nchunks;
    if (more) {
      load_x(xv, c + 1);
      load_w(ws[buf ^ 1], c + 1);
    }
    compute(ws[buf], buf);
    if (more) store_x(xv, buf ^ 1);
    __syncthreads();
  };
  for (int c = 0; c < nchunks; c += 2) {
    step(c, std::integral_constant<int, 0>{});
    if (c + 1 < nchunks) step(c + 1, std::integral_constant<int, 1>{});
  }

  // Lane (r, g), register e of tile (i, t): Y[m0 + 16 i + 4 g + e][16 (t0 + t) + r].
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = (t0 + t) * kTileRows + r;
    if (n >= N) continue;
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + i * 16 + 4 * g + e;
        if (m < M) store_y<YDT>(Y, (int64_t)m * ldy + n, acc[i][t][e]);
      }
  }
}

template <int FMT, int XDT, int YDT, int MT, int NT>
static void launch_tile(const void* W, int64_t N, int64_t K, const void* X, int64_t ldx, int64_t M, void* Y,
                        int64_t ldy, hipStream_t s, const LaunchEvents& ev) {
  const int m_tiles = (int)((M + 16 * MT - 1) / (16 * MT));
  const int n_tiles = (int)((N + 64 * NT - 1) / (64 * NT));
  launch(qgemm_kernel<FMT, XDT, YDT, MT, NT>, dim3((unsigned)(m_tiles * n_tiles)), dim3(256), 0, s, ev,
         (const uint8_t*)W, (int)N, (int)K, (const uint16_t*)X, ldx, (int)M, Y, ldy, m_tiles, n_tiles);
}

// Tile shape: 128 rows x 4 waves x NT weight tiles; NT = 3 when 4 would
// leave CUs idle (e.g. M = 512, N = 12288: 256 workgroups instead of 192).
template <int FMT, int XDT, int YDT>
static void launch_shape(const void* W, int64_t N, int64_t K, const void* X, int64_t ldx, int64_t M, void* Y,
                         int64_t ldy, hipStream_t s, const LaunchEvents& ev) {
  const int64_t mt = (M + 127) / 128;
  const int64_t wg4 = mt * ((N + 255) / 256);
  const int64_t wg3 = mt * ((N + 191) / 192);
  if (M <= 64)
    launch_tile<FMT, XDT, YDT, 4, 4>(W, N, K, X, ldx, M, Y, ldy, s, ev);
  else if (wg4 < 256 && wg3 <= 256)
    launch_tile<FMT, XDT, YDT, 8, 3>(W, N, K, X, ldx, M, Y, ldy, s, ev);
  else
    launch_tile<FMT, XDT, YDT, 8, 4>(W, N, K, X, ldx, M, Y, ldy, s, ev);
}

template <int FMT, int XDT>
static void launch_ydt(int ydt, const void* W, int64_t N, int64_t K, const void* X, int64_t ldx, int64_t M, void* Y,
                       int64_t ldy, hipStream_t s, const LaunchEvents& ev) {
  if (ydt == kBF16) launch_shape<FMT, XDT, kBF16>(W, N, K, X, ldx, M, Y, ldy, s, ev);
  else if (ydt == kF16) launch_shape<FMT, XDT, kF16>(W, N, K, X, ldx, M, Y, ldy, s, ev);
  else launch_shape<FMT, XDT, kF32>(W, N, K, X, ldx, M, Y, ldy, s, ev);
}

hipError_t launch_qgemm(int fmt, int xdt, int ydt, const void* W, int64_t N, int64_t K, const void* X, int64_t ldx,
                        int64_t M, void* Y, int64_t ldy, hipStream_t s, const LaunchEvents& ev) {
  if (fmt == kQ4_0) {
    if (xdt == kBF16) launch_ydt<kQ4_0, kBF16>(ydt, W, N, K, X, ldx, M, Y, ldy, s, ev);
    else launch_ydt<kQ4_0, kF16>(ydt, W, N, K, X, ldx, M, Y, ldy, s, ev);
  } else {
    if (xdt == kBF16) launch_ydt<kQ8_0, kBF16>(ydt, W, N, K, X, ldx, M, Y, ldy, s, ev);
    else launch_ydt<kQ8_0, kF16>(ydt, W, N, K, X, ldx, M, Y, ldy, s, ev);
  }
  return hipGetLastError();
}

}  // namespace q4q8
