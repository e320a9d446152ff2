// Prefill GEMM over repacked Q4_0 / Q8_0 (or plain fp16) weights:
// Y[M, N] = X[M, K] W[N, K]^T.
//
// The pages run prefill on tiled GEMM kernels on matrix intrinsics, one per
// quantisation format, dequantising in the inner loop ("BaseRT:
// Best-in-Class LLM Inference on Apple Silicon via Native Metal", technical
// summary, "Methodologie", prefill optimisation and kernel specialisation;
// the M5 follow-up review, "Method", routes the prefill GEMM to the matrix
// units).  Here one workgroup computes a 128 x 192 block (64 x 64 for small
// M) with the tile engine of qgemm_core.h.  BF16 activations are converted
// once to fp16 by a small pre-pass into the caller's workspace (exact for
// 2^-14 <= |x| < 65520).  Workgroup ids are remapped so each XCD (ids
// i % 8) works through a contiguous range of weight slabs: a slab is read
// from HBM once per XCD and then served by that XCD's L2.
#include "q4q8_dev.h"
#include "q4q8_internal.h"
#include "qgemm_core.h"

// Pipeline depth per format: Q8_0 weight stages take 15 registers a lane
// each, so its ring is one stage shorter to stay within 256 registers.
#ifndef Q4Q8_GEMM_STAGES_Q4
#define Q4Q8_GEMM_STAGES_Q4 4
#endif
#ifndef Q4Q8_GEMM_STAGES_Q8
#define Q4Q8_GEMM_STAGES_Q8 3
#endif
#ifndef Q4Q8_GEMM_STAGES_F16
#define Q4Q8_GEMM_STAGES_F16 4
#endif

namespace q4q8 {

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

// MT m-tiles of 16 rows (BM = 16 MT), NT weight tiles per wave (BN = 64 NT),
// S pipeline stages.  X is fp16 [M, ldx].  TAIL: K is not a multiple of 128,
// so the last chunk's copies are masked per column.
template <int FMT, int YDT, int MT, int NT, int S, bool TAIL>
__global__ __launch_bounds__(512) void qgemm_kernel(const uint8_t* __restrict__ W, int N, int K,
                                                    const uint16_t* __restrict__ X, int64_t ldx, int M,
                                                    void* __restrict__ Y, int64_t ldy, int m_tiles, int n_tiles) {
  using C = TileCfg<FMT, MT, NT, 1, S>;
  __shared__ __attribute__((aligned(1024))) uint16_t xs[C::LDS_HALFS];

  // Tile order: when the column tiles split evenly over the 8 XCDs, XCD x
  // (workgroups i with i % 8 == x) takes column tiles [x n/8, (x+1) n/8),
  // column-fastest, so the workgroups resident on one XCD share a few
  // activation row tiles and that XCD's weight slabs through its L2.
  int nt_id, mt_id;
  if (n_tiles % 8 == 0) {
    const int per = n_tiles / 8, li = blockIdx.x / 8;
    nt_id = (blockIdx.x % 8) * per + li % per;
    mt_id = li / per;
  } else {
    nt_id = blockIdx.x / m_tiles;
    mt_id = blockIdx.x % m_tiles;
  }
  const int m0 = mt_id * C::BM;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nw = wave & 3;
  const int r = lane & 15, g = lane >> 4;
  const int nchunks = (K + kChunkK - 1) / kChunkK;
  const int tiles = (N + kTileRows - 1) / kTileRows;

  // This wave's weight tiles (past the last tile: zero).
  const int t0 = (nt_id * 4 + nw) * NT;
  const int tv = tiles - t0 < NT ? (tiles - t0 > 0 ? tiles - t0 : 0) : NT;
  const __amdgpu_buffer_rsrc_t wres[1] = {
      uniform_rsrc(W + (int64_t)(t0 < tiles ? t0 : 0) * nchunks * C::REC, tv * nchunks * C::REC)};
  // Activation rows m0 .. m0 + BM - 1; rows >= M are out of range by their
  // lane offset alone.
  const __amdgpu_buffer_rsrc_t xres =
      uniform_rsrc(X + (int64_t)m0 * ldx, (int)((int64_t)(M - m0 < C::BM ? M - m0 : C::BM) * ldx * 2));
  uint32_t xv[C::XLOADS];
#pragma unroll
  for (int p = 0; p < C::XLOADS; ++p) {
    int row, cg;
    x_slot(p, tid, row, cg);
    xv[p] = (uint32_t)((row * ldx + cg * 8) * 2);
  }

  float4_t acc[MT * NT];
  tile_mainloop<FMT, MT, NT, 1, S, TAIL>(wres, tv, K, nchunks, xres, xv, xs, acc);
  float4_t kept[(MT / 2) * NT];
  khalf_reduce<MT, NT, 1>(acc, (float4_t*)xs, kept);

  // Lane (r, g), register e of kept tile (i, t):
  // Y[m0 + 16 (kw MT/2 + i) + 4 g + e][16 (t0 + t) + r].
  const int mk = m0 + (wave >> 2) * (MT / 2) * 16 + 4 * g;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = (t0 + t) * kTileRows + r;
    if (n < N) {
#pragma unroll
      for (int i = 0; i < MT / 2; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = mk + i * 16 + e;
          if (m < M) store_y<YDT>(Y, (int64_t)m * ldy + n, kept[i * NT + t][e]);
        }
    }
  }
}

// bf16 -> fp16, 8 values per thread (exact for fp16-normal magnitudes;
// round-toward-zero otherwise).  Block (x, y) covers row y, groups of 8
// columns 256 x .. 256 x + 255; row y of dst holds cols8p groups: the
// converted cols8 groups, then zeros.
__global__ __launch_bounds__(256) void bf16_to_f16_kernel(const uint16_t* __restrict__ src, int64_t lds_,
                                                          uint16_t* __restrict__ dst, int64_t ldd, int cols8,
                                                          int cols8p) {
  const int c8 = blockIdx.x * 256 + threadIdx.x;
  if (c8 >= cols8p) return;
  const int64_t row = blockIdx.y;
  u32x4_t o = {0u, 0u, 0u, 0u};
  if (c8 < cols8) {
    const u32x4_t v = *(const u32x4_t*)(src + row * lds_ + c8 * 8);
    const uint32_t v0 = v[0], v1 = v[1], v2 = v[2], v3 = v[3];
    o[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__builtin_bit_cast(float, v0 << 16),
                                                                    __builtin_bit_cast(float, v0 & 0xFFFF0000u)));
    o[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__builtin_bit_cast(float, v1 << 16),
                                                                    __builtin_bit_cast(float, v1 & 0xFFFF0000u)));
    o[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__builtin_bit_cast(float, v2 << 16),
                                                                    __builtin_bit_cast(float, v2 & 0xFFFF0000u)));
    o[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(__builtin_bit_cast(float, v3 << 16),
                                                                    __builtin_bit_cast(float, v3 & 0xFFFF0000u)));
  }
  *(u32x4_t*)(dst + row * ldd + c8 * 8) = o;
}

// rows <= 2^30 (grid y is 32-bit on gfx950; larger M is rejected earlier).
hipError_t launch_bf16_to_f16(const void* src, int64_t lds_, void* dst, int64_t ldd, int64_t rows, int64_t cols,
                              int64_t colsp, hipStream_t s, const LaunchEvents& ev) {
  const int cols8 = (int)(cols / 8), cols8p = (int)(colsp / 8);
  launch(bf16_to_f16_kernel, dim3((unsigned)((cols8p + 255) / 256), (unsigned)rows), dim3(256), 0, s, ev,
         (const uint16_t*)src, lds_, (uint16_t*)dst, ldd, cols8, cols8p);
  return hipGetLastError();
}

template <int FMT, int YDT, int MT, int NT, int S>
static void launch_tile(const void* W, int64_t N, int64_t K, const void* X, int64_t ldx, int64_t M, void* Y,
                        int64_t ldy, hipStream_t s, const LaunchEvents& ev) {
  const int m_tiles = (int)((M + 16 * MT - 1) / (16 * MT));
  const int n_tiles = (int)((N + 64 * NT - 1) / (64 * NT));
  if (K % kChunkK)
    launch(qgemm_kernel<FMT, YDT, MT, NT, S, true>, dim3((unsigned)(m_tiles * n_tiles)), dim3(512), 0, s, ev,
           (const uint8_t*)W, (int)N, (int)K, (const uint16_t*)X, ldx, (int)M, Y, ldy, m_tiles, n_tiles);
  else
    launch(qgemm_kernel<FMT, YDT, MT, NT, S, false>, dim3((unsigned)(m_tiles * n_tiles)), dim3(512), 0, s, ev,
           (const uint8_t*)W, (int)N, (int)K, (const uint16_t*)X, ldx, (int)M, Y, ldy, m_tiles, n_tiles);
}

// Tile shape: 128 rows x 192 columns (3 weight tiles per wave); 64 x 64 for
// small M, where more workgroups matter more than operand reuse.
template <int FMT, int YDT>
static void launch_shape(const void* W, int64_t N, int64_t K, const void* X, int64_t ldx, int64_t M, void* Y,
                         int64_t ldy, hipStream_t s, const LaunchEvents& ev) {
  constexpr int S = FMT == kQ4_0 ? Q4Q8_GEMM_STAGES_Q4 : FMT == kQ8_0 ? Q4Q8_GEMM_STAGES_Q8 : Q4Q8_GEMM_STAGES_F16;
  if (M <= 64)
    launch_tile<FMT, YDT, 4, 1, S>(W, N, K, X, ldx, M, Y, ldy, s, ev);
  else
    launch_tile<FMT, YDT, 8, 3, S>(W, N, K, X, ldx, M, Y, ldy, s, ev);
}

// BF16 activations: one fp16 copy [M, Kp], Kp = K rounded up to 128 and the
// extra columns zero (the weights there are zero too), so the GEMM never
// masks columns.
static int64_t padded_k(int64_t K) { return (K + kChunkK - 1) / kChunkK * kChunkK; }

size_t qgemm_workspace_bytes(int xdt, int64_t M, int64_t K) {
  if (xdt != kBF16) return 0;
  return (size_t)(((M * padded_k(K) * 2) + 255) / 256 * 256);
}

hipError_t launch_qgemm(int fmt, int xdt, int ydt, const void* W, int64_t N, int64_t K, const void* X, int64_t ldx,
                        int64_t M, void* Y, int64_t ldy, void* ws, hipStream_t s, const LaunchEvents& ev) {
  const void* Xh = X;
  int64_t ldh = ldx;
  LaunchEvents gev = ev;
  if (xdt == kBF16) {   // the timed span covers both kernels
    LaunchEvents pev;
    pev.start = ev.start;
    gev.start = nullptr;
    const int64_t Kp = padded_k(K);
    const hipError_t e = launch_bf16_to_f16(X, ldx, ws, Kp, M, K, Kp, s, pev);
    if (e != hipSuccess) return e;
    Xh = ws;
    ldh = Kp;
    K = Kp;
  }
  if (fmt == kQ4_0) {
    if (ydt == kBF16) launch_shape<kQ4_0, kBF16>(W, N, K, Xh, ldh, M, Y, ldy, s, gev);
    else if (ydt == kF16) launch_shape<kQ4_0, kF16>(W, N, K, Xh, ldh, M, Y, ldy, s, gev);
    else launch_shape<kQ4_0, kF32>(W, N, K, Xh, ldh, M, Y, ldy, s, gev);
  } else if (fmt == kQ8_0) {
    if (ydt == kBF16) launch_shape<kQ8_0, kBF16>(W, N, K, Xh, ldh, M, Y, ldy, s, gev);
    else if (ydt == kF16) launch_shape<kQ8_0, kF16>(W, N, K, Xh, ldh, M, Y, ldy, s, gev);
    else launch_shape<kQ8_0, kF32>(W, N, K, Xh, ldh, M, Y, ldy, s, gev);
  } else {
    if (ydt == kBF16) launch_shape<kFP16W, kBF16>(W, N, K, Xh, ldh, M, Y, ldy, s, gev);
    else if (ydt == kF16) launch_shape<kFP16W, kF16>(W, N, K, Xh, ldh, M, Y, ldy, s, gev);
    else launch_shape<kFP16W, kF32>(W, N, K, Xh, ldh, M, Y, ldy, s, gev);
  }
  return hipGetLastError();
}

}  // namespace q4q8
