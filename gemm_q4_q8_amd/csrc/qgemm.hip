// Prefill GEMM over repacked Q4_0 / Q8_0 (or plain fp16) weights:
// Y[M, N] = X[M, K] W[N, K]^T.
//
// The pages run prefill on tiled GEMM kernels on matrix intrinsics, one per
// quantisation format, dequantising in the inner loop ("BaseRT:
// Best-in-Class LLM Inference on Apple Silicon via Native Metal", technical
// summary, "Methodologie", prefill optimisation and kernel specialisation;
// the M5 follow-up review, "Method", routes the prefill GEMM to the matrix
// units).  Here one workgroup computes a 128 x 192 block (narrower blocks
// when M is too small to give every CU one) with the tile engine of
// qgemm_core.h.  BF16 activations are converted
// once to fp16 by a small pre-pass into the caller's workspace, each row
// scaled by a power of two so its largest magnitude lands in [4, 8); the
// epilogue multiplies the row's results back.  Workgroup ids are remapped so each XCD (ids
// i % 8) works through a contiguous range of weight slabs: a slab is read
// from HBM once per XCD and then served by that XCD's L2.
#include "q4q8_dev.h"
#include "q4q8_internal.h"
#include "qgemm_core.h"

// Pipeline depth per format.  Q8_0 weight stages take 15 registers a lane
// each, so its ring is one stage shorter to stay within 256 registers; Q4_0
// with two or three weight tiles a wave measured 1.5-2 % faster with 3
// stages than with 4 (MI355X, K 4096, N 12288: M 256 37.2 -> 36.4 us, M 512
// 56.2 -> 55.5 us, M 2048 201.9 -> 198.4 us a call).
#ifndef Q4Q8_GEMM_STAGES_Q4
#define Q4Q8_GEMM_STAGES_Q4 3
#endif
#ifndef Q4Q8_GEMM_STAGES_Q8
#define Q4Q8_GEMM_STAGES_Q8 3
#endif
#ifndef Q4Q8_GEMM_STAGES_F16
#define Q4Q8_GEMM_STAGES_F16 4
#endif
// The wide tile: 16 MT rows x 64 NT columns.
#ifndef Q4Q8_GEMM_WIDE_MT
#define Q4Q8_GEMM_WIDE_MT 8
#endif
#ifndef Q4Q8_GEMM_WIDE_NT
#define Q4Q8_GEMM_WIDE_NT 3
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
// so the last chunk's copies are masked per column.  rexp (nullable): row m
// of X holds the activations times 2^-rexp[m]; results are scaled back.
template <int FMT, int YDT, int MT, int NT, int S, bool TAIL>
__global__ __launch_bounds__(512) void qgemm_kernel(const uint8_t* __restrict__ W, int N, int K,
                                                    const uint16_t* __restrict__ X, int64_t ldx, int M,
                                                    const int32_t* __restrict__ rexp, void* __restrict__ Y,
                                                    int64_t ldy, int m_tiles, int n_tiles) {
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
  int ex[MT / 2][4];
#pragma unroll
  for (int i = 0; i < MT / 2; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = mk + i * 16 + e;
      ex[i][e] = (rexp && m < M) ? rexp[m] : 0;
    }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    const int n = (t0 + t) * kTileRows + r;
    if (n < N) {
#pragma unroll
      for (int i = 0; i < MT / 2; ++i)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int m = mk + i * 16 + e;
          if (m < M) store_y<YDT>(Y, (int64_t)m * ldy + n, __builtin_ldexpf(kept[i * NT + t][e], ex[i][e]));
        }
    }
  }
}

// Row scaling to fp16.  Row m of src (bf16 or fp16, row stride lds_) is
// written to dst (fp16, row stride ldd) as x * 2^-e[m], columns cols ..
// colsp - 1 zero, with e[m] = ilogb(max_k |x[m, k]|) - 2, so the row's
// largest magnitude lands in [4, 8) (e = 0 for a zero row or one holding
// inf / NaN).  A power of two is exact both ways: every value of the row
// within 2^20 of its largest magnitude converts exactly (bf16 has 8
// significant bits, fp16 keeps them down to 2^-17), the rest rounds to
// nearest even with an absolute error below 2^-25 of the scaled row, and the
// consumer multiplies its fp32 results by 2^e[m].  One workgroup per row;
// rows of up to kRowRegs x 2048 values stay in registers between the max
// and the conversion, longer ones are read twice (the second time from L2).
constexpr int kRowRegs = 4;

template <int SRC>
__global__ __launch_bounds__(256) void rowscale_f16_kernel(const uint16_t* __restrict__ src, int64_t lds_,
                                                           uint16_t* __restrict__ dst, int64_t ldd, int cols8,
                                                           int cols8p, int32_t* __restrict__ rexp) {
  const int64_t row = blockIdx.x;
  const int tid = threadIdx.x;
  const uint16_t* s = src + row * lds_;
  const bool in_regs = cols8 <= kRowRegs * 256;   // uniform
  u32x4_t v[kRowRegs];
  uint32_t m = 0;
  if (in_regs) {
#pragma unroll
    for (int u = 0; u < kRowRegs; ++u) {
      const int c8 = tid + u * 256;
      v[u] = c8 < cols8 ? *(const u32x4_t*)(s + c8 * 8) : u32x4_t{0u, 0u, 0u, 0u};
      m = max(m, max_mag_bits8(v[u]));
    }
  } else {
    for (int c8 = tid; c8 < cols8; c8 += 256) m = max(m, max_mag_bits8(*(const u32x4_t*)(s + c8 * 8)));
  }
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, off));
  __shared__ uint32_t wmax[4];
  if ((tid & 63) == 0) wmax[tid >> 6] = m;
  __syncthreads();
  m = max(max(wmax[0], wmax[1]), max(wmax[2], wmax[3]));
  const int e = row_exponent<SRC>(m);
  if (tid == 0) rexp[row] = e;
  if (in_regs) {
#pragma unroll
    for (int u = 0; u < kRowRegs; ++u) {
      const int c8 = tid + u * 256;
      if (c8 < cols8p)
        *(u32x4_t*)(dst + row * ldd + c8 * 8) = c8 < cols8 ? f16x8_scaled<SRC>(v[u], -e) : u32x4_t{0u, 0u, 0u, 0u};
    }
    for (int c8 = tid + kRowRegs * 256; c8 < cols8p; c8 += 256) *(u32x4_t*)(dst + row * ldd + c8 * 8) = u32x4_t{0u, 0u, 0u, 0u};
  } else {
    for (int c8 = tid; c8 < cols8p; c8 += 256) {
      const u32x4_t o = c8 < cols8 ? f16x8_scaled<SRC>(*(const u32x4_t*)(s + c8 * 8), -e) : u32x4_t{0u, 0u, 0u, 0u};
      *(u32x4_t*)(dst + row * ldd + c8 * 8) = o;
    }
  }
}

// rows <= 2^31 - 1 (grid x).
hipError_t launch_rowscale_f16(int src_dt, const void* src, int64_t lds_, void* dst, int64_t ldd, int64_t rows,
                               int64_t cols, int64_t colsp, int32_t* rexp, hipStream_t s, const LaunchEvents& ev) {
  const int cols8 = (int)(cols / 8), cols8p = (int)(colsp / 8);
  if (src_dt == kBF16)
    launch(rowscale_f16_kernel<kBF16>, dim3((unsigned)rows), dim3(256), 0, s, ev, (const uint16_t*)src, lds_,
           (uint16_t*)dst, ldd, cols8, cols8p, rexp);
  else
    launch(rowscale_f16_kernel<kF16>, dim3((unsigned)rows), dim3(256), 0, s, ev, (const uint16_t*)src, lds_,
           (uint16_t*)dst, ldd, cols8, cols8p, rexp);
  return hipGetLastError();
}

template <int FMT, int YDT, int MT, int NT, int S>
static void launch_tile(const void* W, int64_t N, int64_t K, const void* X, int64_t ldx, int64_t M,
                        const int32_t* rexp, void* Y, int64_t ldy, hipStream_t s, const LaunchEvents& ev) {
  const int m_tiles = (int)((M + 16 * MT - 1) / (16 * MT));
  const int n_tiles = (int)((N + 64 * NT - 1) / (64 * NT));
  if (K % kChunkK)
    launch(qgemm_kernel<FMT, YDT, MT, NT, S, true>, dim3((unsigned)(m_tiles * n_tiles)), dim3(512), 0, s, ev,
           (const uint8_t*)W, (int)N, (int)K, (const uint16_t*)X, ldx, (int)M, rexp, Y, ldy, m_tiles, n_tiles);
  else
    launch(qgemm_kernel<FMT, YDT, MT, NT, S, false>, dim3((unsigned)(m_tiles * n_tiles)), dim3(512), 0, s, ev,
           (const uint8_t*)W, (int)N, (int)K, (const uint16_t*)X, ldx, (int)M, rexp, Y, ldy, m_tiles, n_tiles);
}

// Tile shape: 128 rows x 192 columns (3 weight tiles per wave) when that
// gives every CU a workgroup; below that, narrower tiles trade operand reuse
// for workgroups (measured on MI355X, K 4096, N 12288, bf16 in and out, call
// time including the pre-pass: M = 128: 51 us with 128 x 192 tiles, 31 us
// with 128 x 64; M = 256: 54 us, 43 us with 128 x 128; 64 x 64 tiles and
// deeper rings (5-8 stages) measured the same or slower).
template <int FMT, int YDT>
static void launch_shape(const void* W, int64_t N, int64_t K, const void* X, int64_t ldx, int64_t M,
                         const int32_t* rexp, void* Y, int64_t ldy, hipStream_t s, const LaunchEvents& ev) {
  constexpr int S = FMT == kQ4_0 ? Q4Q8_GEMM_STAGES_Q4 : FMT == kQ8_0 ? Q4Q8_GEMM_STAGES_Q8 : Q4Q8_GEMM_STAGES_F16;
  // One weight tile a wave issues a third of the loads per chunk: a deeper
  // ring pays there (Q4_0, M 128: 27.0 us with 3 stages, 25.7 with 4).
  constexpr int S1 = FMT == kQ4_0 ? 4 : S;
  constexpr int WMT = Q4Q8_GEMM_WIDE_MT, WNT = Q4Q8_GEMM_WIDE_NT;
  const int64_t wide = (M + 16 * WMT - 1) / (16 * WMT) * ((N + 64 * WNT - 1) / (64 * WNT));
  if (wide >= 256)
    launch_tile<FMT, YDT, WMT, WNT, S>(W, N, K, X, ldx, M, rexp, Y, ldy, s, ev);
  else if (M > 128)
    launch_tile<FMT, YDT, 8, 2, S>(W, N, K, X, ldx, M, rexp, Y, ldy, s, ev);
  else if (M > 64)
    launch_tile<FMT, YDT, 8, 1, S1>(W, N, K, X, ldx, M, rexp, Y, ldy, s, ev);
  else
    launch_tile<FMT, YDT, 4, 1, S1>(W, N, K, X, ldx, M, rexp, Y, ldy, s, ev);
}

// BF16 activations: one row-scaled fp16 copy [M, Kp], Kp = K rounded up to
// 128 and the extra columns zero (the weights there are zero too), so the
// GEMM never masks columns, then the rows' exponents (int32 [M]).
static int64_t padded_k(int64_t K) { return (K + kChunkK - 1) / kChunkK * kChunkK; }
static size_t round256(size_t b) { return (b + 255) / 256 * 256; }

size_t qgemm_workspace_bytes(int xdt, int64_t M, int64_t K) {
  if (xdt != kBF16) return 0;
  return round256((size_t)(M * padded_k(K) * 2)) + round256((size_t)M * 4);
}

hipError_t launch_qgemm(int fmt, int xdt, int ydt, const void* W, int64_t N, int64_t K, const void* X, int64_t ldx,
                        int64_t M, void* Y, int64_t ldy, void* ws, hipStream_t s, const LaunchEvents& ev) {
  const void* Xh = X;
  int64_t ldh = ldx;
  const int32_t* rexp = nullptr;
  LaunchEvents gev = ev;
  if (xdt == kBF16) {   // the timed span covers both kernels
    LaunchEvents pev;
    pev.start = ev.start;
    gev.start = nullptr;
    const int64_t Kp = padded_k(K);
    int32_t* ex = (int32_t*)((uint8_t*)ws + round256((size_t)(M * Kp * 2)));
    const hipError_t e = launch_rowscale_f16(kBF16, X, ldx, ws, Kp, M, K, Kp, ex, s, pev);
    if (e != hipSuccess) return e;
    Xh = ws;
    ldh = Kp;
    K = Kp;
    rexp = ex;
  }
  if (fmt == kQ4_0) {
    if (ydt == kBF16) launch_shape<kQ4_0, kBF16>(W, N, K, Xh, ldh, M, rexp, Y, ldy, s, gev);
    else if (ydt == kF16) launch_shape<kQ4_0, kF16>(W, N, K, Xh, ldh, M, rexp, Y, ldy, s, gev);
    else launch_shape<kQ4_0, kF32>(W, N, K, Xh, ldh, M, rexp, Y, ldy, s, gev);
  } else if (fmt == kQ8_0) {
    if (ydt == kBF16) launch_shape<kQ8_0, kBF16>(W, N, K, Xh, ldh, M, rexp, Y, ldy, s, gev);
    else if (ydt == kF16) launch_shape<kQ8_0, kF16>(W, N, K, Xh, ldh, M, rexp, Y, ldy, s, gev);
    else launch_shape<kQ8_0, kF32>(W, N, K, Xh, ldh, M, rexp, Y, ldy, s, gev);
  } else {
    if (ydt == kBF16) launch_shape<kFP16W, kBF16>(W, N, K, Xh, ldh, M, rexp, Y, ldy, s, gev);
    else if (ydt == kF16) launch_shape<kFP16W, kF16>(W, N, K, Xh, ldh, M, rexp, Y, ldy, s, gev);
    else launch_shape<kFP16W, kF32>(W, N, K, Xh, ldh, M, rexp, Y, ldy, s, gev);
  }
  return hipGetLastError();
}

}  // namespace q4q8
