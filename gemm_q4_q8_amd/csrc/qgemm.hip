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
//     <= 2^-11).  Activations enter as fp16: bf16 inputs are converted once
//     by a small pre-pass into the caller's workspace (exact for
//     2^-14 <= |x| < 65520).  Applying the block scale in fp32 after each
//     MFMA would cost one VALU FMA per output per block -- as much issue time
//     as the MFMAs themselves -- so the scale goes into the operand;
//   * a workgroup computes a BM x BN tile with 4 waves side by side along N:
//     each wave owns NT 16-row weight tiles, streams their records straight
//     from HBM into a 3-stage register ring (buffer loads, two chunks ahead)
//     and unpacks them once per chunk for all BM rows;
//   * the BM x 128 fp16 activation chunk is copied global -> LDS by the
//     buffer loads' LDS path (no registers), into a 3-stage ring.  The copy
//     writes 1 KB per wave instruction contiguously, so rows cannot be
//     padded; instead lane L of the copy picks its source so that LDS slot
//     16 row + (cg ^ row % 16) holds 16-byte column group cg of that row, and
//     the A-fragment reads (16 rows x 4 column groups per instruction) hit
//     distinct banks;
//   * one barrier per chunk; copies past the end (chunk or row) read zero
//     into stages that are not consumed, so the wait counts stay uniform;
//   * workgroup ids are remapped so each XCD (ids i % 8) works through a
//     contiguous range of weight slabs for all M tiles: a slab is read from
//     HBM once per XCD and then served by that XCD's L2.
#include "q4q8_dev.h"
#include "q4q8_internal.h"

#include <type_traits>

// Pipeline depth per format: Q8_0 weight stages take 15 registers a lane
// each, so its ring is one stage shorter to stay within 256 registers.
#ifndef Q4Q8_GEMM_STAGES_Q4
#define Q4Q8_GEMM_STAGES_Q4 4
#endif
#ifndef Q4Q8_GEMM_STAGES_Q8
#define Q4Q8_GEMM_STAGES_Q8 3
#endif

namespace q4q8 {

constexpr uint32_t kOOB = 0x80000000u;          // buffer offset past any range: reads 0

// f(integral_constant<I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
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

// MT m-tiles of 16 rows (BM = 16 MT), NT weight tiles per wave (BN = 64 NT),
// S pipeline stages (S - 1 chunks in flight).  X is fp16 [M, ldx].  TAIL:
// K is not a multiple of 128, so the last chunk's copies are masked per
// column.  Eight waves: wave w covers weight tiles
// t0 .. t0 + NT - 1 with t0 = (4 n_tile + w % 4) NT, and blocks 2 (w / 4) and
// 2 (w / 4) + 1 of every chunk; the two K halves are summed at the end.
template <int FMT, int YDT, int MT, int NT, int S, bool TAIL>
__global__ __launch_bounds__(512) void qgemm_kernel(const uint8_t* __restrict__ W, int N, int K,
                                                    const uint16_t* __restrict__ X, int64_t ldx, int M,
                                                    void* __restrict__ Y, int64_t ldy, int m_tiles, int n_tiles) {
  static_assert(MT % 2 == 0 && NT <= 3, "the K-half reduction reuses the activation ring");
  constexpr int BM = 16 * MT;
  constexpr int REC = Fmt<FMT>::kRecBytes;
  constexpr int CODE = Fmt<FMT>::kCodeBytes;
  constexpr int XLOADS = MT / 2;                  // 16-byte copies per thread per chunk (BM * 16 / 512)
  constexpr int WLOADS = 2 * NT;                  // weight loads per wave per chunk
  constexpr int STAGE_HALFS = BM * kChunkK;
  static_assert(S >= 3 && 8 * (MT / 2) * NT * 1024 <= S * STAGE_HALFS * 2, "ring too small");
  __shared__ __attribute__((aligned(1024))) uint16_t xs[S * STAGE_HALFS];

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
  const int m0 = mt_id * BM;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nw = wave & 3, kw = wave >> 2;
  const int r = lane & 15, g = lane >> 4;
  const int nchunks = (K + kChunkK - 1) / kChunkK;
  const int tiles = (N + kTileRows - 1) / kTileRows;

  // This wave's weight tiles (past the last tile: zero).
  const int t0 = (nt_id * 4 + nw) * NT;
  const int tv = tiles - t0 < NT ? (tiles - t0 > 0 ? tiles - t0 : 0) : NT;
  const __amdgpu_buffer_rsrc_t wres = uniform_rsrc(W + (int64_t)(t0 < tiles ? t0 : 0) * nchunks * REC,
                                                   tv * nchunks * REC);
  // Activation rows m0 .. m0 + BM - 1; rows >= M read as zero.
  const __amdgpu_buffer_rsrc_t xres =
      uniform_rsrc(X + (int64_t)m0 * ldx, (int)((int64_t)(M - m0 < BM ? M - m0 : BM) * ldx * 2));

  // One chunk of this wave's weights: the codes and scales of blocks 2 kw and
  // 2 kw + 1.  Q4_0: dwords 2 kw, 2 kw + 1 of the lane's slot; Q8_0: the
  // lane's slot in half kw.  Per-lane offsets are loop-invariant; the chunk
  // enters through the scalar offset.  Tiles past the last read zero (their
  // lane offset is out of range); chunks past the last re-read the last one.
  typedef typename std::conditional<FMT == kQ4_0, u32x2_t, u32x4_t>::type CodeT;
  struct WStage {
    CodeT codes[NT];
    uint32_t sc[NT];
  };
  const uint32_t wv_code = FMT == kQ4_0 ? lane * 16 + kw * 8 : kw * 1024 + lane * 16;
  const uint32_t wv_scale = CODE + r * 8 + kw * 4;
  auto load_w = [&](WStage& s, int c) __attribute__((always_inline)) {
    const int cc = c < nchunks ? c : nchunks - 1;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int so = (t * nchunks + cc) * REC;
      const uint32_t vc = t < tv ? wv_code : kOOB, vs = t < tv ? wv_scale : kOOB;
      if constexpr (FMT == kQ4_0)
        s.codes[t] = __builtin_amdgcn_raw_buffer_load_b64(wres, vc, so, 0);
      else
        s.codes[t] = __builtin_amdgcn_raw_buffer_load_b128(wres, vc, so, 0);
      s.sc[t] = __builtin_amdgcn_raw_buffer_load_b32(wres, vs, so, 0);
    }
  };
  // Copy chunk c of the activation tile into LDS stage st.  Copy p of this
  // thread fills slot S = 512 p + tid: row S / 16, column group
  // (S % 16) ^ (row % 16).  Rows past M are out of range by their lane
  // offset alone.  Chunks past the last re-read the last one (into a stage
  // nobody reads), so every step issues the same loads; with TAIL, columns
  // past K are sent out of range.
  uint32_t xv[XLOADS];
#pragma unroll
  for (int p = 0; p < XLOADS; ++p) {
    const int slot = p * 512 + tid;
    const int row = slot >> 4;
    const int cg = (slot & 15) ^ (row & 15);
    xv[p] = (uint32_t)((row * ldx + cg * 8) * 2);
  }
  auto copy_x = [&](int c, int st) __attribute__((always_inline)) {
    const int cc = c < nchunks ? c : nchunks - 1;
#pragma unroll
    for (int p = 0; p < XLOADS; ++p) {
      uint32_t v = xv[p];
      if constexpr (TAIL) {
        const int slot = p * 512 + tid;
        const int cg = (slot & 15) ^ ((slot >> 4) & 15);
        v = cg * 8 < K - cc * kChunkK ? v : kOOB;
      }
      uint16_t* dst = xs + st * STAGE_HALFS + (p * 512 + wave * 64) * 8;   // wave-uniform
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xres, (__attribute__((address_space(3))) void*)dst, 16, v,
                                               cc * kChunkK * 2, 0, 0);
    }
  };

  float4_t acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[i][t] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // Unpacked, scaled B operands of block jj (0 or 1) of a weight stage.
  auto dequant = [&](const WStage& s, int jj, half8_t (&b)[NT]) __attribute__((always_inline)) {
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      u32x4_t q;
      if constexpr (FMT == kQ4_0) {
        const uint32_t w = s.codes[t][jj];
        q = deq_q4_f16(w);
      } else {
        const uint32_t d0 = s.codes[t][2 * jj], d1 = s.codes[t][2 * jj + 1];
        q = deq_q8<kF16>(d0, d1);
      }
      const uint32_t sbits = jj ? (s.sc[t] >> 16) : (s.sc[t] & 0xFFFFu);
      const _Float16 sh = __builtin_bit_cast(_Float16, (uint16_t)sbits);
      const half2_t s2 = {sh, sh};
      b[t] = __builtin_bit_cast(half8_t, scale_f16x8(q, s2));
    }
  };
  // MT x NT MFMAs of block jj of the chunk in LDS stage st.
  auto mma = [&](int st, int jj, const half8_t (&b)[NT]) __attribute__((always_inline)) {
    const uint16_t* xb = xs + st * STAGE_HALFS;
    const int j = 2 * kw + jj;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int row = i * 16 + r;
      const half8_t a = *(const half8_t*)(xb + (row * 16 + ((4 * j + g) ^ r)) * 8);
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[i][t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[t], acc[i][t], 0, 0, 0);
    }
  };

  // Prologue: chunks 0 .. S - 2 in flight, weights then activations per
  // chunk.  The scheduling barriers keep that order, so the wait count below
  // holds on every path into the loop head.
  WStage ws[S];
  static_for<0, S - 1>([&](auto ic) __attribute__((always_inline)) {
    constexpr int i = decltype(ic)::value;
    load_w(ws[i], i);
    copy_x(i, i);
    __builtin_amdgcn_sched_barrier(0);
  });
  // Block 0 of chunk 0 is unpacked ahead; afterwards each step unpacks its
  // block 1 during block 0's products and the next chunk's block 0 during
  // block 1's, so the VALU work runs under the matrix-core work.
  half8_t b0[NT], b1[NT];
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"((S - 2) * (XLOADS + WLOADS) + XLOADS) : "memory");
  dequant(ws[0], 0, b0);

  // Chunk c: wait until chunk c's copies and chunk c + 1's weights have
  // landed (chunk c + 1's copies and S - 3 later chunks may still be in
  // flight), barrier (all waves done with chunk c - 1, whose stage is
  // refilled next), start chunk c + S - 1, multiply chunk c.  Register stage
  // indices are compile-time (the loop is unrolled by S).
  auto step = [&](int c, auto stc) __attribute__((always_inline)) {
    constexpr int st = decltype(stc)::value;
    constexpr int nx = (st + S - 1) % S;
    // __syncthreads() would also wait for the later chunks' copies (its
    // fence covers every outstanding LDS write); this barrier waits only for
    // the loads named above, and its memory clobber keeps every load and
    // store on its side of it.
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"((S - 3) * (XLOADS + WLOADS) +
                                                                                      XLOADS)
                 : "memory");
    __builtin_amdgcn_sched_barrier(0);
    load_w(ws[nx], c + S - 1);
    copy_x(c + S - 1, nx);
    dequant(ws[st], 1, b1);
    mma(st, 0, b0);
    dequant(ws[(st + 1) % S], 0, b0);
    mma(st, 1, b1);
  };
  // Full groups of S steps, then the remainder, so every path into the loop
  // head carries the same outstanding loads.
  int c = 0;
  for (; c + S <= nchunks; c += S)
    static_for<0, S>([&](auto ic) __attribute__((always_inline)) { step(c + decltype(ic)::value, ic); });
  static_for<0, S - 1>([&](auto ic) __attribute__((always_inline)) {
    if (c + decltype(ic)::value < nchunks) step(c + decltype(ic)::value, ic);
  });
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // copies issued past the end land before the ring is reused
  __syncthreads();

  // Sum the two K halves through LDS.  Wave (nw, kw) keeps m-tiles
  // [kw MT/2, (kw+1) MT/2) and hands the other half to its partner
  // (nw, 1 - kw): one float4 per lane per tile, 1 KB rows, fixed order.
  // Register tiles are indexed with compile-time constants only (a runtime
  // index would move acc to scratch), hence the branches on kw.
  constexpr int HALF = MT / 2 * NT;
  float4_t* red = (float4_t*)xs;
  auto give = [&](auto kwc) __attribute__((always_inline)) {
    constexpr int G0 = (1 - decltype(kwc)::value) * (MT / 2);
#pragma unroll
    for (int i = 0; i < MT / 2; ++i)
#pragma unroll
      for (int t = 0; t < NT; ++t) red[((nw * 2 + kw) * HALF + i * NT + t) * 64 + lane] = acc[G0 + i][t];
  };
  // Lane (r, g), register e of tile (i, t): Y[m0 + 16 i + 4 g + e][16 (t0 + t) + r].
  auto keep = [&](auto kwc) __attribute__((always_inline)) {
    constexpr int K0 = decltype(kwc)::value * (MT / 2);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int n = (t0 + t) * kTileRows + r;
#pragma unroll
      for (int i = 0; i < MT / 2; ++i) {
        const float4_t v = acc[K0 + i][t] + red[((nw * 2 + (1 - kw)) * HALF + i * NT + t) * 64 + lane];
        if (n < N) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int m = m0 + (K0 + i) * 16 + 4 * g + e;
            if (m < M) store_y<YDT>(Y, (int64_t)m * ldy + n, v[e]);
          }
        }
      }
    }
  };
  if (kw == 0) give(std::integral_constant<int, 0>{});
  else give(std::integral_constant<int, 1>{});
  __syncthreads();
  if (kw == 0) keep(std::integral_constant<int, 0>{});
  else keep(std::integral_constant<int, 1>{});
}

// bf16 -> fp16, 8 values per thread, grid-stride (exact for fp16-normal
// magnitudes; round-toward-zero otherwise).  Row r of dst holds cols8p
// groups of 8: the converted cols8 groups, then zeros.
__global__ __launch_bounds__(256) void bf16_to_f16_kernel(const uint16_t* __restrict__ src, int64_t lds_,
                                                          uint16_t* __restrict__ dst, int64_t ldd, int64_t rows,
                                                          int64_t cols8, int64_t cols8p) {
  const int64_t n = rows * cols8p;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t row = i / cols8p, c8 = i - row * cols8p;
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
}

static hipError_t launch_bf16_to_f16(const void* src, int64_t lds_, void* dst, int64_t ldd, int64_t rows,
                                     int64_t cols, int64_t colsp, hipStream_t s, const LaunchEvents& ev) {
  const int64_t n = rows * (colsp / 8);
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  launch(bf16_to_f16_kernel, dim3((unsigned)blocks), dim3(256), 0, s, ev, (const uint16_t*)src, lds_,
         (uint16_t*)dst, ldd, rows, cols / 8, colsp / 8);
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
  constexpr int S = FMT == kQ4_0 ? Q4Q8_GEMM_STAGES_Q4 : Q4Q8_GEMM_STAGES_Q8;
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
  } else {
    if (ydt == kBF16) launch_shape<kQ8_0, kBF16>(W, N, K, Xh, ldh, M, Y, ldy, s, gev);
    else if (ydt == kF16) launch_shape<kQ8_0, kF16>(W, N, K, Xh, ldh, M, Y, ldy, s, gev);
    else launch_shape<kQ8_0, kF32>(W, N, K, Xh, ldh, M, Y, ldy, s, gev);
  }
  return hipGetLastError();
}

}  // namespace q4q8
