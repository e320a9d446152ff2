// The tile engine of the prefill GEMM: one 512-thread workgroup computes a
// BM x BN block of X W^T for NW weight matrices at once (NW = 2 would give
// gate and up of the same rows).
//
//   * matrix cores: v_mfma_f32_16x16x32_f16, fp32 accumulation.  Weights are
//     unpacked in registers and scaled to fp16 (one rounding, relative error
//     <= 2^-11); activations are fp16.  Applying the block scale in fp32
//     after each MFMA would cost one VALU FMA per output per block -- as much
//     issue time as the MFMAs themselves -- so the scale goes into the
//     operand.
//   * eight waves: wave w owns weight tiles t0 .. t0 + NT - 1 (t0 chosen by
//     the caller from w % 4) and blocks 2 (w / 4), 2 (w / 4) + 1 of every
//     128-wide chunk of K.  Two waves share each SIMD, so one's dequant VALU
//     work runs under the other's MFMAs; the two K halves are summed through
//     LDS at the end (khalf_reduce).
//   * weights stream from HBM into an S-stage register ring (buffer loads,
//     S - 1 chunks ahead).  Each step unpacks the next block during the
//     current block's MFMAs, including the next chunk's first block.
//   * the BM x 128 activation chunk is copied global -> LDS by the buffer
//     loads' LDS path (no registers) into an S-stage ring.  The copy writes
//     1 KB per wave instruction contiguously, so rows cannot be padded;
//     instead lane L picks its source so that LDS slot 16 row + (cg ^ row%16)
//     holds 16-byte column group cg of that row, and the A-fragment reads
//     (16 rows x 4 column groups per instruction) hit distinct banks.  The
//     caller gives each copy's per-lane source offset, so rows may be
//     gathered from anywhere in the activation buffer.
//   * one barrier per chunk that waits only for the loads that chunk needs.
#pragma once

#include "q4q8_dev.h"

#include <type_traits>

namespace q4q8 {

constexpr uint32_t kOOB = 0x80000000u;   // buffer offset past any range: reads 0

// f(integral_constant<I>) for I = B .. E-1, unrolled at compile time.
template <int B, int E, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// Activation copy p of thread tid fills LDS slot 512 p + tid of a stage:
// tile row `row`, 16-byte column group `cg`.
__device__ __forceinline__ void x_slot(int p, int tid, int& row, int& cg) {
  const int slot = p * 512 + tid;
  row = slot >> 4;
  cg = (slot & 15) ^ (row & 15);
}

template <int FMT, int MT, int NT, int NW, int S>
struct TileCfg {
  static constexpr int BM = 16 * MT;
  static constexpr int REC = Fmt<FMT>::kRecBytes;
  static constexpr int CODE = Fmt<FMT>::kCodeBytes;
  static constexpr int XLOADS = MT / 2;          // 16-byte copies per thread per chunk (BM * 16 / 512)
  static constexpr int WLOADS = 2 * NT * NW;     // weight loads per wave per chunk
  static constexpr int STAGE_HALFS = BM * kChunkK;
  static constexpr int RED_HALFS = 8 * NW * (MT / 2) * NT * 512;   // the K-half reduction (1 KB per tile and wave)
  static constexpr int LDS_HALFS = S * STAGE_HALFS > RED_HALFS ? S * STAGE_HALFS : RED_HALFS;
  static_assert(MT % 2 == 0 && S >= 3, "tile shape");
  static_assert(LDS_HALFS * 2 <= 160 * 1024, "LDS per workgroup");
};

// Main loop.  wres[w]: weight matrix w restricted to this wave's tiles
// (tile t of the wave at record t * nchunks); tv of them are valid, the rest
// read zero.  xres/xv: activation buffer and, per copy p, this lane's byte
// offset of (its row, column group 0 of chunk 0) -- kOOB for rows that must
// read zero.  K: columns of X that exist (TAIL masks past it); nchunks:
// chunks of the weight records.  acc (tile (w, i, t) at (w MT + i) NT + t,
// a flat array so every element stays in registers) is overwritten.
template <int FMT, int MT, int NT, int NW, int S, bool TAIL>
__device__ __forceinline__ void tile_mainloop(const __amdgpu_buffer_rsrc_t (&wres)[NW], int tv, int K, int nchunks,
                                              __amdgpu_buffer_rsrc_t xres, const uint32_t (&xv)[MT / 2],
                                              uint16_t* xs, float4_t (&acc)[NW * MT * NT]) {
  using C = TileCfg<FMT, MT, NT, NW, S>;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kw = wave >> 2;
  const int r = lane & 15, g = lane >> 4;

  // One chunk of this wave's weights: codes and scales of blocks 2 kw and
  // 2 kw + 1.  Q4_0: dwords 2 kw, 2 kw + 1 of the lane's slot; Q8_0: the
  // lane's slot in half kw.  Lane offsets are loop-invariant; the chunk
  // enters through the scalar offset.  Chunks past the last re-read the last.
  // Plain fp16: the lane's slot of blocks 2 kw and 2 kw + 1 (two 16-byte
  // loads, no scales).
  struct F16Pair {
    u32x4_t h[2];
  };
  typedef typename std::conditional<FMT == kQ4_0, u32x2_t,
                                    typename std::conditional<FMT == kQ8_0, u32x4_t, F16Pair>::type>::type CodeT;
  struct WStage {
    CodeT codes[NW][NT];
    uint32_t sc[NW][NT];
  };
  const uint32_t wv_code = FMT == kQ4_0 ? lane * 16 + kw * 8 : FMT == kQ8_0 ? kw * 1024 + lane * 16
                                                                             : 2 * kw * 1024 + lane * 16;
  const uint32_t wv_scale = C::CODE + r * 8 + kw * 4;
  auto load_w = [&](WStage& s, int c) __attribute__((always_inline)) {
    const int cc = c < nchunks ? c : nchunks - 1;
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const int so = (t * nchunks + cc) * C::REC;
        const uint32_t vc = t < tv ? wv_code : kOOB, vs = t < tv ? wv_scale : kOOB;
        if constexpr (FMT == kFP16W) {   // two loads, as the quantised formats' codes + scales
          s.codes[w][t].h[0] = __builtin_amdgcn_raw_buffer_load_b128(wres[w], vc, so, 0);
          s.codes[w][t].h[1] = __builtin_amdgcn_raw_buffer_load_b128(wres[w], t < tv ? vc + 1024 : kOOB, so, 0);
        } else {
          if constexpr (FMT == kQ4_0)
            s.codes[w][t] = __builtin_amdgcn_raw_buffer_load_b64(wres[w], vc, so, 0);
          else
            s.codes[w][t] = __builtin_amdgcn_raw_buffer_load_b128(wres[w], vc, so, 0);
          s.sc[w][t] = __builtin_amdgcn_raw_buffer_load_b32(wres[w], vs, so, 0);
        }
      }
  };
  // Copy chunk c of the activation tile into LDS stage st.  Chunks past the
  // last re-read the last one (into a stage nobody reads), so every step
  // issues the same loads; with TAIL, columns past K are sent out of range.
  auto copy_x = [&](int c, int st) __attribute__((always_inline)) {
    const int cc = c < nchunks ? c : nchunks - 1;
#pragma unroll
    for (int p = 0; p < C::XLOADS; ++p) {
      uint32_t v = xv[p];
      if constexpr (TAIL) {
        int row, cg;
        x_slot(p, tid, row, cg);
        v = cg * 8 < K - cc * kChunkK ? v : kOOB;
      }
      uint16_t* dst = xs + st * C::STAGE_HALFS + (p * 512 + wave * 64) * 8;   // wave-uniform
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xres, (__attribute__((address_space(3))) void*)dst, 16, v,
                                               cc * kChunkK * 2, 0, 0);
    }
  };

#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[(w * MT + i) * NT + t] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};

  // Unpacked, scaled B operands of block jj (0 or 1) of a weight stage.
  typedef half8_t BOps[NW][NT];
  auto dequant = [&](const WStage& s, int jj, BOps& b) __attribute__((always_inline)) {
#pragma unroll
    for (int w = 0; w < NW; ++w)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if constexpr (FMT == kFP16W) {
          b[w][t] = __builtin_bit_cast(half8_t, s.codes[w][t].h[jj]);
        } else {
          u32x4_t q;
          if constexpr (FMT == kQ4_0) {
            const uint32_t wd = s.codes[w][t][jj];
            q = deq_q4_f16(wd);
          } else {
            const uint32_t d0 = s.codes[w][t][2 * jj], d1 = s.codes[w][t][2 * jj + 1];
            q = deq_q8<kF16>(d0, d1);
          }
          const uint32_t sbits = jj ? (s.sc[w][t] >> 16) : (s.sc[w][t] & 0xFFFFu);
          const _Float16 sh = __builtin_bit_cast(_Float16, (uint16_t)sbits);
          const half2_t s2 = {sh, sh};
          b[w][t] = __builtin_bit_cast(half8_t, scale_f16x8(q, s2));
        }
      }
  };
  // NW x MT x NT MFMAs of block jj of the chunk in LDS stage st.
  auto mma = [&](int st, int jj, const BOps& b) __attribute__((always_inline)) {
    const uint16_t* xb = xs + st * C::STAGE_HALFS;
    const int j = 2 * kw + jj;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
      const int row = i * 16 + r;
      const half8_t a = *(const half8_t*)(xb + (row * 16 + ((4 * j + g) ^ r)) * 8);
#pragma unroll
      for (int w = 0; w < NW; ++w)
#pragma unroll
        for (int t = 0; t < NT; ++t)
          acc[(w * MT + i) * NT + t] =
              __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b[w][t], acc[(w * MT + i) * NT + t], 0, 0, 0);
    }
  };

  // Prologue: chunks 0 .. S - 2 in flight, weights then activations per
  // chunk.  The scheduling barriers keep that order, so the wait counts
  // below hold on every path into the loop head.
  WStage ws[S];
  static_for<0, S - 1>([&](auto ic) __attribute__((always_inline)) {
    constexpr int i = decltype(ic)::value;
    load_w(ws[i], i);
    copy_x(i, i);
    __builtin_amdgcn_sched_barrier(0);
  });
  // Block 0 of chunk 0 is unpacked ahead; afterwards each step unpacks its
  // block 1 during block 0's products and the next chunk's block 0 during
  // block 1's.
  BOps b0, b1;
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"((S - 2) * (C::XLOADS + C::WLOADS) + C::XLOADS) : "memory");
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
    asm volatile("s_waitcnt vmcnt(%0)\n\ts_waitcnt lgkmcnt(0)\n\ts_barrier" ::"n"(
                     (S - 3) * (C::XLOADS + C::WLOADS) + C::XLOADS)
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
}

// Sum the two K halves through LDS (red: the activation ring, free once the
// main loop is done).  Wave (nw, kw) keeps m-tiles [kw MT/2, (kw+1) MT/2)
// and hands the other half to its partner (nw, 1 - kw): one float4 per lane
// per tile, 1 KB rows, fixed order, so the result is deterministic.
// kept[(w MT/2 + i) NT + t] = full sum of tile (w, kw MT/2 + i, t).  The
// halves are chosen with value selects on kw, not branches: merged branches
// would index acc through a pointer select and push it to scratch.
template <int MT, int NT, int NW>
__device__ __forceinline__ void khalf_reduce(const float4_t (&acc)[NW * MT * NT], float4_t* red,
                                             float4_t (&kept)[NW * (MT / 2) * NT]) {
  constexpr int H = MT / 2, HALF = NW * H * NT;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nw = wave & 3, kw = wave >> 2;
  const bool hi = kw != 0;
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int i = 0; i < H; ++i)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float4_t lo_v = acc[(w * MT + i) * NT + t], hi_v = acc[(w * MT + H + i) * NT + t];
        red[((nw * 2 + kw) * HALF + (w * H + i) * NT + t) * 64 + lane] = hi ? lo_v : hi_v;
      }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < NW; ++w)
#pragma unroll
    for (int i = 0; i < H; ++i)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float4_t lo_v = acc[(w * MT + i) * NT + t], hi_v = acc[(w * MT + H + i) * NT + t];
        kept[(w * H + i) * NT + t] =
            (hi ? hi_v : lo_v) + red[((nw * 2 + (1 - kw)) * HALF + (w * H + i) * NT + t) * 64 + lane];
      }
}

}  // namespace q4q8
