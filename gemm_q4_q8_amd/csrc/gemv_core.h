// Weight streaming and block products shared by the GEMV kernels (decode
// GEMV and the mixture-of-experts decode path); plain fp16 weights use the
// same tiles with the weights themselves as the B operand.
//
// A wavefront owns a tile of 16 weight rows.  Per chunk of 128 k (4 blocks)
// each lane loads 16 (Q4_0) or 32 (Q8_0) contiguous bytes of codes -- the
// wave reads 1 or 2 KB contiguous -- plus its row's 4 fp16 scales.  The codes
// unpack in registers straight into the B operand of one
// v_mfma_f32_16x16x32 per block (exact in fp16 and bf16); the block scale is
// applied to the fp32 block product, so only the fp32 accumulation rounds.
// Activation row m feeds A row 4 (m % 4) + m / 4: for m < 4 the result lands
// in the first accumulator register of each lane (m < 8: the first two).
#pragma once

#include "q4q8_dev.h"

namespace q4q8 {

constexpr int kGemvBufFlags = 0x00020000;   // raw buffer, 32-bit data format (gfx9)
#ifndef Q4Q8_WEIGHT_AUX
#define Q4Q8_WEIGHT_AUX 2                   // cache policy of the weight loads: nt (streamed once; measured
                                            // +9% on the decode step over the default policy)
#endif

// One chunk of a tile's weights in registers.
template <int FMT>
struct GemvStage {
  static constexpr int NV = FMT == kQ4_0 ? 1 : FMT == kQ8_0 ? 2 : 4;
  u32x4_t codes[NV];
  u32x2_t sc;   // unused for plain fp16 weights
};

// Loads chunk c of the tile behind `wres` (a buffer over the tile's records:
// reads past its end return zero, i.e. scale 0).  Lane l = 16 g + r.
template <int FMT>
__device__ __forceinline__ void gemv_load(GemvStage<FMT>& st, __amdgpu_buffer_rsrc_t wres, int c, int lane, int r) {
  const int off = c * Fmt<FMT>::kRecBytes;
#pragma unroll
  for (int v = 0; v < GemvStage<FMT>::NV; ++v)
    st.codes[v] = __builtin_amdgcn_raw_buffer_load_b128(wres, off + v * 1024 + lane * 16, 0, Q4Q8_WEIGHT_AUX);
  if constexpr (FMT != kFP16W)
    st.sc = __builtin_amdgcn_raw_buffer_load_b64(wres, off + Fmt<FMT>::kCodeBytes + r * 8, 0, Q4Q8_WEIGHT_AUX);
}

// Plain fp16 weights: the slots are the B operands themselves; the A
// fragments are fp16 (bf16 activations are converted by the caller).
template <int NI>
__device__ __forceinline__ void gemv_mma_fp16w(const GemvStage<kFP16W>& s, const half8_t (&a)[kBlocksPerChunk],
                                               float (&acc)[NI]) {
  float4_t d = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int j = 0; j < kBlocksPerChunk; ++j)
    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[j], __builtin_bit_cast(half8_t, s.codes[j]), d, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < NI; ++i) acc[i] += d[i];
}

// bf16 -> fp16 of one A fragment, round to nearest even (exact for
// 2^-14 <= |x| < 65520).
__device__ __forceinline__ half8_t bf16x8_to_half8(bf16x8_t v) {
  typedef float float8_t __attribute__((ext_vector_type(8)));
  return __builtin_convertvector(__builtin_convertvector(v, float8_t), half8_t);
}

// acc[i] += sum over the chunk's 4 blocks of scale_j * (A_j . B_j)[register i].
template <int FMT, int XDT, int NI>
__device__ __forceinline__ void gemv_mma(const GemvStage<FMT>& s, const typename Op<XDT>::vec (&a)[kBlocksPerChunk],
                                         float (&acc)[NI]) {
  typedef typename Op<XDT>::vec vec;
  float4_t d[kBlocksPerChunk];
#pragma unroll
  for (int j = 0; j < kBlocksPerChunk; ++j) {
    const u32x4_t b = deq_block<FMT, XDT>(s.codes, j);
    d[j] = Op<XDT>::mfma(a[j], __builtin_bit_cast(vec, b), float4_t{0.0f, 0.0f, 0.0f, 0.0f});
  }
#pragma unroll
  for (int j = 0; j < kBlocksPerChunk; ++j) {
    const uint32_t sbits = (j & 1) ? (s.sc[j >> 1] >> 16) : (s.sc[j >> 1] & 0xFFFFu);
    const float sf = half_bits_to_float(sbits);
#pragma unroll
    for (int i = 0; i < NI; ++i) acc[i] = __builtin_fmaf(sf, d[j][i], acc[i]);
  }
}

}  // namespace q4q8
