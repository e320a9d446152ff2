// Device-side building blocks shared by the gfx950 kernels: the repacked
// weight layout, in-register dequantisation and the 16x16x32 MFMA wrappers.
//
// Repacked layout (one layout serves GEMV, GEMM and the MoE GEMMs):
//   * rows in tiles of 16, K in chunks of 128 (4 blocks of 32);
//   * record (tile t, chunk c) at byte (t * nchunks + c) * kRecBytes;
//   * codes first: 64 lane slots; slot l = 16 g + r holds, for row r of the
//     tile and each block j of the chunk, the 8 codes k = 32 j + 8 g + e
//     (e = 0..7).  That is exactly the B operand lane l feeds to
//     v_mfma_f32_16x16x32_{f16,bf16} when B = W^T restricted to one block:
//     B[k][n] with n = l % 16 and k = 8 (l / 16) + e.
//       Q4_0: 16 bytes per slot, one dword per block; code e sits at bit
//             4 * ((e & 1) * 4 + (e >> 1)), so masking with 0x000F000F /
//             0x00F000F0 (before and after an 8-bit shift) yields the fp16
//             pairs (e0,e1) (e2,e3) (e4,e5) (e6,e7) directly.
//       Q8_0: 32 bytes per slot in two 16-byte halves; half h (first or
//             second kilobyte of the record) carries blocks 2h and 2h+1, 8
//             bytes each, in natural order.
//   * then 128 bytes of scales, fp16 [row r][block j].
// Padding rows / blocks carry scale 0 and code 0.  Plain fp16 weights use the
// same tiles with the weights themselves in the slots (Fmt<kFP16W>).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4q8 {

enum { kQ4_0 = 1, kQ8_0 = 2, kFP16W = 3 };   // weight formats (kFP16W: plain fp16 weights)
enum { kF16 = 1, kBF16 = 2, kF32 = 3 };

constexpr int kTileRows = 16;
constexpr int kChunkK = 128;
constexpr int kBlocksPerChunk = 4;
constexpr int kScaleBytes = 128;

template <int FMT> struct Fmt;
template <> struct Fmt<kQ4_0> {
  static constexpr int kCanonBlock = 18;
  static constexpr int kCodeBytes = 1024;
  static constexpr int kRecBytes = 1024 + kScaleBytes;
};
template <> struct Fmt<kQ8_0> {
  static constexpr int kCanonBlock = 34;
  static constexpr int kCodeBytes = 2048;
  static constexpr int kRecBytes = 2048 + kScaleBytes;
};
// Plain fp16: four 1 KB planes per record (block j at j * 1024, lane slot l
// at l * 16 holding row r's 8 weights k = 32 j + 8 g .. + 7), no scales.
template <> struct Fmt<kFP16W> {
  static constexpr int kCanonBlock = 64;
  static constexpr int kCodeBytes = 4096;
  static constexpr int kRecBytes = 4096;
};

__host__ __device__ constexpr int q4_nibble_shift(int e) { return 4 * ((e & 1) * 4 + (e >> 1)); }

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// Operand types: XDT selects fp16 or bf16 matrix-core operands.
// ---------------------------------------------------------------------------
template <int XDT> struct Op;
template <> struct Op<kF16> {
  typedef half8_t vec;
  static __device__ __forceinline__ float4_t mfma(vec a, vec b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    // Exact for the small integers and fp16-representable values packed here.
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
  }
};
template <> struct Op<kBF16> {
  typedef bf16x8_t vec;
  static __device__ __forceinline__ float4_t mfma(vec a, vec b, float4_t c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack(float lo, float hi) {
    // One v_cvt_pk_bf16_f32 (round to nearest even) for the pair; two scalar
    // casts compile to a conversion each plus a merge.
    typedef float float2_t __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{lo, hi}, bf16x2_t));
  }
};

// ---------------------------------------------------------------------------
// Exact dequantisation of one lane's 8 codes of one block into an MFMA
// operand (values q-8 or q, scale not applied).
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4_t deq_q4_f16(uint32_t w) {
  // (nibble | 0x6400) is the fp16 1024 + n; (16n | 0x6400) is 1024 + 16n.
  // (w & mask) | magic is one v_bitop3_b32 (truth table 0xEA for
  // (a & b) | c).  No inline asm here: the hazard recognizer does not see
  // VALU writes made from inline asm next to in-flight MFMAs.
  const uint32_t kMagic = 0x64006400u;
  const uint32_t w2 = w >> 8;
  half2_t h0 = __builtin_bit_cast(half2_t, __builtin_amdgcn_bitop3_b32(w, 0x000F000Fu, kMagic, 0xEA));
  half2_t h1 = __builtin_bit_cast(half2_t, __builtin_amdgcn_bitop3_b32(w, 0x00F000F0u, kMagic, 0xEA));
  half2_t h2 = __builtin_bit_cast(half2_t, __builtin_amdgcn_bitop3_b32(w2, 0x000F000Fu, kMagic, 0xEA));
  half2_t h3 = __builtin_bit_cast(half2_t, __builtin_amdgcn_bitop3_b32(w2, 0x00F000F0u, kMagic, 0xEA));
  const half2_t off = {(_Float16)1032.0f, (_Float16)1032.0f};
  const half2_t sixteenth = {(_Float16)0.0625f, (_Float16)0.0625f};
  const half2_t off16 = {(_Float16)-72.0f, (_Float16)-72.0f};
  h0 = h0 - off;
  h1 = h1 * sixteenth + off16;   // (1024 + 16n) / 16 - 72 = n - 8, exact
  h2 = h2 - off;
  h3 = h3 * sixteenth + off16;
  u32x4_t r;
  r[0] = __builtin_bit_cast(uint32_t, h0);
  r[1] = __builtin_bit_cast(uint32_t, h1);
  r[2] = __builtin_bit_cast(uint32_t, h2);
  r[3] = __builtin_bit_cast(uint32_t, h3);
  return r;
}

__device__ __forceinline__ u32x4_t deq_q4_bf16(uint32_t w) {
  u32x4_t r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    int e0 = 2 * p, e1 = 2 * p + 1;
    float lo = (float)(int)((w >> q4_nibble_shift(e0)) & 0xFu) - 8.0f;
    float hi = (float)(int)((w >> q4_nibble_shift(e1)) & 0xFu) - 8.0f;
    r[p] = Op<kBF16>::pack(lo, hi);
  }
  return r;
}

template <int XDT>
__device__ __forceinline__ u32x4_t deq_q8(uint32_t d0, uint32_t d1) {
  u32x4_t r;
  r[0] = Op<XDT>::pack((float)(int)(int8_t)(d0), (float)(int)(int8_t)(d0 >> 8));
  r[1] = Op<XDT>::pack((float)(int)(int8_t)(d0 >> 16), (float)(int)(int8_t)(d0 >> 24));
  r[2] = Op<XDT>::pack((float)(int)(int8_t)(d1), (float)(int)(int8_t)(d1 >> 8));
  r[3] = Op<XDT>::pack((float)(int)(int8_t)(d1 >> 16), (float)(int)(int8_t)(d1 >> 24));
  return r;
}

template <int FMT, int XDT>
__device__ __forceinline__ u32x4_t deq_block(const u32x4_t* codes, int j);

// Q4_0: one 16-byte slot, dword j is block j.
template <> __device__ __forceinline__ u32x4_t deq_block<kQ4_0, kF16>(const u32x4_t* c, int j) {
  return deq_q4_f16(c[0][j]);
}
template <> __device__ __forceinline__ u32x4_t deq_block<kQ4_0, kBF16>(const u32x4_t* c, int j) {
  return deq_q4_bf16(c[0][j]);
}
// Q8_0: two 16-byte halves; block j is dwords 2(j&1), 2(j&1)+1 of half j>>1.
template <> __device__ __forceinline__ u32x4_t deq_block<kQ8_0, kF16>(const u32x4_t* c, int j) {
  return deq_q8<kF16>(c[j >> 1][2 * (j & 1)], c[j >> 1][2 * (j & 1) + 1]);
}
template <> __device__ __forceinline__ u32x4_t deq_block<kQ8_0, kBF16>(const u32x4_t* c, int j) {
  return deq_q8<kBF16>(c[j >> 1][2 * (j & 1)], c[j >> 1][2 * (j & 1) + 1]);
}

// Multiply 8 fp16 values (4 packed pairs) by the scale pair s2.  Each element
// is copied into a scalar first: hipcc (clang 22) miscompiles
// __builtin_bit_cast applied directly to an ext_vector element inside an
// unrolled read-modify-write loop (every element came out as element 0).
__device__ __forceinline__ u32x4_t scale_f16x8(const u32x4_t q, const half2_t s2) {
  const uint32_t q0 = q[0], q1 = q[1], q2 = q[2], q3 = q[3];
  u32x4_t o;
  o[0] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, q0) * s2);
  o[1] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, q1) * s2);
  o[2] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, q2) * s2);
  o[3] = __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, q3) * s2);
  return o;
}

// Activation row scaling (the GEMM and MoE paths): exponent of a row whose
// largest magnitude has the bits m (sign cleared; the bits order bf16 and
// fp16 magnitudes, inf and NaN above every finite value): ilogb(max) - 2,
// so the row times 2^-e has its largest magnitude in [4, 8); 0 for a zero
// or non-finite row.
template <int SRC>
__device__ __forceinline__ int row_exponent(uint32_t m) {
  constexpr uint32_t kInf = SRC == kBF16 ? 0x7F80u : 0x7C00u;
  if (m == 0 || m >= kInf) return 0;
  const float big =
      SRC == kBF16 ? __builtin_bit_cast(float, m << 16) : (float)__builtin_bit_cast(_Float16, (uint16_t)m);
  return __builtin_amdgcn_frexp_expf(big) - 3;   // big = f 2^x, f in [0.5, 1): ilogb = x - 1
}

// Two bf16 / fp16 values (one word) -> fp16 of x 2^sh, round to nearest even.
template <int SRC>
__device__ __forceinline__ uint32_t f16x2_scaled(uint32_t w, int sh) {
  float lo, hi;
  if constexpr (SRC == kBF16) {
    lo = __builtin_bit_cast(float, w << 16);
    hi = __builtin_bit_cast(float, w & 0xFFFF0000u);
  } else {
    lo = (float)__builtin_bit_cast(_Float16, (uint16_t)(w & 0xFFFFu));
    hi = (float)__builtin_bit_cast(_Float16, (uint16_t)(w >> 16));
  }
  const half2_t r = {(_Float16)__builtin_ldexpf(lo, sh), (_Float16)__builtin_ldexpf(hi, sh)};
  return __builtin_bit_cast(uint32_t, r);
}

// Eight values; the words are copied to scalars first (see scale_f16x8).
template <int SRC>
__device__ __forceinline__ u32x4_t f16x8_scaled(const u32x4_t v, int sh) {
  const uint32_t w0 = v[0], w1 = v[1], w2 = v[2], w3 = v[3];
  u32x4_t o;
  o[0] = f16x2_scaled<SRC>(w0, sh);
  o[1] = f16x2_scaled<SRC>(w1, sh);
  o[2] = f16x2_scaled<SRC>(w2, sh);
  o[3] = f16x2_scaled<SRC>(w3, sh);
  return o;
}

// Largest magnitude bits (sign cleared) of eight bf16 / fp16 values.
__device__ __forceinline__ uint32_t max_mag_bits8(const u32x4_t v) {
  const uint32_t w0 = v[0], w1 = v[1], w2 = v[2], w3 = v[3];
  const uint32_t a = max(max(w0 & 0x7FFFu, (w0 >> 16) & 0x7FFFu), max(w1 & 0x7FFFu, (w1 >> 16) & 0x7FFFu));
  const uint32_t b = max(max(w2 & 0x7FFFu, (w2 >> 16) & 0x7FFFu), max(w3 & 0x7FFFu, (w3 >> 16) & 0x7FFFu));
  return max(a, b);
}

// A raw buffer resource whose base and size are provably wave-uniform (built
// from readfirstlane'd values), so loads through it take the descriptor from
// SGPRs instead of a per-lane waterfall loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, int bytes) {
  const uint64_t b = (uint64_t)base;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)b);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(b >> 32));
  const int n = __builtin_amdgcn_readfirstlane(bytes);
  return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), (short)0, n, 0x00020000);
}

// silu(z) = z sigmoid(z) = z / (1 + 2^(-z log2(e))), fp32 (the SwiGLU gate
// activation), on the hardware's base-2 exponential and reciprocal (each
// within about one ulp; the argument's own rounding adds a relative error
// near 2^-24 |z|).  For finite z the result is within about 1e-5 relative of
// the exact silu, far below h's bf16 rounding (2^-9).  Large negative z give
// 2^(+big) = inf and a zero reciprocal, so silu -> -0; large positive z give
// sigmoid 1.
__device__ __forceinline__ float silu_f32(float z) {
  const float e = __builtin_amdgcn_exp2f(-z * 1.44269504088896341f);
  return z * __builtin_amdgcn_rcpf(1.0f + e);
}

__device__ __forceinline__ float half_bits_to_float(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16);
}

}  // namespace q4q8
