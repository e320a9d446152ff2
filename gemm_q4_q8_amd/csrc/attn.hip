// Prefill attention on the matrix cores: tiles of queries against tiles of
// keys with an online softmax, so the S x S score matrix never exists in
// memory ("BaseRT: Best-in-Class LLM Inference on Apple Silicon via Native
// Metal", technical summary, "Methodologie", prefill optimisation; the M5
// review, "Method", routes this prefill attention to the matrix units).
//
// Per workgroup: 8 waves x 16 queries of one (batch, query head); K and V of
// the matching key/value head (GQA: head h reads kv head h / (Hq / Hkv)) pass
// through two LDS buffers in blocks of 64 keys: the next block's global loads
// are in flight while the current one is used, then written to the other
// buffer (one barrier per block).  Per wave and key block, with
// v_mfma_f32_16x16x32 on bf16 (or fp16) operands:
//   * S^T = K Q^T  (A = K rows from LDS, B = the wave's Q^T held in
//     registers).  Lane (r, g) ends up with the scores of query r against
//     keys 16 t + 4 g + v, i.e. every lane's values belong to one query, so
//     the running max and sum need only the 4 lanes r, r+16, r+32, r+48;
//   * P^T = exp2(S^T * scale * log2 e - m) rounded to the operand type is
//     already the B operand of O^T = V^T P^T when the 32 keys of an MFMA
//     step are taken in the order (4 g .. 4 g + 3, 16 + 4 g .. 16 + 4 g + 3)
//     for lane group g; V is stored transposed in LDS ([d][key]) so that the
//     A operand reads those keys as two 8-byte runs;
//   * O^T accumulates in fp32 (lane (r, g) holds O[query r][d 16 t + 4 g + v])
//     and is rescaled by exp2(m_old - m_new) when the max moves.
// Causal masking skips key blocks past the workgroup's last query and masks
// the diagonal block per element; query blocks run heaviest first.
#include "q4q8_dev.h"
#include "q4q8_internal.h"

namespace q4q8 {

constexpr int kAttnD = 128;          // head dimension
constexpr int kAttnWaves = 8;
constexpr int kAttnBM = 16 * kAttnWaves;   // queries per workgroup
constexpr int kAttnBN = 64;          // keys per block
constexpr int kKStride = kAttnD + 8;       // K rows in LDS (halfs)
constexpr int kVStride = kAttnBN + 12;     // V^T rows in LDS (halfs; +8 measured slower)

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int32_t B, S, Hq, Hkv;
  int32_t causal;
  int32_t mblocks;
  float scale_log2;   // scale * log2(e)
};

typedef float float2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// Two fp32 values rounded to nearest-even in the operand type, packed
// (one v_cvt_pk_bf16_f32 for bf16).
template <int DT>
__device__ __forceinline__ uint32_t pack_rn(float lo, float hi) {
  if constexpr (DT == kBF16) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{lo, hi}, bf16x2_t));
  } else {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(float2_t{lo, hi}, half2_t));
  }
}

template <int DT>
__global__ __launch_bounds__(kAttnWaves * 64, 4) void attn_prefill_kernel(const AttnArgs a) {
  typedef typename Op<DT>::vec vec;
  // Two buffers of K (row-major) and V^T: block j + 1 is written while block
  // j is read.
  __shared__ __attribute__((aligned(16))) uint16_t ks_buf[2][kAttnBN * kKStride];
  __shared__ __attribute__((aligned(16))) uint16_t vts_buf[2][kAttnD * kVStride];

  // Dispatch order: the first half of the grid takes query blocks heaviest
  // first, the second half lightest first, so the two workgroups that share
  // a CU (block b and b + half) carry about equal causal work together.
  const int total = gridDim.x, half = (total + 1) / 2;
  const int bid = blockIdx.x;
  const int rank = bid < half ? bid : total - 1 - (bid - half);   // 0 = heaviest
  const int mb = a.mblocks - 1 - rank / (a.Hq * a.B);
  const int bh = rank % (a.Hq * a.B);
  const int h = bh % a.Hq, b = bh / a.Hq;
  const int hk = h / (a.Hq / a.Hkv);
  const int S = a.S;
  const int64_t qstride = (int64_t)a.Hq * kAttnD;     // between positions
  const int64_t kvstride = (int64_t)a.Hkv * kAttnD;
  const uint16_t* qb = a.q + (int64_t)b * S * qstride + (int64_t)h * kAttnD;
  const uint16_t* kb = a.k + (int64_t)b * S * kvstride + (int64_t)hk * kAttnD;
  const uint16_t* vb = a.v + (int64_t)b * S * kvstride + (int64_t)hk * kAttnD;
  uint16_t* ob = a.o + (int64_t)b * S * qstride + (int64_t)h * kAttnD;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int m0 = mb * kAttnBM;
  const int qi = m0 + wave * 16 + r;           // this lane's query
  const bool qvalid = qi < S;

  // The wave's Q^T fragments: lane (r, g) holds Q[qi][32 s + 8 g .. + 7].
  vec qf[kAttnD / 32];
#pragma unroll
  for (int s = 0; s < kAttnD / 32; ++s) {
    u32x4_t t = u32x4_t{0, 0, 0, 0};
    if (qvalid) t = *(const u32x4_t*)(qb + (int64_t)qi * qstride + 32 * s + 8 * g);
    qf[s] = __builtin_bit_cast(vec, t);
  }

  // Key blocks: all of them, or up to the last query of the block (causal).
  const int kend = a.causal ? min(S, m0 + kAttnBM) : S;
  const int nblocks = (kend + kAttnBN - 1) / kAttnBN;

  // Global -> register staging.  Waves 0-3 move V: thread t takes keys
  // 4 (t % 16) .. + 3 at d 8 (t / 16) .. + 7 and writes, for each d, the four
  // keys as one 8-byte word of V^T.  Waves 4-7 move K: key u / 4, d 32 (u % 4)
  // .. + 31 (u = t - 256), row-major.
  const bool vrole = tid < 256;   // uniform per wave
  const int u = vrole ? tid : tid - 256;
  const int vk0 = 4 * (u & 15), vd0 = 8 * (u >> 4);
  const int kkey = u >> 2, kd0 = 32 * (u & 3);
  u32x4_t st[4];
  auto fetch = [&](int blk) {
    const int n0 = blk * kAttnBN;
    if (vrole) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int key = n0 + vk0 + i;
        st[i] = key < S ? *(const u32x4_t*)(vb + (int64_t)key * kvstride + vd0) : u32x4_t{0, 0, 0, 0};
      }
    } else {
      const int key = n0 + kkey;
#pragma unroll
      for (int i = 0; i < 4; ++i)
        st[i] = key < S ? *(const u32x4_t*)(kb + (int64_t)key * kvstride + kd0 + 8 * i) : u32x4_t{0, 0, 0, 0};
    }
  };
  auto stash = [&](int buf) {
    if (vrole) {
      uint16_t* vt = vts_buf[buf];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        // Half j of the four keys' words: low halves (j even) or high halves.
        const int w = j >> 1;
        const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
        *(u32x2_t*)(vt + (vd0 + j) * kVStride + vk0) =
            u32x2_t{__builtin_amdgcn_perm(st[1][w], st[0][w], sel), __builtin_amdgcn_perm(st[3][w], st[2][w], sel)};
      }
    } else {
      uint16_t* kt = ks_buf[buf];
#pragma unroll
      for (int i = 0; i < 4; ++i) *(u32x4_t*)(kt + kkey * kKStride + kd0 + 8 * i) = st[i];
    }
  };

  float4_t acc_o[kAttnD / 16];
#pragma unroll
  for (int t = 0; t < kAttnD / 16; ++t) acc_o[t] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
  float m_run = -INFINITY, l_run = 0.0f;

  fetch(0);
  stash(0);
  __syncthreads();
  for (int blk = 0; blk < nblocks; ++blk) {
    const int buf = blk & 1;
    if (blk + 1 < nblocks) fetch(blk + 1);   // in flight during this block's math
    const uint16_t* ks = ks_buf[buf];
    const uint16_t* vts = vts_buf[buf];

    // S^T for 64 keys x the wave's 16 queries.
    float4_t sc[kAttnBN / 16];
#pragma unroll
    for (int t = 0; t < kAttnBN / 16; ++t) {
      float4_t c = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < kAttnD / 32; ++s) {
        const vec kf = *(const vec*)(ks + (16 * t + r) * kKStride + 32 * s + 8 * g);
        c = Op<DT>::mfma(kf, qf[s], c);
      }
      sc[t] = c;
    }
    // Mask (causal diagonal, keys past S) and the block max for query r, on
    // the raw scores (scale > 0 commutes with max).
    const int n0 = blk * kAttnBN;
    const bool edge = n0 + kAttnBN > S || (a.causal && n0 + kAttnBN - 1 > m0 + wave * 16);
    if (edge) {
#pragma unroll
      for (int t = 0; t < kAttnBN / 16; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int key = n0 + 16 * t + 4 * g + v;
          sc[t][v] = (key >= S || (a.causal && key > qi)) ? -INFINITY : sc[t][v];
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int t = 0; t < kAttnBN / 16; ++t) mx = fmaxf(fmaxf(mx, fmaxf(sc[t][0], sc[t][1])), fmaxf(sc[t][2], sc[t][3]));
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(m_run, mx * a.scale_log2);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;   // a row with nothing visible yet
    const float alpha = __builtin_amdgcn_exp2f(m_run - m_use);
    m_run = m_new;
    // p = 2^(s * scale * log2 e - m): one FMA and one v_exp per score.
    float lsum = 0.0f;
    uint32_t pb[kAttnBN / 16][2];
#pragma unroll
    for (int t = 0; t < kAttnBN / 16; ++t) {
      float p[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        p[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[t][v], a.scale_log2, -m_use));
        lsum += p[v];
      }
      pb[t][0] = pack_rn<DT>(p[0], p[1]);
      pb[t][1] = pack_rn<DT>(p[2], p[3]);
    }
    l_run = l_run * alpha + lsum;
    if (__any(alpha != 1.0f)) {   // the max moved for some query of the wave
#pragma unroll
      for (int t = 0; t < kAttnD / 16; ++t) acc_o[t] *= alpha;
    }

    // O^T += V^T P^T, two MFMA steps of 32 keys.
#pragma unroll
    for (int s = 0; s < kAttnBN / 32; ++s) {
      const vec pf = __builtin_bit_cast(vec, u32x4_t{pb[2 * s][0], pb[2 * s][1], pb[2 * s + 1][0], pb[2 * s + 1][1]});
#pragma unroll
      for (int t = 0; t < kAttnD / 16; ++t) {
        const uint16_t* vrow = vts + (16 * t + r) * kVStride + 32 * s + 4 * g;
        const u32x2_t lo = *(const u32x2_t*)vrow;
        const u32x2_t hi = *(const u32x2_t*)(vrow + 16);
        const vec vf = __builtin_bit_cast(vec, u32x4_t{lo[0], lo[1], hi[0], hi[1]});
        acc_o[t] = Op<DT>::mfma(vf, pf, acc_o[t]);
      }
    }
    // The other buffer was last read before the previous barrier.
    if (blk + 1 < nblocks) stash(buf ^ 1);
    __syncthreads();
  }

  // Normalise and store: lane (r, g) writes O[qi][16 t + 4 g .. + 3].
  float l = l_run;
  l += __shfl_xor(l, 16);
  l += __shfl_xor(l, 32);
  const float inv = 1.0f / l;
  if (!qvalid) return;
#pragma unroll
  for (int t = 0; t < kAttnD / 16; ++t) {
    const float4_t o = acc_o[t] * inv;
    *(u32x2_t*)(ob + (int64_t)qi * qstride + 16 * t + 4 * g) = u32x2_t{pack_rn<DT>(o[0], o[1]), pack_rn<DT>(o[2], o[3])};
  }
}

hipError_t launch_attn_prefill(int dt, const void* q, const void* k, const void* v, void* o, int B, int S, int Hq,
                               int Hkv, int causal, float scale, hipStream_t s, const LaunchEvents& ev) {
  AttnArgs a;
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.o = (uint16_t*)o;
  a.B = B;
  a.S = S;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.causal = causal;
  a.mblocks = (S + kAttnBM - 1) / kAttnBM;
  a.scale_log2 = scale * 1.4426950408889634f;
  const dim3 grid((unsigned)(a.mblocks * Hq * B)), block(kAttnWaves * 64);
  if (dt == kBF16) launch(attn_prefill_kernel<kBF16>, grid, block, 0, s, ev, a);
  else launch(attn_prefill_kernel<kF16>, grid, block, 0, s, ev, a);
  return hipGetLastError();
}

}  // namespace q4q8
