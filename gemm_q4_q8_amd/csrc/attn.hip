// Prefill attention on the matrix cores: tiles of queries against tiles of
// keys with an online softmax, so the S x S score matrix never exists in
// memory ("BaseRT: Best-in-Class LLM Inference on Apple Silicon via Native
// Metal", technical summary, "Methodologie", prefill optimisation; the M5
// review, "Method", routes this prefill attention to the matrix units).
//
// Per workgroup: 4 waves x 2 tiles of 16 queries of one (batch, query head);
// K and V of the matching key/value head (GQA: head h reads kv head
// h / (Hq / Hkv)) pass through two LDS buffers in blocks of 64 keys: the next
// block's loads are in flight while the current one is used (K straight to
// LDS by the buffer loads' LDS path, V through registers for the transpose),
// one barrier per block.  Each LDS fragment feeds both query tiles of a
// wave, and the two tiles' independent softmax and MFMA chains interleave.
// Per wave, tile and key block, with v_mfma_f32_16x16x32 on bf16 (or fp16)
// operands:
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
// Causal masking skips key blocks past the query block's last query and
// masks the diagonal blocks per element (in a separate instance of the block
// step); each workgroup takes a light and a heavy query block in turn.
#include "q4q8_dev.h"
#include "q4q8_internal.h"

#include <type_traits>

namespace q4q8 {

constexpr int kAttnD = 128;                  // head dimension
constexpr int kAttnWaves = 4;
// 16-query tiles per wave: QT (2, or 1 when the grid would leave CUs
// without a second workgroup); 16 QT kAttnWaves queries per workgroup.
constexpr int kAttnBN = 64;                  // keys per block
constexpr int kVStride = kAttnBN + 12;       // V^T rows in LDS (halfs; +8 measured slower)

struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  int32_t B, S, Hq, Hkv;
  int32_t causal;
  int32_t mblocks;    // query blocks per (batch, head)
  int32_t per_bh;     // workgroups per (batch, head)
  int32_t paired;     // causal pairing of query blocks i and mblocks - 1 - i
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

template <int DT, int QT>
__global__ __launch_bounds__(kAttnWaves * 64, 2) void attn_prefill_kernel(const AttnArgs a) {
  typedef typename Op<DT>::vec vec;
  constexpr int kAttnQT = QT;
  constexpr int kAttnBM = 16 * QT * kAttnWaves;   // queries per workgroup
  // Two buffers of K and V^T: block j + 1 is written while block j is read.
  // K: 16-byte column group cg of key k at slot 16 k + (cg ^ (k % 16)),
  // written by the buffer loads' LDS path (1 KB contiguous per wave
  // instruction, so no row padding: the XOR keeps the fragment reads on
  // distinct banks).  V^T: [d][key], rows kVStride halfs apart.
  __shared__ __attribute__((aligned(1024))) uint16_t ks_buf[2][kAttnBN * kAttnD];
  __shared__ __attribute__((aligned(16))) uint16_t vts_buf[2][kAttnD * kVStride];

  // Work split.  Paired (causal, enough work for two workgroups per CU):
  // workgroup i of a (batch, head) takes query blocks i and mblocks - 1 - i
  // (one if they coincide), so every workgroup carries about the same number
  // of key blocks wherever it runs; consecutive workgroups share a head.
  // Otherwise one query block each, and the dispatch order puts heavy blocks
  // first in the first half of the grid and light ones first in the second,
  // so workgroups b and b + half, which tend to share a CU, balance.
  const int bid = blockIdx.x;
  int pi, bh, nparts;
  if (a.paired) {
    pi = bid % a.per_bh;
    bh = bid / a.per_bh;
    nparts = pi != a.mblocks - 1 - pi ? 2 : 1;
  } else {
    const int total = gridDim.x, half = (total + 1) / 2;
    const int rank = bid < half ? bid : total - 1 - (bid - half);   // 0 = heaviest
    pi = a.mblocks - 1 - rank / (a.Hq * a.B);
    bh = rank % (a.Hq * a.B);
    nparts = 1;
  }
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
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int r = lane & 15, g = lane >> 4;
  // Per query block (set by the part loop below): its first query m0, the
  // wave's first query wq0, the key blocks it needs.
  int m0 = 0, wq0 = 0, nblocks = 0;
  vec qf[kAttnQT][kAttnD / 32];

  // K: global -> LDS by the buffer loads' LDS path, 4 copies of 16 bytes per
  // lane; copy p of wave w fills slots 64 (4 p + w) .. + 63.
  const __amdgpu_buffer_rsrc_t kres = uniform_rsrc(kb, (int)((int64_t)S * kvstride * 2));
  auto copy_k = [&](int blk, int buf) {
    const int n0 = blk * kAttnBN;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int slot = (4 * p + wave) * 64 + lane;
      const int key = slot >> 4, cg = (slot & 15) ^ (key & 15);
      const uint32_t off = n0 + key < S ? (uint32_t)(((int64_t)(n0 + key) * kvstride + cg * 8) * 2) : 0x80000000u;
      uint16_t* dst = ks_buf[buf] + (4 * p + wave) * 64 * 8;   // wave-uniform
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kres, (__attribute__((address_space(3))) void*)dst, 16, off, 0, 0,
                                               0);
    }
  };
  // V: global -> registers -> LDS transposed.  Thread t takes keys
  // 4 (t % 16) .. + 3 at d 8 (t / 16) .. + 7 and writes, for each d, the four
  // keys as one 8-byte word of V^T.
  const int vk0 = 4 * (tid & 15), vd0 = 8 * (tid >> 4);
  u32x4_t st[4];
  auto fetch_v = [&](int blk) {
    const int n0 = blk * kAttnBN;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int key = n0 + vk0 + i;
      st[i] = key < S ? *(const u32x4_t*)(vb + (int64_t)key * kvstride + vd0) : u32x4_t{0, 0, 0, 0};
    }
  };
  auto stash_v = [&](int buf) {
    uint16_t* vt = vts_buf[buf];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // Half j of the four keys' words: low halves (j even) or high halves.
      const int w = j >> 1;
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
      *(u32x2_t*)(vt + (vd0 + j) * kVStride + vk0) =
          u32x2_t{__builtin_amdgcn_perm(st[1][w], st[0][w], sel), __builtin_amdgcn_perm(st[3][w], st[2][w], sel)};
    }
  };

  float4_t acc_o[kAttnQT][kAttnD / 16];
  float m_run[kAttnQT], l_run[kAttnQT];

  // Per-lane LDS offsets (halfs): K fragment of key tile t, d step s at
  // 2048 t + kofs[s]; V^T fragment of d tile t, key step s at
  // 1216 t + 32 s + vofs (the rest folds into instruction offsets).
  int kofs[kAttnD / 32];
#pragma unroll
  for (int s = 0; s < kAttnD / 32; ++s) kofs[s] = 128 * r + 8 * ((4 * s + g) ^ r);
  const int vofs = r * kVStride + 4 * g;

  // One key block, read from LDS buffer blk % 2.  MASK: the block reaches
  // past S or the diagonal for some query of the workgroup (a separate
  // instance, so full blocks carry no mask arithmetic).
  auto block = [&](int blk, auto maskc) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(maskc)::value;
    const int BUF = blk & 1;
    if (blk + 1 < nblocks) {   // in flight during this block's math
      copy_k(blk + 1, BUF ^ 1);
      fetch_v(blk + 1);
    }
    const uint16_t* ks = ks_buf[BUF];
    const uint16_t* vts = vts_buf[BUF];

    // S^T for 64 keys x the wave's two 16-query tiles; each K fragment
    // serves both tiles.
    float4_t sc[kAttnQT][kAttnBN / 16];
#pragma unroll
    for (int t = 0; t < kAttnBN / 16; ++t) {
#pragma unroll
      for (int u = 0; u < kAttnQT; ++u) sc[u][t] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int s = 0; s < kAttnD / 32; ++s) {
        const vec kf = *(const vec*)(ks + 2048 * t + kofs[s]);
#pragma unroll
        for (int u = 0; u < kAttnQT; ++u) sc[u][t] = Op<DT>::mfma(kf, qf[u][s], sc[u][t]);
      }
    }
    const int n0 = blk * kAttnBN;
    vec pf[kAttnQT][kAttnBN / 32];
#pragma unroll
    for (int u = 0; u < kAttnQT; ++u) {
      if constexpr (MASK) {
        // Key n0 + 16 t + 4 g + v is visible to query qi when 16 t + v <= lim.
        const int qi = wq0 + 16 * u + r;
        const int lim = min(a.causal ? qi - n0 : kAttnBN, S - 1 - n0) - 4 * g;
#pragma unroll
        for (int t = 0; t < kAttnBN / 16; ++t)
#pragma unroll
          for (int v = 0; v < 4; ++v) sc[u][t][v] = 16 * t + v <= lim ? sc[u][t][v] : -INFINITY;
      }
      // Block max for the lane's query on the raw scores (scale > 0
      // commutes with max).
      float mx = -INFINITY;
#pragma unroll
      for (int t = 0; t < kAttnBN / 16; ++t)
        mx = fmaxf(fmaxf(mx, fmaxf(sc[u][t][0], sc[u][t][1])), fmaxf(sc[u][t][2], sc[u][t][3]));
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m_run[u], mx * a.scale_log2);
      const float m_use = m_new == -INFINITY ? 0.0f : m_new;   // a row with nothing visible yet
      const float alpha = __builtin_amdgcn_exp2f(m_run[u] - m_use);
      m_run[u] = m_new;
      // p = 2^(s * scale * log2 e - m): one FMA and one v_exp per score.
      float lsum = 0.0f;
      uint32_t pb[kAttnBN / 16][2];
#pragma unroll
      for (int t = 0; t < kAttnBN / 16; ++t) {
        float p[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          p[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[u][t][v], a.scale_log2, -m_use));
          lsum += p[v];
        }
        pb[t][0] = pack_rn<DT>(p[0], p[1]);
        pb[t][1] = pack_rn<DT>(p[2], p[3]);
      }
      l_run[u] = l_run[u] * alpha + lsum;
      if (__any(alpha != 1.0f)) {   // the max moved for some query of the tile
#pragma unroll
        for (int t = 0; t < kAttnD / 16; ++t) acc_o[u][t] *= alpha;
      }
#pragma unroll
      for (int s = 0; s < kAttnBN / 32; ++s)
        pf[u][s] = __builtin_bit_cast(vec, u32x4_t{pb[2 * s][0], pb[2 * s][1], pb[2 * s + 1][0], pb[2 * s + 1][1]});
    }

    // O^T += V^T P^T, two MFMA steps of 32 keys; each V^T fragment serves
    // both query tiles.
#pragma unroll
    for (int s = 0; s < kAttnBN / 32; ++s) {
#pragma unroll
      for (int t = 0; t < kAttnD / 16; ++t) {
        const uint16_t* vrow = vts + 16 * kVStride * t + 32 * s + vofs;
        const u32x2_t lo = *(const u32x2_t*)vrow;
        const u32x2_t hi = *(const u32x2_t*)(vrow + 16);
        const vec vf = __builtin_bit_cast(vec, u32x4_t{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
        for (int u = 0; u < kAttnQT; ++u) acc_o[u][t] = Op<DT>::mfma(vf, pf[u][s], acc_o[u][t]);
      }
    }
    // The other buffer was last read before the previous barrier.
    if (blk + 1 < nblocks) stash_v(BUF ^ 1);
    __syncthreads();   // also waits for the K copies of the next block
  };

  typedef std::integral_constant<bool, false> Full;
  typedef std::integral_constant<bool, true> Masked;
  for (int part = 0; part < nparts; ++part) {
    const int mb = part == 0 ? pi : a.mblocks - 1 - pi;
    m0 = mb * kAttnBM;
    wq0 = m0 + wave * 16 * kAttnQT;
    // Key blocks: all of them, or up to the last query of the block (causal).
    const int kend = a.causal ? min(S, m0 + kAttnBM) : S;
    nblocks = (kend + kAttnBN - 1) / kAttnBN;
    // The wave's Q^T fragments: tile u, lane (r, g) holds Q[q][32 s + 8 g ..
    // + 7] for its query q = wq0 + 16 u + r.
#pragma unroll
    for (int u = 0; u < kAttnQT; ++u) {
      const int qi = wq0 + 16 * u + r;
#pragma unroll
      for (int s = 0; s < kAttnD / 32; ++s) {
        u32x4_t t = u32x4_t{0, 0, 0, 0};
        if (qi < S) t = *(const u32x4_t*)(qb + (int64_t)qi * qstride + 32 * s + 8 * g);
        qf[u][s] = __builtin_bit_cast(vec, t);
      }
    }
#pragma unroll
    for (int u = 0; u < kAttnQT; ++u) {
      m_run[u] = -INFINITY;
      l_run[u] = 0.0f;
#pragma unroll
      for (int t = 0; t < kAttnD / 16; ++t) acc_o[u][t] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // Blocks before nfull need no mask for any query of the workgroup.
    const int nfull = min(S / kAttnBN, a.causal ? m0 / kAttnBN : nblocks);
    copy_k(0, 0);   // both buffers are free: the previous part ended on a barrier
    fetch_v(0);
    stash_v(0);
    __syncthreads();   // its fence also waits for the LDS copies
    int blk = 0;
    for (; blk < nfull; ++blk) block(blk, Full());
    for (; blk < nblocks; ++blk) block(blk, Masked());

    // Normalise and store: lane (r, g) writes O[q][16 t + 4 g .. + 3].
#pragma unroll
    for (int u = 0; u < kAttnQT; ++u) {
      float l = l_run[u];
      l += __shfl_xor(l, 16);
      l += __shfl_xor(l, 32);
      const float inv = 1.0f / l;
      const int qi = wq0 + 16 * u + r;
      if (qi < S) {
#pragma unroll
        for (int t = 0; t < kAttnD / 16; ++t) {
          const float4_t o = acc_o[u][t] * inv;
          *(u32x2_t*)(ob + (int64_t)qi * qstride + 16 * t + 4 * g) =
              u32x2_t{pack_rn<DT>(o[0], o[1]), pack_rn<DT>(o[2], o[3])};
        }
      }
    }
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
  // Two 16-query tiles per wave (every K / V^T fragment serves both), or one
  // when 128-query workgroups would not give every CU two of them (short
  // sequences: S 512, 32 heads is 128 workgroups) -- four for causal grids,
  // whose uneven blocks balance better in smaller pieces (measured, 32 heads:
  // S 512 22.9 -> 17.1 us; S 2048 causal 85 -> 79 us, non-causal 107 us kept
  // on two tiles, which one tile would take to 137 us).
  const int64_t wg128 = (int64_t)((S + 127) / 128) * Hq * B;
  const int qt = wg128 >= (causal ? 1024 : 512) ? 2 : 1;
  const int bm = 16 * qt * kAttnWaves;
  a.mblocks = (S + bm - 1) / bm;
  // Pair query blocks when the paired grid still fills two workgroups per CU
  // (measured: S 4096 causal 249 -> 230 us; at S 2048, 32 heads, pairing
  // would leave half the CU slots empty).
  a.paired = causal && (int64_t)((a.mblocks + 1) / 2) * Hq * B >= 512;
  a.per_bh = a.paired ? (a.mblocks + 1) / 2 : a.mblocks;
  a.scale_log2 = scale * 1.4426950408889634f;
  const dim3 grid((unsigned)(a.per_bh * Hq * B)), block(kAttnWaves * 64);
  if (qt == 2) {
    if (dt == kBF16) launch(attn_prefill_kernel<kBF16, 2>, grid, block, 0, s, ev, a);
    else launch(attn_prefill_kernel<kF16, 2>, grid, block, 0, s, ev, a);
  } else {
    if (dt == kBF16) launch(attn_prefill_kernel<kBF16, 1>, grid, block, 0, s, ev, a);
    else launch(attn_prefill_kernel<kF16, 1>, grid, block, 0, s, ev, a);
  }
  return hipGetLastError();
}

}  // namespace q4q8
