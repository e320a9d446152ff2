// Prefill attention on the matrix cores: tiles of queries against tiles of
// keys with an online softmax, so the S x S score matrix never exists in
// memory ("BaseRT: Best-in-Class LLM Inference on Apple Silicon via Native
// Metal", technical summary, "Methodologie", prefill optimisation; the M5
// review, "Method", routes this prefill attention to the matrix units).
//
// Per workgroup: 4 waves x 2 (or 1) tiles of 16 queries of one (batch, query
// head); K and V of the matching key/value head (GQA: head h reads kv head
// h / (Hq / Hkv)) pass through two LDS buffers in blocks of 64 keys: the next
// block's loads are in flight while the current one is used (both straight
// to LDS by the buffer loads' LDS path, V read back transposed), one barrier
// per block.  Each LDS fragment feeds both query tiles of a wave, and the two
// tiles' independent softmax and MFMA chains interleave.  Causal grids too
// small to give every CU two 4-wave workgroups run two such groups of 4 waves
// per workgroup over the two halves of every query block's key range, merged
// at the end; with two tiles a wave and paired query blocks, the first group
// runs the light block whole and then the heavy block's first key blocks,
// the second group the rest of the heavy one, and only the heavy block is
// merged (the K / V copies run on across the switch, its Q waits in LDS).
// Per wave, tile and key block, with v_mfma_f32_16x16x32 on bf16 (or fp16)
// operands:
//   * S^T = K Q^T  (A = K rows from LDS, B = the wave's Q^T held in
//     registers).  Lane (r, g) ends up with the scores of query r against
//     keys 16 t + 4 g + v, i.e. every lane's values belong to one query, so
//     the running max needs only the 4 lanes r, r+16, r+32, r+48;
//   * P^T = exp2(S^T * scale * log2 e - m) rounded to the operand type is
//     already the B operand of O^T = V^T P^T when the 32 keys of an MFMA
//     step are taken in the order (4 g .. 4 g + 3, 16 + 4 g .. 16 + 4 g + 3)
//     for lane group g; V stays [key][d] in LDS and the transposed LDS read
//     gives the A operand those keys as two runs of four;
//   * O^T accumulates in fp32 (lane (r, g) holds O[query r][d 16 t + 4 g + v])
//     and is rescaled by exp2(m_old - m_new) when the reference max moves
//     (only by more than a fixed headroom, so rarely); the row sums come
//     from one more MFMA per key step against a V^T tile of ones.
// Causal masking skips key blocks past the query block's last query and
// masks the diagonal blocks per element (in a separate instance of the block
// step); in paired grids each workgroup takes a light and a heavy query
// block in turn.
#include "q4q8_dev.h"
#include "q4q8_internal.h"

#include <type_traits>

namespace q4q8 {

constexpr int kAttnD = 128;                  // head dimension
constexpr int kAttnWaves = 4;
// 16-query tiles per wave: QT (2, or 1 when the grid would leave CUs
// without a second workgroup); 16 QT kAttnWaves queries per workgroup.
constexpr int kAttnBN = 64;                  // keys per block
// Headroom of the softmax's reference max (log2 units): P values stay at or
// below 2^8, well inside the fp16 and bf16 operand ranges.
constexpr float kAttnSlack = 8.0f;

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

// Transposed LDS read of four 16-bit values (ds_read_b64_tr_b16).
__device__ __forceinline__ u32x2_t read_tr16(const uint16_t* p) {
  typedef short short4_t __attribute__((ext_vector_type(4)));
  return __builtin_bit_cast(
      u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) short4_t*)(p)));
}

// max(a, b) and max(a, b, c) that return NaN if any operand is NaN
// (v_maximum_f32 / v_maximum3_f32; fmaxf would first canonicalise every
// operand that comes out of an MFMA).
__device__ __forceinline__ float maxf(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float max3f(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}

// max over lanes l, l ^ 16, l ^ 32 and l ^ 48 (the four lanes that hold one
// query's scores) by the cross-lane swap instructions, which stay in the
// VALU: v_permlane16_swap of a value with itself gives rows (0, 0, 2, 2) and
// (1, 1, 3, 3) of 16 lanes, v_permlane32_swap halves (0, 0) and (1, 1).
__device__ __forceinline__ float max_lanes4(float m) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  m = maxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(m), __float_as_uint(m), false, false);
  return maxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// KS groups of kAttnWaves waves per workgroup.  KS = 2 splits every query
// block's key range between the groups (group 0 the first half of the key
// blocks, group 1 the rest, both over the same queries, each with its own K/V
// buffers), and group 1 merges group 0's partial O, max and sum through LDS at
// the end: a causal grid of 128-query blocks then fills every CU once with two
// waves a SIMD while each wave keeps two query tiles.
template <int DT, int QT, int KS>
__global__ __launch_bounds__(kAttnWaves * 64 * KS, KS == 1 ? 2 : 1) void attn_prefill_kernel(const AttnArgs a) {
  typedef typename Op<DT>::vec vec;
  constexpr uint32_t kOnes2 = DT == kBF16 ? 0x3F803F80u : 0x3C003C00u;   // (1, 1) in the operand type
  constexpr int kAttnQT = QT;
  constexpr int kAttnBM = 16 * QT * kAttnWaves;   // queries per workgroup
  // Two buffers of K and V per group: block j + 1 is written while block j is
  // read, both by the buffer loads' LDS path (1 KB contiguous per wave
  // instruction, so rows cannot be padded; XOR swizzles of the 16-byte column
  // groups keep the fragment reads on distinct banks).  K: column group cg of
  // key k at slot 16 k + (cg ^ (k % 16)).  V: column group cg of key k at slot
  // 16 k + (cg ^ 2 (k % 8)), read transposed (ds_read_b64_tr_b16).
  // kv_lds[group][0: K, 1: V][buffer].
  __shared__ __attribute__((aligned(1024))) uint16_t kv_lds[KS][2][2][kAttnBN * kAttnD];
  // The paired two-group form (KS = 2, two tiles a wave) keeps the heavy
  // query block's Q here: 16-byte column group cg of query row q (of the
  // block) at slot 16 q + (cg ^ (q % 16)).
  constexpr bool kSeg = KS == 2 && QT == 2;
  __shared__ __attribute__((aligned(1024))) uint16_t q_lds[kSeg ? kAttnBM * kAttnD : 8];

  // Work split.  Paired (causal, enough work for two workgroups per CU):
  // workgroup i of a (batch, head) takes query blocks i and mblocks - 1 - i
  // (one if they coincide), so every workgroup carries about the same number
  // of key blocks wherever it runs; consecutive workgroups share a head.
  // Otherwise one query block each, and the dispatch order puts heavy blocks
  // first in the first half of the grid and light ones first in the second,
  // so workgroups b and b + half, which tend to share a CU, balance.
  // Workgroup i runs on XCD i % 8: with the paired split each XCD takes a
  // contiguous range of (batch, head) pairs, so a key/value head's K and V
  // stay in one XCD's L2 (measured: S 2048 causal 80.6 -> 77.3 us).
  int bid = blockIdx.x;
  if (a.paired && gridDim.x % 8 == 0) bid = (bid % 8) * (gridDim.x / 8) + bid / 8;
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
  const int grp = wave / kAttnWaves, wv = wave % kAttnWaves;   // key group, wave in the group
  const int r = lane & 15, g = lane >> 4;
  // Per query block (set by the part loop below): its first query m0, the
  // wave's first query wq0, the key blocks it needs.
  int m0 = 0, wq0 = 0, nblocks = 0;
  vec qf[kAttnQT][kAttnD / 32];

  // K and V of key block blk are read through a buffer resource that starts
  // at the block's first key and ends at key S - 1, so keys past S read zero
  // by the resource's range check and the per-lane offsets stay fixed.
  auto block_rsrc = [&](const uint16_t* base, int blk) __attribute__((always_inline)) {
    const int n0 = blk * kAttnBN;
    return uniform_rsrc(base + (int64_t)n0 * kvstride, (int)((int64_t)min(S - n0, kAttnBN) * kvstride * 2));
  };
  // K: global -> LDS by the buffer loads' LDS path, 4 copies of 16 bytes per
  // lane; copy p of wave w (of the group) fills slots 64 (4 p + w) .. + 63,
  // i.e. key 16 p + 4 w + g of the block, column group r ^ (key % 16).
  uint32_t koff[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int key = 16 * p + 4 * wv + g, cg = r ^ (key & 15);
    koff[p] = (uint32_t)((key * kvstride + cg * 8) * 2);
  }
  auto copy_k = [&](int blk, int buf) {
    const __amdgpu_buffer_rsrc_t kres = block_rsrc(kb, blk);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint16_t* dst = kv_lds[grp][0][buf] + (4 * p + wv) * 64 * 8;   // wave-uniform
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kres, (__attribute__((address_space(3))) void*)dst, 16, koff[p], 0,
                                               0, 0);
    }
  };
  // V: the same copies as K with V's swizzle: slot 16 key + r holds column
  // group r ^ 2 (key % 8) of key 16 p + 4 w + g.
  uint32_t voff[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int key = 16 * p + 4 * wv + g, cg = r ^ (2 * (key & 7));
    voff[p] = (uint32_t)((key * kvstride + cg * 8) * 2);
  }
  auto copy_v = [&](int blk, int buf) {
    const __amdgpu_buffer_rsrc_t vres = block_rsrc(vb, blk);
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      uint16_t* dst = kv_lds[grp][1][buf] + (4 * p + wv) * 64 * 8;   // wave-uniform
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vres, (__attribute__((address_space(3))) void*)dst, 16, voff[p], 0,
                                               0, 0);
    }
  };

  float4_t acc_o[kAttnQT][kAttnD / 16];
  // Row sums of P by the matrix cores: O^T's extra tile with V^T all ones
  // (every register of lane (r, g) then holds the sum for query r, taken over
  // the rounded P that the product uses).
  float4_t acc_l[kAttnQT];
  float m_run[kAttnQT];
  const vec ones = __builtin_bit_cast(vec, u32x4_t{kOnes2, kOnes2, kOnes2, kOnes2});

  // Per-lane LDS offsets (halfs): K fragment of key tile t, d step s at
  // 2048 t + kofs[s]; V fragment of d tile t, keys 32 s + 16 h + .. at
  // 4096 s + 2048 h + vofs[t] (the rest folds into instruction offsets).
  int kofs[kAttnD / 32];
#pragma unroll
  for (int s = 0; s < kAttnD / 32; ++s) kofs[s] = 128 * r + 8 * ((4 * s + g) ^ r);
  // The transposed read: in each 16-lane group, lane 4 i + q names four
  // adjacent halfs of row i of a 4 x 16 block, and lane j receives column j,
  // rows 0..3.  Lane (r, g) names key 4 g + i (i = r / 4), d 16 t + 4 q
  // (q = r % 4), so it receives V[4 g + 0..3][16 t + r]: the A operand's keys
  // 4 g .. 4 g + 3 of V^T (and, 16 keys on, 16 + 4 g ..), in the key order
  // the P^T operand uses.
  int vofs[kAttnD / 16];
#pragma unroll
  for (int t = 0; t < kAttnD / 16; ++t) {
    const int key = 4 * g + (r >> 2), q = r & 3;
    vofs[t] = key * kAttnD + (((2 * t + (q >> 1)) ^ (2 * (key & 7))) * 8) + (q & 1) * 4;
  }

  // One key block, read from LDS buffer blk % 2.  MASK: the block reaches
  // past S or the diagonal for some query of the workgroup (a separate
  // instance, so full blocks carry no mask arithmetic).
  // bend: the end of this group's key blocks.
  // BUF: the LDS buffers holding block blk; nxt: the key block the group
  // takes next (copied into the other buffers during this one), or -1.
  auto block = [&](int blk, int BUF, int nxt, auto maskc) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(maskc)::value;
    if (nxt >= 0) {   // in flight during this block's math
      copy_k(nxt, BUF ^ 1);
      copy_v(nxt, BUF ^ 1);
    }
    const uint16_t* ks = kv_lds[grp][0][BUF];
    const uint16_t* vsb = kv_lds[grp][1][BUF];

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
      // commutes with max).  The NaN-propagating maximum takes three operands
      // per instruction with no canonicalising moves in front (a NaN score
      // makes its row NaN either way).
      float mx = max3f(sc[u][0][0], sc[u][0][1], sc[u][0][2]);
      mx = max3f(mx, sc[u][0][3], sc[u][1][0]);
      mx = max3f(mx, sc[u][1][1], sc[u][1][2]);
      mx = max3f(mx, sc[u][1][3], sc[u][2][0]);
      mx = max3f(mx, sc[u][2][1], sc[u][2][2]);
      mx = max3f(mx, sc[u][2][3], sc[u][3][0]);
      mx = max3f(mx, sc[u][3][1], sc[u][3][2]);
      mx = maxf(mx, sc[u][3][3]);
      mx = max_lanes4(mx);
      // The reference max m moves only when the block's max exceeds it by
      // more than kAttnSlack (log2 units), so p <= 2^kAttnSlack and most
      // blocks skip the rescale of O; O and the row sum share m, so the
      // quotient is unchanged.
      const float m_cand = maxf(m_run[u], mx * a.scale_log2);
      const bool move = m_cand > m_run[u] + kAttnSlack;   // m = -inf: any finite max moves it
      const float m_new = move ? m_cand : m_run[u];
      const float m_use = m_new == -INFINITY ? 0.0f : m_new;   // a row with nothing visible yet
      const float alpha = move ? __builtin_amdgcn_exp2f(m_run[u] - m_use) : 1.0f;
      m_run[u] = m_new;
      // p = 2^(s * scale * log2 e - m): one FMA and one v_exp per score.
      uint32_t pb[kAttnBN / 16][2];
#pragma unroll
      for (int t = 0; t < kAttnBN / 16; ++t) {
        float p[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) p[v] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[u][t][v], a.scale_log2, -m_use));
        pb[t][0] = pack_rn<DT>(p[0], p[1]);
        pb[t][1] = pack_rn<DT>(p[2], p[3]);
      }
      if (__any(move)) {   // the reference max moved for some query of the tile
#pragma unroll
        for (int t = 0; t < kAttnD / 16; ++t) acc_o[u][t] *= alpha;
        acc_l[u] *= alpha;
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
        const u32x2_t lo = read_tr16(vsb + 4096 * s + vofs[t]);
        const u32x2_t hi = read_tr16(vsb + 4096 * s + 2048 + vofs[t]);
        const vec vf = __builtin_bit_cast(vec, u32x4_t{lo[0], lo[1], hi[0], hi[1]});
#pragma unroll
        for (int u = 0; u < kAttnQT; ++u) acc_o[u][t] = Op<DT>::mfma(vf, pf[u][s], acc_o[u][t]);
      }
#pragma unroll
      for (int u = 0; u < kAttnQT; ++u) acc_l[u] = Op<DT>::mfma(ones, pf[u][s], acc_l[u]);
    }
    __syncthreads();   // also waits for the K and V copies of the next block
  };

  typedef std::integral_constant<bool, false> Full;
  typedef std::integral_constant<bool, true> Masked;
  if constexpr (kSeg) {
    // Paired blocks L = pi (light; absent when it is the middle block) and
    // H = mblocks - 1 - pi (heavy) of one (batch, head).  Group 0 takes all
    // of L's key blocks, then H's first pH; group 1 the rest of H's, so both
    // carry about the same number; only H's two partial results are merged.
    // The K / V copies run on across group 0's switch from L to H (the same
    // head's keys), and H's Q comes from LDS, so the switch costs no load
    // latency.
    const int mbH = a.mblocks - 1 - pi;
    const bool hasL = nparts == 2;
    const int m0L = pi * kAttnBM, m0H = mbH * kAttnBM;
    const int nL = hasL ? (min(S, m0L + kAttnBM) + kAttnBN - 1) / kAttnBN : 0;
    const int nH = (min(S, m0H + kAttnBM) + kAttnBN - 1) / kAttnBN;
    const int nfullL = min(S / kAttnBN, m0L / kAttnBN), nfullH = min(S / kAttnBN, m0H / kAttnBN);
    const int pH = max(0, (nH - nL) / 2);
    const int mysteps = grp == 0 ? nL + pH : nH - pH;
    const int nsteps = max(nL + pH, nH - pH);
    auto kb_of = [&](int i) __attribute__((always_inline)) { return grp == 0 ? (i < nL ? i : i - nL) : pH + i; };

    // H's Q into LDS (rows past S read zero), copy p of wave w at slots
    // 64 (8 p + w) .. + 63.
    {
      const __amdgpu_buffer_rsrc_t qres =
          uniform_rsrc(qb + (int64_t)m0H * qstride, (int)((int64_t)min(S - m0H, kAttnBM) * qstride * 2));
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int slot = (8 * p + wave) * 64 + lane;
        const int qrow = slot >> 4, cg = (slot & 15) ^ (qrow & 15);
        uint16_t* dst = q_lds + (8 * p + wave) * 64 * 8;   // wave-uniform
        __builtin_amdgcn_raw_ptr_buffer_load_lds(qres, (__attribute__((address_space(3))) void*)dst, 16,
                                                 (uint32_t)((qrow * qstride + cg * 8) * 2), 0, 0, 0);
      }
    }
    auto q_from_lds = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < kAttnQT; ++u) {
        const int qrow = wv * 16 * kAttnQT + 16 * u + r;
#pragma unroll
        for (int s2 = 0; s2 < kAttnD / 32; ++s2)
          qf[u][s2] = *(const vec*)(q_lds + (qrow * 16 + ((4 * s2 + g) ^ (qrow & 15))) * 8);
      }
    };
    auto reset = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < kAttnQT; ++u) {
        m_run[u] = -INFINITY;
        acc_l[u] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int t = 0; t < kAttnD / 16; ++t) acc_o[u][t] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
      }
    };
    // Normalise and store the wave's tiles of the query block at m0.
    auto store_o = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int u = 0; u < kAttnQT; ++u) {
        const float inv = 1.0f / acc_l[u][0];
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
    };
    const bool startL = grp == 0 && hasL;
    m0 = startL ? m0L : m0H;
    wq0 = m0 + wv * 16 * kAttnQT;
    if (startL) {   // L's Q from global memory (the barrier below waits for it)
#pragma unroll
      for (int u = 0; u < kAttnQT; ++u) {
        const int qi = wq0 + 16 * u + r;
#pragma unroll
        for (int s2 = 0; s2 < kAttnD / 32; ++s2) {
          u32x4_t t = u32x4_t{0, 0, 0, 0};
          if (qi < S) t = *(const u32x4_t*)(qb + (int64_t)qi * qstride + 32 * s2 + 8 * g);
          qf[u][s2] = __builtin_bit_cast(vec, t);
        }
      }
    }
    reset();
    if (mysteps > 0) {
      copy_k(kb_of(0), 0);
      copy_v(kb_of(0), 0);
    }
    __syncthreads();   // its fence also waits for the LDS copies (Q of H included)
    if (!startL) q_from_lds();
    // Two segments a group: group 0 runs L's blocks, then H's first pH;
    // group 1 runs H's from pH on (its second segment is empty).  Each
    // segment is a loop over blocks without a mask, then one over masked.
    int i = 0;   // step count: the K/V buffer parity
#pragma unroll 1
    for (int seg = 0; seg < 2; ++seg) {
      const bool segL = grp == 0 && seg == 0;
      const int kb0 = grp == 0 ? 0 : (seg == 0 ? pH : nH);
      const int kb1 = grp == 0 ? (seg == 0 ? nL : pH) : nH;
      const int nfull = segL ? nfullL : nfullH;
      const int nxt_after = segL && pH > 0 ? 0 : -1;
      const int f1 = min(max(nfull, kb0), kb1);
      for (int j = kb0; j < f1; ++j, ++i) block(j, i & 1, j + 1 < kb1 ? j + 1 : nxt_after, Full());
      for (int j = f1; j < kb1; ++j, ++i) block(j, i & 1, j + 1 < kb1 ? j + 1 : nxt_after, Masked());
      if (segL && hasL) {   // L done: store it, continue with H
        store_o();
        reset();
        q_from_lds();
        m0 = m0H;
        wq0 = m0 + wv * 16 * kAttnQT;
      }
    }
    for (; i < nsteps; ++i) __syncthreads();   // one barrier per step of the other group
    // Group 0 hands its partial O of H (relative to its reference max), max
    // and sum to group 1 through the LDS (group 0's K/V buffers for O, group
    // 1's for the max and sum; every block read ended on the last barrier).
    float4_t* po = (float4_t*)&kv_lds[0][0][0][0];
    float2_t* pml = (float2_t*)&kv_lds[1][0][0][0];
    if (grp == 0) {
#pragma unroll
      for (int u = 0; u < kAttnQT; ++u) {
#pragma unroll
        for (int t = 0; t < kAttnD / 16; ++t) po[((wv * kAttnQT + u) * (kAttnD / 16) + t) * 64 + lane] = acc_o[u][t];
        pml[(wv * kAttnQT + u) * 64 + lane] = float2_t{m_run[u], acc_l[u][0]};
      }
    }
    __syncthreads();
    if (grp == 1) {
#pragma unroll
      for (int u = 0; u < kAttnQT; ++u) {
        const float2_t ml = pml[(wv * kAttnQT + u) * 64 + lane];
        const float m = maxf(ml[0], m_run[u]);
        const float f0 = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ml[0] - m);
        const float f1 = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run[u] - m);
        acc_l[u][0] = acc_l[u][0] * f1 + ml[1] * f0;
#pragma unroll
        for (int t = 0; t < kAttnD / 16; ++t)
          acc_o[u][t] = acc_o[u][t] * f1 + po[((wv * kAttnQT + u) * (kAttnD / 16) + t) * 64 + lane] * f0;
      }
      store_o();
    }
    return;
  }
  for (int part = 0; part < nparts; ++part) {
    const int mb = part == 0 ? pi : a.mblocks - 1 - pi;
    m0 = mb * kAttnBM;
    wq0 = m0 + wv * 16 * kAttnQT;
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
      acc_l[u] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int t = 0; t < kAttnD / 16; ++t) acc_o[u][t] = float4_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
    // Blocks before nfull need no mask for any query of the workgroup.
    const int nfull = min(S / kAttnBN, a.causal ? m0 / kAttnBN : nblocks);
    // This group's key blocks [b0, b1); both groups take nsteps steps (one
    // barrier each), group 0 idling through its last one when it has fewer.
    const int ksplit = KS == 2 ? nblocks / 2 : nblocks;
    const int b0 = grp == 0 ? 0 : ksplit, b1 = grp == 0 ? ksplit : nblocks;
    const int nsteps = KS == 2 ? nblocks - ksplit : nblocks;
    if (b0 < b1) {   // both buffers are free: the previous part ended on a barrier
      copy_k(b0, b0 & 1);
      copy_v(b0, b0 & 1);
    }
    __syncthreads();   // its fence also waits for the LDS copies
    int blk = b0;
    for (; blk < min(b1, nfull); ++blk) block(blk, blk & 1, blk + 1 < b1 ? blk + 1 : -1, Full());
    for (; blk < b1; ++blk) block(blk, blk & 1, blk + 1 < b1 ? blk + 1 : -1, Masked());
    for (int i = b1 - b0; i < nsteps; ++i) __syncthreads();   // one barrier per step of the other group

    bool store = true;
    if constexpr (KS == 2) {
      // Group 0 hands its partial O (relative to its reference max), max and
      // sum to group 1 through the LDS (its own K/V buffers for O, group 1's
      // for the max and sum; every block read ended on the last barrier).
      float4_t* po = (float4_t*)&kv_lds[0][0][0][0];
      float2_t* pml = (float2_t*)&kv_lds[1][0][0][0];
      if (grp == 0) {
#pragma unroll
        for (int u = 0; u < kAttnQT; ++u) {
#pragma unroll
          for (int t = 0; t < kAttnD / 16; ++t) po[((wv * kAttnQT + u) * (kAttnD / 16) + t) * 64 + lane] = acc_o[u][t];
          pml[(wv * kAttnQT + u) * 64 + lane] = float2_t{m_run[u], acc_l[u][0]};
        }
      }
      __syncthreads();
      if (grp == 1) {
#pragma unroll
        for (int u = 0; u < kAttnQT; ++u) {
          const float2_t ml = pml[(wv * kAttnQT + u) * 64 + lane];
          const float m = maxf(ml[0], m_run[u]);
          // exp2(-inf) = 0 drops a group that saw no key of the row; a row
          // that saw none at all (past S) is not stored.
          const float f0 = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(ml[0] - m);
          const float f1 = m == -INFINITY ? 0.0f : __builtin_amdgcn_exp2f(m_run[u] - m);
          acc_l[u][0] = acc_l[u][0] * f1 + ml[1] * f0;
#pragma unroll
          for (int t = 0; t < kAttnD / 16; ++t)
            acc_o[u][t] = acc_o[u][t] * f1 + po[((wv * kAttnQT + u) * (kAttnD / 16) + t) * 64 + lane] * f0;
        }
      }
      store = grp == 1;
    }

    // Normalise and store: lane (r, g) writes O[q][16 t + 4 g .. + 3].
    if (store) {
#pragma unroll
      for (int u = 0; u < kAttnQT; ++u) {
        const float inv = 1.0f / acc_l[u][0];
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
    if constexpr (KS == 2) __syncthreads();   // the merge's LDS reads end before the next part's copies
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
  // Grid choice, in order: the two key-split forms for causal grids that
  // would otherwise leave CUs with one 4-wave workgroup or none, then the
  // one-group form (KS = 1).
  const int64_t wg128 = (int64_t)((S + 127) / 128) * Hq * B;
  a.scale_log2 = scale * 1.4426950408889634f;
  // Causal grids whose paired 128-query blocks give every CU one 8-wave
  // workgroup, but not two 4-wave ones, split their key ranges between two
  // wave groups (KS = 2; measured, S 2048, 32 heads: 51.5 -> 45.5 us against
  // one tile a wave in paired 64-query workgroups, medians of five runs).
  const int64_t pairs128 = (int64_t)((S + 255) / 256) * Hq * B;
  if (causal && pairs128 >= 256 && pairs128 < 512) {
    a.mblocks = (S + 127) / 128;
    a.paired = 1;
    a.per_bh = (a.mblocks + 1) / 2;
    const dim3 grid((unsigned)(a.per_bh * Hq * B)), block(2 * kAttnWaves * 64);
    if (dt == kBF16) launch(attn_prefill_kernel<kBF16, 2, 2>, grid, block, 0, s, ev, a);
    else launch(attn_prefill_kernel<kF16, 2, 2>, grid, block, 0, s, ev, a);
    return hipGetLastError();
  }
  // Small causal grids (64-query blocks give at most one workgroup per CU):
  // one tile a wave, two wave groups over each block's key range.
  const int64_t wg64 = (int64_t)((S + 63) / 64) * Hq * B;
  if (causal && wg64 <= 256) {
    a.mblocks = (S + 63) / 64;
    a.paired = 0;
    a.per_bh = a.mblocks;
    const dim3 grid((unsigned)(a.per_bh * Hq * B)), block(2 * kAttnWaves * 64);
    if (dt == kBF16) launch(attn_prefill_kernel<kBF16, 1, 2>, grid, block, 0, s, ev, a);
    else launch(attn_prefill_kernel<kF16, 1, 2>, grid, block, 0, s, ev, a);
    return hipGetLastError();
  }
  // One group: two 16-query tiles per wave (every K / V^T fragment serves
  // both), or one when 128-query workgroups would not give every CU two of
  // them -- four for causal grids, whose uneven blocks balance better in
  // smaller pieces (measured, 32 heads: S 512 22.9 -> 17.1 us; non-causal
  // S 2048 107 us kept on two tiles, which one tile would take to 137 us).
  const int qt = wg128 >= (causal ? 1024 : 512) ? 2 : 1;
  const int bm = 16 * qt * kAttnWaves;
  a.mblocks = (S + bm - 1) / bm;
  // Pair query blocks when the paired grid still fills two workgroups per CU
  // (measured: S 4096 causal 249 -> 230 us; at S 2048, 32 heads, pairing
  // would leave half the CU slots empty).
  a.paired = causal && (int64_t)((a.mblocks + 1) / 2) * Hq * B >= 512;
  a.per_bh = a.paired ? (a.mblocks + 1) / 2 : a.mblocks;
  const dim3 grid((unsigned)(a.per_bh * Hq * B)), block(kAttnWaves * 64);
  if (qt == 2) {
    if (dt == kBF16) launch(attn_prefill_kernel<kBF16, 2, 1>, grid, block, 0, s, ev, a);
    else launch(attn_prefill_kernel<kF16, 2, 1>, grid, block, 0, s, ev, a);
  } else {
    if (dt == kBF16) launch(attn_prefill_kernel<kBF16, 1, 1>, grid, block, 0, s, ev, a);
    else launch(attn_prefill_kernel<kF16, 1, 1>, grid, block, 0, s, ev, a);
  }
  return hipGetLastError();
}

}  // namespace q4q8
