// Load-time conversion of canonical Q4_0 / Q8_0 blocks (and plain fp16
// weights) into the gfx950 tile layout described in q4q8_dev.h.  The runtime on the pages converts
// checkpoints once into its own weight format ("BaseRT: Advancing
// Best-in-Class LLM Inference with Apple M5 Neural Accelerators", review,
// section "Comparison"); this is that step for MI355X.  Only bytes move: the
// fp16 scales and the codes are copied unchanged, the codes are reordered.
#include "q4q8_dev.h"
#include "q4q8_internal.h"

namespace q4q8 {

// Write lane slot `slot` of record (tile, chunk) -- its codes, and for
// slots 0..15 the four scales of row `slot` -- from canonical blocks.
// Shared verbatim by the device kernel and the host conversion.
template <int FMT>
__host__ __device__ inline void repack_slot(const uint8_t* canon, uint8_t* rec, int64_t N, int64_t K,
                                            int64_t tile, int64_t chunk, int slot) {
  constexpr int CB = Fmt<FMT>::kCanonBlock;
  const int r = slot & 15, g = slot >> 4;
  const int64_t n = tile * kTileRows + r;
  const int64_t nblocks = K / 32;
  for (int j = 0; j < kBlocksPerChunk; ++j) {
    const int64_t blk = chunk * kBlocksPerChunk + j;
    const bool valid = n < N && blk < nblocks;
    const uint8_t* b = canon + (n * nblocks + blk) * CB;
    if (FMT == kFP16W) {   // 8 weights (16 bytes) of row n, block blk, elements 8 g .. 8 g + 7
      uint8_t* dst = rec + j * 1024 + slot * 16;
      for (int e = 0; e < 16; ++e) dst[e] = valid ? b[16 * g + e] : 0;
      continue;
    }
    if (FMT == kQ4_0) {
      uint32_t word = 0;
      if (valid) {
        for (int e = 0; e < 8; ++e) {
          const int i = 8 * g + e;  // element within the block
          const uint32_t q = i < 16 ? (b[2 + i] & 0xFu) : (b[2 + i - 16] >> 4);
          word |= q << q4_nibble_shift(e);
        }
      }
      uint8_t* dst = rec + slot * 16 + 4 * j;
      for (int t = 0; t < 4; ++t) dst[t] = (uint8_t)(word >> (8 * t));
    } else {
      uint8_t* dst = rec + (j >> 1) * 1024 + slot * 16 + (j & 1) * 8;
      for (int e = 0; e < 8; ++e) dst[e] = valid ? b[2 + 8 * g + e] : 0;
    }
    if (g == 0) {
      uint8_t* sc = rec + Fmt<FMT>::kCodeBytes + r * 8 + j * 2;
      sc[0] = valid ? b[0] : 0;
      sc[1] = valid ? b[1] : 0;
    }
  }
}

template <int FMT>
__global__ __launch_bounds__(256) void repack_kernel(const uint8_t* __restrict__ canon, uint8_t* __restrict__ dst,
                                                     int64_t N, int64_t K, int64_t nchunks, int64_t nslots) {
  const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (gid >= nslots) return;
  const int slot = (int)(gid & 63);
  const int64_t rec = gid >> 6;
  const int64_t tile = rec / nchunks, chunk = rec % nchunks;
  repack_slot<FMT>(canon, dst + rec * Fmt<FMT>::kRecBytes, N, K, tile, chunk, slot);
}

hipError_t launch_repack(int fmt, const void* canon, int64_t N, int64_t K, void* dst, hipStream_t stream) {
  const int64_t tiles = (N + kTileRows - 1) / kTileRows;
  const int64_t nchunks = (K + kChunkK - 1) / kChunkK;
  const int64_t nslots = tiles * nchunks * 64;
  const int64_t grid = (nslots + 255) / 256;
  if (fmt == kQ4_0)
    repack_kernel<kQ4_0><<<dim3((unsigned)grid), dim3(256), 0, stream>>>((const uint8_t*)canon, (uint8_t*)dst, N, K,
                                                                         nchunks, nslots);
  else if (fmt == kQ8_0)
    repack_kernel<kQ8_0><<<dim3((unsigned)grid), dim3(256), 0, stream>>>((const uint8_t*)canon, (uint8_t*)dst, N, K,
                                                                         nchunks, nslots);
  else
    repack_kernel<kFP16W><<<dim3((unsigned)grid), dim3(256), 0, stream>>>((const uint8_t*)canon, (uint8_t*)dst, N,
                                                                          K, nchunks, nslots);
  return hipGetLastError();
}

void repack_host(int fmt, const void* canon, int64_t N, int64_t K, void* dst) {
  const int64_t tiles = (N + kTileRows - 1) / kTileRows;
  const int64_t nchunks = (K + kChunkK - 1) / kChunkK;
  const int rb = fmt == kQ4_0 ? Fmt<kQ4_0>::kRecBytes : fmt == kQ8_0 ? Fmt<kQ8_0>::kRecBytes : Fmt<kFP16W>::kRecBytes;
  for (int64_t rec = 0; rec < tiles * nchunks; ++rec) {
    uint8_t* out = (uint8_t*)dst + rec * rb;
    for (int slot = 0; slot < 64; ++slot) {
      if (fmt == kQ4_0)
        repack_slot<kQ4_0>((const uint8_t*)canon, out, N, K, rec / nchunks, rec % nchunks, slot);
      else if (fmt == kQ8_0)
        repack_slot<kQ8_0>((const uint8_t*)canon, out, N, K, rec / nchunks, rec % nchunks, slot);
      else
        repack_slot<kFP16W>((const uint8_t*)canon, out, N, K, rec / nchunks, rec % nchunks, slot);
    }
  }
}

}  // namespace q4q8
