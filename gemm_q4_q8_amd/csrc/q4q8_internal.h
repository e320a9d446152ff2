// Host-side declarations shared by the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4q8 {

constexpr int kMaxGroup = 8;

// One GEMV problem as the kernel sees it (tile0: first global tile index).
struct GemvProb {
  const uint8_t* W;
  const uint16_t* x;
  float* y;
  int64_t ldx, ldy;
  int32_t N, K;
  int32_t tile0;
  int32_t pad;
};

struct GemvArgs {
  GemvProb p[kMaxGroup];
  int32_t count;
  int32_t M;
  int32_t total_tiles;
  int32_t pad;
};

hipError_t launch_repack(int fmt, const void* canon, int64_t N, int64_t K, void* dst, hipStream_t stream);
void repack_host(int fmt, const void* canon, int64_t N, int64_t K, void* dst);

hipError_t launch_qgemv(int fmt, int xdt, const GemvArgs& args, int max_chunks, hipStream_t stream);

hipError_t launch_qgemm(int fmt, int xdt, int ydt, const void* W, int64_t N, int64_t K, const void* X, int64_t ldx,
                        int64_t M, void* Y, int64_t ldy, hipStream_t stream);

hipError_t launch_moe_route(const float* logits, int T, int E, int topk, int32_t* ids, float* gates,
                            int32_t* counts, int32_t* offsets, int32_t* sorted_pairs, hipStream_t stream);

size_t moe_workspace_bytes(int fmt, int T, int E, int topk, int H, int F);

hipError_t launch_moe_qgemm(int fmt, int xdt, const void* Wg, const void* Wu, const void* Wd, int E, int H, int F,
                            const void* X, int T, int topk, const float* gates, const int32_t* offsets,
                            const int32_t* sorted_pairs, float* out, void* h_out, void* ws, hipStream_t stream);

}  // namespace q4q8
