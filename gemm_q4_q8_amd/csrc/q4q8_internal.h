// Host-side declarations shared by the C-ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace q4q8 {

// Optional start/stop events recorded by the dispatch itself
// (hipExtLaunchKernel), so their elapsed time is the kernel's own duration.
struct LaunchEvents {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};

template <typename K, typename... A>
inline void launch(K kernel, dim3 grid, dim3 block, uint32_t shmem, hipStream_t s, const LaunchEvents& ev,
                   A... args) {
  if (ev.start || ev.stop)
    hipExtLaunchKernelGGL(kernel, grid, block, shmem, s, ev.start, ev.stop, 0, args...);
  else
    kernel<<<grid, block, shmem, s>>>(args...);
}

constexpr int kMaxGroup = 8;

// Internal GEMV output dtype (SwiGLU pairs only): rounded to bf16, stored as
// fp16 (the decode FFN's h).
constexpr int kYF16ViaBF16 = 4;

// One GEMV problem as the kernel sees it.  A SwiGLU pair has W = gate and
// W2 = up weights (same shape, same x) and stores h = silu(W x) * (W2 x) as
// ydt; a plain problem has W2 = null and stores fp32 dot products.
struct GemvProb {
  const uint8_t* W;
  const uint8_t* W2;
  const uint16_t* x;
  void* y;
  int64_t ldx, ldy;
  int32_t N, K;
  int32_t ydt;   // output dtype of a pair (kF16, kBF16, kF32); unused otherwise
  int32_t pad;
};

struct GemvArgs {
  int32_t wg0[kMaxGroup];   // first workgroup of each problem (set by the launcher)
  int32_t ks[kMaxGroup];    // waves per tile of each problem (a pair: 2 x its K-shares), a power of 2
                            // dividing the waves per workgroup
  int32_t count;
  int32_t M;
  int32_t total_tiles;
  int32_t xk;               // problems with K <= xk stage x in LDS (set by the launcher)
  GemvProb p[kMaxGroup];
};

hipError_t launch_repack(int fmt, const void* canon, int64_t N, int64_t K, void* dst, hipStream_t stream);
void repack_host(int fmt, const void* canon, int64_t N, int64_t K, void* dst);

hipError_t launch_qgemv(int fmt, int xdt, GemvArgs args, int max_chunks, int max_k, hipStream_t stream,
                        const LaunchEvents& ev);

size_t qgemm_workspace_bytes(int xdt, int64_t M, int64_t K);
// bf16 / fp16 (src_dt) [rows, cols] (row stride lds_) -> fp16 [rows, colsp]
// (row stride ldd), columns cols .. colsp - 1 zero, row m scaled by 2^-rexp[m]
// so its largest magnitude lands in [4, 8) (rexp[m] = 0 for a zero or
// non-finite row).  cols and colsp multiples of 8.
hipError_t launch_rowscale_f16(int src_dt, const void* src, int64_t lds_, void* dst, int64_t ldd, int64_t rows,
                               int64_t cols, int64_t colsp, int32_t* rexp, hipStream_t s, const LaunchEvents& ev);
hipError_t launch_qgemm(int fmt, int xdt, int ydt, const void* W, int64_t N, int64_t K, const void* X, int64_t ldx,
                        int64_t M, void* Y, int64_t ldy, void* ws, hipStream_t stream, const LaunchEvents& ev);

hipError_t launch_moe_route(const float* logits, int T, int E, int topk, int32_t* ids, float* gates,
                            int32_t* counts, int32_t* offsets, int32_t* sorted_pairs, hipStream_t stream);

size_t moe_workspace_bytes(int fmt, int T, int E, int topk, int H, int F);

// Decode path of the expert products (GEMV kernels), used for T <= 8 tokens
// when the token rows fit the workgroup's activation buffer.  h: bf16
// [T*topk, F] in sorted-pair order; y16: fp16 [T*topk, H] by pair id, in
// the token's scale (y 2^-2 xexp[t]); xexp: int32 [T], each token row's
// power-of-two exponent (written by the gate/up kernel).
// Returns true when it also formed out (down fused with the combine);
// otherwise y16 holds the per-pair outputs for the combine kernel.
constexpr int kMoeDecodeMaxTokens = 8;
bool moe_decode_fits(int T, int H, int F);
bool launch_moe_decode(int fmt, int xdt, const void* Wg, const void* Wu, const void* Wd, int E, int H, int F,
                       const void* X, int T, int topk, const float* gates, const int32_t* offsets,
                       const int32_t* sorted_pairs, uint16_t* h, uint16_t* y16, int32_t* xexp, float* out,
                       hipStream_t s);

// The routed decode call: the gate/up kernel derives the routing from the
// logits (as launch_moe_route would) and stores it in these arrays.
struct MoeRouteOut {
  const float* logits;
  int32_t* ids;
  float* gates;
  int32_t* counts;
  int32_t* offsets;
  int32_t* sorted_pairs;
};
bool launch_moe_decode_routed(int fmt, int xdt, const void* Wg, const void* Wu, const void* Wd, int E, int H, int F,
                              const void* X, int T, int topk, const MoeRouteOut& ro, uint16_t* h, uint16_t* y16,
                              int32_t* xexp, float* out, hipStream_t s);
hipError_t launch_moe_decode_call(int fmt, int xdt, const void* Wg, const void* Wu, const void* Wd, int E, int H,
                                  int F, const void* X, int T, int topk, const MoeRouteOut& ro, float* out,
                                  void* h_out, void* ws, hipStream_t s);

// The one-call MoE layer: q4q8_moe_route + q4q8_moe_qgemm's results for any
// T (the decode call for the few tokens it takes).
hipError_t launch_moe_forward(int fmt, int xdt, const void* Wg, const void* Wu, const void* Wd, int E, int H, int F,
                              const void* X, int T, int topk, const MoeRouteOut& ro, float* out, void* h_out,
                              void* ws, hipStream_t s);

hipError_t launch_moe_qgemm(int fmt, int xdt, const void* Wg, const void* Wu, const void* Wd, int E, int H, int F,
                            const void* X, int T, int topk, const float* gates, const int32_t* offsets,
                            const int32_t* sorted_pairs, float* out, void* h_out, void* ws, hipStream_t stream);

// Prefill attention, head dimension 128: Q/O [B, S, Hq, 128], K/V
// [B, S, Hkv, 128], dtype dt (kF16 or kBF16).
hipError_t launch_attn_prefill(int dt, const void* q, const void* k, const void* v, void* o, int B, int S, int Hq,
                               int Hkv, int causal, float scale, hipStream_t s, const LaunchEvents& ev);

}  // namespace q4q8
