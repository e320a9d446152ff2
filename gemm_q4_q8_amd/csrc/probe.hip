// Measurement helper: an HBM read ceiling for the decode GEMV.
//
// Reads a buffer once with 16-byte non-temporal loads (the policy the GEMV's
// weight loads use), four loads in flight per thread, over a fixed grid of
// many short workgroups (measured on MI355X: 512-thread workgroups, 64 per
// CU, beat longer grid-stride loops over fewer of them for GiB-sized reads;
// a caller may pick a smaller grid for a short read); each wave folds
// what it read into one XOR digest word so the loads cannot be dropped.
// Bytes read / kernel time is the streaming read rate the quantised GEMV is
// compared with.
#include "q4q8_dev.h"
#include "q4q8_internal.h"

namespace q4q8 {

namespace {

constexpr int kProbeThreads = 512;
constexpr int kProbeBlocks = 256 * 64;  // 64 workgroups per CU, in waves of residency
constexpr int kProbeUnroll = 4;

__global__ __launch_bounds__(kProbeThreads) void stream_read_kernel(const u32x4_t* __restrict__ p, int64_t n16,
                                                                    uint32_t* __restrict__ digest) {
  const int64_t stride = (int64_t)gridDim.x * kProbeThreads;
  uint32_t acc = 0;
  int64_t i = (int64_t)blockIdx.x * kProbeThreads + threadIdx.x;
  for (; i + (kProbeUnroll - 1) * stride < n16; i += kProbeUnroll * stride) {
    u32x4_t v[kProbeUnroll];
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
    for (int u = 0; u < kProbeUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  for (; i < n16; i += stride) {
    const u32x4_t v = __builtin_nontemporal_load(p + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
  if ((threadIdx.x & 63) == 0) digest[blockIdx.x * (kProbeThreads / 64) + (threadIdx.x >> 6)] = acc;
}

}  // namespace

size_t stream_read_digest_bytes() { return (size_t)kProbeBlocks * (kProbeThreads / 64) * sizeof(uint32_t); }

int stream_read_max_workgroups() { return kProbeBlocks; }

// workgroups: 1 .. kProbeBlocks (the caller checks).
hipError_t launch_stream_read(const void* buf, size_t bytes, int workgroups, uint32_t* digest, hipStream_t s,
                              const LaunchEvents& ev) {
  launch(stream_read_kernel, dim3((unsigned)workgroups), dim3(kProbeThreads), 0, s, ev, (const u32x4_t*)buf,
         (int64_t)(bytes / 16), digest);
  return hipGetLastError();
}

}  // namespace q4q8
