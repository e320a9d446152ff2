// C-ABI layer: argument validation (pure host code, before anything is
// enqueued), error reporting and dispatch to the kernel launchers.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>

#include "../../include/q4q8.h"
#include "../../include/q4q8_measure.h"
#include "q4q8_internal.h"

namespace q4q8 {
// HBM read-ceiling probe (csrc/probe.hip), a measurement helper.
size_t stream_read_digest_bytes();
int stream_read_max_workgroups();
hipError_t launch_stream_read(const void* buf, size_t bytes, int workgroups, uint32_t* digest, hipStream_t s,
                              const LaunchEvents& ev);
}  // namespace q4q8

namespace {

thread_local char g_last_error[512];

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
  va_end(ap);
  return status;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return Q4Q8_OK;
  return fail(Q4Q8_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool fmt_ok(int fmt) { return fmt == Q4Q8_Q4_0 || fmt == Q4Q8_Q8_0; }   // quantised formats
bool any_fmt_ok(int fmt) { return fmt_ok(fmt) || fmt == Q4Q8_FP16; }    // + plain fp16 (layout, GEMV)
bool act_ok(int dt) { return dt == Q4Q8_F16 || dt == Q4Q8_BF16; }
bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

int64_t canon_block(int fmt) { return fmt == Q4Q8_Q4_0 ? 18 : fmt == Q4Q8_Q8_0 ? 34 : 64; }
int64_t rec_bytes(int fmt) { return fmt == Q4Q8_Q4_0 ? 1152 : fmt == Q4Q8_Q8_0 ? 2176 : 4096; }

// Shape rules common to every weight matrix (any format; the products that
// take only the quantised formats check that themselves).
int check_matrix(int fmt, int64_t N, int64_t K) {
  if (!any_fmt_ok(fmt)) return fail(Q4Q8_ERR_UNSUPPORTED, "unknown weight format %d", fmt);
  if (N < 1 || K < 32) return fail(Q4Q8_ERR_INVALID_ARG, "bad shape N=%lld K=%lld", (long long)N, (long long)K);
  if (K % 32) return fail(Q4Q8_ERR_INVALID_ARG, "K=%lld is not a multiple of 32", (long long)K);
  if (N > (1LL << 30) || K > (1LL << 24))
    return fail(Q4Q8_ERR_UNSUPPORTED, "shape N=%lld K=%lld beyond N <= 2^30, K <= 2^24", (long long)N,
                (long long)K);
  return Q4Q8_OK;
}

int64_t repacked(int fmt, int64_t N, int64_t K) {
  return ((N + 15) / 16) * ((K + 127) / 128) * rec_bytes(fmt);
}

void clear_hip_error() { (void)hipGetLastError(); }

}  // namespace

extern "C" {

int q4q8_abi_version(void) { return Q4Q8_ABI_VERSION; }

const char* q4q8_status_string(int s) {
  switch (s) {
    case Q4Q8_OK: return "ok";
    case Q4Q8_ERR_INVALID_ARG: return "invalid argument";
    case Q4Q8_ERR_UNSUPPORTED: return "unsupported";
    case Q4Q8_ERR_WORKSPACE: return "workspace too small";
    case Q4Q8_ERR_ALIGNMENT: return "misaligned pointer or leading dimension";
    case Q4Q8_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* q4q8_last_error(void) { return g_last_error; }

// Sizes beyond the shape limits every product call enforces (N <= 2^30,
// K <= 2^24) are bad arguments too: the byte counts would overflow.
size_t q4q8_canonical_bytes(int fmt, int64_t N, int64_t K) {
  if (!any_fmt_ok(fmt) || N < 1 || K < 32 || K % 32 || N > (1LL << 30) || K > (1LL << 24)) return 0;
  return (size_t)(N * (K / 32) * canon_block(fmt));
}

size_t q4q8_repacked_bytes(int fmt, int64_t N, int64_t K) {
  if (!any_fmt_ok(fmt) || N < 1 || K < 32 || K % 32 || N > (1LL << 30) || K > (1LL << 24)) return 0;
  return (size_t)repacked(fmt, N, K);
}

int q4q8_repack(int fmt, const void* canon, int64_t N, int64_t K, void* dst, size_t dst_bytes, void* stream) {
  int st = check_matrix(fmt, N, K);
  if (st) return st;
  if (!canon || !dst) return fail(Q4Q8_ERR_INVALID_ARG, "repack: null pointer");
  if (!aligned(dst, 16)) return fail(Q4Q8_ERR_ALIGNMENT, "repack: destination not 16-byte aligned");
  if (dst_bytes < (size_t)repacked(fmt, N, K))
    return fail(Q4Q8_ERR_INVALID_ARG, "repack: destination holds %zu bytes, needs %lld", dst_bytes,
                (long long)repacked(fmt, N, K));
  clear_hip_error();
  return hip_status(q4q8::launch_repack(fmt, canon, N, K, dst, (hipStream_t)stream), "repack launch");
}

int q4q8_repack_host(int fmt, const void* canon, int64_t N, int64_t K, void* dst, size_t dst_bytes) {
  int st = check_matrix(fmt, N, K);
  if (st) return st;
  if (!canon || !dst) return fail(Q4Q8_ERR_INVALID_ARG, "repack_host: null pointer");
  if (dst_bytes < (size_t)repacked(fmt, N, K))
    return fail(Q4Q8_ERR_INVALID_ARG, "repack_host: destination holds %zu bytes, needs %lld", dst_bytes,
                (long long)repacked(fmt, N, K));
  q4q8::repack_host(fmt, canon, N, K, dst);
  return Q4Q8_OK;
}

}  // extern "C"

// One GEMV problem as the entry points hand it over: plain (W2 null, fp32 y)
// or a SwiGLU pair (W gate, W2 up, y of dtype ydt).
struct GemvIn {
  const void* W;
  const void* W2;
  const void* x;
  void* y;
  int64_t N, K, ldx, ldy;
  int ydt;
};

static int check_gemv_prob(int fmt, const GemvIn& d, int M, int idx) {
  int st = check_matrix(fmt, d.N, d.K);
  if (st) return st;
  if (!d.W || !d.x || !d.y) return fail(Q4Q8_ERR_INVALID_ARG, "qgemv[%d]: null pointer", idx);
  if (!aligned(d.W, 16) || (d.W2 && !aligned(d.W2, 16)))
    return fail(Q4Q8_ERR_ALIGNMENT, "qgemv[%d]: weights not 16-byte aligned", idx);
  if (!aligned(d.x, 16)) return fail(Q4Q8_ERR_ALIGNMENT, "qgemv[%d]: x not 16-byte aligned", idx);
  if (d.ydt != Q4Q8_F16 && d.ydt != Q4Q8_BF16 && d.ydt != Q4Q8_F32)
    return fail(Q4Q8_ERR_UNSUPPORTED, "qgemv[%d]: output dtype %d", idx, d.ydt);
  const size_t ysz = d.ydt == Q4Q8_F32 ? 4 : 2;
  if (!aligned(d.y, ysz))
    return fail(Q4Q8_ERR_ALIGNMENT, "qgemv[%d]: y not aligned to its %zu-byte element", idx, ysz);
  if (M > 1) {
    if (d.ldx < d.K || d.ldy < d.N)
      return fail(Q4Q8_ERR_INVALID_ARG, "qgemv[%d]: ldx=%lld < K or ldy=%lld < N", idx, (long long)d.ldx,
                  (long long)d.ldy);
    if (d.ldx % 8) return fail(Q4Q8_ERR_ALIGNMENT, "qgemv[%d]: ldx=%lld not a multiple of 8", idx, (long long)d.ldx);
    if (d.ldx > (1LL << 40) || d.ldy > (1LL << 40))
      return fail(Q4Q8_ERR_UNSUPPORTED, "qgemv[%d]: leading dimension beyond 2^40", idx);
  }
  return Q4Q8_OK;
}

static int check_gemv_common(int fmt, int xdt, int M, int count) {
  if (!any_fmt_ok(fmt)) return fail(Q4Q8_ERR_UNSUPPORTED, "unknown weight format %d", fmt);
  if (!act_ok(xdt)) return fail(Q4Q8_ERR_UNSUPPORTED, "qgemv: activation dtype %d not F16/BF16", xdt);
  if (M < 1 || M > 8) return fail(Q4Q8_ERR_INVALID_ARG, "qgemv: M=%d outside 1..8", M);
  if (count < 1 || count > Q4Q8_MAX_GROUP)
    return fail(Q4Q8_ERR_INVALID_ARG, "qgemv: %d problems (1..%d allowed)", count, Q4Q8_MAX_GROUP);
  return Q4Q8_OK;
}

// Enqueues one launch over already validated problems.
static int run_gemv(int fmt, const GemvIn* in, int count, int xdt, int M, void* stream,
                    const q4q8::LaunchEvents& ev) {
  q4q8::GemvArgs args;
  memset(&args, 0, sizeof(args));
  int64_t tiles = 0;
  int max_chunks = 0, max_k = 0;
  for (int i = 0; i < count; ++i) {
    q4q8::GemvProb& p = args.p[i];
    p.W = (const uint8_t*)in[i].W;
    p.W2 = (const uint8_t*)in[i].W2;
    p.x = (const uint16_t*)in[i].x;
    p.y = in[i].y;
    p.ldx = M > 1 ? in[i].ldx : 0;
    p.ldy = M > 1 ? in[i].ldy : 0;
    p.N = (int32_t)in[i].N;
    p.K = (int32_t)in[i].K;
    p.ydt = in[i].ydt;
    tiles += (in[i].W2 ? 2 : 1) * ((in[i].N + 15) / 16);
    const int chunks = (int)((in[i].K + 127) / 128);
    if (chunks > max_chunks) max_chunks = chunks;
    if (in[i].K > max_k) max_k = (int)in[i].K;
  }
  if (tiles > (1LL << 31) - 1) return fail(Q4Q8_ERR_UNSUPPORTED, "qgemv: too many row tiles");
  args.count = count;
  args.M = M;
  args.total_tiles = (int32_t)tiles;
  clear_hip_error();
  return hip_status(q4q8::launch_qgemv(fmt, xdt, args, max_chunks, max_k, (hipStream_t)stream, ev),
                    "qgemv launch");
}

static int qgemv_grouped(int fmt, const q4q8_gemv_desc* descs, int count, int xdt, int M, void* stream,
                         const q4q8::LaunchEvents& ev) {
  if (!descs) return fail(Q4Q8_ERR_INVALID_ARG, "qgemv: null descriptor array");
  int st = check_gemv_common(fmt, xdt, M, count);
  if (st) return st;
  GemvIn in[Q4Q8_MAX_GROUP];
  for (int i = 0; i < count; ++i) {
    in[i] = GemvIn{descs[i].W, nullptr, descs[i].x, descs[i].y, descs[i].N, descs[i].K, descs[i].ldx,
                   descs[i].ldy, Q4Q8_F32};
    st = check_gemv_prob(fmt, in[i], M, i);
    if (st) return st;
  }
  return run_gemv(fmt, in, count, xdt, M, stream, ev);
}

extern "C" {

int q4q8_qgemv_grouped(int fmt, const q4q8_gemv_desc* descs, int count, int xdt, int M, void* stream) {
  return qgemv_grouped(fmt, descs, count, xdt, M, stream, q4q8::LaunchEvents());
}

int q4q8_qgemv_grouped_timed(int fmt, const q4q8_gemv_desc* descs, int count, int xdt, int M, void* stream,
                             void* ev_start, void* ev_stop) {
  q4q8::LaunchEvents ev;
  ev.start = (hipEvent_t)ev_start;
  ev.stop = (hipEvent_t)ev_stop;
  return qgemv_grouped(fmt, descs, count, xdt, M, stream, ev);
}

int q4q8_qgemv(int fmt, const void* W, int64_t N, int64_t K, const void* x, int xdt, int64_t ldx, int M, float* y,
               int64_t ldy, void* stream) {
  q4q8_gemv_desc d;
  d.W = W;
  d.x = x;
  d.y = y;
  d.N = N;
  d.K = K;
  d.ldx = ldx;
  d.ldy = ldy;
  return q4q8_qgemv_grouped(fmt, &d, 1, xdt, M, stream);
}

}  // extern "C"

static int swiglu_impl(int fmt, const void* Wg, const void* Wu, int64_t F, int64_t K, const void* x, int xdt,
                       int64_t ldx, int M, void* h, int hdt, int64_t ldh, void* stream,
                       const q4q8::LaunchEvents& ev) {
  int st = check_gemv_common(fmt, xdt, M, 1);
  if (st) return st;
  if (!Wu) return fail(Q4Q8_ERR_INVALID_ARG, "qgemv_swiglu: null pointer");
  const GemvIn in{Wg, Wu, x, h, F, K, ldx, ldh, hdt};
  st = check_gemv_prob(fmt, in, M, 0);
  if (st) return st;
  return run_gemv(fmt, &in, 1, xdt, M, stream, ev);
}

static size_t ffn_ws(int M, int64_t F) { return (size_t)(((int64_t)M * F * 2 + 255) / 256 * 256); }

static int ffn_impl(int fmt, const void* Wg, const void* Wu, const void* Wd, int64_t H, int64_t F, const void* x,
                    int xdt, int64_t ldx, int M, float* y, int64_t ldy, void* ws, size_t ws_bytes, void* stream,
                    const q4q8::LaunchEvents& ev) {
  int st = check_gemv_common(fmt, xdt, M, 1);
  if (st) return st;
  if (!Wg || !Wu || !Wd) return fail(Q4Q8_ERR_INVALID_ARG, "ffn_decode: null pointer");
  if (F < 32 || F % 32) return fail(Q4Q8_ERR_INVALID_ARG, "ffn_decode: F=%lld not a positive multiple of 32", (long long)F);
  const size_t need = ffn_ws(M, F);
  if (!ws || ws_bytes < need)
    return fail(Q4Q8_ERR_WORKSPACE, "ffn_decode: workspace holds %zu bytes, needs %zu", ws ? ws_bytes : 0, need);
  if (!aligned(ws, 256)) return fail(Q4Q8_ERR_ALIGNMENT, "ffn_decode: workspace not 256-byte aligned");
  // Validate both launches before enqueuing either: gate/up writes h (rows
  // of F, 2 bytes each) into ws, down reads it.  h is rounded to bf16 and
  // stored as fp16, so the down GEMV takes fp16 operands.
  GemvIn gu{Wg, Wu, x, ws, F, H, ldx, F, Q4Q8_BF16};
  st = check_gemv_prob(fmt, gu, M, 0);
  if (st) return st;
  const GemvIn dn{Wd, nullptr, ws, y, H, F, F, ldy, Q4Q8_F32};
  st = check_gemv_prob(fmt, dn, M, 1);
  if (st) return st;
  gu.ydt = q4q8::kYF16ViaBF16;
  q4q8::LaunchEvents e1, e2;
  e1.start = ev.start;
  e2.stop = ev.stop;
  st = run_gemv(fmt, &gu, 1, xdt, M, stream, e1);
  if (st) return st;
  return run_gemv(fmt, &dn, 1, Q4Q8_F16, M, stream, e2);
}

extern "C" {

int q4q8_qgemv_swiglu(int fmt, const void* Wg, const void* Wu, int64_t F, int64_t K, const void* x, int xdt,
                      int64_t ldx, int M, void* h, int hdt, int64_t ldh, void* stream) {
  return swiglu_impl(fmt, Wg, Wu, F, K, x, xdt, ldx, M, h, hdt, ldh, stream, q4q8::LaunchEvents());
}

int q4q8_qgemv_swiglu_timed(int fmt, const void* Wg, const void* Wu, int64_t F, int64_t K, const void* x, int xdt,
                            int64_t ldx, int M, void* h, int hdt, int64_t ldh, void* stream, void* ev_start,
                            void* ev_stop) {
  q4q8::LaunchEvents ev;
  ev.start = (hipEvent_t)ev_start;
  ev.stop = (hipEvent_t)ev_stop;
  return swiglu_impl(fmt, Wg, Wu, F, K, x, xdt, ldx, M, h, hdt, ldh, stream, ev);
}

size_t q4q8_ffn_decode_workspace(int M, int64_t F) {
  if (M < 1 || M > 8 || F < 32 || F % 32 || F > (1LL << 24)) return 0;
  return ffn_ws(M, F);
}

int q4q8_ffn_decode(int fmt, const void* Wg, const void* Wu, const void* Wd, int64_t H, int64_t F, const void* x,
                    int xdt, int64_t ldx, int M, float* y, int64_t ldy, void* ws, size_t ws_bytes, void* stream) {
  return ffn_impl(fmt, Wg, Wu, Wd, H, F, x, xdt, ldx, M, y, ldy, ws, ws_bytes, stream, q4q8::LaunchEvents());
}

int q4q8_ffn_decode_timed(int fmt, const void* Wg, const void* Wu, const void* Wd, int64_t H, int64_t F,
                          const void* x, int xdt, int64_t ldx, int M, float* y, int64_t ldy, void* ws,
                          size_t ws_bytes, void* stream, void* ev_start, void* ev_stop) {
  q4q8::LaunchEvents ev;
  ev.start = (hipEvent_t)ev_start;
  ev.stop = (hipEvent_t)ev_stop;
  return ffn_impl(fmt, Wg, Wu, Wd, H, F, x, xdt, ldx, M, y, ldy, ws, ws_bytes, stream, ev);
}

}  // extern "C"

extern "C" {

static int qgemm_impl(int fmt, const void* W, int64_t N, int64_t K, const void* X, int xdt, int64_t ldx, int64_t M,
                      void* Y, int ydt, int64_t ldy, void* ws, size_t ws_bytes, void* stream,
                      const q4q8::LaunchEvents& ev) {
  if (!any_fmt_ok(fmt)) return fail(Q4Q8_ERR_UNSUPPORTED, "qgemm: weight format %d", fmt);
  int st = check_matrix(fmt, N, K);
  if (st) return st;
  if (!act_ok(xdt)) return fail(Q4Q8_ERR_UNSUPPORTED, "qgemm: activation dtype %d not F16/BF16", xdt);
  if (ydt != Q4Q8_F16 && ydt != Q4Q8_BF16 && ydt != Q4Q8_F32)
    return fail(Q4Q8_ERR_UNSUPPORTED, "qgemm: output dtype %d", ydt);
  if (M < 1 || M > (1LL << 30)) return fail(Q4Q8_ERR_INVALID_ARG, "qgemm: M=%lld", (long long)M);
  if (((M + 63) / 64) * ((N + 63) / 64) >= (1LL << 23))
    return fail(Q4Q8_ERR_UNSUPPORTED, "qgemm: M x N too large for one launch (split it)");
  if (!W || !X || !Y) return fail(Q4Q8_ERR_INVALID_ARG, "qgemm: null pointer");
  if (ldx < K || ldy < N) return fail(Q4Q8_ERR_INVALID_ARG, "qgemm: ldx < K or ldy < N");
  if (ldx > (1LL << 22)) return fail(Q4Q8_ERR_UNSUPPORTED, "qgemm: ldx=%lld beyond 2^22", (long long)ldx);
  const int ysz = ydt == Q4Q8_F32 ? 4 : 2;
  if (!aligned(W, 16) || !aligned(X, 16) || !aligned(Y, ysz) || ldx % 8)
    return fail(Q4Q8_ERR_ALIGNMENT,
                "qgemm: W and X must be 16-byte aligned, ldx a multiple of 8, Y aligned to its element size");
  const size_t need = q4q8::qgemm_workspace_bytes(xdt, M, K);
  if (need && (!ws || ws_bytes < need))
    return fail(Q4Q8_ERR_WORKSPACE, "qgemm: workspace holds %zu bytes, needs %zu", ws ? ws_bytes : 0, need);
  if (need && !aligned(ws, 256)) return fail(Q4Q8_ERR_ALIGNMENT, "qgemm: workspace not 256-byte aligned");
  clear_hip_error();
  return hip_status(q4q8::launch_qgemm(fmt, xdt, ydt, W, N, K, X, ldx, M, Y, ldy, ws, (hipStream_t)stream, ev),
                    "qgemm launch");
}

size_t q4q8_qgemm_workspace(int xdt, int64_t M, int64_t K) {
  if (!act_ok(xdt) || M < 1 || K < 1) return 0;
  return q4q8::qgemm_workspace_bytes(xdt, M, K);
}

int q4q8_qgemm(int fmt, const void* W, int64_t N, int64_t K, const void* X, int xdt, int64_t ldx, int64_t M, void* Y,
               int ydt, int64_t ldy, void* ws, size_t ws_bytes, void* stream) {
  return qgemm_impl(fmt, W, N, K, X, xdt, ldx, M, Y, ydt, ldy, ws, ws_bytes, stream, q4q8::LaunchEvents());
}

int q4q8_qgemm_timed(int fmt, const void* W, int64_t N, int64_t K, const void* X, int xdt, int64_t ldx, int64_t M,
                     void* Y, int ydt, int64_t ldy, void* ws, size_t ws_bytes, void* stream, void* ev_start,
                     void* ev_stop) {
  q4q8::LaunchEvents ev;
  ev.start = (hipEvent_t)ev_start;
  ev.stop = (hipEvent_t)ev_stop;
  return qgemm_impl(fmt, W, N, K, X, xdt, ldx, M, Y, ydt, ldy, ws, ws_bytes, stream, ev);
}

size_t q4q8_stream_read_digest_bytes(void) { return q4q8::stream_read_digest_bytes(); }

int q4q8_stream_read_grid_timed(const void* buf, size_t bytes, int workgroups, uint32_t* digest,
                                size_t digest_bytes, void* stream, void* ev_start, void* ev_stop) {
  if (!buf || !digest) return fail(Q4Q8_ERR_INVALID_ARG, "stream_read: null pointer");
  if (bytes < 16 || bytes % 16) return fail(Q4Q8_ERR_INVALID_ARG, "stream_read: bytes=%zu is not a positive multiple of 16", bytes);
  if (workgroups < 1 || workgroups > q4q8::stream_read_max_workgroups())
    return fail(Q4Q8_ERR_INVALID_ARG, "stream_read: workgroups=%d outside 1..%d", workgroups,
                q4q8::stream_read_max_workgroups());
  if (digest_bytes < q4q8::stream_read_digest_bytes())
    return fail(Q4Q8_ERR_INVALID_ARG, "stream_read: digest needs %zu bytes, got %zu", q4q8::stream_read_digest_bytes(),
                digest_bytes);
  if (!aligned(buf, 16) || !aligned(digest, 4))
    return fail(Q4Q8_ERR_ALIGNMENT, "stream_read: buf must be 16-byte and digest 4-byte aligned");
  q4q8::LaunchEvents ev;
  ev.start = (hipEvent_t)ev_start;
  ev.stop = (hipEvent_t)ev_stop;
  clear_hip_error();
  return hip_status(q4q8::launch_stream_read(buf, bytes, workgroups, digest, (hipStream_t)stream, ev), "stream_read");
}

int q4q8_stream_read_timed(const void* buf, size_t bytes, uint32_t* digest, size_t digest_bytes, void* stream,
                           void* ev_start, void* ev_stop) {
  return q4q8_stream_read_grid_timed(buf, bytes, q4q8::stream_read_max_workgroups(), digest, digest_bytes, stream,
                                     ev_start, ev_stop);
}

int q4q8_moe_route(const float* logits, int T, int E, int topk, int32_t* ids, float* gates, int32_t* counts,
                   int32_t* offsets, int32_t* sorted_pairs, void* stream) {
  if (!logits || !ids || !gates || !counts || !offsets || !sorted_pairs)
    return fail(Q4Q8_ERR_INVALID_ARG, "moe_route: null pointer");
  if (T < 1 || E < 1 || topk < 1 || topk > E)
    return fail(Q4Q8_ERR_INVALID_ARG, "moe_route: T=%d E=%d topk=%d", T, E, topk);
  if (E > 1024 || topk > 16) return fail(Q4Q8_ERR_UNSUPPORTED, "moe_route: E=%d > 1024 or topk=%d > 16", E, topk);
  if ((int64_t)T * topk > (1LL << 22))
    return fail(Q4Q8_ERR_UNSUPPORTED, "moe_route: T*topk=%lld beyond 2^22", (long long)T * topk);
  clear_hip_error();
  return hip_status(q4q8::launch_moe_route(logits, T, E, topk, ids, gates, counts, offsets, sorted_pairs,
                                           (hipStream_t)stream),
                    "moe_route launch");
}

size_t q4q8_moe_workspace(int fmt, int T, int E, int topk, int H, int F) {
  if (!fmt_ok(fmt) || T < 1 || E < 1 || topk < 1 || topk > E || H < 128 || F < 128) return 0;
  return q4q8::moe_workspace_bytes(fmt, T, E, topk, H, F);
}

int q4q8_moe_qgemm(int fmt, const void* Wg, const void* Wu, const void* Wd, int E, int H, int F, const void* X,
                   int xdt, int T, int topk, const float* gates, const int32_t* offsets,
                   const int32_t* sorted_pairs, float* out, void* h_out, void* ws, size_t ws_bytes, void* stream) {
  if (!fmt_ok(fmt)) return fail(Q4Q8_ERR_UNSUPPORTED, "unknown weight format %d", fmt);
  if (!act_ok(xdt)) return fail(Q4Q8_ERR_UNSUPPORTED, "moe_qgemm: activation dtype %d not F16/BF16", xdt);
  if (!Wg || !Wu || !Wd || !X || !gates || !offsets || !sorted_pairs || !out)
    return fail(Q4Q8_ERR_INVALID_ARG, "moe_qgemm: null pointer");
  if (T < 1 || E < 1 || topk < 1 || topk > E || topk > 16 || E > 1024)
    return fail(Q4Q8_ERR_INVALID_ARG, "moe_qgemm: T=%d E=%d topk=%d", T, E, topk);
  if (H < 128 || F < 128 || H % 128 || F % 128)
    return fail(Q4Q8_ERR_INVALID_ARG, "moe_qgemm: H=%d and F=%d must be positive multiples of 128", H, F);
  const int64_t P = (int64_t)T * topk;
  if (P > (1LL << 22) || H > (1 << 20) || F > (1 << 20) || (int64_t)T * H * 2 >= (1LL << 31) ||
      P * F * 2 >= (1LL << 31) || P * H * 2 >= (1LL << 31))
    return fail(Q4Q8_ERR_UNSUPPORTED, "moe_qgemm: sizes beyond limits (T*topk <= 2^22, T*H, T*topk*F and "
                                      "T*topk*H below 2^30 elements)");
  const size_t need = q4q8::moe_workspace_bytes(fmt, T, E, topk, H, F);
  if (!ws || ws_bytes < need)
    return fail(Q4Q8_ERR_WORKSPACE, "moe_qgemm: workspace holds %zu bytes, needs %zu", ws_bytes, need);
  if (!aligned(ws, 256)) return fail(Q4Q8_ERR_ALIGNMENT, "moe_qgemm: workspace not 256-byte aligned");
  if (!aligned(Wg, 16) || !aligned(Wu, 16) || !aligned(Wd, 16) || !aligned(X, 16) || !aligned(out, 16) ||
      (h_out && !aligned(h_out, 16)))
    return fail(Q4Q8_ERR_ALIGNMENT, "moe_qgemm: weights, X, out and h_out must be 16-byte aligned");
  clear_hip_error();
  return hip_status(q4q8::launch_moe_qgemm(fmt, xdt, Wg, Wu, Wd, E, H, F, X, T, topk, gates, offsets, sorted_pairs,
                                           out, h_out, ws, (hipStream_t)stream),
                    "moe_qgemm launch");
}

}  // extern "C"

namespace {

// The no-allocation decode call's scratch: one array per GPU, resident from
// module load until the process ends.  Host code never passes `scratch`
// itself to a kernel (on the host it names a stand-in, not device memory);
// it uses the device address hipGetSymbolAddress returns, looked up once per
// device with that device current.
constexpr size_t kScratchBytes = (size_t)1 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on the device that runs `stream`.
int scratch_for(void* stream, void** out) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "moe_decode_noalloc: device of the stream");
  if (dev < 0 || dev >= kMaxDevices) return fail(Q4Q8_ERR_UNSUPPORTED, "moe_decode_noalloc: device %d", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void* p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return hip_status(e, "moe_decode_noalloc: scratch address");
    if (!p) return fail(Q4Q8_ERR_HIP, "moe_decode_noalloc: scratch address is null");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return Q4Q8_OK;
}

int moe_decode_impl(int fmt, const void* Wg, const void* Wu, const void* Wd, int E, int H, int F, const float* logits,
                    const void* X, int xdt, int T, int topk, int32_t* ids, float* gates, int32_t* counts,
                    int32_t* offsets, int32_t* sorted_pairs, float* out, void* h_out, void* ws, size_t ws_bytes,
                    void* stream, bool use_scratch, bool any_t = false) {
  if (!fmt_ok(fmt)) return fail(Q4Q8_ERR_UNSUPPORTED, "unknown weight format %d", fmt);
  if (!act_ok(xdt)) return fail(Q4Q8_ERR_UNSUPPORTED, "moe_decode: activation dtype %d not F16/BF16", xdt);
  if (!Wg || !Wu || !Wd || !logits || !X || !ids || !gates || !counts || !offsets || !sorted_pairs || !out)
    return fail(Q4Q8_ERR_INVALID_ARG, "moe_decode: null pointer");
  if (T < 1 || E < 1 || topk < 1 || topk > E || topk > 16 || E > 1024)
    return fail(Q4Q8_ERR_INVALID_ARG, "moe_decode: T=%d E=%d topk=%d", T, E, topk);
  if (H < 128 || F < 128 || H % 128 || F % 128)
    return fail(Q4Q8_ERR_INVALID_ARG, "moe_decode: H=%d and F=%d must be positive multiples of 128", H, F);
  if (any_t) {
    const int64_t P = (int64_t)T * topk;
    if (P > (1LL << 22) || H > (1 << 20) || F > (1 << 20) || (int64_t)T * H * 2 >= (1LL << 31) ||
        P * F * 2 >= (1LL << 31) || P * H * 2 >= (1LL << 31))
      return fail(Q4Q8_ERR_UNSUPPORTED, "moe_forward: sizes beyond limits (T*topk <= 2^22, T*H, T*topk*F and "
                                        "T*topk*H below 2^30 elements)");
  } else if (H > (1 << 20) || F > (1 << 20) || !q4q8::moe_decode_fits(T, H, F)) {
    return fail(Q4Q8_ERR_UNSUPPORTED,
                "moe_decode: T=%d H=%d F=%d beyond the decode path (T <= 8 and T*(max(H,F)+8)*2 + 512 <= 52 KB; "
                "use q4q8_moe_forward, or q4q8_moe_route + q4q8_moe_qgemm)",
                T, H, F);
  }
  const size_t need = q4q8::moe_workspace_bytes(fmt, T, E, topk, H, F);
  if (use_scratch) {
    if (need > kScratchBytes)
      return fail(Q4Q8_ERR_UNSUPPORTED,
                  "moe_decode_noalloc: T=%d topk=%d H=%d F=%d need %zu bytes of scratch, beyond its %zu (use "
                  "q4q8_moe_decode with a workspace)",
                  T, topk, H, F, need, kScratchBytes);
  } else {
    if (!ws || ws_bytes < need)
      return fail(Q4Q8_ERR_WORKSPACE, "moe_decode: workspace holds %zu bytes, needs %zu", ws_bytes, need);
    if (!aligned(ws, 256)) return fail(Q4Q8_ERR_ALIGNMENT, "moe_decode: workspace not 256-byte aligned");
  }
  if (!aligned(Wg, 16) || !aligned(Wu, 16) || !aligned(Wd, 16) || !aligned(X, 16) || !aligned(out, 16) ||
      (h_out && !aligned(h_out, 16)) || !aligned(logits, 4) || !aligned(ids, 4) || !aligned(gates, 4) ||
      !aligned(counts, 4) || !aligned(offsets, 4) || !aligned(sorted_pairs, 4))
    return fail(Q4Q8_ERR_ALIGNMENT, "moe_decode: weights, X, out and h_out must be 16-byte aligned, the routing "
                                    "arrays 4-byte aligned");
  if (use_scratch) {
    const int st = scratch_for(stream, &ws);
    if (st != Q4Q8_OK) return st;
  }
  clear_hip_error();
  const q4q8::MoeRouteOut ro = {logits, ids, gates, counts, offsets, sorted_pairs};
  if (any_t)
    return hip_status(q4q8::launch_moe_forward(fmt, xdt, Wg, Wu, Wd, E, H, F, X, T, topk, ro, out, h_out, ws,
                                               (hipStream_t)stream),
                      "moe_forward launch");
  return hip_status(q4q8::launch_moe_decode_call(fmt, xdt, Wg, Wu, Wd, E, H, F, X, T, topk, ro, out, h_out, ws,
                                                 (hipStream_t)stream),
                    "moe_decode launch");
}

}  // namespace

extern "C" {

int q4q8_moe_decode(int fmt, const void* Wg, const void* Wu, const void* Wd, int E, int H, int F,
                    const float* logits, const void* X, int xdt, int T, int topk, int32_t* ids, float* gates,
                    int32_t* counts, int32_t* offsets, int32_t* sorted_pairs, float* out, void* h_out, void* ws,
                    size_t ws_bytes, void* stream) {
  return moe_decode_impl(fmt, Wg, Wu, Wd, E, H, F, logits, X, xdt, T, topk, ids, gates, counts, offsets,
                         sorted_pairs, out, h_out, ws, ws_bytes, stream, false);
}

int q4q8_moe_forward(int fmt, const void* Wg, const void* Wu, const void* Wd, int E, int H, int F,
                     const float* logits, const void* X, int xdt, int T, int topk, int32_t* ids, float* gates,
                     int32_t* counts, int32_t* offsets, int32_t* sorted_pairs, float* out, void* h_out, void* ws,
                     size_t ws_bytes, void* stream) {
  return moe_decode_impl(fmt, Wg, Wu, Wd, E, H, F, logits, X, xdt, T, topk, ids, gates, counts, offsets,
                         sorted_pairs, out, h_out, ws, ws_bytes, stream, false, true);
}

int q4q8_moe_decode_noalloc(int fmt, const void* Wg, const void* Wu, const void* Wd, int E, int H, int F,
                            const float* logits, const void* X, int xdt, int T, int topk, int32_t* ids,
                            float* gates, int32_t* counts, int32_t* offsets, int32_t* sorted_pairs, float* out,
                            void* h_out, void* stream) {
  return moe_decode_impl(fmt, Wg, Wu, Wd, E, H, F, logits, X, xdt, T, topk, ids, gates, counts, offsets,
                         sorted_pairs, out, h_out, nullptr, 0, stream, true);
}

size_t q4q8_moe_decode_noalloc_max_scratch(void) { return kScratchBytes; }

static int attn_impl(int dt, const void* Q, const void* K, const void* V, void* O, int B, int S, int Hq, int Hkv,
                     int D, int causal, float scale, void* stream, const q4q8::LaunchEvents& ev) {
  if (!act_ok(dt)) return fail(Q4Q8_ERR_UNSUPPORTED, "attn_prefill: dtype %d not F16/BF16", dt);
  if (D != 128) return fail(Q4Q8_ERR_UNSUPPORTED, "attn_prefill: head dimension %d (128 supported)", D);
  if (!Q || !K || !V || !O) return fail(Q4Q8_ERR_INVALID_ARG, "attn_prefill: null pointer");
  if (B < 1 || S < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv)
    return fail(Q4Q8_ERR_INVALID_ARG, "attn_prefill: B=%d S=%d Hq=%d Hkv=%d (Hq a multiple of Hkv)", B, S, Hq, Hkv);
  if (!(scale > 0.0f) || scale > 1e30f) return fail(Q4Q8_ERR_INVALID_ARG, "attn_prefill: scale must be positive");
  if ((int64_t)B * Hq * ((S + 127) / 128) >= (1LL << 31) || (int64_t)B * S * Hq * D >= (1LL << 40) ||
      (int64_t)S * Hkv * D * 2 >= (1LL << 31))
    return fail(Q4Q8_ERR_UNSUPPORTED, "attn_prefill: sizes beyond limits (S * Hkv * D below 2^30)");
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 8))
    return fail(Q4Q8_ERR_ALIGNMENT, "attn_prefill: Q, K, V must be 16-byte aligned, O 8-byte aligned");
  clear_hip_error();
  return hip_status(q4q8::launch_attn_prefill(dt, Q, K, V, O, B, S, Hq, Hkv, causal ? 1 : 0, scale,
                                              (hipStream_t)stream, ev),
                    "attn_prefill launch");
}

int q4q8_attn_prefill(int dt, const void* Q, const void* K, const void* V, void* O, int B, int S, int Hq, int Hkv,
                      int D, int causal, float scale, void* stream) {
  return attn_impl(dt, Q, K, V, O, B, S, Hq, Hkv, D, causal, scale, stream, q4q8::LaunchEvents());
}

int q4q8_attn_prefill_timed(int dt, const void* Q, const void* K, const void* V, void* O, int B, int S, int Hq,
                            int Hkv, int D, int causal, float scale, void* stream, void* ev_start, void* ev_stop) {
  q4q8::LaunchEvents ev;
  ev.start = (hipEvent_t)ev_start;
  ev.stop = (hipEvent_t)ev_stop;
  return attn_impl(dt, Q, K, V, O, B, S, Hq, Hkv, D, causal, scale, stream, ev);
}

}  // extern "C"
