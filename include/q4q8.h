/*
 * q4q8.h -- C ABI of the block-quantised weight-product library for AMD MI355X
 * (gfx950 / CDNA4).
 *
 * What the library computes.  "BaseRT: Best-in-Class LLM Inference on Apple
 * Silicon via Native Metal" (gist.science technical summary, section
 * "Methodologie", kernel specialisation) describes GEMV kernels for decode and
 * GEMM kernels for prefill, one variant per quantisation format, that
 * dequantise inside the inner loop so weights are never materialised in
 * global memory.  Its follow-up, "BaseRT: Advancing Best-in-Class LLM
 * Inference with Apple M5 Neural Accelerators" (review, section "Method"),
 * adds grouped mixture-of-experts GEMMs with fused expert projections on the
 * matrix units, with memory-bound decode kept on the GEMV path.  The same
 * pages say weights are converted once to the runtime's own format (review,
 * section "Comparison") and that the decode loop allocates nothing (technical
 * summary, "Methodologie", zero-allocation decode loop).
 *
 * Formats (32 weights per block along K, one fp16 scale s per block):
 *   Q4_0: 4-bit codes q in 0..15, weight = s * (q - 8)
 *   Q8_0: int8 codes q,          weight = s * q
 * Canonical (interchange) blocks: Q4_0 = 18 bytes [s][16 bytes, byte i =
 * q[i] | q[i+16] << 4]; Q8_0 = 34 bytes [s][32 int8].  Blocks run along K,
 * rows n = 0..N-1 follow one another.  FP16 (plain weights, the top of the
 * technical summary's Q2..FP16 format range, abstract): row-major fp16
 * [N, K], 64 bytes per 32 weights.  Repacked FP16 records are 4096 bytes:
 * four 1 KB planes, block j's lane slot l at j * 1024 + l * 16 holding the
 * slot's 8 weights; no scales.  In the GEMV, BF16 activations meet FP16
 * weights as fp16 operands (converted to nearest: exact for
 * 2^-14 <= |x| < 65520, |x| >= 65520 becomes +-inf).
 *
 * Conventions for every call below.
 *   - Ownership: the caller allocates and frees everything (weights,
 *     activations, outputs, workspace).  The library allocates no memory and
 *     keeps no device state, except q4q8_moe_decode_noalloc's static scratch
 *     array (one per GPU, described there).
 *   - Measurement: dispatch-timed forms of some calls (q4q8_*_timed) and an
 *     HBM read probe are exported too; they are declared in q4q8_measure.h,
 *     apart from the product interface.
 *   - Streams: `stream` is a hipStream_t passed as void* (NULL = the null
 *     stream).  Calls enqueue work and return without synchronising; results
 *     are ready once the stream reaches that point.
 *   - Errors: arguments are validated on the host before anything is
 *     enqueued.  On a validation failure the call returns a negative status,
 *     enqueues nothing and leaves every output untouched.  A launch failure
 *     returns Q4Q8_ERR_HIP.  A fault while a kernel runs surfaces at the
 *     caller's next synchronisation.  q4q8_last_error() gives a one-line
 *     description of the last failure on the calling thread.  No C++
 *     exception crosses this interface.
 *   - Threading: calls are re-entrant; calls on different streams may run
 *     concurrently (they share no library state).
 *   - Determinism: all outputs are bitwise reproducible run to run (no
 *     floating-point atomics; every reduction has a fixed order).
 *   - Shapes: K % 32 == 0, N >= 1, K >= 32.  Repacked weights and activation
 *     rows must be 16-byte aligned (leading dimensions multiples of 8
 *     elements).  Activation values are finite.
 *   - Activations of dtype F16 are used as fp16.  BF16 activations are
 *     exact in the GEMV.  In the GEMM and the MoE calls every activation
 *     row is scaled by a power of two 2^-e chosen so that its largest
 *     magnitude lands in [4, 8), converted to fp16 for the matrix cores
 *     (exact for every value within a factor 2^20 of the row's largest;
 *     smaller ones round to nearest with an absolute error below 2^-25 of
 *     the scaled row) and the results are multiplied back by 2^e, so any
 *     finite bf16 row is accepted.  In the MoE calls h and y carry the
 *     token's 2^-2e inside the library (|h| <= |x W_gate^T| |x W_up^T|), and
 *     F16 rows are scaled the same way.
 */
#ifndef Q4Q8_H
#define Q4Q8_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define Q4Q8_ABI_VERSION 1

typedef enum {
  Q4Q8_OK = 0,
  Q4Q8_ERR_INVALID_ARG = -1,   /* null pointer, bad shape or count          */
  Q4Q8_ERR_UNSUPPORTED = -2,   /* unknown format / dtype, or size limit      */
  Q4Q8_ERR_WORKSPACE = -3,     /* workspace missing or too small             */
  Q4Q8_ERR_ALIGNMENT = -4,     /* pointer or leading dimension misaligned    */
  Q4Q8_ERR_HIP = -5            /* the HIP runtime refused a launch or copy   */
} q4q8_status;

/* Q4Q8_FP16: plain fp16 weights (no quantisation), accepted by the layout
 * calls, the GEMV entry points (q4q8_qgemv, _grouped, _swiglu,
 * q4q8_ffn_decode) and q4q8_qgemm; the MoE calls take Q4_0 and Q8_0 only. */
typedef enum { Q4Q8_Q4_0 = 1, Q4Q8_Q8_0 = 2, Q4Q8_FP16 = 3 } q4q8_format;
typedef enum { Q4Q8_F16 = 1, Q4Q8_BF16 = 2, Q4Q8_F32 = 3 } q4q8_dtype;

/* Version of this interface (Q4Q8_ABI_VERSION of the built library). */
int q4q8_abi_version(void);

/* Human-readable name of a status code (static string). */
const char* q4q8_status_string(int status);

/* Detail of the last failing call on this thread ("" if none).  The string
 * is thread-local and valid until the next failing call on this thread. */
const char* q4q8_last_error(void);

/* ------------------------------------------------------------------------ */
/* Weight layout (load time)                                                */
/* ------------------------------------------------------------------------ */

/* Bytes of a canonical N x K matrix: N * (K/32) * (18 | 34).  0 on bad args
 * (including N > 2^30 or K > 2^24, the product calls' shape limits). */
size_t q4q8_canonical_bytes(int fmt, int64_t N, int64_t K);

/* Bytes of the repacked N x K matrix.  Rows are padded to a multiple of 16
 * and K to a multiple of 128; when N % 16 == 0 and K % 128 == 0 this equals
 * the canonical size (no byte is added).  0 on bad args (as for
 * q4q8_canonical_bytes). */
size_t q4q8_repacked_bytes(int fmt, int64_t N, int64_t K);

/* Convert canonical blocks to the gfx950 layout every product call reads
 * (the "native weight format" conversion, done once at load time).
 * Layout: 16-row tiles; each tile holds K/128 records of 4 blocks; a record
 * is 64 lane slots of codes (16 B per slot for Q4_0, 32 B for Q8_0, slot
 * l = 16*g + r holds row r, codes 8g..8g+7 of each of the 4 blocks, nibbles
 * pre-permuted for the in-register unpack) followed by the 16 x 4 fp16
 * scales [row][block].  Padding rows and blocks get scale 0 and code 0.
 *   canon:     device pointer, q4q8_canonical_bytes(fmt, N, K) bytes, any
 *              alignment, read only.
 *   dst:       device pointer, 16-byte aligned, dst_bytes >=
 *              q4q8_repacked_bytes(fmt, N, K).  Written entirely.
 * Asynchronous on `stream`. */
int q4q8_repack(int fmt, const void* canon, int64_t N, int64_t K,
                void* dst, size_t dst_bytes, void* stream);

/* The same conversion on the host, for offline checkpoint conversion: both
 * pointers are host memory; synchronous; touches no GPU.  Produces exactly
 * the bytes q4q8_repack produces. */
int q4q8_repack_host(int fmt, const void* canon, int64_t N, int64_t K,
                     void* dst, size_t dst_bytes);

/* ------------------------------------------------------------------------ */
/* Decode: quantised GEMV, M = 1..8 activation rows                          */
/* (technical summary, "Methodologie": a GEMV per quantisation format for   */
/*  decode, dequantisation inside the inner loop)                           */
/* ------------------------------------------------------------------------ */

/* y[m, n] = sum_k W[n, k] * x[m, k]   for m < M, n < N.
 *   W:   repacked weights (device), from q4q8_repack with the same fmt,N,K.
 *   x:   device, M rows of K activations of dtype xdt (F16 or BF16),
 *        row m at x + m*ldx elements; 16-byte aligned, ldx % 8 == 0,
 *        ldx >= K when M > 1.
 *   y:   device fp32, row m at y + m*ldy; ldy >= N when M > 1.  Written only
 *        at [0, M) x [0, N).
 * fp32 accumulation; the weights are exact in the matrix-core operand type
 * and the block scales are applied in fp32. */
int q4q8_qgemv(int fmt, const void* W, int64_t N, int64_t K,
               const void* x, int xdt, int64_t ldx, int M,
               float* y, int64_t ldy, void* stream);

/* One GEMV problem of a grouped launch. */
typedef struct {
  const void* W;      /* repacked weights (device)             */
  const void* x;      /* activations, M rows (device)           */
  float* y;           /* fp32 output, M rows (device)           */
  int64_t N, K;       /* matrix shape                           */
  int64_t ldx, ldy;   /* leading dimensions (elements)          */
} q4q8_gemv_desc;

#define Q4Q8_MAX_GROUP 8

/* Up to Q4Q8_MAX_GROUP independent GEMVs of one format, dtype and M in a
 * single launch (e.g. the q/k/v projections of a layer, or gate and up).
 * `descs` is host memory, read during the call only.  Each problem obeys
 * the rules of q4q8_qgemv; outputs must not overlap. */
int q4q8_qgemv_grouped(int fmt, const q4q8_gemv_desc* descs, int count,
                       int xdt, int M, void* stream);

/* ------------------------------------------------------------------------ */
/* Decode FFN: fused gate/up GEMV with a SwiGLU epilogue, then down          */
/* (technical summary, "Methodologie": kernel fusion of FFN blocks, which    */
/*  matters in decode where kernels are short; the SwiGLU expert form is    */
/*  this library's reading, as for the mixture-of-experts path below)       */
/* ------------------------------------------------------------------------ */

/* h[m, f] = silu(zg) * zu  with  zg = sum_k Wg[f, k] x[m, k],
 *                               zu = sum_k Wu[f, k] x[m, k],
 * silu(z) = z / (1 + exp(-z)), for m < M <= 8, f < F, in one launch: both
 * matrices stream in the same workgroups and h is formed in registers, so
 * neither zg nor zu reaches memory.
 *   Wg, Wu: repacked [F, K] weights of one format (device, 16-byte aligned).
 *   x:      as for q4q8_qgemv (shared by both products).
 *   h:      device, dtype hdt (F16, BF16 or F32), row m at h + m*ldh,
 *           ldh >= F when M > 1, aligned to its element size.  Rounded once
 *           from the fp32 value.
 * Rules and errors as for q4q8_qgemv. */
int q4q8_qgemv_swiglu(int fmt, const void* Wg, const void* Wu, int64_t F,
                      int64_t K, const void* x, int xdt, int64_t ldx, int M,
                      void* h, int hdt, int64_t ldh, void* stream);

/* Workspace bytes of q4q8_ffn_decode: the h rows (2 bytes each), M * F * 2
 * rounded up to 256.  0 for M outside 1..8 or F not a positive multiple of 32. */
size_t q4q8_ffn_decode_workspace(int M, int64_t F);

/* The decode FFN of a layer, two launches on `stream`:
 *   h = silu(x Wg^T) * (x Wu^T)   (q4q8_qgemv_swiglu, rounded to bf16)
 *   y = h Wd^T                    (q4q8_qgemv, fp32)
 * h is held in ws as fp16: its bf16 values, converted to nearest (exact for
 * 2^-14 <= |h| < 65520; |h| >= 65520 becomes +-inf), so that the down
 * product takes fp16 operands and the Q4_0 unpack's fp16 form.
 *   Wg, Wu: repacked [F, H]; Wd: repacked [H, F]; one format.
 *   x:      M rows of H activations (F16/BF16), as for q4q8_qgemv.
 *   y:      device fp32, row m at y + m*ldy, ldy >= H when M > 1.
 *   ws:     device, >= q4q8_ffn_decode_workspace(M, F) bytes, 256-byte
 *           aligned; overwritten.  Once the stream has run the call it
 *           holds h, fp16 [M, F] row-major (row stride F).
 * Every argument of both launches is validated before the first is
 * enqueued.  Errors: as q4q8_qgemv, plus Q4Q8_ERR_WORKSPACE. */
int q4q8_ffn_decode(int fmt, const void* Wg, const void* Wu, const void* Wd,
                    int64_t H, int64_t F, const void* x, int xdt,
                    int64_t ldx, int M, float* y, int64_t ldy, void* ws,
                    size_t ws_bytes, void* stream);

/* ------------------------------------------------------------------------ */
/* Prefill: quantised GEMM                                                   */
/* (technical summary, "Methodologie", prefill optimisation: tiled GEMM on  */
/*  matrix intrinsics; review, "Method": prefill GEMM on the matrix units)  */
/* ------------------------------------------------------------------------ */

/* Workspace bytes q4q8_qgemm needs: for BF16 activations their row-scaled
 * fp16 copy, M * Kp * 2 with Kp = K rounded up to 128, rounded up to 256
 * bytes, then the rows' exponents, M * 4 rounded up to 256; 0 for F16.
 * 0 also for invalid xdt/M/K. */
size_t q4q8_qgemm_workspace(int xdt, int64_t M, int64_t K);

/* Y[m, n] = sum_k X[m, k] * W[n, k]   for m < M, n < N.
 *   X:   device, BF16 or F16 (xdt), row m at X + m*ldx; 16-byte aligned,
 *        ldx % 8 == 0, K <= ldx <= 2^22.
 *   Y:   device, ydt = BF16, F16 or F32, row m at Y + m*ldy, ldy >= N,
 *        aligned to its element size.
 *   ws:  device workspace of >= q4q8_qgemm_workspace(xdt, M, K) bytes,
 *        256-byte aligned (may be NULL when that is 0); clobbered.
 *   fmt: Q4Q8_Q4_0, Q4Q8_Q8_0 or Q4Q8_FP16 (plain fp16 weights, the same
 *        repacked tiles; the pages' format list runs up to FP16).
 * fp32 accumulation on fp16 matrix-core operands (weights dequantised and
 * scaled to fp16, relative rounding <= 2^-11, or fp16 weights as they are;
 * BF16 activation rows scaled by a power of two and converted to fp16 as
 * the conventions above state); result rounded once to ydt.
 * M >= 1 (any).  Errors: Q4Q8_ERR_WORKSPACE if ws is missing or short. */
int q4q8_qgemm(int fmt, const void* W, int64_t N, int64_t K,
               const void* X, int xdt, int64_t ldx, int64_t M,
               void* Y, int ydt, int64_t ldy, void* ws, size_t ws_bytes,
               void* stream);

/* ------------------------------------------------------------------------ */
/* Mixture of experts (review, "Method": MoE expert GEMM and fused expert    */
/* projections on the matrix units; the routing rule is this library's)     */
/* ------------------------------------------------------------------------ */

/* Route T tokens over E experts and sort the (token, slot) pairs by expert.
 *   logits:  device fp32 [T, E] row-major.
 *   ids:     device int32 [T, topk]: per token the topk experts with the
 *            largest logits, descending; equal logits -> lower id first.
 *   gates:   device fp32 [T, topk]: softmax over the topk selected logits.
 *   counts:  device int32 [E]: pairs routed to each expert.
 *   offsets: device int32 [E+1]: exclusive scan of counts (offsets[E] =
 *            T*topk).
 *   sorted_pairs: device int32 [T*topk]: pair ids p = t*topk + j ordered by
 *            (expert, p) -- a stable counting sort, bit-exact.
 * Limits: 1 <= topk <= min(E, 16), 1 <= E <= 1024, T >= 1.  No workspace. */
int q4q8_moe_route(const float* logits, int T, int E, int topk,
                   int32_t* ids, float* gates, int32_t* counts,
                   int32_t* offsets, int32_t* sorted_pairs, void* stream);

/* Workspace bytes q4q8_moe_qgemm needs for these sizes. */
size_t q4q8_moe_workspace(int fmt, int T, int E, int topk, int H, int F);

/* Expert SwiGLU over every pair and the weighted combine:
 *   h_p   = silu(x_t W_gate[e]^T) * (x_t W_up[e]^T)      (F values, fp32,
 *           stored as bf16 in sorted-pair order)
 *   y_p   = h_p W_down[e]^T                              (H values, fp32)
 *   out_t = sum_j gates[t, j] * y_{t*topk + j}           (fp32)
 *   Wg, Wu: device, E repacked [F, H] matrices, expert e at
 *           e * q4q8_repacked_bytes(fmt, F, H).
 *   Wd:     device, E repacked [H, F] matrices, expert e at
 *           e * q4q8_repacked_bytes(fmt, H, F).
 *   X:      device BF16 (or F16, xdt) [T, H] row-major, 16-byte aligned.
 *   gates, offsets, sorted_pairs: as produced by q4q8_moe_route.
 *   out:    device fp32 [T, H].
 *   h_out:  optional (NULL to skip) device bf16 [T*topk, F]: the h rows in
 *           sorted-pair order, for inspection.
 *   ws:     device workspace of >= q4q8_moe_workspace(...) bytes, 256-byte
 *           aligned; contents need no initialisation and are clobbered.
 * H % 128 == 0 and F % 128 == 0.  Pairs of one expert are processed
 * together, so each expert's weights are streamed once per call.
 * Kernel choice (review, "Method": memory-bound decode stays on the GEMV
 * kernels, compute-bound prefill goes to the matrix-unit tiles): up to 8
 * tokens whose rows fit 52 KB of LDS (8 x max(H, F) halfs) run on GEMV
 * kernels, each expert's routed tokens as its activation rows; larger T on
 * 64-row matrix-core tiles.  Both paths round h to bf16 and y to fp16 and
 * combine in the same fixed order. */
int q4q8_moe_qgemm(int fmt, const void* Wg, const void* Wu, const void* Wd,
                   int E, int H, int F, const void* X, int xdt, int T,
                   int topk, const float* gates,
                   const int32_t* offsets, const int32_t* sorted_pairs,
                   float* out, void* h_out, void* ws, size_t ws_bytes,
                   void* stream);

/* MoE decode in one call: q4q8_moe_route followed by q4q8_moe_qgemm for a
 * few tokens, with the routing derived inside the first expert kernel
 * instead of by a kernel of its own (one launch fewer on the short decode
 * step; review, "Method": decode on the GEMV kernels).
 *   logits:  device fp32 [T, E].
 *   ids, gates, counts, offsets, sorted_pairs: outputs, exactly as
 *            q4q8_moe_route defines them (same bits), 4-byte aligned.
 *   Wg, Wu, Wd, X, xdt, out, h_out, ws: as q4q8_moe_qgemm (ws of
 *            q4q8_moe_workspace(fmt, T, E, topk, H, F) bytes).
 * Up to 4 tokens the routing runs inside the first expert kernel; past 4
 * (where one wave per token in every workgroup costs more than a launch) the
 * call runs the routing kernel first.
 * out and h_out equal those of q4q8_moe_route + q4q8_moe_qgemm bit for bit.
 * Limits: the decode path only -- T <= 8 and T * (max(H, F) + 8) * 2 + 512
 * <= 52 KB, else Q4Q8_ERR_UNSUPPORTED; otherwise as q4q8_moe_route and
 * q4q8_moe_qgemm. */
int q4q8_moe_decode(int fmt, const void* Wg, const void* Wu, const void* Wd,
                    int E, int H, int F, const float* logits, const void* X,
                    int xdt, int T, int topk, int32_t* ids, float* gates,
                    int32_t* counts, int32_t* offsets, int32_t* sorted_pairs,
                    float* out, void* h_out, void* ws, size_t ws_bytes,
                    void* stream);

/* The whole MoE layer in one call for any T: q4q8_moe_route followed by
 * q4q8_moe_qgemm, with the same results bit for bit (routing arrays, out,
 * h_out).  Up to the decode path's limits (T <= 8 and T * (max(H, F) + 8)
 * * 2 + 512 <= 52 KB) it is q4q8_moe_decode.  Above, three launches precede
 * the combine: top-k plus the activation row scaling (one wave per token),
 * then gate+up, whose workgroups find their expert's rows from the routed
 * experts in pair order -- the stable sort, formed in the expert kernel
 * instead of by a sort kernel (the expert's first workgroup stores its
 * count, offset and slice of sorted_pairs) -- then down.
 *   Arguments as q4q8_moe_decode; ws of q4q8_moe_workspace(fmt, T, E, topk,
 *   H, F) bytes.  Limits as q4q8_moe_route and q4q8_moe_qgemm. */
int q4q8_moe_forward(int fmt, const void* Wg, const void* Wu, const void* Wd,
                     int E, int H, int F, const float* logits, const void* X,
                     int xdt, int T, int topk, int32_t* ids, float* gates,
                     int32_t* counts, int32_t* offsets, int32_t* sorted_pairs,
                     float* out, void* h_out, void* ws, size_t ws_bytes,
                     void* stream);

/* q4q8_moe_decode without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The call allocates nothing and calls
 * no allocating routine: its scratch is a static device array of
 * q4q8_moe_decode_noalloc_max_scratch() bytes (1 MiB) that the library's
 * module holds on every GPU it runs on until the process ends; its address
 * on the stream's device is looked up once, on that device's first call.
 * Arguments, results and limits are those of q4q8_moe_decode (same kernels,
 * same bits); a call whose q4q8_moe_workspace(fmt, T, E, topk, H, F)
 * exceeds the scratch returns Q4Q8_ERR_UNSUPPORTED and enqueues nothing
 * (the MoE shape of E 128, top-8, H 2048, F 768 needs 0.4 MB at T = 8).
 * The scratch needs no initialisation and keeps the last call's contents.
 * Every call on one GPU shares that GPU's scratch: calls that can overlap on
 * one GPU (different streams, or different threads without ordering) race
 * and must be serialised by the caller. */
int q4q8_moe_decode_noalloc(int fmt, const void* Wg, const void* Wu,
                            const void* Wd, int E, int H, int F,
                            const float* logits, const void* X, int xdt,
                            int T, int topk, int32_t* ids, float* gates,
                            int32_t* counts, int32_t* offsets,
                            int32_t* sorted_pairs, float* out, void* h_out,
                            void* stream);

/* Bytes of q4q8_moe_decode_noalloc's per-GPU scratch. */
size_t q4q8_moe_decode_noalloc_max_scratch(void);

/* ------------------------------------------------------------------------ */
/* Prefill attention (technical summary, "Methodologie", prefill            */
/* optimisation: tiled attention with an online softmax, O(n) memory;       */
/* review, "Method": prefill attention on the matrix units)                 */
/* ------------------------------------------------------------------------ */

/* O[b, i, h, :] = sum_j p_j V[b, j, h / (Hq/Hkv), :],
 *   p = softmax_j(scale * Q[b, i, h, :] . K[b, j, h / (Hq/Hkv), :])
 * over keys j < S, and j <= i when causal != 0.  The S x S scores are never
 * stored: keys are processed in blocks with a running max and sum.
 *   Q, O: device [B, S, Hq, D] row-major; K, V: device [B, S, Hkv, D]; all
 *         of dtype dt (F16 or BF16).  Q, K, V 16-byte aligned, O 8-byte.
 *   D:    head dimension, 128.  Hq a multiple of Hkv.  scale > 0 (usually
 *         1/sqrt(D)).
 * Scores and the softmax statistics are fp32; the probabilities enter the
 * P.V product and the row sums rounded to dt; O is rounded once to dt.
 * Errors: Q4Q8_ERR_UNSUPPORTED for other D or dtypes. */
int q4q8_attn_prefill(int dt, const void* Q, const void* K, const void* V,
                      void* O, int B, int S, int Hq, int Hkv, int D,
                      int causal, float scale, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* Q4Q8_H */
