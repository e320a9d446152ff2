/*
 * q4q8_measure.h -- measurement entry points of the q4q8 library (MI355X,
 * gfx950), apart from the product interface in q4q8.h.
 *
 * The *_timed calls compute exactly what the call of the same name without
 * the suffix computes (same kernels, same results); the kernel dispatch
 * itself records the two hipEvent_t handles passed as void* (either may be
 * NULL), so hipEventElapsedTime gives the kernels' own duration without the
 * host's launch gaps.  q4q8_stream_read_timed measures the HBM read rate the
 * decode GEMV is compared with.  Conventions (streams, errors, ownership)
 * are those of q4q8.h.
 */
#ifndef Q4Q8_MEASURE_H
#define Q4Q8_MEASURE_H

#include "q4q8.h"

#ifdef __cplusplus
extern "C" {
#endif

/* As q4q8_qgemv_grouped, and the dispatch itself records ev_start when the
 * kernel starts and ev_stop when it ends (hipEvent_t handles, either may be
 * NULL), so hipEventElapsedTime gives the kernel's own duration.  For
 * measurement; the result is identical. */
int q4q8_qgemv_grouped_timed(int fmt, const q4q8_gemv_desc* descs, int count,
                             int xdt, int M, void* stream,
                             void* ev_start, void* ev_stop);

/* As q4q8_qgemv_swiglu, with dispatch-recorded events (see
 * q4q8_qgemv_grouped_timed).  For measurement; the result is identical. */
int q4q8_qgemv_swiglu_timed(int fmt, const void* Wg, const void* Wu,
                            int64_t F, int64_t K, const void* x, int xdt,
                            int64_t ldx, int M, void* h, int hdt,
                            int64_t ldh, void* stream, void* ev_start,
                            void* ev_stop);

/* As q4q8_ffn_decode, with ev_start recorded when the first kernel starts
 * and ev_stop when the second ends.  For measurement. */
int q4q8_ffn_decode_timed(int fmt, const void* Wg, const void* Wu,
                          const void* Wd, int64_t H, int64_t F,
                          const void* x, int xdt, int64_t ldx, int M,
                          float* y, int64_t ldy, void* ws, size_t ws_bytes,
                          void* stream, void* ev_start, void* ev_stop);

/* As q4q8_qgemm, with dispatch-recorded events (see
 * q4q8_qgemv_grouped_timed): ev_start when the first kernel of the call
 * starts, ev_stop when the last ends.  For measurement; the result is
 * identical. */
int q4q8_qgemm_timed(int fmt, const void* W, int64_t N, int64_t K,
                     const void* X, int xdt, int64_t ldx, int64_t M,
                     void* Y, int ydt, int64_t ldy, void* ws,
                     size_t ws_bytes, void* stream,
                     void* ev_start, void* ev_stop);

/* As q4q8_attn_prefill, with dispatch-recorded events (see
 * q4q8_qgemv_grouped_timed).  For measurement; the result is identical. */
int q4q8_attn_prefill_timed(int dt, const void* Q, const void* K,
                            const void* V, void* O, int B, int S, int Hq,
                            int Hkv, int D, int causal, float scale,
                            void* stream, void* ev_start, void* ev_stop);

/* ------------------------------------------------------------------------ */
/* Measurement helper: the HBM read ceiling the decode GEMV is compared      */
/* with (not a quantised product)                                           */
/* ------------------------------------------------------------------------ */

/* Bytes the digest of q4q8_stream_read_timed needs (one word per wave of its
 * fixed grid). */
size_t q4q8_stream_read_digest_bytes(void);

/* Reads bytes of device memory at buf once, with 16-byte non-temporal loads
 * (the GEMV's weight-load policy) over a grid that fills every CU, and writes
 * per-wave XOR digests of the 32-bit words read to digest, so that XOR-ing
 * every digest word gives the XOR of the buffer.  ev_start / ev_stop
 * (optional, as in q4q8_qgemv_grouped_timed) bracket the kernel; bytes / that
 * time is the streaming read rate.
 *   buf:    device, 16-byte aligned; bytes a multiple of 16 (>= 16).
 *   digest: device, >= q4q8_stream_read_digest_bytes() bytes, 4-byte aligned;
 *           overwritten.
 * Errors: Q4Q8_ERR_INVALID_ARG (null, size), Q4Q8_ERR_ALIGNMENT. */
int q4q8_stream_read_timed(const void* buf, size_t bytes, uint32_t* digest,
                           size_t digest_bytes, void* stream,
                           void* ev_start, void* ev_stop);

/* As q4q8_stream_read_timed over a grid of `workgroups` 512-thread
 * workgroups (1 .. 16384; q4q8_stream_read_timed takes 16384, the best
 * grid for GiB-sized reads), so that a short read can be timed on the grid
 * that suits its size.  Only the digest words of those workgroups (the
 * first workgroups * 8) are written.
 * Errors: as q4q8_stream_read_timed, and Q4Q8_ERR_INVALID_ARG for
 * workgroups outside 1 .. 16384. */
int q4q8_stream_read_grid_timed(const void* buf, size_t bytes, int workgroups,
                                uint32_t* digest, size_t digest_bytes,
                                void* stream, void* ev_start, void* ev_stop);

#ifdef __cplusplus
}
#endif

#endif /* Q4Q8_MEASURE_H */
