"""Python binding of libq4q8.so (ctypes), with torch tensors for memory and streams.

Argument marshalling only: every computation runs in the library's HIP
kernels.  Tensors are passed by data pointer together with the current HIP
stream of their device.  If the library is not built the first call raises;
there is no fallback path.

Formats: Q4_0 = 1, Q8_0 = 2, FP16 = 3 (plain fp16 weights: layout, GEMV and
GEMM calls).  Activation dtypes: torch.float16 or torch.bfloat16.  Weights
are uint8 tensors holding repacked blocks (see repack()).
"""
from __future__ import annotations

import ctypes
import os

import torch

Q4_0 = 1
Q8_0 = 2
FP16 = 3
F16 = 1
BF16 = 2
F32 = 3
MAX_GROUP = 8

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libq4q8.so")
_lib = None

_DT = {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32}


class Q4Q8Error(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: status {status} ({status_string(status)}): {last_error()}")
        self.status = status


class GemvDesc(ctypes.Structure):
    _fields_ = [("W", ctypes.c_void_p), ("x", ctypes.c_void_p), ("y", ctypes.c_void_p),
                ("N", ctypes.c_int64), ("K", ctypes.c_int64),
                ("ldx", ctypes.c_int64), ("ldy", ctypes.c_int64)]


def _declare(lib):
    i64, i32, vp, sz = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t
    sig = {
        "q4q8_abi_version": (i32, []),
        "q4q8_status_string": (ctypes.c_char_p, [i32]),
        "q4q8_last_error": (ctypes.c_char_p, []),
        "q4q8_canonical_bytes": (sz, [i32, i64, i64]),
        "q4q8_repacked_bytes": (sz, [i32, i64, i64]),
        "q4q8_repack": (i32, [i32, vp, i64, i64, vp, sz, vp]),
        "q4q8_repack_host": (i32, [i32, vp, i64, i64, vp, sz]),
        "q4q8_qgemv": (i32, [i32, vp, i64, i64, vp, i32, i64, i32, vp, i64, vp]),
        "q4q8_qgemv_grouped": (i32, [i32, ctypes.POINTER(GemvDesc), i32, i32, i32, vp]),
        "q4q8_qgemv_grouped_timed": (i32, [i32, ctypes.POINTER(GemvDesc), i32, i32, i32, vp, vp, vp]),
        "q4q8_qgemv_swiglu": (i32, [i32, vp, vp, i64, i64, vp, i32, i64, i32, vp, i32, i64, vp]),
        "q4q8_qgemv_swiglu_timed": (i32, [i32, vp, vp, i64, i64, vp, i32, i64, i32, vp, i32, i64, vp, vp, vp]),
        "q4q8_ffn_decode_workspace": (sz, [i32, i64]),
        "q4q8_ffn_decode": (i32, [i32, vp, vp, vp, i64, i64, vp, i32, i64, i32, vp, i64, vp, sz, vp]),
        "q4q8_ffn_decode_timed": (i32, [i32, vp, vp, vp, i64, i64, vp, i32, i64, i32, vp, i64, vp, sz, vp,
                                        vp, vp]),
        "q4q8_attn_prefill": (i32, [i32, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, ctypes.c_float, vp]),
        "q4q8_attn_prefill_timed": (i32, [i32, vp, vp, vp, vp, i32, i32, i32, i32, i32, i32, ctypes.c_float, vp,
                                          vp, vp]),
        "q4q8_qgemm_workspace": (sz, [i32, i64, i64]),
        "q4q8_qgemm": (i32, [i32, vp, i64, i64, vp, i32, i64, i64, vp, i32, i64, vp, sz, vp]),
        "q4q8_qgemm_timed": (i32, [i32, vp, i64, i64, vp, i32, i64, i64, vp, i32, i64, vp, sz, vp, vp, vp]),
        "q4q8_moe_route": (i32, [vp, i32, i32, i32, vp, vp, vp, vp, vp, vp]),
        "q4q8_moe_workspace": (sz, [i32, i32, i32, i32, i32, i32]),
        "q4q8_moe_qgemm": (i32, [i32, vp, vp, vp, i32, i32, i32, vp, i32, i32, i32,
                                 vp, vp, vp, vp, vp, vp, sz, vp]),
        "q4q8_moe_decode": (i32, [i32, vp, vp, vp, i32, i32, i32, vp, vp, i32, i32, i32,
                                  vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "q4q8_moe_forward": (i32, [i32, vp, vp, vp, i32, i32, i32, vp, vp, i32, i32, i32,
                                   vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]),
        "q4q8_moe_decode_noalloc": (i32, [i32, vp, vp, vp, i32, i32, i32, vp, vp, i32, i32, i32,
                                          vp, vp, vp, vp, vp, vp, vp, vp]),
        "q4q8_moe_decode_noalloc_max_scratch": (sz, []),
        "q4q8_stream_read_digest_bytes": (sz, []),
        "q4q8_stream_read_timed": (i32, [vp, sz, vp, sz, vp, vp, vp]),
        "q4q8_stream_read_grid_timed": (i32, [vp, sz, i32, vp, sz, vp, vp, vp]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


def lib():
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(or python gemm_q4_q8_amd/build.py)")
        _lib = _declare(ctypes.CDLL(LIB_PATH))
    return _lib


def status_string(s: int) -> str:
    return lib().q4q8_status_string(s).decode()


def last_error() -> str:
    return lib().q4q8_last_error().decode()


def _check(st: int, what: str):
    if st != 0:
        raise Q4Q8Error(st, what)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None else ctypes.c_void_p(0)


def _dev(t: torch.Tensor, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# ----------------------------------------------------------------------------
# Layout
# ----------------------------------------------------------------------------
def canonical_bytes(fmt: int, N: int, K: int) -> int:
    return int(lib().q4q8_canonical_bytes(fmt, N, K))


def repacked_bytes(fmt: int, N: int, K: int) -> int:
    return int(lib().q4q8_repacked_bytes(fmt, N, K))


def repack(fmt: int, canon: torch.Tensor, N: int, K: int, out: torch.Tensor | None = None) -> torch.Tensor:
    """Canonical blocks (uint8 GPU tensor) -> repacked weights (uint8 GPU tensor)."""
    _dev(canon, "canon")
    nb = repacked_bytes(fmt, N, K)
    if out is None:
        out = torch.empty(nb, dtype=torch.uint8, device=canon.device)
    _dev(out, "out")
    if canon.numel() * canon.element_size() != canonical_bytes(fmt, N, K):
        raise ValueError("canonical tensor has the wrong size")
    _check(lib().q4q8_repack(fmt, _ptr(canon), N, K, _ptr(out), out.numel() * out.element_size(),
                             _stream(canon)), "repack")
    return out


def repack_host(fmt: int, canon, N: int, K: int):
    """Host-side conversion (numpy uint8 in, numpy uint8 out); touches no GPU."""
    import numpy as np
    src = np.ascontiguousarray(canon, dtype=np.uint8)
    if src.size != canonical_bytes(fmt, N, K):
        raise ValueError("canonical buffer has the wrong size")
    dst = np.empty(repacked_bytes(fmt, N, K), dtype=np.uint8)
    _check(lib().q4q8_repack_host(fmt, src.ctypes.data_as(ctypes.c_void_p), N, K,
                                  dst.ctypes.data_as(ctypes.c_void_p), dst.size), "repack_host")
    return dst


# ----------------------------------------------------------------------------
# Products
# ----------------------------------------------------------------------------
def qgemv(fmt: int, W: torch.Tensor, N: int, K: int, x: torch.Tensor,
          out: torch.Tensor | None = None) -> torch.Tensor:
    """y[M, N] fp32 = x[M, K] (fp16/bf16) @ W^T, M = 1..8."""
    _dev(W, "W")
    if x.dim() != 2 or x.shape[1] != K:
        raise ValueError("x must be [M, K]")
    if x.stride(1) != 1:
        raise ValueError("x rows must be contiguous")
    M = x.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=x.device)
    _check(lib().q4q8_qgemv(fmt, _ptr(W), N, K, _ptr(x), _DT[x.dtype], x.stride(0), M,
                            _ptr(out), out.stride(0), _stream(x)), "qgemv")
    return out


def gemv_descs(problems):
    """ctypes descriptor array for problems [(W, N, K, x [M,K], y [M,N] fp32)]."""
    arr = (GemvDesc * max(len(problems), 1))()
    for i, (W, N, K, x, y) in enumerate(problems):
        _dev(W, "W")
        arr[i] = GemvDesc(W.data_ptr(), x.data_ptr(), y.data_ptr(), N, K, x.stride(0), y.stride(0))
    return arr


def qgemv_grouped(fmt: int, problems, M: int, descs=None, events=None):
    """problems: list of (W, N, K, x [M,K], y [M,N] fp32); one launch.

    descs: a prebuilt gemv_descs(problems) (saves rebuilding it per call).
    events: optional (start, stop) raw hipEvent_t handles recorded by the
    dispatch itself.
    """
    n = len(problems)
    arr = descs if descs is not None else gemv_descs(problems)
    xdt = _DT[problems[0][3].dtype]
    stream = _stream(problems[0][3])
    if events is None:
        st = lib().q4q8_qgemv_grouped(fmt, arr, n, xdt, M, stream)
    else:
        st = lib().q4q8_qgemv_grouped_timed(fmt, arr, n, xdt, M, stream,
                                            ctypes.c_void_p(events[0]), ctypes.c_void_p(events[1]))
    _check(st, "qgemv_grouped")


def qgemv_swiglu(fmt: int, Wg: torch.Tensor, Wu: torch.Tensor, F: int, K: int, x: torch.Tensor,
                 out: torch.Tensor | None = None, out_dtype=torch.bfloat16, events=None) -> torch.Tensor:
    """h[M, F] = silu(x @ Wg^T) * (x @ Wu^T), one launch, output out_dtype."""
    _dev(Wg, "Wg")
    _dev(Wu, "Wu")
    if x.dim() != 2 or x.shape[1] != K or x.stride(1) != 1:
        raise ValueError("x must be [M, K] with contiguous rows")
    M = x.shape[0]
    if out is None:
        out = torch.empty((M, F), dtype=out_dtype, device=x.device)
    args = (fmt, _ptr(Wg), _ptr(Wu), F, K, _ptr(x), _DT[x.dtype], x.stride(0), M, _ptr(out), _DT[out.dtype],
            out.stride(0), _stream(x))
    if events is None:
        st = lib().q4q8_qgemv_swiglu(*args)
    else:
        st = lib().q4q8_qgemv_swiglu_timed(*args, ctypes.c_void_p(events[0]), ctypes.c_void_p(events[1]))
    _check(st, "qgemv_swiglu")
    return out


def ffn_decode_workspace(M: int, F: int) -> int:
    return int(lib().q4q8_ffn_decode_workspace(M, F))


def ffn_decode(fmt: int, Wg: torch.Tensor, Wu: torch.Tensor, Wd: torch.Tensor, H: int, F: int, x: torch.Tensor,
               out: torch.Tensor | None = None, ws: torch.Tensor | None = None, events=None) -> torch.Tensor:
    """y[M, H] fp32 = (silu(x Wg^T) * (x Wu^T)) Wd^T, h rounded to bf16 and held as fp16; two launches.

    ws: optional uint8 workspace of >= ffn_decode_workspace(M, F) bytes (the
    h rows, fp16; allocated per call if omitted).
    """
    for t, n in ((Wg, "Wg"), (Wu, "Wu"), (Wd, "Wd")):
        _dev(t, n)
    if x.dim() != 2 or x.shape[1] != H or x.stride(1) != 1:
        raise ValueError("x must be [M, H] with contiguous rows")
    M = x.shape[0]
    if out is None:
        out = torch.empty((M, H), dtype=torch.float32, device=x.device)
    if ws is None:
        ws = torch.empty(max(ffn_decode_workspace(M, F), 1), dtype=torch.uint8, device=x.device)
    args = (fmt, _ptr(Wg), _ptr(Wu), _ptr(Wd), H, F, _ptr(x), _DT[x.dtype], x.stride(0), M, _ptr(out),
            out.stride(0), _ptr(ws), ws.numel() * ws.element_size(), _stream(x))
    if events is None:
        st = lib().q4q8_ffn_decode(*args)
    else:
        st = lib().q4q8_ffn_decode_timed(*args, ctypes.c_void_p(events[0]), ctypes.c_void_p(events[1]))
    _check(st, "ffn_decode")
    return out


def qgemm_workspace(xdt: int, M: int, K: int) -> int:
    return int(lib().q4q8_qgemm_workspace(xdt, M, K))


def qgemm(fmt: int, W: torch.Tensor, N: int, K: int, X: torch.Tensor,
          out: torch.Tensor | None = None, out_dtype=torch.bfloat16, ws: torch.Tensor | None = None,
          events=None) -> torch.Tensor:
    """Y[M, N] = X[M, K] @ W^T, fp32 accumulation, output out_dtype.

    ws: optional uint8 workspace of >= qgemm_workspace() bytes (allocated per
    call if omitted).  events: optional (start, stop) raw hipEvent_t handles.
    """
    _dev(W, "W")
    if X.dim() != 2 or X.shape[1] != K or X.stride(1) != 1:
        raise ValueError("X must be [M, K] with contiguous rows")
    M = X.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=X.device)
    xdt = _DT[X.dtype]
    nws = qgemm_workspace(xdt, M, K)
    if ws is None and nws:
        ws = torch.empty(nws, dtype=torch.uint8, device=X.device)
    nbytes = ws.numel() * ws.element_size() if ws is not None else 0
    args = (fmt, _ptr(W), N, K, _ptr(X), xdt, X.stride(0), M, _ptr(out), _DT[out.dtype], out.stride(0),
            _ptr(ws), nbytes, _stream(X))
    if events is None:
        st = lib().q4q8_qgemm(*args)
    else:
        st = lib().q4q8_qgemm_timed(*args, ctypes.c_void_p(events[0]), ctypes.c_void_p(events[1]))
    _check(st, "qgemm")
    return out


def moe_route(logits: torch.Tensor, topk: int, out=None):
    """-> ids [T,k] int32, gates [T,k] fp32, counts [E], offsets [E+1], sorted_pairs [T*k].

    out: optional preallocated (ids, gates, counts, offsets, sorted_pairs).
    """
    _dev(logits, "logits")
    T, E = logits.shape
    d = logits.device
    if out is not None:
        ids, gates, counts, offsets, sp = out
    else:
        ids = torch.empty((T, topk), dtype=torch.int32, device=d)
        gates = torch.empty((T, topk), dtype=torch.float32, device=d)
        counts = torch.empty(E, dtype=torch.int32, device=d)
        offsets = torch.empty(E + 1, dtype=torch.int32, device=d)
        sp = torch.empty(T * topk, dtype=torch.int32, device=d)
    _check(lib().q4q8_moe_route(_ptr(logits), T, E, topk, _ptr(ids), _ptr(gates), _ptr(counts),
                                _ptr(offsets), _ptr(sp), _stream(logits)), "moe_route")
    return ids, gates, counts, offsets, sp


def moe_workspace(fmt: int, T: int, E: int, topk: int, H: int, F: int) -> int:
    return int(lib().q4q8_moe_workspace(fmt, T, E, topk, H, F))


def moe_qgemm(fmt: int, Wg, Wu, Wd, E: int, H: int, F: int, X: torch.Tensor, topk: int,
              gates, offsets, sorted_pairs, out=None, h_out=None, ws=None):
    """Expert SwiGLU + weighted combine -> out [T, H] fp32."""
    T = X.shape[0]
    d = X.device
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=d)
    nws = moe_workspace(fmt, T, E, topk, H, F)
    if ws is None:
        ws = torch.empty(nws, dtype=torch.uint8, device=d)
    _check(lib().q4q8_moe_qgemm(fmt, _ptr(Wg), _ptr(Wu), _ptr(Wd), E, H, F, _ptr(X), _DT[X.dtype], T, topk,
                                _ptr(gates), _ptr(offsets), _ptr(sorted_pairs), _ptr(out),
                                _ptr(h_out), _ptr(ws), ws.numel() * ws.element_size(), _stream(X)),
           "moe_qgemm")
    return out


def moe_decode(fmt: int, Wg, Wu, Wd, E: int, H: int, F: int, logits: torch.Tensor, X: torch.Tensor, topk: int,
               route=None, out=None, h_out=None, ws=None):
    """Routing and expert products of a few tokens in one call ->
    (out [T, H] fp32, (ids, gates, counts, offsets, sorted_pairs)).

    route: optional preallocated routing arrays, as moe_route's out."""
    _dev(logits, "logits")
    T = X.shape[0]
    d = X.device
    if logits.shape != (T, E):
        raise ValueError("logits must be [T, E]")
    if route is None:
        route = (torch.empty((T, topk), dtype=torch.int32, device=d), torch.empty((T, topk), dtype=torch.float32, device=d),
                 torch.empty(E, dtype=torch.int32, device=d), torch.empty(E + 1, dtype=torch.int32, device=d),
                 torch.empty(T * topk, dtype=torch.int32, device=d))
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=d)
    nws = moe_workspace(fmt, T, E, topk, H, F)
    if ws is None:
        ws = torch.empty(nws, dtype=torch.uint8, device=d)
    ids, gates, counts, offsets, sp = route
    _check(lib().q4q8_moe_decode(fmt, _ptr(Wg), _ptr(Wu), _ptr(Wd), E, H, F, _ptr(logits), _ptr(X), _DT[X.dtype], T,
                                 topk, _ptr(ids), _ptr(gates), _ptr(counts), _ptr(offsets), _ptr(sp), _ptr(out),
                                 _ptr(h_out), _ptr(ws), ws.numel() * ws.element_size(), _stream(X)),
           "moe_decode")
    return out, route


def moe_forward(fmt: int, Wg, Wu, Wd, E: int, H: int, F: int, logits: torch.Tensor, X: torch.Tensor, topk: int,
                route=None, out=None, h_out=None, ws=None):
    """The whole MoE layer for any T in one call (q4q8_moe_forward) ->
    (out [T, H] fp32, (ids, gates, counts, offsets, sorted_pairs))."""
    _dev(logits, "logits")
    T = X.shape[0]
    d = X.device
    if logits.shape != (T, E):
        raise ValueError("logits must be [T, E]")
    if route is None:
        route = (torch.empty((T, topk), dtype=torch.int32, device=d), torch.empty((T, topk), dtype=torch.float32, device=d),
                 torch.empty(E, dtype=torch.int32, device=d), torch.empty(E + 1, dtype=torch.int32, device=d),
                 torch.empty(T * topk, dtype=torch.int32, device=d))
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=d)
    nws = moe_workspace(fmt, T, E, topk, H, F)
    if ws is None:
        ws = torch.empty(nws, dtype=torch.uint8, device=d)
    ids, gates, counts, offsets, sp = route
    _check(lib().q4q8_moe_forward(fmt, _ptr(Wg), _ptr(Wu), _ptr(Wd), E, H, F, _ptr(logits), _ptr(X), _DT[X.dtype],
                                  T, topk, _ptr(ids), _ptr(gates), _ptr(counts), _ptr(offsets), _ptr(sp), _ptr(out),
                                  _ptr(h_out), _ptr(ws), ws.numel() * ws.element_size(), _stream(X)),
           "moe_forward")
    return out, route


def moe_decode_noalloc(fmt: int, Wg, Wu, Wd, E: int, H: int, F: int, logits: torch.Tensor, X: torch.Tensor,
                       topk: int, route=None, out=None, h_out=None):
    """moe_decode on the library's static per-GPU scratch (no workspace, no
    allocation inside the call; the route/out/h_out tensors are allocated
    here only when not given).  Calls that overlap on one GPU race."""
    _dev(logits, "logits")
    T = X.shape[0]
    d = X.device
    if logits.shape != (T, E):
        raise ValueError("logits must be [T, E]")
    if route is None:
        route = (torch.empty((T, topk), dtype=torch.int32, device=d), torch.empty((T, topk), dtype=torch.float32, device=d),
                 torch.empty(E, dtype=torch.int32, device=d), torch.empty(E + 1, dtype=torch.int32, device=d),
                 torch.empty(T * topk, dtype=torch.int32, device=d))
    if out is None:
        out = torch.empty((T, H), dtype=torch.float32, device=d)
    ids, gates, counts, offsets, sp = route
    _check(lib().q4q8_moe_decode_noalloc(fmt, _ptr(Wg), _ptr(Wu), _ptr(Wd), E, H, F, _ptr(logits), _ptr(X),
                                         _DT[X.dtype], T, topk, _ptr(ids), _ptr(gates), _ptr(counts), _ptr(offsets),
                                         _ptr(sp), _ptr(out), _ptr(h_out), _stream(X)),
           "moe_decode_noalloc")
    return out, route


def attn_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, causal: bool = True, scale=None,
                 out: torch.Tensor | None = None, events=None) -> torch.Tensor:
    """O [B, S, Hq, D] = softmax(scale Q K^T) V per head (GQA), bf16/fp16."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _dev(t, n)
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if k.shape != (B, S, Hkv, D) or v.shape != k.shape or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("k and v must be [B, S, Hkv, D] of q's dtype")
    if out is None:
        out = torch.empty_like(q)
    _dev(out, "out")
    sc = (1.0 / D ** 0.5) if scale is None else float(scale)
    args = (_DT[q.dtype], _ptr(q), _ptr(k), _ptr(v), _ptr(out), B, S, Hq, Hkv, D, 1 if causal else 0, sc, _stream(q))
    if events is None:
        st = lib().q4q8_attn_prefill(*args)
    else:
        st = lib().q4q8_attn_prefill_timed(*args, ctypes.c_void_p(events[0]), ctypes.c_void_p(events[1]))
    _check(st, "attn_prefill")
    return out


# ----------------------------------------------------------------------------
# Measurement helper
# ----------------------------------------------------------------------------
def stream_read(buf: torch.Tensor, digest: torch.Tensor = None, events=None, workgroups: int = None) -> torch.Tensor:
    """Read every byte of buf once on the GPU (the HBM read-ceiling probe);
    returns the per-wave XOR digests (int32).  events: optional (start, stop)
    hipEvent_t handles recorded around the kernel.  workgroups: the probe's
    grid (default: the library's, tuned for GiB-sized reads)."""
    _dev(buf, "buf")
    n = int(lib().q4q8_stream_read_digest_bytes())
    if digest is None:
        digest = torch.empty(n // 4, dtype=torch.int32, device=buf.device)
    ev = events or (None, None)
    if workgroups is None:
        st = lib().q4q8_stream_read_timed(_ptr(buf), buf.numel() * buf.element_size(), _ptr(digest),
                                          digest.numel() * digest.element_size(), _stream(buf),
                                          ctypes.c_void_p(ev[0]), ctypes.c_void_p(ev[1]))
    else:
        st = lib().q4q8_stream_read_grid_timed(_ptr(buf), buf.numel() * buf.element_size(), int(workgroups),
                                               _ptr(digest), digest.numel() * digest.element_size(), _stream(buf),
                                               ctypes.c_void_p(ev[0]), ctypes.c_void_p(ev[1]))
    _check(st, "stream_read")
    return digest
