"""CPU oracle for the block-quantised weight products (fp64, NumPy).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import or call
this package; only the tests, the smoke check and the benchmark's CPU-baseline
leg do.  It shares no code with the HIP library or its Python binding: it has
its own block decoder and computes every result from the plain definitions.

What it follows (all from "BaseRT: Best-in-Class LLM Inference on Apple
Silicon via Native Metal", gist.science technical summary, section
"Methodologie", paragraph on kernel specialisation; and the follow-up review
"BaseRT: Advancing Best-in-Class LLM Inference with Apple M5 Neural
Accelerators", section "Method"):

* decode uses a GEMV and prefill a GEMM, one variant per quantisation format,
  with dequantisation inside the inner loop, so the product equals
  "dequantise the block, then take the dot product";
* mixture-of-experts prefill runs grouped expert GEMMs with fused expert
  projections.

The block formats, the routing rule and the SwiGLU expert are not defined on
the pages; the oracle takes these readings:

* Q4_0: 32 weights per block, fp16 scale s, 4-bit codes q; w = s*(q-8).
  Byte i of the 16 code bytes holds q[i] (low nibble) and q[i+16] (high).
* Q8_0: 32 weights per block, fp16 scale s, int8 codes q; w = s*q.
* FP16: plain fp16 weights, row-major little-endian (the pages' format list
  runs up to FP16; technical summary abstract).
* Routing: per token, the top-k experts by logit, descending, equal logits
  broken towards the lower expert id, NaN ranked as -inf; gates = softmax
  over the k selected logits.
* Sorting: pairs p = t*k + j are ordered by (expert, p); counts and offsets are
  the histogram and its exclusive scan.
* Attention (prefill): softmax(scale q k^T) v per head, causal, GQA by
  contiguous groups of query heads (readings: the pages name the tiled
  online-softmax method but no masking, head layout or scale).
* Expert: h = silu(x W_gate^T) * (x W_up^T), y = h W_down^T,
  out[t] = sum_j gate[t, j] * y[pair(t, j)].  The decode FFN (ffn) is the
  same SwiGLU block on a dense layer; the pages credit fusing such
  feed-forward operator sequences for decode (technical summary,
  "Methodologie", fusion).

Every function returns float64 (or exact integers).  Error bounds returned
next to the values are the sums of |w*x| that the acceptance rule scales.

Parity pins: see tests/test_oracle.py (brute force in exact rationals, closed
forms, invariants, textbook special cases).  Every function here is pinned.
"""
from __future__ import annotations

import numpy as np

Q4_0 = 1
Q8_0 = 2
FP16 = 3
QK = 32
_BLOCK_BYTES = {Q4_0: 18, Q8_0: 34}


# ----------------------------------------------------------------------------
# Block decoding
# ----------------------------------------------------------------------------
def _blocks(fmt: int, canon, N: int, K: int) -> np.ndarray:
    if K % QK:
        raise ValueError("K must be a multiple of 32")
    b = np.frombuffer(np.ascontiguousarray(canon, dtype=np.uint8).tobytes(), dtype=np.uint8)
    nb = K // QK
    if b.size != N * nb * _BLOCK_BYTES[fmt]:
        raise ValueError("canonical buffer has the wrong size")
    return b.reshape(N, nb, _BLOCK_BYTES[fmt])


def _scale(blocks: np.ndarray) -> np.ndarray:
    """The leading fp16 (little-endian) of each block, exactly, as fp64."""
    raw = blocks[:, :, 0].astype(np.uint16) | (blocks[:, :, 1].astype(np.uint16) << 8)
    return raw.view(np.float16).astype(np.float64)


def decode(fmt: int, canon, N: int, K: int):
    """Return (scale [N, K/32] fp64, q [N, K] int64) of a canonical matrix."""
    blk = _blocks(fmt, canon, N, K)
    s = _scale(blk)
    body = blk[:, :, 2:]
    if fmt == Q4_0:
        lo = (body & 0x0F).astype(np.int64)          # elements 0..15
        hi = (body >> 4).astype(np.int64)            # elements 16..31
        q = np.concatenate([lo, hi], axis=2)
    elif fmt == Q8_0:
        q = body.view(np.int8).astype(np.int64)
    else:
        raise ValueError(fmt)
    return s, q.reshape(N, K)


def dequant(fmt: int, canon, N: int, K: int) -> np.ndarray:
    """W [N, K] fp64: s*(q-8) for Q4_0, s*q for Q8_0 (exact in fp64); for
    FP16 the little-endian fp16 values themselves."""
    if fmt == FP16:
        if K % QK:
            raise ValueError("K must be a multiple of 32")
        b = np.frombuffer(np.ascontiguousarray(canon, dtype=np.uint8).tobytes(), dtype=np.uint8)
        if b.size != N * K * 2:
            raise ValueError("canonical buffer has the wrong size")
        raw = b[0::2].astype(np.uint16) | (b[1::2].astype(np.uint16) << 8)
        return raw.view(np.float16).astype(np.float64).reshape(N, K)
    s, q = decode(fmt, canon, N, K)
    off = 8 if fmt == Q4_0 else 0
    return (np.repeat(s, QK, axis=1) * (q - off)).astype(np.float64)


# ----------------------------------------------------------------------------
# Dense products
# ----------------------------------------------------------------------------
def qgemv(fmt: int, canon, N: int, K: int, x: np.ndarray):
    """y[m, n] = sum_k W[n, k] x[m, k] and its bound sum_k |W[n, k] x[m, k]|.

    x is [M, K] float64 (the exact stored activation values).
    """
    W = dequant(fmt, canon, N, K)
    x = np.asarray(x, dtype=np.float64)
    return x @ W.T, np.abs(x) @ np.abs(W).T


def qgemm(fmt: int, canon, N: int, K: int, X: np.ndarray):
    """Y = X W^T (same definition as the GEMV, any M)."""
    return qgemv(fmt, canon, N, K, X)


def qgemm_rows(fmt: int, canon, N: int, K: int, X: np.ndarray, rows, cols):
    """Y[rows[i], cols[i]] and bounds for sampled output elements only."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    ucols = np.unique(cols)
    pos = {int(c): i for i, c in enumerate(ucols)}
    if fmt == FP16:
        nbytes = K * 2
        c = np.ascontiguousarray(canon, dtype=np.uint8).reshape(N, nbytes)[ucols]
        W = dequant(FP16, c.reshape(-1), len(ucols), K)
    else:
        s, q = decode_rows(fmt, canon, N, K, ucols)
        off = 8 if fmt == Q4_0 else 0
        W = np.repeat(s, QK, axis=1) * (q - off)
    Xr = np.asarray(X, dtype=np.float64)
    y = np.empty(rows.size)
    b = np.empty(rows.size)
    for i, (r, c) in enumerate(zip(rows, cols)):
        w = W[pos[int(c)]]
        y[i] = float(np.dot(Xr[r], w))
        b[i] = float(np.dot(np.abs(Xr[r]), np.abs(w)))
    return y, b


def decode_rows(fmt: int, canon, N: int, K: int, rows):
    """decode() restricted to the given output rows (for large matrices)."""
    nbytes = (K // QK) * _BLOCK_BYTES[fmt]
    c = np.ascontiguousarray(canon, dtype=np.uint8).reshape(N, nbytes)
    sub = c[np.asarray(rows)]
    return decode(fmt, sub.reshape(-1), len(rows), K)


# ----------------------------------------------------------------------------
# Mixture of experts
# ----------------------------------------------------------------------------
def silu(z):
    """z * sigmoid(z), written so that large |z| does not overflow."""
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(-np.abs(z))
    sig = np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return z * sig


def silu_prime(z):
    z = np.asarray(z, dtype=np.float64)
    e = np.exp(-np.abs(z))
    sig = np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))
    return sig * (1.0 + z * (1.0 - sig))


def moe_route(logits: np.ndarray, topk: int):
    """ids [T, k] int32 and gates [T, k] fp64 from fp32 logits [T, E].

    Order: descending logit, ties to the lower expert id.  The comparison is
    on the fp32 values themselves (exact in fp64).  Gates are the softmax over
    the k selected logits, taken relative to the largest one.

    A NaN logit ranks as -inf (reading for degenerate router rows: the pages
    define no routing; a NaN expert is then chosen only after every finite
    one, among the -inf entries by expert id, and its gate is 0).  A row whose
    selected logits are all -inf has no softmax; its gates come out NaN.
    """
    lg = np.asarray(logits, dtype=np.float32).astype(np.float64)
    lg = np.where(np.isnan(lg), -np.inf, lg)
    T, E = lg.shape
    if not (1 <= topk <= E):
        raise ValueError("topk out of range")
    order = np.argsort(-lg, axis=1, kind="stable")[:, :topk]
    sel = np.take_along_axis(lg, order, axis=1)
    ex = np.exp(sel - sel[:, :1])
    gates = ex / ex.sum(axis=1, keepdims=True)
    return order.astype(np.int32), gates


def moe_sort(ids: np.ndarray, E: int):
    """counts [E], offsets [E+1] (exclusive scan) and the stable pair order."""
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    sorted_pairs = np.argsort(flat, kind="stable").astype(np.int32)
    return counts, offsets, sorted_pairs


def moe_ffn(fmt: int, wg, wu, wd, x: np.ndarray, ids: np.ndarray, gates: np.ndarray,
            sorted_pairs: np.ndarray, H: int, F: int, h_override=None):
    """Expert SwiGLU over every (token, slot) pair and the weighted combine.

    wg, wu: per-expert canonical [F, H]; wd: per-expert canonical [H, F].
    x: [T, H] fp64.  Returns a dict with, in sorted-pair order,
      zg, zu, bg, bu : gate/up pre-activations and their |w*x| bounds  [P, F]
      h              : silu(zg) * zu                                    [P, F]
    and per token
      out            : sum_j g[t,j] * (W_down[e] h)                     [T, H]
      bout           : sum_j g[t,j] * sum_f |W_down[e][n,f] h[f]|        [T, H]
      y, by          : per-pair down outputs and bounds (sorted order)  [P, H]
    If h_override [P, F] is given, it replaces h as the input of the down
    projection (used to check the down stage on its own).
    """
    T, k = ids.shape
    P = T * k
    x = np.asarray(x, dtype=np.float64)
    flat = np.asarray(ids).reshape(-1)
    zg = np.zeros((P, F))
    zu = np.zeros((P, F))
    bg = np.zeros((P, F))
    bu = np.zeros((P, F))
    y = np.zeros((P, H))
    by = np.zeros((P, H))
    dense_cache = {}

    def W(which, e):
        key = (which, e)
        if key not in dense_cache:
            src = {"g": wg, "u": wu, "d": wd}[which][e]
            n, kk = (F, H) if which in "gu" else (H, F)
            dense_cache[key] = dequant(fmt, src, n, kk)
        return dense_cache[key]

    sp = np.asarray(sorted_pairs)
    experts = flat[sp]
    for e in np.unique(experts):
        rows = np.nonzero(experts == e)[0]          # positions in sorted order
        toks = sp[rows] // k
        xe = x[toks]
        Wg, Wu = W("g", e), W("u", e)
        zg[rows] = xe @ Wg.T
        zu[rows] = xe @ Wu.T
        bg[rows] = np.abs(xe) @ np.abs(Wg).T
        bu[rows] = np.abs(xe) @ np.abs(Wu).T
    h = silu(zg) * zu
    hin = h if h_override is None else np.asarray(h_override, dtype=np.float64)
    for e in np.unique(experts):
        rows = np.nonzero(experts == e)[0]
        Wd = W("d", e)
        y[rows] = hin[rows] @ Wd.T
        by[rows] = np.abs(hin[rows]) @ np.abs(Wd).T
    out = np.zeros((T, H))
    bout = np.zeros((T, H))
    g = np.asarray(gates, dtype=np.float64).reshape(-1)
    inv = np.empty(P, dtype=np.int64)
    inv[sp] = np.arange(P)
    for p in range(P):
        t = p // k
        r = inv[p]
        out[t] += g[p] * y[r]
        bout[t] += g[p] * by[r]
    return dict(zg=zg, zu=zu, bg=bg, bu=bu, h=h, y=y, by=by, out=out, bout=bout)


def ffn(fmt: int, wg, wu, wd, x: np.ndarray, H: int, F: int, h_override=None):
    """Dense SwiGLU FFN of a decode step (the fused gate/up GEMV, then down).

    wg, wu: canonical [F, H]; wd: canonical [H, F]; x: [M, H] fp64.
    Returns zg, zu, bg, bu, h = silu(zg) * zu  [M, F]; y = h W_down^T and its
    bound by = |h| |W_down|^T  [M, H] (omitted when wd is None: the gate/up
    stage alone).  h_override replaces h as the input of the down projection
    (to check that stage on its own).
    """
    x = np.asarray(x, dtype=np.float64)
    Wg, Wu = dequant(fmt, wg, F, H), dequant(fmt, wu, F, H)
    zg, zu = x @ Wg.T, x @ Wu.T
    h = silu(zg) * zu
    r = dict(zg=zg, zu=zu, bg=np.abs(x) @ np.abs(Wg).T, bu=np.abs(x) @ np.abs(Wu).T, h=h)
    if wd is not None:
        Wd = dequant(fmt, wd, H, F)
        hin = h if h_override is None else np.asarray(h_override, dtype=np.float64)
        r.update(y=hin @ Wd.T, by=np.abs(hin) @ np.abs(Wd).T)
    return r


def ffn_out_bound(fmt: int, wd, r: dict, hb: np.ndarray, H: int, F: int, rel: float = 2e-3,
                  abs_tol: float = 1e-5) -> np.ndarray:
    """First-order bound on |y_gpu - y| of the FFN: the down dot products'
    own tolerance plus the input error hb carried through |W_down|."""
    Wd = dequant(fmt, wd, H, F)
    return rel * r["by"] + hb @ np.abs(Wd).T + abs_tol


def moe(fmt: int, wg, wu, wd, x, logits, topk: int, H: int, F: int):
    """The whole MoE layer: route, sort, experts, combine."""
    E = len(wg)
    ids, gates = moe_route(logits, topk)
    counts, offsets, sp = moe_sort(ids, E)
    r = moe_ffn(fmt, wg, wu, wd, x, ids, gates, sp, H, F)
    r.update(ids=ids, gates=gates, counts=counts, offsets=offsets, sorted_pairs=sp)
    return r


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool = True, scale=None, rows=None):
    """Prefill attention: per query head h and query i,
        s_j = scale * q_i . k_j   over keys j (j <= i when causal),
        p   = softmax(s),  o_i = sum_j p_j v_j,
    with GQA: query head h reads key/value head h // (Hq / Hkv).

    q [B, S, Hq, D], k and v [B, S, Hkv, D] (fp64 values).  Returns o and the
    bound sum_j p_j |v_j| (both [B, S, Hq, D]; with rows given, only those
    query positions, [B, len(rows), Hq, D]).  scale defaults to 1/sqrt(D).
    The technical summary ("Methodologie", prefill optimisation) names tiled
    attention with an online softmax; this is the quantity it computes.
    """
    q, k, v = (np.asarray(a, dtype=np.float64) for a in (q, k, v))
    B, S, Hq, D = q.shape
    Hkv = k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    group = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    rows = np.arange(S) if rows is None else np.asarray(rows)
    o = np.zeros((B, len(rows), Hq, D))
    bound = np.zeros_like(o)
    for b in range(B):
        for h in range(Hq):
            kk, vv = k[b, :, h // group], v[b, :, h // group]
            s = scale * (q[b, rows, h] @ kk.T)                  # [len(rows), S]
            if causal:
                s = np.where(np.arange(S)[None, :] <= rows[:, None], s, -np.inf)
            s = s - s.max(axis=1, keepdims=True)
            e = np.exp(s)
            p = e / e.sum(axis=1, keepdims=True)
            o[b, :, h] = p @ vv
            bound[b, :, h] = p @ np.abs(vv)
    return o, bound


def h_bound(r: dict, rel: float = 2e-3, storage_rel: float = 2.0 ** -8, abs_tol: float = 1e-5):
    """First-order bound on |h_gpu - h| from the per-dot-product tolerance.

    Each of the two projections may be off by rel*B + abs_tol; the stored h may
    additionally carry its own rounding (storage_rel relative, e.g. bf16).
    """
    ez_g = rel * r["bg"] + abs_tol
    ez_u = rel * r["bu"] + abs_tol
    sg = silu(r["zg"])
    return (np.abs(silu_prime(r["zg"])) * np.abs(r["zu"]) * ez_g + np.abs(sg) * ez_u
            + storage_rel * np.abs(r["h"]) + abs_tol)


def moe_out_bound(fmt: int, wd, r: dict, ids: np.ndarray, gates: np.ndarray,
                  sorted_pairs: np.ndarray, H: int, F: int, hb: np.ndarray,
                  rel: float = 2e-3, abs_tol: float = 1e-5) -> np.ndarray:
    """First-order bound on |out_gpu - out| through the whole expert chain.

    Each gate may be off by rel*g + abs_tol, each down-projection dot product
    by rel*B + abs_tol on top of what its input h carries (hb, from h_bound):
      sum_j [ g_j (rel*by + |W_down| hb + abs_tol) + (rel*g_j + abs_tol) |y| ]
    """
    T, k = ids.shape
    P = T * k
    flat = np.asarray(ids).reshape(-1)
    sp = np.asarray(sorted_pairs)
    experts = flat[sp]
    prop = np.zeros((P, H))
    for e in np.unique(experts):
        rows = np.nonzero(experts == e)[0]
        Wd = dequant(fmt, wd[e], H, F)
        prop[rows] = hb[rows] @ np.abs(Wd).T
    inv = np.empty(P, dtype=np.int64)
    inv[sp] = np.arange(P)
    g = np.asarray(gates, dtype=np.float64).reshape(-1)
    bound = np.full((T, H), abs_tol)
    for p in range(P):
        t = p // k
        i = inv[p]
        bound[t] += g[p] * (rel * r["by"][i] + prop[i] + abs_tol) + (rel * g[p] + abs_tol) * np.abs(r["y"][i])
    return bound
