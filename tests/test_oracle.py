"""Pins for the CPU oracle: each check is independent of the oracle's own code.

The pages print no worked example for any format or kernel, so the oracle is
pinned by hand-built blocks (tests/golden), exact rational brute force, closed
forms, textbook special cases and invariants.  A plausible slip anywhere in the
oracle (nibble order, offset, sign, transposed operand, softmax over the wrong
set, unstable sort, gate applied to the wrong pair) fails at least one test.
"""
import math
import os
from collections import Counter
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    bytes_, values = None, []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            if line.startswith("bytes"):
                bytes_ = bytes.fromhex("".join(line.split()[1:]))
            elif line.startswith("values"):
                values.append([float(v) for v in line.split()[1:]])
    return np.frombuffer(bytes_, dtype=np.uint8), np.concatenate(values)


def _f16(v):
    return float(np.float16(v))


def _f16_bytes(v):
    return list(np.array([v], dtype=np.float16).view(np.uint8))


# ----------------------------------------------------------------------------
# Block decoding
# ----------------------------------------------------------------------------
def test_golden_q4_0():
    raw, want = _read_golden("q4_0_blocks.txt")
    got = oracle.dequant(oracle.Q4_0, raw, 1, 64)
    assert got.shape == (1, 64)
    assert np.array_equal(got[0], want)


def test_golden_q8_0():
    raw, want = _read_golden("q8_0_blocks.txt")
    got = oracle.dequant(oracle.Q8_0, raw, 1, 32)
    assert np.array_equal(got[0], want)


@pytest.mark.parametrize("scale", [1.0, 2.0 ** -7, 0.002, 0.02, -0.5])
def test_dequant_every_q4_code(scale):
    """Every code 0..15 in every position: w == s*(q-8) exactly."""
    s = _f16(scale)
    rows = []
    expect = []
    for shift in range(16):
        q = [(i + shift) % 16 for i in range(32)]
        body = [q[i] | (q[i + 16] << 4) for i in range(16)]
        rows.append(_f16_bytes(s) + body)
        expect.append([s * (c - 8) for c in q])
    raw = np.array(rows, dtype=np.uint8).reshape(-1)
    got = oracle.dequant(oracle.Q4_0, raw, 16, 32)
    assert np.array_equal(got, np.array(expect))


@pytest.mark.parametrize("scale", [1.0, 2.0 ** -7, 0.0002, 0.002])
def test_dequant_every_q8_code(scale):
    """Every int8 code -128..127: w == s*q exactly."""
    s = _f16(scale)
    codes = np.arange(-128, 128, dtype=np.int64).reshape(8, 32)
    rows = [_f16_bytes(s) + [int(c) & 0xFF for c in row] for row in codes]
    raw = np.array(rows, dtype=np.uint8).reshape(-1)
    got = oracle.dequant(oracle.Q8_0, raw, 8, 32)
    assert np.array_equal(got, s * codes.astype(np.float64))


@pytest.mark.parametrize("fmt", [synth.Q4_0, synth.Q8_0])
def test_decode_returns_the_drawn_codes(fmt):
    w = synth.q_weight(synth.rng_for(7, fmt), fmt, 5, 96)
    s, q = oracle.decode(fmt, w.canon, 5, 96)
    assert np.array_equal(s, w.scales.astype(np.float64))
    assert np.array_equal(q, w.codes.astype(np.int64))


def test_decode_rejects_bad_sizes():
    with pytest.raises(ValueError):
        oracle.decode(oracle.Q4_0, np.zeros(18, np.uint8), 1, 48)
    with pytest.raises(ValueError):
        oracle.decode(oracle.Q4_0, np.zeros(17, np.uint8), 1, 32)


# ----------------------------------------------------------------------------
# Products: exact rational brute force and closed forms
# ----------------------------------------------------------------------------
def _exact_gemv(fmt, w, x_values):
    """Exact y and |w*x| bound from the logical draw, in Fractions."""
    N, K = w.codes.shape
    M = x_values.shape[0]
    off = 8 if fmt == synth.Q4_0 else 0
    y = [[Fraction(0)] * N for _ in range(M)]
    b = [[Fraction(0)] * N for _ in range(M)]
    for n in range(N):
        for kk in range(K):
            wv = Fraction(float(w.scales[n, kk // 32])) * (int(w.codes[n, kk]) - off)
            for m in range(M):
                t = wv * Fraction(float(x_values[m, kk]))
                y[m][n] += t
                b[m][n] += abs(t)
    return y, b


@pytest.mark.parametrize("fmt,xdt", [(synth.Q4_0, synth.F16), (synth.Q8_0, synth.BF16),
                                     (synth.Q4_0, synth.BF16), (synth.Q8_0, synth.F16)])
@pytest.mark.parametrize("K", [32, 64, 96])
def test_gemv_matches_exact_rationals(fmt, xdt, K):
    N, M = 4, 3
    w = synth.q_weight(synth.rng_for(11, K + fmt), fmt, N, K)
    x = synth.activation(synth.rng_for(12, K + xdt), (M, K), xdt)
    y, b = oracle.qgemv(fmt, w.canon, N, K, x.values)
    ye, be = _exact_gemv(fmt, w, x.values)
    for m in range(M):
        for n in range(N):
            bound = float(be[m][n])
            assert abs(y[m, n] - float(ye[m][n])) <= 1e-15 * bound + 1e-300
            assert abs(b[m, n] - bound) <= 1e-15 * bound


def test_gemv_one_hot_picks_a_column():
    w = synth.q_weight(synth.rng_for(3, 0), synth.Q4_0, 8, 128)
    W = w.scales.astype(np.float64).repeat(32, axis=1) * (w.codes.astype(np.float64) - 8)
    for k in [0, 5, 31, 32, 127]:
        x = np.zeros((1, 128))
        x[0, k] = 1.0
        y, _ = oracle.qgemv(synth.Q4_0, w.canon, 8, 128, x)
        assert np.array_equal(y[0], W[:, k])


def test_gemv_all_ones_closed_form():
    """x = 1: y[n] = sum_b s[n,b] * (sum_i q[n,b,i] - 256) for Q4_0."""
    w = synth.q_weight(synth.rng_for(4, 0), synth.Q4_0, 6, 256)
    y, _ = oracle.qgemv(synth.Q4_0, w.canon, 6, 256, np.ones((1, 256)))
    q = w.codes.astype(np.int64).reshape(6, 8, 32).sum(axis=2) - 256
    want = (w.scales.astype(np.float64) * q).sum(axis=1)
    assert np.allclose(y[0], want, rtol=1e-14, atol=0)
    w8 = synth.q_weight(synth.rng_for(4, 1), synth.Q8_0, 6, 256)
    y8, _ = oracle.qgemv(synth.Q8_0, w8.canon, 6, 256, np.ones((1, 256)))
    q8 = w8.codes.astype(np.int64).reshape(6, 8, 32).sum(axis=2)
    assert np.allclose(y8[0], (w8.scales.astype(np.float64) * q8).sum(axis=1), rtol=1e-14, atol=0)


def test_gemv_zero_codes_give_zero():
    scales = np.full((3, 4), np.float16(0.01))
    codes = np.full((3, 128), 8, dtype=np.uint8)
    raw = synth.pack_blocks(synth.Q4_0, scales, codes)
    x = synth.activation(synth.rng_for(5, 0), (2, 128), synth.F16).values
    y, b = oracle.qgemv(synth.Q4_0, raw, 3, 128, x)
    assert np.all(y == 0) and np.all(b == 0)
    raw8 = synth.pack_blocks(synth.Q8_0, scales, np.zeros((3, 128), np.int8))
    y8, _ = oracle.qgemv(synth.Q8_0, raw8, 3, 128, x)
    assert np.all(y8 == 0)


def test_gemv_doubling_scales_doubles_y():
    w = synth.q_weight(synth.rng_for(6, 0), synth.Q4_0, 5, 160)
    x = synth.activation(synth.rng_for(6, 1), (2, 160), synth.F16).values
    y1, _ = oracle.qgemv(synth.Q4_0, w.canon, 5, 160, x)
    raw2 = synth.pack_blocks(synth.Q4_0, (w.scales.astype(np.float32) * 2).astype(np.float16), w.codes)
    y2, _ = oracle.qgemv(synth.Q4_0, raw2, 5, 160, x)
    assert np.array_equal(y2, 2 * y1)


def test_gemv_linear_in_x():
    w = synth.q_weight(synth.rng_for(8, 0), synth.Q8_0, 7, 96)
    a = synth.activation(synth.rng_for(8, 1), (1, 96), synth.BF16).values
    c = synth.activation(synth.rng_for(8, 2), (1, 96), synth.BF16).values
    ya, ba = oracle.qgemv(synth.Q8_0, w.canon, 7, 96, a)
    yc, bc = oracle.qgemv(synth.Q8_0, w.canon, 7, 96, c)
    ys, _ = oracle.qgemv(synth.Q8_0, w.canon, 7, 96, 3 * a - c)
    assert np.allclose(ys, 3 * ya - yc, rtol=0, atol=1e-13 * (3 * ba + bc).max())


@pytest.mark.parametrize("fmt", [synth.Q4_0, synth.FP16])
def test_gemm_rows_agree_with_full_product(fmt):
    w = synth.weight(synth.rng_for(9, 0), fmt, 40, 128)
    X = synth.activation(synth.rng_for(9, 1), (17, 128), synth.BF16).values
    Y, B = oracle.qgemm(fmt, w.canon, 40, 128, X)
    rows = [0, 3, 16, 16, 9]
    cols = [39, 0, 7, 8, 20]
    y, b = oracle.qgemm_rows(fmt, w.canon, 40, 128, X, rows, cols)
    assert np.allclose(y, Y[rows, cols], rtol=1e-14, atol=1e-14)
    assert np.allclose(b, B[rows, cols], rtol=1e-14)
    if fmt == synth.FP16:
        # brute force from the generator's fp16 matrix (not the byte decode)
        for i, (r, c) in enumerate(zip(rows, cols)):
            exact = sum(float(w.codes[c, k]) * float(X[r, k]) for k in range(128))
            assert abs(y[i] - exact) <= 1e-12 * b[i]


# ----------------------------------------------------------------------------
# Routing and sorting
# ----------------------------------------------------------------------------
def _brute_route(lg, k):
    ids, gates = [], []
    for row in lg:
        order = sorted(range(len(row)), key=lambda e: (-float(row[e]), e))[:k]
        sel = [float(row[e]) for e in order]
        m = max(sel)
        ex = [math.exp(v - m) for v in sel]
        s = math.fsum(ex)
        ids.append(order)
        gates.append([v / s for v in ex])
    return np.array(ids), np.array(gates)


def test_route_matches_brute_force_with_ties():
    rng = synth.rng_for(21, 0)
    lg = synth.router_logits(rng, 40, 16)
    lg[0, :] = 0.5                       # all tied: ids 0..k-1
    lg[1, [3, 9, 12]] = 4.0              # three-way tie at the top
    lg[2, [15, 0]] = 3.0                 # tie across the ends
    lg[3, :] = -1.0
    lg[3, 5] = np.float32(1.0) + np.float32(2.0 ** -23)
    lg[3, 4] = 1.0                       # one ulp apart: 5 before 4
    ids, gates = oracle.moe_route(lg, 4)
    bi, bg = _brute_route(lg, 4)
    assert np.array_equal(ids, bi)
    assert np.allclose(gates, bg, rtol=1e-15, atol=0)
    assert list(ids[0]) == [0, 1, 2, 3]
    assert list(ids[1][:3]) == [3, 9, 12]
    assert list(ids[2][:2]) == [0, 15]
    assert list(ids[3][:2]) == [5, 4]


def test_route_nan_ranks_as_minus_infinity():
    """Reading for degenerate router rows: a NaN logit ranks as -inf (after
    every finite logit, among the -inf entries by expert id) and gets gate 0."""
    lg = np.array([[1.0, np.nan, 0.5, -np.inf, -np.inf],
                   [np.nan, 0.0, 0.5, np.nan, 2.0],
                   [-np.inf, np.nan, 3.0, -np.inf, 3.0]], dtype=np.float32)
    ids, g = oracle.moe_route(lg, 4)
    assert ids.tolist() == [[0, 2, 1, 3], [4, 2, 1, 0], [2, 4, 0, 1]]
    e = math.exp(-0.5)
    assert np.allclose(g[0], [1 / (1 + e), e / (1 + e), 0.0, 0.0], rtol=1e-15, atol=0)
    assert np.all(np.isfinite(g)) and np.allclose(g.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert g[2].tolist() == [0.5, 0.5, 0.0, 0.0]
    # Brute force on random rows mixing NaN, -inf and exact ties: sort key
    # (class, -value, id) with class 0 for numbers above -inf, 1 for -inf and NaN.
    rng = synth.rng_for(24, 0)
    lg = rng.integers(-2, 3, size=(300, 9)).astype(np.float32)
    lg[rng.random(lg.shape) < 0.2] = np.nan
    lg[rng.random(lg.shape) < 0.2] = -np.inf
    lg[:, 0] = np.where(np.all(~np.isfinite(lg), axis=1), 1.0, lg[:, 0])   # keep one finite logit
    for k in (1, 4, 9):
        ids, g = oracle.moe_route(lg, k)
        for t, row in enumerate(lg):
            key = lambda i: (1, 0.0, i) if (np.isnan(row[i]) or row[i] == -np.inf) else (0, -float(row[i]), i)
            want = sorted(range(9), key=key)[:k]
            assert ids[t].tolist() == want
            fin = [float(row[i]) for i in want if np.isfinite(row[i])]
            m = max(fin)
            ex = [math.exp(float(row[i]) - m) if np.isfinite(row[i]) else 0.0 for i in want]
            assert np.allclose(g[t], np.array(ex) / math.fsum(ex), rtol=1e-15, atol=0)


def test_route_gates_are_a_softmax():
    lg = synth.router_logits(synth.rng_for(22, 0), 64, 128)
    ids, g = oracle.moe_route(lg, 8)
    assert np.allclose(g.sum(axis=1), 1.0, rtol=0, atol=1e-15)
    assert np.all(np.diff(g, axis=1) <= 0)
    sel = np.take_along_axis(lg.astype(np.float64), ids.astype(np.int64), axis=1)
    assert np.allclose(g, scipy.special.softmax(sel, axis=1), rtol=1e-14, atol=0)
    # k = E: the gates are the softmax over all experts, in sorted order.
    idsE, gE = oracle.moe_route(lg, 128)
    full = scipy.special.softmax(lg.astype(np.float64), axis=1)
    assert np.allclose(gE, np.take_along_axis(full, idsE.astype(np.int64), axis=1), rtol=1e-13, atol=0)
    # k = 1: the arg-max with gate 1.
    id1, g1 = oracle.moe_route(lg, 1)
    assert np.array_equal(id1[:, 0], np.argmax(lg, axis=1))
    assert np.all(g1 == 1.0)


def test_route_rejects_bad_topk():
    with pytest.raises(ValueError):
        oracle.moe_route(np.zeros((2, 4), np.float32), 5)


def test_sort_matches_brute_force():
    rng = synth.rng_for(23, 0)
    E, T, k = 16, 50, 4
    ids, _ = oracle.moe_route(synth.router_logits(rng, T, E), k)
    counts, offsets, sp = oracle.moe_sort(ids, E)
    pairs = sorted((int(ids.reshape(-1)[p]), p) for p in range(T * k))
    assert list(sp) == [p for _, p in pairs]
    c = Counter(ids.reshape(-1).tolist())
    assert list(counts) == [c.get(e, 0) for e in range(E)]
    assert offsets[0] == 0 and offsets[-1] == T * k
    assert np.all(np.diff(offsets) == counts)
    assert sorted(sp.tolist()) == list(range(T * k))
    e_sorted = ids.reshape(-1)[sp]
    assert np.all(np.diff(e_sorted) >= 0)
    for e in range(E):
        seg = sp[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)          # stable: ascending pair id


def test_sort_with_empty_experts():
    ids = np.array([[3, 1], [3, 1], [1, 3]], dtype=np.int32)
    counts, offsets, sp = oracle.moe_sort(ids, 6)
    assert list(counts) == [0, 3, 0, 3, 0, 0]
    assert list(offsets) == [0, 0, 3, 3, 6, 6, 6]
    assert list(sp) == [1, 3, 4, 0, 2, 5]


# ----------------------------------------------------------------------------
# Expert SwiGLU and combine
# ----------------------------------------------------------------------------
def test_silu_textbook_values():
    for z in [-40.0, -3.0, -1.0, 0.0, 0.5, 1.0, 3.0, 40.0, 800.0, -800.0]:
        want = z / (1.0 + math.exp(-z)) if z > -700 else 0.0
        assert abs(float(oracle.silu(z)) - want) <= 1e-15 * max(1.0, abs(z))
    zs = np.linspace(-6, 6, 25)
    h = 1e-6
    fd = (oracle.silu(zs + h) - oracle.silu(zs - h)) / (2 * h)
    assert np.allclose(oracle.silu_prime(zs), fd, rtol=0, atol=1e-8)


def _small_moe(E=6, T=9, H=64, F=32, k=3, seed=31, same=False):
    logits, x, wg, wu, wd = synth.moe(seed=seed, T=T, E=E, H=H, F=F)
    if same:
        wg = [wg[0]] * E
        wu = [wu[0]] * E
        wd = [wd[0]] * E
    return logits, x, wg, wu, wd


def _dense_ffn(w_g, w_u, w_d, xv):
    """Dense SwiGLU from the logical draw (independent of the oracle decoder)."""
    def deq(w):
        return w.scales.astype(np.float64).repeat(32, axis=1) * (w.codes.astype(np.float64) - 8)
    zg = xv @ deq(w_g).T
    zu = xv @ deq(w_u).T
    h = zg / (1.0 + np.exp(-zg)) * zu
    return h @ deq(w_d).T


def test_identical_experts_equal_a_dense_ffn():
    E, T, H, F, k = 6, 9, 64, 32, 3
    logits, x, wg, wu, wd = _small_moe(E, T, H, F, k, same=True)
    r = oracle.moe(synth.Q4_0, [w.canon for w in wg], [w.canon for w in wu],
                   [w.canon for w in wd], x.values, logits, k, H, F)
    dense = _dense_ffn(wg[0], wu[0], wd[0], x.values)
    assert np.allclose(r["out"], dense, rtol=1e-12, atol=1e-12)


def test_top1_picks_the_argmax_expert():
    E, T, H, F = 5, 7, 64, 32
    logits, x, wg, wu, wd = _small_moe(E, T, H, F, seed=32)
    r = oracle.moe(synth.Q4_0, [w.canon for w in wg], [w.canon for w in wu],
                   [w.canon for w in wd], x.values, logits, 1, H, F)
    for t in range(T):
        e = int(np.argmax(logits[t]))
        want = _dense_ffn(wg[e], wu[e], wd[e], x.values[t:t + 1])[0]
        assert np.allclose(r["out"][t], want, rtol=1e-12, atol=1e-12)


def test_one_hot_token_closed_form():
    """x_t = e_c: z_g[f] = W_g[f, c] and z_u[f] = W_u[f, c] exactly."""
    E, T, H, F, k = 4, 4, 64, 32, 2
    logits, x, wg, wu, wd = _small_moe(E, T, H, F, k, seed=33)
    xv = np.zeros((T, H))
    cols = [0, 17, 33, 63]
    for t, c in enumerate(cols):
        xv[t, c] = 1.0
    r = oracle.moe(synth.Q4_0, [w.canon for w in wg], [w.canon for w in wu],
                   [w.canon for w in wd], xv, logits, k, H, F)
    ids, gates = r["ids"], r["gates"]
    for t, c in enumerate(cols):
        acc = np.zeros(H)
        for j in range(k):
            e = int(ids[t, j])
            g_col = wg[e].scales[:, c // 32].astype(np.float64) * (wg[e].codes[:, c].astype(np.float64) - 8)
            u_col = wu[e].scales[:, c // 32].astype(np.float64) * (wu[e].codes[:, c].astype(np.float64) - 8)
            h = [gv / (1.0 + math.exp(-gv)) * uv for gv, uv in zip(g_col, u_col)]
            Wd = wd[e].scales.astype(np.float64).repeat(32, axis=1) * (wd[e].codes.astype(np.float64) - 8)
            acc += gates[t, j] * (Wd @ np.array(h))
        assert np.allclose(r["out"][t], acc, rtol=1e-12, atol=1e-13)


def test_relabelling_experts_changes_nothing():
    E, T, H, F, k = 6, 8, 64, 32, 3
    logits, x, wg, wu, wd = _small_moe(E, T, H, F, k, seed=34)
    perm = np.array([4, 2, 5, 0, 1, 3])          # new label i is old expert perm[i]
    cg = [w.canon for w in wg]
    cu = [w.canon for w in wu]
    cd = [w.canon for w in wd]
    r1 = oracle.moe(synth.Q4_0, cg, cu, cd, x.values, logits, k, H, F)
    r2 = oracle.moe(synth.Q4_0, [cg[i] for i in perm], [cu[i] for i in perm], [cd[i] for i in perm],
                    x.values, logits[:, perm], k, H, F)
    assert np.allclose(r1["out"], r2["out"], rtol=1e-12, atol=1e-13)


def test_moe_bounds_catch_a_planted_error():
    """The propagated bound accepts the oracle and rejects plausible slips.

    The acceptance rule scales sum|w*x|, which exceeds |y| by about sqrt(K) on
    random data, so the slips planted here are the structural ones: silu on
    the up projection instead of the gate, and gates applied to the wrong slot.
    """
    E, T, H, F, k = 6, 9, 64, 32, 3
    logits, x, wg, wu, wd = _small_moe(E, T, H, F, k, seed=35)
    cg, cu, cd = [w.canon for w in wg], [w.canon for w in wu], [w.canon for w in wd]
    r = oracle.moe(synth.Q4_0, cg, cu, cd, x.values, logits, k, H, F)
    hb = oracle.h_bound(r)
    ob = oracle.moe_out_bound(synth.Q4_0, cd, r, r["ids"], r["gates"], r["sorted_pairs"], H, F, hb)
    assert np.all(ob > 0)
    assert np.all(np.abs(r["h"] - r["h"]) <= hb)
    swapped = oracle.silu(r["zu"]) * r["zg"]
    assert np.any(np.abs(swapped - r["h"]) > hb)
    bad = oracle.moe_ffn(synth.Q4_0, cg, cu, cd, x.values, r["ids"], r["gates"], r["sorted_pairs"],
                         H, F, h_override=swapped)
    assert np.any(np.abs(bad["out"] - r["out"]) > ob)
    g_bad = r["gates"][:, ::-1].copy()
    bad2 = oracle.moe_ffn(synth.Q4_0, cg, cu, cd, x.values, r["ids"], g_bad, r["sorted_pairs"], H, F)
    assert np.any(np.abs(bad2["out"] - r["out"]) > ob)


# ----------------------------------------------------------------------------
# Dense decode FFN (fused gate/up SwiGLU, then down)
# ----------------------------------------------------------------------------
def _logical(w, fmt):
    """Dense weights from the logical draw (scales and codes, not the bytes)."""
    off = 8 if fmt == synth.Q4_0 else 0
    return w.scales.astype(np.float64).repeat(32, axis=1) * (w.codes.astype(np.float64) - off)


def _ffn_weights(fmt, H, F, seed):
    rng = [synth.rng_for(seed, i) for i in range(3)]
    return (synth.q_weight(rng[0], fmt, F, H), synth.q_weight(rng[1], fmt, F, H),
            synth.q_weight(rng[2], fmt, H, F))


@pytest.mark.parametrize("fmt", [synth.Q4_0, synth.Q8_0])
def test_ffn_matches_the_logical_draw(fmt):
    H, F, M = 96, 64, 3
    wg, wu, wd = _ffn_weights(fmt, H, F, 36)
    x = synth.activation(synth.rng_for(36, 9), (M, H), synth.BF16).values
    r = oracle.ffn(fmt, wg.canon, wu.canon, wd.canon, x, H, F)
    zg, zu = x @ _logical(wg, fmt).T, x @ _logical(wu, fmt).T
    h = [[a / (1.0 + math.exp(-a)) * b for a, b in zip(ra, rb)] for ra, rb in zip(zg, zu)]
    assert np.allclose(r["h"], h, rtol=1e-12, atol=1e-13)
    assert np.allclose(r["y"], np.array(h) @ _logical(wd, fmt).T, rtol=1e-12, atol=1e-12)


def test_ffn_one_hot_closed_form():
    """x = e_c: h[f] = silu(Wg[f, c]) * Wu[f, c], y = Wd h, from one column of codes."""
    H, F = 64, 32
    wg, wu, wd = _ffn_weights(synth.Q4_0, H, F, 37)
    for c in (0, 31, 32, 63):
        x = np.zeros((1, H))
        x[0, c] = 1.0
        r = oracle.ffn(synth.Q4_0, wg.canon, wu.canon, wd.canon, x, H, F)
        g = [float(wg.scales[f, c // 32]) * (int(wg.codes[f, c]) - 8) for f in range(F)]
        u = [float(wu.scales[f, c // 32]) * (int(wu.codes[f, c]) - 8) for f in range(F)]
        h = np.array([a / (1.0 + math.exp(-a)) * b for a, b in zip(g, u)])
        assert np.allclose(r["h"][0], h, rtol=1e-13, atol=1e-15)
        y = [sum(float(wd.scales[n, f // 32]) * (int(wd.codes[n, f]) - 8) * h[f] for f in range(F))
             for n in range(H)]
        assert np.allclose(r["y"][0], y, rtol=1e-12, atol=1e-14)


def test_ffn_is_a_one_expert_moe():
    """With one expert and top-1 the gate is exactly 1 and the MoE layer is the FFN."""
    H, F, T = 64, 32, 5
    wg, wu, wd = _ffn_weights(synth.Q8_0, H, F, 38)
    x = synth.activation(synth.rng_for(38, 9), (T, H), synth.F16).values
    logits = synth.router_logits(synth.rng_for(38, 10), T, 1)
    m = oracle.moe(synth.Q8_0, [wg.canon], [wu.canon], [wd.canon], x, logits, 1, H, F)
    r = oracle.ffn(synth.Q8_0, wg.canon, wu.canon, wd.canon, x, H, F)
    assert np.all(m["gates"] == 1.0)
    assert np.array_equal(m["out"], r["y"])


def test_ffn_bounds_catch_a_planted_error():
    """h_bound / ffn_out_bound accept the oracle and reject silu on the wrong
    projection and a transposed down matrix."""
    H = F = 64
    wg, wu, wd = _ffn_weights(synth.Q4_0, H, F, 39)
    x = synth.activation(synth.rng_for(39, 9), (4, H), synth.BF16).values
    r = oracle.ffn(synth.Q4_0, wg.canon, wu.canon, wd.canon, x, H, F)
    hb = oracle.h_bound(r)
    ob = oracle.ffn_out_bound(synth.Q4_0, wd.canon, r, hb, H, F)
    assert np.all(ob > 0)
    swapped = oracle.silu(r["zu"]) * r["zg"]
    assert np.any(np.abs(swapped - r["h"]) > hb)
    bad = oracle.ffn(synth.Q4_0, wg.canon, wu.canon, wd.canon, x, H, F, h_override=swapped)
    assert np.any(np.abs(bad["y"] - r["y"]) > ob)
    yt = r["h"] @ _logical(wd, synth.Q4_0)
    assert np.any(np.abs(yt - r["y"]) > ob)


# ----------------------------------------------------------------------------
# Prefill attention
# ----------------------------------------------------------------------------
def _qkv(B, S, Hq, Hkv, D, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((B, S, Hq, D)), rng.standard_normal((B, S, Hkv, D)),
            rng.standard_normal((B, S, Hkv, D)))


def test_attention_zero_queries_give_prefix_means():
    """q = 0: every visible score is 0, so o_i is the mean of v_0..v_i
    (causal) or of all v (not causal)."""
    _, k, v = _qkv(2, 9, 4, 2, 8, 70)
    q = np.zeros((2, 9, 4, 8))
    o, _ = oracle.attention(q, k, v, causal=True)
    for h in range(4):
        want = np.cumsum(v[:, :, h // 2], axis=1) / np.arange(1, 10)[None, :, None]
        assert np.allclose(o[:, :, h], want, rtol=1e-13, atol=1e-14)
    o, _ = oracle.attention(q, k, v, causal=False)
    assert np.allclose(o[:, :, 3], v[:, :, 1].mean(axis=1, keepdims=True), rtol=1e-13, atol=1e-14)


def test_attention_two_keys_is_a_sigmoid_mix():
    q, k, v = _qkv(1, 2, 1, 1, 16, 71)
    o, _ = oracle.attention(q, k, v, causal=False, scale=0.3)
    for i in range(2):
        s0, s1 = 0.3 * q[0, i, 0] @ k[0, 0, 0], 0.3 * q[0, i, 0] @ k[0, 1, 0]
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        assert np.allclose(o[0, i, 0], w0 * v[0, 0, 0] + (1 - w0) * v[0, 1, 0], rtol=1e-13, atol=1e-14)


def test_attention_dominant_key_selects_its_value():
    """One key scores 200 above the rest: o equals its v to e^-200."""
    B, S, D = 1, 6, 4
    q = np.zeros((B, S, 1, D))
    k = np.zeros((B, S, 1, D))
    v = np.random.default_rng(72).standard_normal((B, S, 1, D))
    q[0, 5, 0, 0] = 400.0
    k[0, 3, 0, 0] = 1.0
    o, _ = oracle.attention(q, k, v, causal=True, scale=0.5)
    assert np.allclose(o[0, 5, 0], v[0, 3, 0], rtol=0, atol=1e-60)
    assert np.allclose(o[0, 0, 0], v[0, 0, 0], rtol=0, atol=0)      # causal: query 0 sees key 0 only


def test_attention_gqa_maps_contiguous_head_groups():
    """Query head h reads kv head h // (Hq/Hkv): each head equals a one-head
    call on its own kv head, and differs from the call on the other one."""
    q, k, v = _qkv(1, 7, 4, 2, 8, 73)
    o, _ = oracle.attention(q, k, v)
    for h in range(4):
        one, _ = oracle.attention(q[:, :, h:h + 1], k[:, :, h // 2:h // 2 + 1], v[:, :, h // 2:h // 2 + 1])
        other, _ = oracle.attention(q[:, :, h:h + 1], k[:, :, 1 - h // 2:2 - h // 2], v[:, :, 1 - h // 2:2 - h // 2])
        assert np.array_equal(o[:, :, h:h + 1], one)
        assert not np.allclose(o[:, 1:, h:h + 1], other[:, 1:])


def test_attention_key_permutation_invariance_without_mask():
    q, k, v = _qkv(1, 11, 2, 1, 8, 74)
    perm = np.random.default_rng(75).permutation(11)
    o1, b1 = oracle.attention(q, k, v, causal=False)
    o2, b2 = oracle.attention(q, k[:, perm], v[:, perm], causal=False)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-13) and np.allclose(b1, b2, rtol=1e-12, atol=1e-13)


def test_attention_rows_subset_and_bound():
    q, k, v = _qkv(2, 13, 2, 2, 8, 76)
    o, b = oracle.attention(q, k, v)
    rows = [0, 5, 12]
    o2, b2 = oracle.attention(q, k, v, rows=rows)
    assert np.array_equal(o[:, rows], o2) and np.array_equal(b[:, rows], b2)
    assert np.all(b >= np.abs(o) - 1e-12)
    # the acceptance bound rejects the plausible slips: no causal mask, scale missing
    tol = 2.0 ** -7 * b + 1e-5
    bad, _ = oracle.attention(q, k, v, causal=False)
    assert np.any(np.abs(bad - o) > tol)
    bad, _ = oracle.attention(q, k, v, scale=1.0)
    assert np.any(np.abs(bad - o) > tol)


# ----------------------------------------------------------------------------
# Plain fp16 weights
# ----------------------------------------------------------------------------
def test_fp16_dequant_reads_little_endian_rows():
    """Hand-built bytes: 1.0 = 0x3C00, -2.0 = 0xC000, 0.5 = 0x3800, 65504 = 0x7BFF."""
    vals = [1.0, -2.0, 0.5, 65504.0]
    raw = []
    for v in ([0x3C00, 0xC000, 0x3800, 0x7BFF] * 16):
        raw += [v & 0xFF, v >> 8]
    W = oracle.dequant(oracle.FP16, np.array(raw, dtype=np.uint8), 2, 32)
    assert W.shape == (2, 32)
    assert list(W[0, :4]) == vals and list(W[1, -4:]) == vals


def test_fp16_gemv_matches_exact_rationals():
    w = synth.fp16_weight(synth.rng_for(44, 0), 5, 64)
    x = synth.activation(synth.rng_for(44, 1), (2, 64), synth.BF16)
    y, b = oracle.qgemv(oracle.FP16, w.canon, 5, 64, x.values)
    for m in range(2):
        for n in range(5):
            exact = sum(Fraction(float(w.codes[n, k])) * Fraction(float(x.values[m, k])) for k in range(64))
            assert abs(Fraction(y[m, n]) - exact) <= Fraction(1, 2 ** 40) * (1 + abs(exact))
            assert b[m, n] == pytest.approx(sum(abs(float(w.codes[n, k]) * x.values[m, k]) for k in range(64)))
