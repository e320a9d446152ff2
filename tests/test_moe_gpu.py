"""GPU parity of the MoE path against the CPU oracle.

Two kernel paths sit behind q4q8_moe_qgemm: MFMA row tiles for prefill
(T > 8 tokens) and GEMV kernels for decode (T <= 8); the cases below cover
both, including the benchmark's MoE shape at T = 1 and 8.

Routing and the permutation (ids, counts, offsets, sorted_pairs) must match
bit for bit; gates within 2e-3 relative; h (the bf16 SwiGLU output, read back
through h_out) within the first-order bound propagated from the per-dot-
product tolerance; out within the bound propagated through the whole chain,
and again, tighter, against the oracle fed the GPU's own h (down projection
and combine checked on their own).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from util import act_tensor, bytes_tensor, dev, values

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import gemm_q4_q8_amd as q
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    q.lib()
    return q


def _route(q, logits, k):
    L = torch.from_numpy(np.ascontiguousarray(logits, dtype=np.float32)).to(dev())
    got = q.moe_route(L, k)
    torch.cuda.synchronize()
    return [a.cpu().numpy() for a in got]


def _check_route(logits, k, got):
    ids, gates, counts, offsets, sp = got
    rid, rg = oracle.moe_route(logits, k)
    rc, ro, rsp = oracle.moe_sort(rid, logits.shape[1])
    assert np.array_equal(ids, rid), "ids differ"
    assert np.array_equal(counts, rc), "counts differ"
    assert np.array_equal(offsets, ro), "offsets differ"
    assert np.array_equal(sp, rsp), "sorted_pairs differ"
    assert np.all(np.abs(gates - rg) <= 2e-3 * rg + 1e-5), np.abs(gates - rg).max()


ROUTE_CASES = [(512, 128, 8), (37, 10, 3), (1, 1, 1), (5, 16, 16), (64, 65, 4), (300, 1024, 16),
               (1000, 64, 1), (3, 200, 7)]


@pytest.mark.parametrize("T,E,k", ROUTE_CASES)
def test_route_parity(q, T, E, k):
    logits = synth.router_logits(synth.rng_for(70, T * 7 + E * 3 + k), T, E)
    _check_route(logits, k, _route(q, logits, k))


def test_route_ties_and_infinities(q):
    """Many exact ties (integer logits), a row of equal values, -inf entries
    (a row keeps two finite logits: with every selected logit -inf the
    softmax is undefined)."""
    rng = synth.rng_for(71, 0)
    logits = rng.integers(-2, 3, size=(200, 40)).astype(np.float32)
    logits[5] = 0.0
    logits[6, ::3] = -np.inf
    logits[7] = -np.inf
    logits[7, [3, 30]] = [1.0, -5.0]
    _check_route(logits, 6, _route(q, logits, 6))


def _nan_logits(seed, T, E):
    """Integer logits (many exact ties) with NaN and -inf entries; every row
    keeps at least one finite logit (with every selected logit -inf the
    softmax is undefined)."""
    rng = synth.rng_for(seed, T * 1000 + E)
    lg = rng.integers(-2, 3, size=(T, E)).astype(np.float32)
    lg[rng.random(lg.shape) < 0.2] = np.nan
    lg[rng.random(lg.shape) < 0.15] = -np.inf
    lg[:, 0] = np.where(np.isfinite(lg[:, 0]), lg[:, 0], 1.0)
    return lg


@pytest.mark.parametrize("T,E,k", [(1, 5, 4), (3, 16, 4), (12, 40, 6), (200, 40, 6), (9, 128, 8), (40, 300, 16)])
def test_route_nan_logits(q, T, E, k):
    """NaN logits rank as -inf, on each routing kernel: the one-workgroup
    kernel with the LDS rank sort (<= 32 pairs) and with the histogram sort,
    and the top-k + sort kernels (T > 16)."""
    logits = _nan_logits(74, T, E)
    if T == 1:
        logits[0] = [1.0, np.nan, 0.5, -np.inf, -np.inf]
    got = _route(q, logits, k)
    if T == 1:
        assert got[0].tolist() == [[0, 2, 1, 3]]
    _check_route(logits, k, got)


def test_moe_nan_logits(q):
    """NaN router logits through the whole layer: the one-call decode entry
    point (routing inside the gate/up kernel at T <= 4, the routing kernel
    above), the two-call decode path, and the prefill path."""
    E, k, H, F = 24, 4, 256, 128
    wg = [synth.q_weight(synth.rng_for(75, 1000 + e), synth.Q4_0, F, H) for e in range(E)]
    wu = [synth.q_weight(synth.rng_for(75, 2000 + e), synth.Q4_0, F, H) for e in range(E)]
    wd = [synth.q_weight(synth.rng_for(75, 3000 + e), synth.Q4_0, H, F) for e in range(E)]
    for T in (2, 6, 40):
        logits = _nan_logits(76, T, E)
        x = synth.activation(synth.rng_for(77, T), (T, H), synth.BF16)
        two = _run_moe(q, synth.Q4_0, logits, x, wg, wu, wd, k, H, F)
        _check_moe(synth.Q4_0, logits, x, wg, wu, wd, k, H, F, two, f"moe NaN logits T{T}")
        if T <= 8:
            one = _run_moe_decode(q, synth.Q4_0, logits, x, wg, wu, wd, k, H, F)
            for key in ("ids", "gates", "offsets", "sp", "h", "out"):
                assert np.array_equal(one[key], two[key]), key


def test_route_many_pairs(q):
    """65536 pairs: every wave of the sort handles several rounds of 64."""
    logits = synth.router_logits(synth.rng_for(72, 0), 8192, 128)
    _check_route(logits, 8, _route(q, logits, 8))


def _stack(q, fmt, ws, n, k):
    return torch.cat([q.repack(fmt, bytes_tensor(w.canon), n, k) for w in ws])


def _run_moe(q, fmt, logits, x, wg, wu, wd, k, H, F):
    E = len(wg)
    Wg, Wu, Wd = _stack(q, fmt, wg, F, H), _stack(q, fmt, wu, F, H), _stack(q, fmt, wd, H, F)
    L = torch.from_numpy(logits).to(dev())
    ids, gates, counts, offsets, sp = q.moe_route(L, k)
    T = logits.shape[0]
    h = torch.full((T * k, F), float("nan"), dtype=torch.bfloat16, device=dev())
    out = q.moe_qgemm(fmt, Wg, Wu, Wd, E, H, F, act_tensor(x), k, gates, offsets, sp, h_out=h)
    torch.cuda.synchronize()
    return dict(ids=ids.cpu().numpy(), gates=gates.cpu().numpy(), offsets=offsets.cpu().numpy(),
                sp=sp.cpu().numpy(), h=values(h), out=out.cpu().numpy().astype(np.float64))


def _check_moe(fmt, logits, x, wg, wu, wd, k, H, F, got, what, abs_tol=1e-5):
    cg, cu, cd = [w.canon for w in wg], [w.canon for w in wu], [w.canon for w in wd]
    r = oracle.moe(fmt, cg, cu, cd, x.values, logits, k, H, F)
    assert np.array_equal(got["ids"], r["ids"]) and np.array_equal(got["sp"], r["sorted_pairs"])
    hb = oracle.h_bound(r, abs_tol=abs_tol)
    herr = np.abs(got["h"] - r["h"])
    assert np.all(np.isfinite(got["h"])), f"{what}: h not finite"
    assert np.all(herr <= hb), f"{what}: h err/bound {(herr / hb).max():.3g}"
    ob = oracle.moe_out_bound(fmt, cd, r, r["ids"], r["gates"], r["sorted_pairs"], H, F, hb, abs_tol=abs_tol)
    oerr = np.abs(got["out"] - r["out"])
    assert np.all(oerr <= ob), f"{what}: out err/bound {(oerr / ob).max():.3g}"
    # Down projection + combine on their own: the oracle takes the GPU's h.
    r2 = oracle.moe_ffn(fmt, cg, cu, cd, x.values, r["ids"], r["gates"], r["sorted_pairs"], H, F,
                        h_override=got["h"])
    ob2 = oracle.moe_out_bound(fmt, cd, r2, r["ids"], r["gates"], r["sorted_pairs"], H, F,
                               np.zeros_like(got["h"]), abs_tol=abs_tol)
    oerr2 = np.abs(got["out"] - r2["out"])
    assert np.all(oerr2 <= ob2), f"{what}: isolated out err/bound {(oerr2 / ob2).max():.3g}"


MOE_CASES = [
    # fmt, xdt, T, E, k, H, F
    (synth.Q4_0, synth.BF16, 40, 8, 2, 256, 128),
    (synth.Q8_0, synth.F16, 33, 5, 3, 384, 256),
    (synth.Q4_0, synth.BF16, 100, 16, 4, 256, 384),
    (synth.Q4_0, synth.F16, 200, 4, 2, 128, 256),    # ~100 pairs per expert: two row tiles
    (synth.Q8_0, synth.BF16, 10, 16, 1, 128, 128),   # most experts empty
    (synth.Q4_0, synth.BF16, 1, 3, 3, 128, 128),     # one token
    # H or F past one 1024-column LDS phase and not a multiple of it: the
    # expert kernels reload a partial second phase.
    (synth.Q4_0, synth.BF16, 64, 4, 2, 1536, 256),
    (synth.Q8_0, synth.BF16, 48, 4, 2, 1536, 1152),
    (synth.Q4_0, synth.F16, 90, 6, 3, 384, 1152),
]


@pytest.mark.parametrize("fmt,xdt,T,E,k,H,F", MOE_CASES)
def test_moe_parity(q, fmt, xdt, T, E, k, H, F):
    seed = 80 + T + E
    logits = synth.router_logits(synth.rng_for(seed, 0), T, E)
    x = synth.activation(synth.rng_for(seed, 1), (T, H), xdt)
    wg = [synth.q_weight(synth.rng_for(seed, 1000 + e), fmt, F, H) for e in range(E)]
    wu = [synth.q_weight(synth.rng_for(seed, 2000 + e), fmt, F, H) for e in range(E)]
    wd = [synth.q_weight(synth.rng_for(seed, 3000 + e), fmt, H, F) for e in range(E)]
    got = _run_moe(q, fmt, logits, x, wg, wu, wd, k, H, F)
    _check_moe(fmt, logits, x, wg, wu, wd, k, H, F, got, f"moe fmt{fmt} T{T} E{E} k{k} H{H} F{F}")


DECODE_CASES = [
    # fmt, xdt, T, E, k, H, F
    (synth.Q8_0, synth.F16, 3, 16, 4, 512, 384),
    (synth.Q4_0, synth.F16, 5, 8, 8, 256, 128),      # topk = E: every expert takes all 5 tokens
    (synth.Q8_0, synth.BF16, 8, 4, 2, 128, 256),     # up to 8 rows per expert
    (synth.Q4_0, synth.BF16, 2, 1024, 16, 128, 128),
    (synth.Q4_0, synth.BF16, 7, 64, 8, 1024, 512),
    (synth.Q8_0, synth.BF16, 1, 32, 1, 384, 128),
    (synth.Q8_0, synth.F16, 2, 32, 16, 256, 1792),  # topk x F past the fused down+combine's buffer
]


@pytest.mark.parametrize("fmt,xdt,T,E,k,H,F", DECODE_CASES)
def test_moe_decode_parity(q, fmt, xdt, T, E, k, H, F):
    seed = 120 + T + E + k
    logits = synth.router_logits(synth.rng_for(seed, 0), T, E)
    x = synth.activation(synth.rng_for(seed, 1), (T, H), xdt)
    wg = [synth.q_weight(synth.rng_for(seed, 1000 + e), fmt, F, H) for e in range(E)]
    wu = [synth.q_weight(synth.rng_for(seed, 2000 + e), fmt, F, H) for e in range(E)]
    wd = [synth.q_weight(synth.rng_for(seed, 3000 + e), fmt, H, F) for e in range(E)]
    got = _run_moe(q, fmt, logits, x, wg, wu, wd, k, H, F)
    _check_moe(fmt, logits, x, wg, wu, wd, k, H, F, got, f"moe decode fmt{fmt} T{T} E{E} k{k} H{H} F{F}")


def _run_moe_decode(q, fmt, logits, x, wg, wu, wd, k, H, F):
    """The one-call decode entry point, with every output read back."""
    E = len(wg)
    Wg, Wu, Wd = _stack(q, fmt, wg, F, H), _stack(q, fmt, wu, F, H), _stack(q, fmt, wd, H, F)
    L = torch.from_numpy(logits).to(dev())
    T = logits.shape[0]
    h = torch.full((T * k, F), float("nan"), dtype=torch.bfloat16, device=dev())
    route = (torch.full((T, k), -7, dtype=torch.int32, device=dev()), torch.full((T, k), -7.0, device=dev()),
             torch.full((E,), -7, dtype=torch.int32, device=dev()), torch.full((E + 1,), -7, dtype=torch.int32, device=dev()),
             torch.full((T * k,), -7, dtype=torch.int32, device=dev()))
    out, (ids, gates, counts, offsets, sp) = q.moe_decode(fmt, Wg, Wu, Wd, E, H, F, L, act_tensor(x), k, route=route,
                                                          h_out=h)
    torch.cuda.synchronize()
    return dict(ids=ids.cpu().numpy(), gates=gates.cpu().numpy(), counts=counts.cpu().numpy(),
                offsets=offsets.cpu().numpy(), sp=sp.cpu().numpy(), h=values(h),
                out=out.cpu().numpy().astype(np.float64))


@pytest.mark.parametrize("fmt,xdt,T,E,k,H,F", DECODE_CASES)
def test_moe_decode_one_call(q, fmt, xdt, T, E, k, H, F):
    """q4q8_moe_decode (routing inside the first expert kernel) against the
    oracle, and bit for bit against q4q8_moe_route + q4q8_moe_qgemm."""
    seed = 120 + T + E + k
    logits = synth.router_logits(synth.rng_for(seed, 0), T, E)
    x = synth.activation(synth.rng_for(seed, 1), (T, H), xdt)
    wg = [synth.q_weight(synth.rng_for(seed, 1000 + e), fmt, F, H) for e in range(E)]
    wu = [synth.q_weight(synth.rng_for(seed, 2000 + e), fmt, F, H) for e in range(E)]
    wd = [synth.q_weight(synth.rng_for(seed, 3000 + e), fmt, H, F) for e in range(E)]
    one = _run_moe_decode(q, fmt, logits, x, wg, wu, wd, k, H, F)
    two = _run_moe(q, fmt, logits, x, wg, wu, wd, k, H, F)
    for key in ("ids", "gates", "offsets", "sp"):
        assert np.array_equal(one[key], two[key]), key
    assert np.array_equal(one["counts"], np.diff(two["offsets"]))
    assert np.array_equal(one["h"], two["h"], equal_nan=False)
    assert np.array_equal(one["out"], two["out"])
    _check_moe(fmt, logits, x, wg, wu, wd, k, H, F, one, f"moe_decode fmt{fmt} T{T} E{E} k{k} H{H} F{F}")


def test_moe_decode_one_call_full_shape(q):
    """The MoE workload's experts at T = 1, 2, 8 through the one-call entry
    point: bitwise equal to the two-call path, and against the oracle."""
    cfg = synth.MOE
    E, k, H, F = cfg["E"], cfg["topk"], cfg["H"], cfg["F"]
    _, _, wg, wu, wd = synth.moe(T=1)
    for T in (1, 2, 8):
        logits = synth.router_logits(synth.rng_for(132, T), T, E)
        x = synth.activation(synth.rng_for(133, T), (T, H), synth.BF16)
        one = _run_moe_decode(q, synth.Q4_0, logits, x, wg, wu, wd, k, H, F)
        two = _run_moe(q, synth.Q4_0, logits, x, wg, wu, wd, k, H, F)
        assert np.array_equal(one["out"], two["out"]) and np.array_equal(one["h"], two["h"])
        assert np.array_equal(one["gates"], two["gates"]) and np.array_equal(one["sp"], two["sp"])
        _check_moe(synth.Q4_0, logits, x, wg, wu, wd, k, H, F, one, f"moe_decode full shape T{T}")


def test_moe_decode_full_shape(q):
    """The MoE workload's experts (E 128, top-8, H 2048, F 768, Q4_0) with
    T = 1, 2, 8 decode tokens (every output), and T = 9 (the first prefill
    size) on the same weights."""
    cfg = synth.MOE
    E, k, H, F = cfg["E"], cfg["topk"], cfg["H"], cfg["F"]
    _, _, wg, wu, wd = synth.moe(T=1)
    for T in (1, 2, 8, 9):
        logits = synth.router_logits(synth.rng_for(130, T), T, E)
        x = synth.activation(synth.rng_for(131, T), (T, H), synth.BF16)
        got = _run_moe(q, synth.Q4_0, logits, x, wg, wu, wd, k, H, F)
        _check_moe(synth.Q4_0, logits, x, wg, wu, wd, k, H, F, got, f"moe full shape T{T}")


def test_moe_deterministic(q):
    T, E, k, H, F = 64, 8, 2, 256, 128
    logits = synth.router_logits(synth.rng_for(90, 0), T, E)
    x = synth.activation(synth.rng_for(90, 1), (T, H), synth.BF16)
    wg = [synth.q_weight(synth.rng_for(90, 1000 + e), synth.Q4_0, F, H) for e in range(E)]
    wu = [synth.q_weight(synth.rng_for(90, 2000 + e), synth.Q4_0, F, H) for e in range(E)]
    wd = [synth.q_weight(synth.rng_for(90, 3000 + e), synth.Q4_0, H, F) for e in range(E)]
    a = _run_moe(q, synth.Q4_0, logits, x, wg, wu, wd, k, H, F)
    b = _run_moe(q, synth.Q4_0, logits, x, wg, wu, wd, k, H, F)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["h"], b["h"])
    # decode path (6 tokens)
    a = _run_moe(q, synth.Q4_0, logits[:6], x6 := synth.act_from_values(x.values[:6], synth.BF16), wg, wu, wd, k,
                 H, F)
    b = _run_moe(q, synth.Q4_0, logits[:6], x6, wg, wu, wd, k, H, F)
    assert np.array_equal(a["out"], b["out"]) and np.array_equal(a["h"], b["h"])


def test_moe_full_size_sampled(q):
    """The MoE workload (T 512, E 128, top-8, H 2048, F 768, Q4_0, bf16 X) in
    the benchmark's launch shape: routing bit-exact; h of every pair of four
    sampled experts against the oracle; out of six sampled tokens against
    the oracle's down projection and combine fed the GPU's h."""
    cfg = synth.MOE
    T, E, k, H, F = cfg["T"], cfg["E"], cfg["topk"], cfg["H"], cfg["F"]
    logits, x, wg, wu, wd = synth.moe()
    got = _run_moe(q, synth.Q4_0, logits, x, wg, wu, wd, k, H, F)
    rid, rg = oracle.moe_route(logits, k)
    rc, ro, rsp = oracle.moe_sort(rid, E)
    assert np.array_equal(got["ids"], rid) and np.array_equal(got["sp"], rsp)
    assert np.array_equal(got["offsets"], ro)
    assert np.all(np.abs(got["gates"] - rg) <= 2e-3 * rg + 1e-5)
    assert np.all(np.isfinite(got["out"]))

    flat = rid.reshape(-1)
    rng = np.random.default_rng(91)
    for e in rng.choice(np.nonzero(rc)[0], 4, replace=False):
        rows = np.arange(ro[e], ro[e + 1])            # sorted-order positions of expert e
        toks = rsp[rows] // k
        xe = x.values[toks]
        Wg = oracle.dequant(synth.Q4_0, wg[e].canon, F, H)
        Wu = oracle.dequant(synth.Q4_0, wu[e].canon, F, H)
        r = dict(zg=xe @ Wg.T, zu=xe @ Wu.T, bg=np.abs(xe) @ np.abs(Wg).T, bu=np.abs(xe) @ np.abs(Wu).T)
        r["h"] = oracle.silu(r["zg"]) * r["zu"]
        hb = oracle.h_bound(r)
        assert np.all(np.abs(got["h"][rows] - r["h"]) <= hb), f"expert {e}: h"

    inv = np.empty(T * k, dtype=np.int64)
    inv[rsp] = np.arange(T * k)
    for t in rng.choice(T, 6, replace=False):
        ref = np.zeros(H)
        bound = np.full(H, 1e-5)
        for j in range(k):
            p = t * k + j
            e = flat[p]
            hrow = got["h"][inv[p]]
            Wd = oracle.dequant(synth.Q4_0, wd[e].canon, H, F)
            y = Wd @ hrow
            by = np.abs(Wd) @ np.abs(hrow)
            ref += rg[t, j] * y
            bound += rg[t, j] * (2e-3 * by + 1e-5) + (2e-3 * rg[t, j] + 1e-5) * np.abs(y)
        assert np.all(np.abs(got["out"][t] - ref) <= bound), f"token {t}: out"


@pytest.mark.parametrize("fmt", [synth.Q4_0, synth.Q8_0])
def test_moe_full_size_chain(q, fmt):
    """The MoE workload (T 512, E 128, top-8, H 2048, F 768, bf16 X) in both
    formats, in the benchmark's launch shape, against the oracle's own chain:
    routing bit-exact, every h value within the propagated bound, every out
    value within the bound carried through the whole chain, and every out
    value against the oracle's down projection and combine fed the GPU's h."""
    cfg = synth.MOE
    T, E, k, H, F = cfg["T"], cfg["E"], cfg["topk"], cfg["H"], cfg["F"]
    logits, x, wg, wu, wd = synth.moe(fmt=fmt)
    got = _run_moe(q, fmt, logits, x, wg, wu, wd, k, H, F)
    _check_moe(fmt, logits, x, wg, wu, wd, k, H, F, got, f"moe full size fmt{fmt}")


def test_moe_malformed_offsets_stay_in_bounds(q):
    """Offsets past T*topk (malformed routing) on the matrix-core path: the
    results are unspecified, but no store may land outside h_out or out."""
    T, E, k, H, F = 24, 4, 2, 256, 128
    P = T * k
    fmt = synth.Q4_0
    wg = [synth.q_weight(synth.rng_for(78, 1000 + e), fmt, F, H) for e in range(E)]
    wu = [synth.q_weight(synth.rng_for(78, 2000 + e), fmt, F, H) for e in range(E)]
    wd = [synth.q_weight(synth.rng_for(78, 3000 + e), fmt, H, F) for e in range(E)]
    Wg, Wu, Wd = _stack(q, fmt, wg, F, H), _stack(q, fmt, wu, F, H), _stack(q, fmt, wd, H, F)
    x = synth.activation(synth.rng_for(78, 1), (T, H), synth.BF16)
    gates = torch.full((T, k), 0.5, device=dev())
    offsets = torch.tensor([0, 10, 30, P + 40, P + 200], dtype=torch.int32, device=dev())
    sp = torch.arange(P, dtype=torch.int32, device=dev())
    guard = 4096
    hbuf = torch.full((P * F + guard,), 7.0, dtype=torch.bfloat16, device=dev())
    obuf = torch.full((T * H + guard,), 7.0, dtype=torch.float32, device=dev())
    ws = torch.full((q.moe_workspace(fmt, T, E, k, H, F) + guard,), 0x5A, dtype=torch.uint8, device=dev())
    q.moe_qgemm(fmt, Wg, Wu, Wd, E, H, F, act_tensor(x), k, gates, offsets, sp,
                out=obuf[:T * H].view(T, H), h_out=hbuf[:P * F].view(P, F), ws=ws[:-guard])
    torch.cuda.synchronize()
    assert torch.all(hbuf[P * F:] == 7.0)
    assert torch.all(obuf[T * H:] == 7.0)
    assert torch.all(ws[-guard:] == 0x5A)


@pytest.mark.parametrize("T", [2, 6, 40])
@pytest.mark.parametrize("xdt", [synth.BF16, synth.F16])
def test_moe_activation_range(q, T, xdt):
    """Token rows far outside the fp16 range: each token row is scaled by a
    power of two before its fp16 conversion and h and y carry the square of
    that factor, so neither saturates.  bf16 tokens scaled by 2^20 next to
    unscaled ones and ones scaled by 2^-20 (standard tolerance), then every
    token scaled by 2^-20 with the absolute term scaled to match (h and out
    scale with the square); fp16 tokens with entries near the fp16 maximum.
    T = 2 (routing inside the first kernel, fused down + combine), 6 (decode
    kernels) and 40 (matrix-core path); the one-call entry point must equal
    the two-call path bit for bit."""
    E, k, H, F = 16, 4, 256, 256
    fmt = synth.Q4_0
    wg = [synth.q_weight(synth.rng_for(79, 1000 + e), fmt, F, H) for e in range(E)]
    wu = [synth.q_weight(synth.rng_for(79, 2000 + e), fmt, F, H) for e in range(E)]
    wd = [synth.q_weight(synth.rng_for(79, 3000 + e), fmt, H, F) for e in range(E)]
    logits = synth.router_logits(synth.rng_for(79, T), T, E)
    base = synth.activation(synth.rng_for(79, 100 + T), (T, H), synth.BF16).values
    if xdt == synth.BF16:
        scale = np.where(np.arange(T) % 3 == 0, 2.0 ** 20, np.where(np.arange(T) % 3 == 1, 1.0, 2.0 ** -20))
        cases = [(scale, 1e-5), (np.full(T, 2.0 ** -20), 1e-5 * 2.0 ** -40)]
    else:
        cases = [(np.full(T, 2.0 ** 13), 1e-5)]       # |x| up to ~4 * 8192: near the fp16 maximum
    for sc, abs_tol in cases:
        x = synth.act_from_values(base * sc[:, None], xdt)
        two = _run_moe(q, fmt, logits, x, wg, wu, wd, k, H, F)
        assert np.all(np.isfinite(two["out"])) and np.all(np.isfinite(two["h"]))
        _check_moe(fmt, logits, x, wg, wu, wd, k, H, F, two, f"moe range T{T} xdt{xdt}", abs_tol=abs_tol)
        if T <= 8:
            one = _run_moe_decode(q, fmt, logits, x, wg, wu, wd, k, H, F)
            for key in ("h", "out"):
                assert np.array_equal(one[key], two[key]), key


def _run_forward(q, fmt, logits, x, wg, wu, wd, k, H, F):
    """The one-call entry point (q4q8_moe_forward), every output read back."""
    E = len(wg)
    Wg, Wu, Wd = _stack(q, fmt, wg, F, H), _stack(q, fmt, wu, F, H), _stack(q, fmt, wd, H, F)
    L = torch.from_numpy(logits).to(dev())
    T = logits.shape[0]
    h = torch.full((T * k, F), float("nan"), dtype=torch.bfloat16, device=dev())
    route = (torch.full((T, k), -7, dtype=torch.int32, device=dev()), torch.full((T, k), -7.0, device=dev()),
             torch.full((E,), -7, dtype=torch.int32, device=dev()), torch.full((E + 1,), -7, dtype=torch.int32, device=dev()),
             torch.full((T * k,), -7, dtype=torch.int32, device=dev()))
    out, (ids, gates, counts, offsets, sp) = q.moe_forward(fmt, Wg, Wu, Wd, E, H, F, L, act_tensor(x), k, route=route,
                                                           h_out=h)
    torch.cuda.synchronize()
    return dict(ids=ids.cpu().numpy(), gates=gates.cpu().numpy(), counts=counts.cpu().numpy(),
                offsets=offsets.cpu().numpy(), sp=sp.cpu().numpy(), h=values(h),
                out=out.cpu().numpy().astype(np.float64))


FORWARD_CASES = [
    # fmt, xdt, T, E, k, H, F
    (synth.Q4_0, synth.BF16, 40, 8, 2, 256, 128),
    (synth.Q8_0, synth.F16, 12, 16, 4, 384, 256),     # just past the decode path
    (synth.Q4_0, synth.F16, 200, 4, 2, 128, 256),     # ~100 rows per expert: two row tiles
    (synth.Q4_0, synth.BF16, 1000, 16, 5, 128, 128),  # 5000 pairs: two rounds of the in-kernel sort
    (synth.Q8_0, synth.BF16, 48, 4, 2, 1536, 1152),   # partial LDS phases
    (synth.Q4_0, synth.BF16, 30, 64, 8, 256, 128),    # many empty experts
    (synth.Q4_0, synth.BF16, 3, 16, 4, 256, 128),     # the decode path
]


@pytest.mark.parametrize("fmt,xdt,T,E,k,H,F", FORWARD_CASES)
def test_moe_forward(q, fmt, xdt, T, E, k, H, F):
    """q4q8_moe_forward (routing and the sort formed inside the expert
    kernels) against the oracle, and bit for bit against q4q8_moe_route +
    q4q8_moe_qgemm (routing arrays, h, out)."""
    seed = 150 + T + E + k
    logits = synth.router_logits(synth.rng_for(seed, 0), T, E)
    x = synth.activation(synth.rng_for(seed, 1), (T, H), xdt)
    wg = [synth.q_weight(synth.rng_for(seed, 1000 + e), fmt, F, H) for e in range(E)]
    wu = [synth.q_weight(synth.rng_for(seed, 2000 + e), fmt, F, H) for e in range(E)]
    wd = [synth.q_weight(synth.rng_for(seed, 3000 + e), fmt, H, F) for e in range(E)]
    one = _run_forward(q, fmt, logits, x, wg, wu, wd, k, H, F)
    two = _run_moe(q, fmt, logits, x, wg, wu, wd, k, H, F)
    for key in ("ids", "gates", "offsets", "sp", "h", "out"):
        assert np.array_equal(one[key], two[key]), key
    assert np.array_equal(one["counts"], np.diff(two["offsets"]))
    _check_moe(fmt, logits, x, wg, wu, wd, k, H, F, one, f"moe_forward fmt{fmt} T{T} E{E} k{k} H{H} F{F}")


@pytest.mark.parametrize("fmt", [synth.Q4_0, synth.Q8_0])
def test_moe_forward_full_size(q, fmt):
    """The MoE workload through q4q8_moe_forward: bit for bit the two-call
    path (whose full-size parity against the oracle's chain is tested above),
    routing arrays against the oracle, NaN-free."""
    cfg = synth.MOE
    T, E, k, H, F = cfg["T"], cfg["E"], cfg["topk"], cfg["H"], cfg["F"]
    logits, x, wg, wu, wd = synth.moe(fmt=fmt)
    one = _run_forward(q, fmt, logits, x, wg, wu, wd, k, H, F)
    two = _run_moe(q, fmt, logits, x, wg, wu, wd, k, H, F)
    for key in ("ids", "gates", "offsets", "sp", "h", "out"):
        assert np.array_equal(one[key], two[key]), key
    rid, _ = oracle.moe_route(logits, k)
    rc, ro, rsp = oracle.moe_sort(rid, E)
    assert np.array_equal(one["ids"], rid) and np.array_equal(one["counts"], rc)
    assert np.array_equal(one["offsets"], ro) and np.array_equal(one["sp"], rsp)
    assert np.all(np.isfinite(one["out"]))


def test_moe_forward_nan_logits(q):
    E, k, H, F = 24, 4, 256, 128
    wg = [synth.q_weight(synth.rng_for(75, 1000 + e), synth.Q4_0, F, H) for e in range(E)]
    wu = [synth.q_weight(synth.rng_for(75, 2000 + e), synth.Q4_0, F, H) for e in range(E)]
    wd = [synth.q_weight(synth.rng_for(75, 3000 + e), synth.Q4_0, H, F) for e in range(E)]
    logits = _nan_logits(76, 40, E)
    x = synth.activation(synth.rng_for(77, 40), (40, H), synth.BF16)
    one = _run_forward(q, synth.Q4_0, logits, x, wg, wu, wd, k, H, F)
    _check_moe(synth.Q4_0, logits, x, wg, wu, wd, k, H, F, one, "moe_forward NaN logits")
