"""Seeded random shapes through every product family against the oracle:
decode GEMV (Q4_0 / Q8_0 / fp16 weights, fp16 / bf16 x, M = 1..8), grouped
GEMV launches of 2-8 problems with different K, prefill GEMM (every format and
output dtype, ragged M and N), the MoE layer through the one-call prefill
entry point and the one-call decode entry point (routing ids and the sorted
pairs bit-exact, h and out within their bounds), and prefill attention
(batch, sequence length, head counts with GQA, causal or not, bf16 / fp16).  Shapes are drawn from a
fixed seed, so every run checks the same cases."""
import numpy as np
import pytest
import torch

import oracle
import synth
from util import act_tensor, bytes_tensor, check, check_rounded, values
import test_moe_gpu as tm

pytestmark = pytest.mark.gpu

OUT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


@pytest.fixture(scope="module")
def q():
    import gemm_q4_q8_amd as q
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    q.lib()
    return q


def _cases(kind, n):
    rng = np.random.default_rng(synth.rng_for(970, {"gemv": 0, "grouped": 1, "gemm": 2, "moe": 3, "dec": 4,
                                                     "attn": 5}[kind])
                                .integers(1 << 62))
    return [int(s) for s in rng.integers(1 << 30, size=n)]


@pytest.mark.parametrize("seed", _cases("gemv", 48))
def test_random_gemv(q, seed):
    r = np.random.default_rng(seed)
    fmt, xdt = int(r.choice([1, 2, 3])), int(r.choice([1, 2]))
    N, K, M = int(r.integers(1, 700)), 32 * int(r.integers(1, 200)), int(r.integers(1, 9))
    w = synth.weight(synth.rng_for(971, seed), fmt, N, K)
    x = synth.activation(synth.rng_for(972, seed), (M, K), xdt)
    y = q.qgemv(fmt, q.repack(fmt, bytes_tensor(w.canon), N, K), N, K, act_tensor(x))
    torch.cuda.synchronize()
    ref, b = oracle.qgemv(fmt, w.canon, N, K, x.values)
    check(y.cpu().numpy(), ref, b, f"gemv fmt{fmt} xdt{xdt} N{N} K{K} M{M}")


@pytest.mark.parametrize("seed", _cases("grouped", 24))
def test_random_grouped_gemv(q, seed):
    r = np.random.default_rng(seed)
    fmt, xdt, M, G = int(r.choice([1, 2])), int(r.choice([1, 2])), int(r.integers(1, 9)), int(r.integers(2, 9))
    probs, refs = [], []
    for g in range(G):
        N, K = int(r.integers(1, 500)), 32 * int(r.integers(1, 160))
        w = synth.weight(synth.rng_for(973, seed + g), fmt, N, K)
        x = synth.activation(synth.rng_for(974, seed + g), (M, K), xdt)
        y = torch.empty((M, N), dtype=torch.float32, device="cuda:0")
        probs.append((q.repack(fmt, bytes_tensor(w.canon), N, K), N, K, act_tensor(x), y))
        refs.append(oracle.qgemv(fmt, w.canon, N, K, x.values))
    q.qgemv_grouped(fmt, probs, M)
    torch.cuda.synchronize()
    for g, ((_, N, K, _, y), (ref, b)) in enumerate(zip(probs, refs)):
        check(y.cpu().numpy(), ref, b, f"grouped fmt{fmt} M{M} problem {g} N{N} K{K}")


@pytest.mark.parametrize("seed", _cases("gemm", 48))
def test_random_gemm(q, seed):
    r = np.random.default_rng(seed)
    fmt, xdt, ydt = int(r.choice([1, 2, 3])), int(r.choice([1, 2])), str(r.choice(["bf16", "f16", "f32"]))
    M, N, K = int(r.integers(1, 700)), int(r.integers(1, 900)), 32 * int(r.integers(1, 64))
    w = synth.weight(synth.rng_for(975, seed), fmt, N, K)
    x = synth.activation(synth.rng_for(976, seed), (M, K), xdt)
    y = q.qgemm(fmt, q.repack(fmt, bytes_tensor(w.canon), N, K), N, K, act_tensor(x), out_dtype=OUT[ydt])
    torch.cuda.synchronize()
    ref, b = oracle.qgemm(fmt, w.canon, N, K, x.values)
    what = f"gemm fmt{fmt} xdt{xdt} M{M} N{N} K{K} {ydt}"
    if ydt == "f32":
        check(values(y), ref, b, what)
    else:
        check_rounded(values(y), ref, b, what, dtype=ydt)


def _moe_case(seed, max_t):
    r = np.random.default_rng(seed)
    fmt, xdt = int(r.choice([1, 2])), int(r.choice([1, 2]))
    T, E = int(r.integers(1, max_t + 1)), int(r.integers(1, 40))
    k = int(r.integers(1, min(E, 8) + 1))
    H, F = 128 * int(r.integers(1, 9)), 128 * int(r.integers(1, 9))
    logits = synth.router_logits(synth.rng_for(seed, 0), T, E)
    x = synth.activation(synth.rng_for(seed, 1), (T, H), xdt)
    wg = [synth.q_weight(synth.rng_for(seed, 1000 + e), fmt, F, H) for e in range(E)]
    wu = [synth.q_weight(synth.rng_for(seed, 2000 + e), fmt, F, H) for e in range(E)]
    wd = [synth.q_weight(synth.rng_for(seed, 3000 + e), fmt, H, F) for e in range(E)]
    return fmt, logits, x, wg, wu, wd, k, H, F


@pytest.mark.parametrize("seed", _cases("moe", 16))
def test_random_moe_forward(q, seed):
    fmt, logits, x, wg, wu, wd, k, H, F = _moe_case(seed, 120)
    got = tm._run_forward(q, fmt, logits, x, wg, wu, wd, k, H, F)
    tm._check_moe(fmt, logits, x, wg, wu, wd, k, H, F, got,
                  f"moe_forward fmt{fmt} T{logits.shape[0]} E{len(wg)} k{k} H{H} F{F}")


@pytest.mark.parametrize("seed", _cases("dec", 12))
def test_random_moe_decode(q, seed):
    fmt, logits, x, wg, wu, wd, k, H, F = _moe_case(seed, 8)
    got = tm._run_moe_decode(q, fmt, logits, x, wg, wu, wd, k, H, F)
    tm._check_moe(fmt, logits, x, wg, wu, wd, k, H, F, got,
                  f"moe_decode fmt{fmt} T{logits.shape[0]} E{len(wg)} k{k} H{H} F{F}")


@pytest.mark.parametrize("seed", _cases("attn", 16))
def test_random_attention(q, seed):
    r = np.random.default_rng(seed)
    B, S = int(r.integers(1, 3)), int(r.integers(1, 1100))
    Hkv = int(r.choice([1, 2, 4, 8]))
    Hq = Hkv * int(r.choice([1, 2, 4]))
    causal, dt = bool(r.integers(0, 2)), int(r.choice([1, 2]))
    qa, ka, va = synth.attention_inputs(B, S, Hq, Hkv, 128, dt, seed)
    o = q.attn_prefill(act_tensor(qa), act_tensor(ka), act_tensor(va), causal=causal)
    torch.cuda.synchronize()
    got = values(o)
    ref, bound = oracle.attention(qa.values, ka.values, va.values, causal=causal)
    tol = 2.0 ** -7 * bound + 2.0 ** -8 * np.abs(ref) + 1e-5   # the attention tests' acceptance rule
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got)) and np.all(err <= tol), \
        f"attn B{B} S{S} Hq{Hq} Hkv{Hkv} causal{causal} dt{dt}: err/tol {(err / tol).max():.3g}"

