"""GPU parity of prefill attention against the CPU oracle.

Acceptance per output: |o - o_ref| <= 2^-7 * sum_j p_j |v_j| + 2^-8 |o_ref| +
1e-5.  The probabilities enter the P.V product and the normalising sum
rounded to the operand type (relative 2^-9 for bf16, so O is a weighted mean
with weights off by at most that much each), and O itself is rounded once to
the storage type: both are covered with a margin; the fp32 scores' own
rounding is far below.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from util import act_tensor, dev, values

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import gemm_q4_q8_amd as q
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    q.lib()
    return q


def _check(got, ref, bound, what):
    tol = 2.0 ** -7 * bound + 2.0 ** -8 * np.abs(ref) + 1e-5
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    i = np.unravel_index(np.argmax(err / tol), err.shape)
    assert np.all(err <= tol), f"{what}: err/tol {(err / tol).max():.3g} at {i}: got {got[i]} ref {ref[i]}"


def _run(q, qa, ka, va, causal):
    o = q.attn_prefill(act_tensor(qa), act_tensor(ka), act_tensor(va), causal=causal)
    torch.cuda.synchronize()
    return values(o)


CASES = [
    # B, S, Hq, Hkv, causal, dtype
    (1, 128, 4, 4, True, synth.BF16),
    (2, 200, 8, 2, True, synth.BF16),      # ragged S, GQA 4:1
    (1, 77, 2, 1, False, synth.F16),
    (1, 1, 4, 2, True, synth.BF16),        # one token
    (1, 1000, 4, 1, False, synth.BF16),
    (3, 300, 6, 3, True, synth.F16),
    (1, 513, 8, 8, True, synth.BF16),      # one query past a block boundary
    (1, 64, 2, 2, True, synth.F16),        # a single key block
]


@pytest.mark.parametrize("B,S,Hq,Hkv,causal,dt", CASES)
def test_attn_parity(q, B, S, Hq, Hkv, causal, dt):
    qa, ka, va = synth.attention_inputs(B, S, Hq, Hkv, 128, dt, 150 + S + Hq)
    got = _run(q, qa, ka, va, causal)
    ref, bound = oracle.attention(qa.values, ka.values, va.values, causal=causal)
    _check(got, ref, bound, f"attn B{B} S{S} Hq{Hq} Hkv{Hkv} causal{causal} dt{dt}")


@pytest.mark.parametrize("B,S", [(8, 512), (8, 640)])
def test_attn_paired_query_blocks(q, B, S):
    """Causal with enough (batch, head) pairs that each workgroup takes query
    blocks i and last - i (640: an odd block count, the middle block alone);
    sampled query positions of every head."""
    Hq, Hkv = 32, 8
    qa, ka, va = synth.attention_inputs(B, S, Hq, Hkv, 128, synth.BF16, 165 + S)
    got = _run(q, qa, ka, va, True)
    rows = sorted({0, 1, 63, 64, 127, 128, 255, 256, 300, S - 129, S - 128, S - 2, S - 1})
    ref, bound = oracle.attention(qa.values, ka.values, va.values, causal=True, rows=rows)
    _check(got[:, rows], ref, bound, f"attn paired B{B} S{S}")


@pytest.mark.parametrize("B,S,Hq,Hkv,dt", [(4, 300, 32, 8, synth.BF16), (4, 520, 32, 4, synth.F16)])
def test_attn_key_split_full(q, B, S, Hq, Hkv, dt):
    """Causal grids large enough for the two-group form (each query block's
    key range split between two wave groups and merged): every output, ragged
    S (the last query block partly past S), paired blocks with a middle block
    alone (300: three 128-query blocks)."""
    qa, ka, va = synth.attention_inputs(B, S, Hq, Hkv, 128, dt, 170 + S)
    got = _run(q, qa, ka, va, True)
    ref, bound = oracle.attention(qa.values, ka.values, va.values, causal=True)
    _check(got, ref, bound, f"attn key split B{B} S{S} Hq{Hq} Hkv{Hkv} dt{dt}")


def test_attn_large_scores(q):
    """Scores far from 0 (inputs x 6): the running max must move often."""
    B, S, Hq, Hkv = 1, 384, 2, 1
    qa, ka, va = synth.attention_inputs(B, S, Hq, Hkv, 128, synth.BF16, 160)
    qa = synth.act_from_values(qa.values * 6.0, synth.BF16)
    got = _run(q, qa, ka, va, True)
    ref, bound = oracle.attention(qa.values, ka.values, va.values, causal=True)
    _check(got, ref, bound, "attn large scores")


def test_attn_full_shape_sampled(q):
    """The attention workload (S 2048, Hq 32, Hkv 8, D 128, causal, bf16):
    every head at sampled query positions incl. block edges; deterministic."""
    c = synth.ATTN
    qa, ka, va = synth.attention_inputs(c["B"], c["S"], c["Hq"], c["Hkv"], c["D"], c["dt"], c["seed"])
    qt, kt, vt = act_tensor(qa), act_tensor(ka), act_tensor(va)
    o1 = q.attn_prefill(qt, kt, vt, causal=True)
    o2 = q.attn_prefill(qt, kt, vt, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    rows = [0, 1, 15, 16, 63, 64, 127, 128, 129, 1000, 1023, 1024, 2046, 2047]
    rows += list(np.random.default_rng(161).choice(2048, 10, replace=False))
    rows = sorted(set(int(r) for r in rows))
    ref, bound = oracle.attention(qa.values, ka.values, va.values, causal=True, rows=rows)
    _check(values(o1)[:, rows], ref, bound, "attn full shape")
