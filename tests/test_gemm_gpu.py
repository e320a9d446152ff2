"""GPU parity of the prefill GEMM against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from util import act_tensor, bytes_tensor, check, check_rounded, dev, values

pytestmark = pytest.mark.gpu

OUT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}


@pytest.fixture(scope="module")
def q():
    import gemm_q4_q8_amd as q
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    q.lib()
    return q


def _compare(got, ref, bound, ydt, what):
    if ydt == "f32":
        return check(got, ref, bound, what)
    return check_rounded(got, ref, bound, what, dtype=ydt)


SMALL = [(1, 16, 128), (17, 48, 160), (64, 256, 256), (100, 200, 1056), (128, 192, 4096),
         (300, 400, 512), (257, 1000, 384), (129, 64, 32), (300, 1536, 256), (70, 3072, 160), (70, 100, 352)]


@pytest.mark.parametrize("fmt,xdt,ydt", [(synth.Q4_0, synth.BF16, "bf16"), (synth.Q4_0, synth.F16, "f32"),
                                         (synth.Q8_0, synth.BF16, "bf16"), (synth.Q8_0, synth.F16, "f16"),
                                         (synth.FP16, synth.BF16, "bf16"), (synth.FP16, synth.F16, "f32")])
@pytest.mark.parametrize("M,N,K", SMALL)
def test_qgemm_parity_small(q, fmt, xdt, ydt, M, N, K):
    w = synth.weight(synth.rng_for(61, M + N + K + fmt), fmt, N, K)
    x = synth.activation(synth.rng_for(62, M * 3 + K + xdt), (M, K), xdt)
    Wd = q.repack(fmt, bytes_tensor(w.canon), N, K)
    y = q.qgemm(fmt, Wd, N, K, act_tensor(x), out_dtype=OUT[ydt])
    torch.cuda.synchronize()
    ref, bound = oracle.qgemm(fmt, w.canon, N, K, x.values)
    _compare(values(y), ref, bound, ydt, f"gemm fmt{fmt} M{M} N{N} K{K} {ydt}")


def test_qgemm_strided_and_deterministic(q):
    M, N, K = 70, 96, 256
    w = synth.q_weight(synth.rng_for(63, 0), synth.Q4_0, N, K)
    x = synth.activation(synth.rng_for(63, 1), (M, K), synth.BF16)
    X = torch.zeros((M, K + 24), dtype=torch.bfloat16, device=dev())
    X[:, :K] = act_tensor(x)
    Y = torch.full((M, N + 8), 3.0, dtype=torch.float32, device=dev())
    Wd = q.repack(synth.Q4_0, bytes_tensor(w.canon), N, K)
    L = q.lib()
    nws = q.qgemm_workspace(2, M, K)
    ws = torch.empty(nws, dtype=torch.uint8, device=dev())
    for _ in range(2):
        st = L.q4q8_qgemm(1, q._ptr(Wd), N, K, q._ptr(X), 2, K + 24, M, q._ptr(Y), 3, N + 8, q._ptr(ws), nws,
                          q._stream(X))
        assert st == 0, q.last_error()
        first = Y.clone() if _ == 0 else first
    torch.cuda.synchronize()
    assert torch.equal(first, Y)
    ref, bound = oracle.qgemm(synth.Q4_0, w.canon, N, K, x.values)
    yh = Y.cpu().numpy()
    check(yh[:, :N], ref, bound)
    assert np.all(yh[:, N:] == 3.0)


def test_qgemm_zero_weights(q):
    N, K, M = 64, 512, 40
    scales = np.full((N, K // 32), np.float16(0.02))
    codes = np.full((N, K), 8, dtype=np.uint8)
    w = synth.QWeight(synth.Q4_0, N, K, synth.pack_blocks(synth.Q4_0, scales, codes), scales, codes)
    x = synth.activation(synth.rng_for(64, 0), (M, K), synth.BF16)
    y = q.qgemm(synth.Q4_0, q.repack(1, bytes_tensor(w.canon), N, K), N, K, act_tensor(x), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.all(y.abs() <= 1e-5)


@pytest.mark.parametrize("fmt,M", [(synth.Q4_0, 128), (synth.Q4_0, 256), (synth.Q4_0, 512), (synth.Q4_0, 2048),
                                   (synth.Q8_0, 256), (synth.Q8_0, 512), (synth.FP16, 512)])
def test_qgemm_prefill_full_size_sampled(q, fmt, M):
    """The prefill shapes (K 4096, N 12288; M 128 and 256 take the narrower
    tiles) in the benchmark's launch shape (Q8_0 and fp16 weights drawn as
    the benchmark draws them); 4096 sampled
    outputs plus every output of the first and last 16-row block against the
    oracle, and NaN/Inf-free everywhere."""
    w, x = synth.prefill(M)
    if fmt != synth.Q4_0:
        w = synth.weight(synth.rng_for(synth.PREFILL["seed"], 50), fmt, w.N, w.K)
    N, K = w.N, w.K
    Wd = q.repack(fmt, bytes_tensor(w.canon), N, K)
    y = q.qgemm(fmt, Wd, N, K, act_tensor(x), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    yv = values(y)
    assert np.all(np.isfinite(yv))
    rng = np.random.default_rng(65 + M)
    rows = np.concatenate([rng.integers(0, M, 4096), np.zeros(64, int), np.full(64, M - 1)])
    cols = np.concatenate([rng.integers(0, N, 4096), np.arange(64), N - 1 - np.arange(64)])
    ref, bound = oracle.qgemm_rows(fmt, w.canon, N, K, x.values, rows, cols)
    check_rounded(yv[rows, cols], ref, bound, f"prefill fmt{fmt} M{M} sampled")
    for r0 in (0, M - 16):
        ref, bound = oracle.qgemm(fmt, w.canon, N, K, x.values[r0:r0 + 16])
        check_rounded(yv[r0:r0 + 16], ref, bound, f"prefill fmt{fmt} M{M} rows {r0}..")


@pytest.mark.parametrize("fmt", [synth.Q4_0, synth.Q8_0, synth.FP16])
def test_qgemm_activation_range(q, fmt):
    """BF16 rows far outside the fp16 range (scaled by 2^20, 2^60, 2^-20,
    2^-60), a zero row, a row with one large outlier and rows spanning 40
    binades: each row is scaled by a power of two before its fp16 conversion,
    so every output keeps the tolerance relative to its own row's scale."""
    M, N, K = 80, 200, 352
    w = synth.weight(synth.rng_for(66, fmt), fmt, N, K)
    base = synth.activation(synth.rng_for(66, 10), (M, K), synth.BF16).values
    row_scale = np.ones(M)
    row_scale[0:10] = 2.0 ** 20
    row_scale[10:20] = 2.0 ** -20
    row_scale[20:25] = 2.0 ** 60
    row_scale[25:30] = 2.0 ** -60
    xv = base * row_scale[:, None]
    xv[30] = 0.0
    xv[31, 7] = 3.0e5                                   # one outlier, the rest N(0, 1)
    span = synth.rng_for(66, 11).uniform(-30, 10, size=(8, K))
    xv[32:40] = np.sign(base[32:40]) * 2.0 ** span      # magnitudes 2^-30 .. 2^10 within a row
    x = synth.act_from_values(xv, synth.BF16)
    Wd = q.repack(fmt, bytes_tensor(w.canon), N, K)
    ref, bound = oracle.qgemm(fmt, w.canon, N, K, x.values)
    y = q.qgemm(fmt, Wd, N, K, act_tensor(x), out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = values(y)
    assert np.all(np.isfinite(got))
    tol = 2e-3 * bound + 1e-5 * row_scale[:, None]
    err = np.abs(got - ref)
    assert np.all(err <= tol), f"max err/tol {(err / tol).max():.3g} at row {np.unravel_index(np.argmax(err / tol), err.shape)}"
    assert np.all(got[30] == 0.0)
    yb = q.qgemm(fmt, Wd, N, K, act_tensor(x), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    check_rounded(values(yb)[:20], ref[:20], bound[:20], "bf16 out, rows scaled by 2^20 / 2^-20 (abs term 1e-5)")
