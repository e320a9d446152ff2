"""GPU parity of the repack kernel and the decode GEMV against the CPU oracle."""
import numpy as np
import pytest
import torch

import oracle
import synth
from util import act_tensor, bytes_tensor, check, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import gemm_q4_q8_amd as q
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    q.lib()
    return q


def _run(q, w, x, out=None):
    Wd = q.repack(w.fmt, bytes_tensor(w.canon), w.N, w.K)
    y = q.qgemv(w.fmt, Wd, w.N, w.K, act_tensor(x), out=out)
    torch.cuda.synchronize()
    return y.cpu().numpy()


@pytest.mark.parametrize("fmt", [synth.Q4_0, synth.Q8_0, synth.FP16])
@pytest.mark.parametrize("N,K", [(16, 128), (17, 160), (1, 32), (300, 1056), (64, 4096)])
def test_repack_device_matches_host(q, fmt, N, K):
    w = synth.weight(synth.rng_for(51, N + K + fmt), fmt, N, K)
    dev_bytes = q.repack(fmt, bytes_tensor(w.canon), N, K)
    torch.cuda.synchronize()
    assert np.array_equal(dev_bytes.cpu().numpy(), q.repack_host(fmt, w.canon, N, K))


SHAPES = [(16, 128), (17, 160), (1, 32), (100, 32), (257, 1056), (64, 4096), (48, 12288)]


@pytest.mark.parametrize("fmt,xdt", [(synth.Q4_0, synth.F16), (synth.Q4_0, synth.BF16),
                                     (synth.Q8_0, synth.BF16), (synth.Q8_0, synth.F16),
                                     (synth.FP16, synth.F16), (synth.FP16, synth.BF16)])
@pytest.mark.parametrize("N,K", SHAPES)
def test_qgemv_parity_small(q, fmt, xdt, N, K):
    """Every M = 1..8 on shapes spanning tiles, ragged rows and a K tail."""
    w = synth.weight(synth.rng_for(52, N * 7 + K + fmt), fmt, N, K)
    Wd = q.repack(fmt, bytes_tensor(w.canon), N, K)
    for M in range(1, 9):
        x = synth.activation(synth.rng_for(53, 100 * M + K + xdt), (M, K), xdt)
        y = q.qgemv(fmt, Wd, N, K, act_tensor(x))
        torch.cuda.synchronize()
        ref, bound = oracle.qgemv(fmt, w.canon, N, K, x.values)
        check(y.cpu().numpy(), ref, bound, f"fmt{fmt} xdt{xdt} N{N} K{K} M{M}")


def test_qgemv_strided_rows(q):
    """ldx > K and ldy > N: only [0,M) x [0,N) is written."""
    N, K, M = 40, 256, 5
    w = synth.q_weight(synth.rng_for(54, 0), synth.Q4_0, N, K)
    x = synth.activation(synth.rng_for(54, 1), (M, K), synth.F16)
    big = torch.zeros((M, K + 64), dtype=torch.float16, device=dev())
    big[:, :K] = act_tensor(x)
    y = torch.full((M, N + 24), 7.0, dtype=torch.float32, device=dev())
    Wd = q.repack(synth.Q4_0, bytes_tensor(w.canon), N, K)
    st = q.lib().q4q8_qgemv(1, q._ptr(Wd), N, K, q._ptr(big), 1, K + 64, M, q._ptr(y), N + 24, q._stream(big))
    assert st == 0
    torch.cuda.synchronize()
    ref, bound = oracle.qgemv(synth.Q4_0, w.canon, N, K, x.values)
    yh = y.cpu().numpy()
    check(yh[:, :N], ref, bound)
    assert np.all(yh[:, N:] == 7.0)


def test_qgemv_zero_weights_give_exact_zero(q):
    """All Q4_0 codes 8 (and Q8_0 codes 0): y must be 0 within 1e-5 absolute."""
    for fmt, code in [(synth.Q4_0, 8), (synth.Q8_0, 0)]:
        N, K = 64, 4096
        scales = np.full((N, K // 32), np.float16(0.02))
        codes = np.full((N, K), code, dtype=np.uint8 if fmt == synth.Q4_0 else np.int8)
        w = synth.QWeight(fmt, N, K, synth.pack_blocks(fmt, scales, codes), scales, codes)
        for xdt in (synth.F16, synth.BF16):
            x = synth.activation(synth.rng_for(55, xdt), (8, K), xdt)
            y = _run(q, w, x)
            assert np.all(np.abs(y) <= 1e-5)


def test_qgemv_one_hot_is_exact(q):
    N, K = 48, 512
    w = synth.q_weight(synth.rng_for(56, 0), synth.Q4_0, N, K)
    W = oracle.dequant(synth.Q4_0, w.canon, N, K)
    cols = [0, 31, 32, 200, 511]
    xv = np.zeros((len(cols), K))
    for i, c in enumerate(cols):
        xv[i, c] = 1.0
    x = synth.act_from_values(xv, synth.F16)
    y = _run(q, w, x)
    assert np.array_equal(y, W[:, cols].T.astype(np.float32))


def test_qgemv_deterministic_and_grouped_equal(q):
    mats = [(4096, 4096), (1024, 4096), (1024, 4096)]
    ws = [synth.q_weight(synth.rng_for(57, i), synth.Q4_0, N, K) for i, (N, K) in enumerate(mats)]
    x = synth.activation(synth.rng_for(57, 9), (4, 4096), synth.F16)
    xt = act_tensor(x)
    Wds = [q.repack(synth.Q4_0, bytes_tensor(w.canon), w.N, w.K) for w in ws]
    single = [q.qgemv(synth.Q4_0, Wd, w.N, w.K, xt) for Wd, w in zip(Wds, ws)]
    again = [q.qgemv(synth.Q4_0, Wd, w.N, w.K, xt) for Wd, w in zip(Wds, ws)]
    ys = [torch.empty((4, w.N), dtype=torch.float32, device=dev()) for w in ws]
    q.qgemv_grouped(synth.Q4_0, [(Wd, w.N, w.K, xt, y) for Wd, w, y in zip(Wds, ws, ys)], 4)
    torch.cuda.synchronize()
    for a, b, c in zip(single, again, ys):
        assert torch.equal(a, b)
        assert torch.equal(a, c)


def _layer_check(q, M, names):
    ws, xs = synth.layer_8b(M, mats=names)
    worst = 0.0
    for name in names:
        w = ws[name]
        x = xs[synth.LAYER_8B_INPUT[name]]
        y = _run(q, w, x)
        ref, bound = oracle.qgemv(synth.Q4_0, w.canon, w.N, w.K, x.values)
        worst = max(worst, check(y, ref, bound, f"8B layer {name} M{M}"))
    return worst


@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_qgemv_layer_8b_full(q, M):
    """The 8B-shaped layer's seven projections at full size, every output."""
    _layer_check(q, M, ["wq", "wk", "wv", "wo", "wg", "wu", "wd"])


def test_qgemv_single_2048(q):
    w, x = synth.gemv_problem(synth.Q4_0, 2048, 2048, 1, synth.F16, synth.GEMV_2048["seed"])
    y = _run(q, w, x)
    ref, bound = oracle.qgemv(synth.Q4_0, w.canon, 2048, 2048, x.values)
    check(y, ref, bound, "gemv 2048")


@pytest.mark.parametrize("M", list(range(1, 9)))
def test_qgemv_q8_3b_full(q, M):
    ws, xs = synth.q8_3b(M)
    for name, w in ws.items():
        y = _run(q, w, xs[name])
        ref, bound = oracle.qgemv(synth.Q8_0, w.canon, w.N, w.K, xs[name].values)
        check(y, ref, bound, f"q8 3B {name} M{M}")


def _grouped_check(q, fmt, ws, xs, M, what):
    """One grouped launch over problems of different K, every output against
    the oracle (each problem takes its own K split inside the launch)."""
    Wds = [q.repack(fmt, bytes_tensor(w.canon), w.N, w.K) for w in ws]
    xts = [act_tensor(x) for x in xs]
    ys = [torch.full((M, w.N), float("nan"), dtype=torch.float32, device=dev()) for w in ws]
    q.qgemv_grouped(fmt, [(Wd, w.N, w.K, xt, y) for Wd, w, xt, y in zip(Wds, ws, xts, ys)], M)
    torch.cuda.synchronize()
    for w, x, y, i in zip(ws, xs, ys, range(len(ws))):
        ref, bound = oracle.qgemv(fmt, w.canon, w.N, w.K, x.values)
        check(y.cpu().numpy(), ref, bound, f"{what} problem {i}")


@pytest.mark.parametrize("M", [1, 3, 8])
def test_qgemv_grouped_mixed_k_ragged(q, M):
    shapes = [(200, 1056), (48, 160), (1000, 4096), (64, 12288), (17, 32)]
    ws = [synth.q_weight(synth.rng_for(58, i), synth.Q4_0, N, K) for i, (N, K) in enumerate(shapes)]
    xs = [synth.activation(synth.rng_for(58, 10 + i), (M, K), synth.F16) for i, (N, K) in enumerate(shapes)]
    _grouped_check(q, synth.Q4_0, ws, xs, M, f"mixed-K group M{M}")


@pytest.mark.parametrize("fmt,xdt,M", [(synth.Q4_0, synth.F16, 4), (synth.Q8_0, synth.BF16, 8),
                                        (synth.FP16, synth.BF16, 5), (synth.Q4_0, synth.BF16, 8)])
def test_qgemv_grouped_lds_and_global_x(q, fmt, xdt, M):
    """A launch where the shorter problems stage x in LDS and the longest
    (K = 26624: its M rows exceed the LDS) reads x from global memory."""
    shapes = [(100, 4096), (64, 26624), (33, 160), (300, 2080)]
    mk = (lambda i, N, K: synth.fp16_weight(synth.rng_for(61, i), N, K)) if fmt == synth.FP16 else \
        (lambda i, N, K: synth.q_weight(synth.rng_for(61, i), fmt, N, K))
    ws = [mk(i, N, K) for i, (N, K) in enumerate(shapes)]
    xs = [synth.activation(synth.rng_for(61, 10 + i), (M, K), xdt) for i, (N, K) in enumerate(shapes)]
    _grouped_check(q, fmt, ws, xs, M, f"LDS + global x group fmt{fmt} M{M}")


@pytest.mark.parametrize("fmt,xdt,M,N,K", [(synth.Q4_0, synth.F16, 8, 300, 26624), (synth.Q4_0, synth.BF16, 5, 77, 20000),
                                           (synth.Q8_0, synth.BF16, 8, 64, 12288), (synth.FP16, synth.F16, 8, 40, 12320)])
def test_qgemv_oversized_x(q, fmt, xdt, M, N, K):
    """One problem whose M activation rows exceed the LDS, so x is read from
    global memory (K not a multiple of 128 in two cases), every output."""
    w = synth.fp16_weight(synth.rng_for(62, 0), N, K) if fmt == synth.FP16 else \
        synth.q_weight(synth.rng_for(62, 0), fmt, N, K)
    x = synth.activation(synth.rng_for(62, 1), (M, K), xdt)
    _grouped_check(q, fmt, [w], [x], M, f"oversized x fmt{fmt} M{M} K{K}")


@pytest.mark.parametrize("M", [1, 2, 3, 5, 8])
def test_qgemv_layer_8b_one_launch(q, M):
    """The 8B-shaped layer's seven projections in one grouped launch (the
    benchmark's headline launch shape), every output."""
    names = ["wq", "wk", "wv", "wo", "wg", "wu", "wd"]
    ws, xs = synth.layer_8b(M, mats=names)
    _grouped_check(q, synth.Q4_0, [ws[n] for n in names], [xs[synth.LAYER_8B_INPUT[n]] for n in names], M,
                   f"8B layer one launch M{M}")


@pytest.mark.parametrize("M", [1, 2, 5, 8])
def test_qgemv_q8_3b_one_launch(q, M):
    ws, xs = synth.q8_3b(M)
    names = list(ws)
    _grouped_check(q, synth.Q8_0, [ws[n] for n in names], [xs[n] for n in names], M, f"q8 3B one launch M{M}")


@pytest.mark.parametrize("M", [1, 8])
def test_fp16_layer_8b_one_launch(q, M):
    """Plain fp16 weights of the 8B-shaped layer's seven projections in one
    grouped launch (bf16 activations meet fp16 weights as fp16 operands)."""
    names = [n for n, _, _ in synth.LAYER_8B["mats"]]
    shapes = {n: (N, K) for n, N, K in synth.LAYER_8B["mats"]}
    ws = [synth.fp16_weight(synth.rng_for(59, i), *shapes[n]) for i, n in enumerate(names)]
    _, xs = synth.layer_8b(M, mats=[])
    xb = {k: synth.act_from_values(v.values, synth.BF16) for k, v in xs.items()}
    _grouped_check(q, synth.FP16, ws, [xb[synth.LAYER_8B_INPUT[n]] for n in names], M, f"fp16 8B layer M{M}")
