"""GPU parity of the fused decode FFN against the CPU oracle.

q4q8_qgemv_swiglu: h = silu(x Wg^T) * (x Wu^T) in one launch, checked against
the oracle's h within the bound propagated from the per-dot-product tolerance
(plus the output type's rounding).  q4q8_ffn_decode: y = h Wd^T with h held as
bf16, within the bound propagated through the chain, and again against the
oracle fed the GPU's own h (read back from the workspace).  Also: q/k/v of a
layer as one grouped launch over a shared x.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from util import act_tensor, bytes_tensor, check, dev, values

pytestmark = pytest.mark.gpu

STORAGE_REL = {torch.bfloat16: 2.0 ** -8, torch.float16: 2.0 ** -11, torch.float32: 2.0 ** -24}


@pytest.fixture(scope="module")
def q():
    import gemm_q4_q8_amd as q
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    q.lib()
    return q


def _weights(fmt, H, F, seed, down=True):
    shapes = [(F, H), (F, H), (H, F)] if down else [(F, H), (F, H)]
    ws = [synth.weight(synth.rng_for(seed, i), fmt, n, k) for i, (n, k) in enumerate(shapes)]
    return ws if down else ws + [None]


def _up(q, w):
    return q.repack(w.fmt, bytes_tensor(w.canon), w.N, w.K)


def _check_h(got, r, hdt, what):
    hb = oracle.h_bound(r, storage_rel=STORAGE_REL[hdt])
    assert np.all(np.isfinite(got)), f"{what}: h not finite"
    err = np.abs(got - r["h"])
    assert np.all(err <= hb), f"{what}: h err/bound {(err / hb).max():.3g}"


SWIGLU_CASES = [
    # fmt, xdt, F, H
    (synth.Q4_0, synth.F16, 200, 1024),
    (synth.Q4_0, synth.BF16, 17, 160),
    (synth.Q8_0, synth.BF16, 300, 1536),
    (synth.Q8_0, synth.F16, 70, 4096),
    (synth.Q4_0, synth.BF16, 1, 32),
    (synth.Q4_0, synth.F16, 48, 12288),
    (synth.FP16, synth.BF16, 100, 640),
]


@pytest.mark.parametrize("fmt,xdt,F,H", SWIGLU_CASES)
@pytest.mark.parametrize("hdt", [torch.bfloat16, torch.float16, torch.float32])
def test_swiglu_parity(q, fmt, xdt, F, H, hdt):
    wg, wu, _ = _weights(fmt, H, F, 60 + F + H, down=False)
    Wg, Wu = _up(q, wg), _up(q, wu)
    for M in (1, 2, 5, 8):
        x = synth.activation(synth.rng_for(61, 10 * M + H), (M, H), xdt)
        h = q.qgemv_swiglu(fmt, Wg, Wu, F, H, act_tensor(x), out_dtype=hdt)
        torch.cuda.synchronize()
        r = oracle.ffn(fmt, wg.canon, wu.canon, None, x.values, H, F)
        _check_h(values(h), r, hdt, f"swiglu fmt{fmt} F{F} H{H} M{M} {hdt}")


def test_swiglu_strided_and_deterministic(q):
    """ldx > H and ldh > F; columns past F untouched; reruns bitwise equal."""
    F, H, M = 40, 256, 6
    wg, wu, _ = _weights(synth.Q4_0, H, F, 62, down=False)
    x = synth.activation(synth.rng_for(62, 9), (M, H), synth.BF16)
    big = torch.zeros((M, H + 32), dtype=torch.bfloat16, device=dev())
    big[:, :H] = act_tensor(x)
    h = torch.full((M, F + 24), 3.0, dtype=torch.float32, device=dev())
    Wg, Wu = _up(q, wg), _up(q, wu)
    q.qgemv_swiglu(synth.Q4_0, Wg, Wu, F, H, big[:, :H], out=h[:, :F])
    again = q.qgemv_swiglu(synth.Q4_0, Wg, Wu, F, H, big[:, :H], out_dtype=torch.float32)
    torch.cuda.synchronize()
    hh = h.cpu().numpy()
    assert np.all(hh[:, F:] == 3.0)
    assert np.array_equal(hh[:, :F], again.cpu().numpy())
    r = oracle.ffn(synth.Q4_0, wg.canon, wu.canon, None, x.values, H, F)
    _check_h(hh[:, :F].astype(np.float64), r, torch.float32, "strided swiglu")


def _ffn_run(q, fmt, wg, wu, wd, x, H, F):
    M = x.values.shape[0]
    ws = torch.empty(q.ffn_decode_workspace(M, F), dtype=torch.uint8, device=dev())
    y = q.ffn_decode(fmt, _up(q, wg), _up(q, wu), _up(q, wd), H, F, act_tensor(x), ws=ws)
    torch.cuda.synchronize()
    h16 = ws[:M * F * 2].view(torch.float16).view(M, F)
    # h is held as fp16 but carries bf16 roundings: every value survives a
    # round trip through bf16 unchanged.
    assert torch.equal(h16.to(torch.bfloat16).to(torch.float16), h16)
    h = values(h16)
    return y.cpu().numpy().astype(np.float64), h


def _ffn_check(fmt, wg, wu, wd, x, H, F, y, h, what):
    r = oracle.ffn(fmt, wg.canon, wu.canon, wd.canon, x.values, H, F)
    _check_h(h, r, torch.bfloat16, what)
    hb = oracle.h_bound(r)
    ob = oracle.ffn_out_bound(fmt, wd.canon, r, hb, H, F)
    err = np.abs(y - r["y"])
    assert np.all(err <= ob), f"{what}: y err/bound {(err / ob).max():.3g}"
    # Down projection on its own: the oracle takes the GPU's h.
    r2 = oracle.ffn(fmt, wg.canon, wu.canon, wd.canon, x.values, H, F, h_override=h)
    check(y, r2["y"], r2["by"], f"{what} (down on the GPU's h)")


FFN_CASES = [
    # fmt, xdt, H, F
    (synth.Q4_0, synth.F16, 256, 384),
    (synth.Q4_0, synth.BF16, 160, 96),
    (synth.Q8_0, synth.BF16, 512, 1056),
    (synth.Q8_0, synth.F16, 96, 32),
    (synth.FP16, synth.F16, 256, 384),
]


@pytest.mark.parametrize("fmt,xdt,H,F", FFN_CASES)
def test_ffn_decode_parity(q, fmt, xdt, H, F):
    wg, wu, wd = _weights(fmt, H, F, 63 + H + F)
    for M in range(1, 9):
        x = synth.activation(synth.rng_for(64, 10 * M + F), (M, H), xdt)
        y, h = _ffn_run(q, fmt, wg, wu, wd, x, H, F)
        _ffn_check(fmt, wg, wu, wd, x, H, F, y, h, f"ffn fmt{fmt} H{H} F{F} M{M}")


@pytest.mark.parametrize("M", [1, 8])
def test_ffn_decode_layer_8b(q, M):
    """The 8B-shaped layer's FFN (H 4096, F 12288, Q4_0) as the benchmark
    runs it, every output."""
    ws, xs = synth.layer_8b(M, mats=["wg", "wu", "wd"])
    H, F = 4096, 12288
    x = xs[synth.LAYER_8B_INPUT["wg"]]
    y, h = _ffn_run(q, synth.Q4_0, ws["wg"], ws["wu"], ws["wd"], x, H, F)
    _ffn_check(synth.Q4_0, ws["wg"], ws["wu"], ws["wd"], x, H, F, y, h, f"8B ffn M{M}")


@pytest.mark.parametrize("M", [1, 4, 8])
def test_qkv_grouped_shared_x(q, M):
    """q, k and v of the 8B-shaped layer in one grouped launch reading one x."""
    names = ["wq", "wk", "wv"]
    ws, xs = synth.layer_8b(M, mats=names)
    x = xs["x_attn"]
    xt = act_tensor(x)
    Wds = [_up(q, ws[n]) for n in names]
    ys = [torch.full((M, ws[n].N), float("nan"), dtype=torch.float32, device=dev()) for n in names]
    q.qgemv_grouped(synth.Q4_0, [(W, ws[n].N, ws[n].K, xt, y) for W, n, y in zip(Wds, names, ys)], M)
    torch.cuda.synchronize()
    for n, y in zip(names, ys):
        ref, bound = oracle.qgemv(synth.Q4_0, ws[n].canon, ws[n].N, ws[n].K, x.values)
        check(y.cpu().numpy(), ref, bound, f"qkv {n} M{M}")
