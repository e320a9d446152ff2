"""The no-allocation MoE decode entry point (q4q8_moe_decode_noalloc, its
scratch a static per-GPU device array) against q4q8_moe_decode with a
caller workspace: same bits for every output, called through the C ABI,
twice in a row with the second call smaller (the scratch keeps the first
call's contents), plus the rejection of sizes beyond the scratch."""
import ctypes

import numpy as np
import pytest
import torch

import synth
from util import act_tensor, bytes_tensor, dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import gemm_q4_q8_amd as q
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    q.lib()
    return q


def _stack(q, fmt, ws, n, k):
    return torch.cat([q.repack(fmt, bytes_tensor(w.canon), n, k) for w in ws])


def _call(q, fmt, W, E, H, F, logits, x, k, noalloc):
    """One call through the C ABI; returns every output (routing, out, h)."""
    L = q.lib()
    T = logits.shape[0]
    lg = torch.from_numpy(logits).to(dev())
    X = act_tensor(x)
    ids = torch.full((T, k), -7, dtype=torch.int32, device=dev())
    gates = torch.full((T, k), -7.0, device=dev())
    counts = torch.full((E,), -7, dtype=torch.int32, device=dev())
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device=dev())
    sp = torch.full((T * k,), -7, dtype=torch.int32, device=dev())
    out = torch.full((T, H), float("nan"), device=dev())
    h = torch.full((T * k, F), float("nan"), dtype=torch.bfloat16, device=dev())
    args = [fmt, q._ptr(W[0]), q._ptr(W[1]), q._ptr(W[2]), E, H, F, q._ptr(lg), q._ptr(X), x.dtype, T, k,
            q._ptr(ids), q._ptr(gates), q._ptr(counts), q._ptr(offsets), q._ptr(sp), q._ptr(out), q._ptr(h)]
    if noalloc:
        st = L.q4q8_moe_decode_noalloc(*args, q._stream(X))
    else:
        nws = q.moe_workspace(fmt, T, E, k, H, F)
        ws = torch.empty(nws, dtype=torch.uint8, device=dev())
        st = L.q4q8_moe_decode(*args, q._ptr(ws), nws, q._stream(X))
    assert st == 0, q.last_error()
    torch.cuda.synchronize()
    return [t.cpu() for t in (ids, gates, counts, offsets, sp, out, h)]


@pytest.mark.parametrize("fmt", [synth.Q4_0, synth.Q8_0])
def test_noalloc_equals_workspace_call(q, fmt):
    # First call: the MoE workload's expert shape at T = 8 (routing kernel
    # first, unfused down); second: a smaller layer at T = 2 (routing inside
    # the gate/up kernel, down fused with the combine).
    cases = [(8, 128, 8, 2048, 768, 140), (2, 24, 4, 512, 256, 141)]
    for T, E, k, H, F, seed in cases:
        wg = [synth.q_weight(synth.rng_for(seed, 1000 + e), fmt, F, H) for e in range(E)]
        wu = [synth.q_weight(synth.rng_for(seed, 2000 + e), fmt, F, H) for e in range(E)]
        wd = [synth.q_weight(synth.rng_for(seed, 3000 + e), fmt, H, F) for e in range(E)]
        W = (_stack(q, fmt, wg, F, H), _stack(q, fmt, wu, F, H), _stack(q, fmt, wd, H, F))
        logits = synth.router_logits(synth.rng_for(seed, 0), T, E)
        x = synth.activation(synth.rng_for(seed, 1), (T, H), synth.BF16)
        a = _call(q, fmt, W, E, H, F, logits, x, k, noalloc=True)
        b = _call(q, fmt, W, E, H, F, logits, x, k, noalloc=False)
        for name, u, v in zip(("ids", "gates", "counts", "offsets", "sorted_pairs", "out", "h"), a, b):
            assert torch.equal(u.view(torch.int16) if u.dtype == torch.bfloat16 else u,
                               v.view(torch.int16) if v.dtype == torch.bfloat16 else v), f"T{T}: {name} differs"
        assert torch.all(torch.isfinite(a[5]))


def test_noalloc_rejects_sizes_beyond_scratch(q):
    """T 8, top-16, H = F = 3200 is a valid decode call whose workspace
    (about 1.7 MB) exceeds the 1 MiB scratch: rejected before anything runs."""
    L = q.lib()
    assert L.q4q8_moe_decode_noalloc_max_scratch() == 1 << 20
    T, E, k, H, F = 8, 32, 16, 3200, 3200
    assert q.moe_workspace(synth.Q4_0, T, E, k, H, F) > 1 << 20
    p = ctypes.c_void_p(0x10000)
    st = L.q4q8_moe_decode_noalloc(synth.Q4_0, p, p, p, E, H, F, p, p, synth.BF16, T, k, p, p, p, p, p, p, None,
                                   None)
    assert st == -2 and "scratch" in q.last_error()
