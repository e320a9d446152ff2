"""The products under HIP graph capture: each call is captured once into a
graph, the graph is replayed several times with other eager work and
synchronisations between replays, and every replay must equal the eager
result bit for bit (the library enqueues no memset or allocation, so a
captured call is the same kernels on the same buffers)."""
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


def _replays_match(fn, outs, eager_noise, replays=4):
    """fn() enqueues the call writing into outs; compare replays to eager."""
    fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()                                   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    for i in range(replays):
        for o in outs:
            o.fill_(float("nan") if o.is_floating_point() else -1)
        eager_noise(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r), f"replay {i} differs from the eager result"


def _noise(q):
    """Unrelated eager GEMV launches between replays."""
    w = synth.q_weight(synth.rng_for(70, 0), synth.Q4_0, 256, 1024)
    W = q.repack(synth.Q4_0, bytes_tensor(w.canon), 256, 1024)
    x = act_tensor(synth.activation(synth.rng_for(70, 1), (3, 1024), synth.F16))

    def run(i):
        for _ in range(i + 1):
            q.qgemv(synth.Q4_0, W, 256, 1024, x)
    return run


@pytest.mark.parametrize("M", [1, 8])
def test_graph_grouped_gemv(q, M):
    names = ["wq", "wk", "wv", "wo", "wg", "wu", "wd"]
    ws, xs = synth.layer_8b(M, mats=names)
    Wds = [q.repack(synth.Q4_0, bytes_tensor(ws[n].canon), ws[n].N, ws[n].K) for n in names]
    xt = {k: act_tensor(v) for k, v in xs.items()}
    ys = [torch.empty((M, ws[n].N), dtype=torch.float32, device=dev()) for n in names]
    probs = [(W, ws[n].N, ws[n].K, xt[synth.LAYER_8B_INPUT[n]], y) for W, n, y in zip(Wds, names, ys)]
    _replays_match(lambda: q.qgemv_grouped(synth.Q4_0, probs, M), ys, _noise(q))


@pytest.mark.parametrize("fmt", [synth.Q4_0, synth.Q8_0])
def test_graph_ffn_decode(q, fmt):
    M, H, F = 3, 1024, 2048
    wg, wu, wd = (synth.q_weight(synth.rng_for(71, i), fmt, n, k) for i, (n, k) in enumerate([(F, H), (F, H), (H, F)]))
    Wg, Wu, Wd = (q.repack(fmt, bytes_tensor(w.canon), w.N, w.K) for w in (wg, wu, wd))
    x = act_tensor(synth.activation(synth.rng_for(71, 9), (M, H), synth.BF16))
    y = torch.empty((M, H), dtype=torch.float32, device=dev())
    ws = torch.empty(q.ffn_decode_workspace(M, F), dtype=torch.uint8, device=dev())
    _replays_match(lambda: q.ffn_decode(fmt, Wg, Wu, Wd, H, F, x, out=y, ws=ws), [y], _noise(q))


@pytest.mark.parametrize("T", [4, 40])
def test_graph_moe(q, T):
    """Routing and the expert products in one graph: the decode path (T = 4)
    and the matrix-core path (T = 40)."""
    E, k, H, F = 16, 4, 256, 384
    logits = torch.from_numpy(synth.router_logits(synth.rng_for(72, T), T, E)).to(dev())
    mk = lambda i, n, kk: synth.q_weight(synth.rng_for(73, i), synth.Q4_0, n, kk)
    Wg = torch.cat([q.repack(synth.Q4_0, bytes_tensor(mk(e, F, H).canon), F, H) for e in range(E)])
    Wu = torch.cat([q.repack(synth.Q4_0, bytes_tensor(mk(100 + e, F, H).canon), F, H) for e in range(E)])
    Wd = torch.cat([q.repack(synth.Q4_0, bytes_tensor(mk(200 + e, H, F).canon), H, F) for e in range(E)])
    X = act_tensor(synth.activation(synth.rng_for(74, T), (T, H), synth.BF16))
    route = (torch.empty((T, k), dtype=torch.int32, device=dev()), torch.empty((T, k), dtype=torch.float32, device=dev()),
             torch.empty(E, dtype=torch.int32, device=dev()), torch.empty(E + 1, dtype=torch.int32, device=dev()),
             torch.empty(T * k, dtype=torch.int32, device=dev()))
    out = torch.empty((T, H), dtype=torch.float32, device=dev())
    ws = torch.empty(q.moe_workspace(synth.Q4_0, T, E, k, H, F), dtype=torch.uint8, device=dev())

    def step():
        ids, gates, counts, offsets, sp = q.moe_route(logits, k, out=route)
        q.moe_qgemm(synth.Q4_0, Wg, Wu, Wd, E, H, F, X, k, gates, offsets, sp, out=out, ws=ws)
    _replays_match(step, [out, *route], _noise(q))


@pytest.mark.parametrize("T", [2, 7])
def test_graph_moe_decode_one_call(q, T):
    """The one-call decode entry point (routing inside the first kernel),
    with the fused down + combine (T = 2) and the separate combine (T = 7)."""
    E, k, H, F = 16, 4, 256, 384
    logits = torch.from_numpy(synth.router_logits(synth.rng_for(76, T), T, E)).to(dev())
    mk = lambda i, n, kk: synth.q_weight(synth.rng_for(77, i), synth.Q4_0, n, kk)
    Wg = torch.cat([q.repack(synth.Q4_0, bytes_tensor(mk(e, F, H).canon), F, H) for e in range(E)])
    Wu = torch.cat([q.repack(synth.Q4_0, bytes_tensor(mk(100 + e, F, H).canon), F, H) for e in range(E)])
    Wd = torch.cat([q.repack(synth.Q4_0, bytes_tensor(mk(200 + e, H, F).canon), H, F) for e in range(E)])
    X = act_tensor(synth.activation(synth.rng_for(78, T), (T, H), synth.BF16))
    route = (torch.empty((T, k), dtype=torch.int32, device=dev()), torch.empty((T, k), dtype=torch.float32, device=dev()),
             torch.empty(E, dtype=torch.int32, device=dev()), torch.empty(E + 1, dtype=torch.int32, device=dev()),
             torch.empty(T * k, dtype=torch.int32, device=dev()))
    out = torch.empty((T, H), dtype=torch.float32, device=dev())
    ws = torch.empty(q.moe_workspace(synth.Q4_0, T, E, k, H, F), dtype=torch.uint8, device=dev())
    _replays_match(lambda: q.moe_decode(synth.Q4_0, Wg, Wu, Wd, E, H, F, logits, X, k, route=route, out=out, ws=ws),
                   [out, *route], _noise(q))


def test_graph_prefill_gemm(q):
    """The bf16 pre-pass and the GEMM in one graph."""
    M, N, K = 200, 640, 1024
    w = synth.q_weight(synth.rng_for(75, 0), synth.Q4_0, N, K)
    W = q.repack(synth.Q4_0, bytes_tensor(w.canon), N, K)
    X = act_tensor(synth.activation(synth.rng_for(75, 1), (M, K), synth.BF16))
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev())
    ws = torch.empty(q.qgemm_workspace(synth.BF16, M, K), dtype=torch.uint8, device=dev())
    _replays_match(lambda: q.qgemm(synth.Q4_0, W, N, K, X, out=Y, ws=ws), [Y], _noise(q))
