#!/usr/bin/env python3
"""Benchmark of the block-quantised weight products on one MI355X.

Headline workload (one "step"): the decode step of one 8B-shaped transformer
layer's projections over Q4_0 weights, M = 1 fp16 activation row: q/k/v
(4096x4096, 2x 1024x4096), o (4096x4096), gate and up (2x 12288x4096), down
(4096x12288).  The workload gives the seven products four independent
activation inputs (x_attn for q/k/v, x_o, x_ffn for gate/up, x_dn), so a
step computes them in one grouped launch, each matrix with its own split of
K so that every wave streams about the same number of chunks.  The same step
in the dependency order of a real layer (q/k/v, then o, then gate+up, then
down: four launches, since attention, norms and SwiGLU would sit between
them) is reported under "workloads".  Consecutive steps use different copies
of the layer's weights (8 copies, 868 MB, more than the 256 MB Infinity
Cache), as consecutive layers of a model would, so the weights stream from
HBM.  The K timed steps are one HIP graph of K launches, as a model's decode
graph holds one launch per layer.

value = algorithmic bytes of K steps / GPU time of K steps (GB/s), inputs
resident in HBM: events on the stream bracket exactly the K graph-replayed
steps, which are all queued (behind a bounded ~300 us spin kernel) before
the first one starts, with a synchronize on both sides.  Algorithmic bytes per step = repacked weight bytes (0.5625
B per weight, exactly the canonical Q4_0 bytes) + activations read (fp16) +
outputs written (fp32).

roofline: the dominant kernel is the step's single grouped launch (108.7 MB);
its duration comes from start/stop events recorded by its own dispatch
(hipExtLaunchKernel), averaged over R launches on rotating weight copies.
traffic: HBM bytes per launch from rocprofv3 FETCH_SIZE/WRITE_SIZE counters
(stored under profiles/ with the hash of the kernel sources they were taken
on; null if the sources changed since).

cpu_baseline: the fp64 NumPy oracle timed on the host on one decode step of
the same layer (all seven matrices, M = 1).

Other workloads (the dependency-order step at M = 1, one-launch steps at
M = 2/4/8, the single 2048x2048 GEMV, the Q8_0 3B-shaped matrices, the
layer with plain fp16 weights, the layer's fused decode FFN at M = 1 and 8,
the prefill GEMM at M = 512 and 2048 (Q8_0 at 512), the MoE layer at 512
tokens (Q4_0 and Q8_0) and its decode at 1 and 8 tokens,
prefill attention at S = 512 and 2048) are reported under "workloads", each
with its own algorithmic bytes / flops and time.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
F16_MFMA_PEAK_TFLOPS = 2500.0    # dense fp16/bf16 matrix-core peak
LAYER_COPIES = 8


def _kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in ("qgemv.hip", "gemv_core.h", "q4q8_dev.h", "q4q8_internal.h"):
        with open(os.path.join(ROOT, "gemm_q4_q8_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


class HipEvents:
    """hipEvent_t pairs from the HIP runtime torch already loaded."""

    def __init__(self):
        self.hip = ctypes.CDLL("libamdhip64.so.7")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventSynchronize.argtypes = [ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]

    def create(self):
        e = ctypes.c_void_p()
        if self.hip.hipEventCreate(ctypes.byref(e)) != 0:
            raise RuntimeError("hipEventCreate failed")
        return e.value

    def elapsed_ms(self, a, b) -> float:
        self.hip.hipEventSynchronize(ctypes.c_void_p(b))
        ms = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(a), ctypes.c_void_p(b)) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return float(ms.value)

    def destroy(self, e):
        self.hip.hipEventDestroy(ctypes.c_void_p(e))


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# After ~50 ms idle the GPU runs the headline step ~10 % slower for its first
# ~10 ms of load (measured on MI355X, 200-step windows: 22.1, 22.0, 20.6,
# 20.2, then 19.9 us a step).  Every timed measurement below is preceded by
# this much of its own work, untimed.
SETTLE_MS = 30.0


def settle(torch, fn, ms: float = SETTLE_MS) -> int:
    """Run fn(i) back to back, untimed, for at least `ms` milliseconds of wall
    time (synchronising after doubling batches); returns the calls made."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i, n = 0, 4
    while True:
        for _ in range(n):
            fn(i)
            i += 1
        torch.cuda.synchronize()
        if (time.perf_counter() - t0) * 1e3 >= ms:
            return i
        n *= 2


class ClockSampler:
    """Samples the GPU's current shader clock (SCLK, MHz) from the device's
    sysfs `pp_dpm_sclk` (the level marked `*`) on a background thread while a
    workload runs.  The device is found by its PCI bus id; where the file is
    missing or unreadable the summary is None."""

    def __init__(self, hip, period_s: float = 0.005):
        import threading
        self.path = None
        try:
            buf = ctypes.create_string_buffer(64)
            hip.hipDeviceGetPCIBusId.argtypes = [ctypes.c_char_p, ctypes.c_int, ctypes.c_int]
            if hip.hipDeviceGetPCIBusId(buf, 64, 0) == 0:
                p = f"/sys/bus/pci/devices/{buf.value.decode().lower()}/pp_dpm_sclk"
                open(p).read()
                self.path = p
        except (OSError, AttributeError, UnicodeDecodeError):
            self.path = None
        self.period = period_s
        self.samples = []
        self._stop = threading.Event()
        self._thread = threading.Thread(target=self._run, daemon=True)

    def _read(self):
        import re
        for line in open(self.path):
            if "*" in line:
                m = re.search(r"(\d+)\s*[Mm][Hh][Zz]", line)
                return int(m.group(1)) if m else None
        return None

    def _run(self):
        while not self._stop.is_set():
            try:
                v = self._read()
            except OSError:
                return
            if v is not None:
                self.samples.append(v)
            time.sleep(self.period)

    def __enter__(self):
        if self.path:
            self._thread.start()
        return self

    def __exit__(self, *exc):
        self._stop.set()
        if self.path:
            self._thread.join()

    def summary(self):
        if not self.samples:
            return None
        d = sorted(self.samples)
        return {"sclk_mhz_median": d[len(d) // 2], "sclk_mhz_min": d[0], "sclk_mhz_max": d[-1],
                "samples": len(d)}


def stream_ceiling(q, torch, ev: HipEvents, launch_bytes: int):
    """Measured HBM ceiling on this machine.  Read: the library's read probe
    (q4q8_stream_read_timed: 16-byte non-temporal loads, the GEMV's policy)
    over 4 GiB, bytes / dispatch-event time.  Copy (context): a 1 GiB device
    copy, bytes read + written / time.  Both far larger than the 256 MB
    Infinity Cache; best and median of 10 repetitions after 2 warm-ups.
    Read at the launch's size: the same probe over launch_bytes, eight
    buffers in turn (870 MB, past the Infinity Cache), launched eagerly one
    after another as the headline's timed launches are, mean of 64, on the
    best of four grids (2048 .. 16384 workgroups): what one plain read of
    that many bytes costs, ramp and tail included."""
    out = {}
    n = launch_bytes // 16 * 16
    bufs = [torch.empty(n, dtype=torch.uint8, device="cuda:0") for _ in range(8)]
    digest = None
    best = None
    for wgs in (2048, 4096, 8192, 16384):
        pairs = [(ev.create(), ev.create()) for _ in range(72)]
        for i, e in enumerate(pairs):
            digest = q.stream_read(bufs[i % 8], digest=digest, events=e, workgroups=wgs)
        ts = [ev.elapsed_ms(*e) * 1e-3 for e in pairs[8:]]
        for e in pairs:
            ev.destroy(e[0])
            ev.destroy(e[1])
        mean = sum(ts) / len(ts)
        if best is None or mean < best[0]:
            best = (mean, wgs)
    out["read_launch_bytes"] = n
    out["read_launch_us_mean"] = round(best[0] * 1e6, 3)
    out["read_launch_GB/s"] = round(n / best[0] / 1e9, 1)
    out["read_launch_workgroups"] = best[1]
    del bufs, digest
    buf = torch.empty(1 << 32, dtype=torch.uint8, device="cuda:0")
    digest = None
    ts = []
    for i in range(12):
        e = (ev.create(), ev.create())
        digest = q.stream_read(buf, digest=digest, events=e)
        if i >= 2:
            ts.append(ev.elapsed_ms(*e) * 1e-3)
        ev.destroy(e[0])
        ev.destroy(e[1])
    ts.sort()
    out["read_GB/s"] = round(buf.numel() / ts[0] / 1e9, 1)
    out["read_GB/s_median"] = round(buf.numel() / ts[len(ts) // 2] / 1e9, 1)
    del buf, digest
    b = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0")
    c = torch.empty_like(b)
    ts = []
    for i in range(12):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        c.copy_(b)
        e1.record()
        torch.cuda.synchronize()
        if i >= 2:
            ts.append(e0.elapsed_time(e1) * 1e-3)
    ts.sort()
    out["copy_GB/s"] = round(2 * b.numel() / ts[0] / 1e9, 1)
    del b, c
    torch.cuda.empty_cache()
    out["how"] = ("read: q4q8_stream_read_timed over 4 GiB (non-temporal 16-byte loads), "
                  "bytes / dispatch-event time, best of 10; read_launch: the same probe over the headline "
                  "launch's bytes, 8 buffers in turn, mean of 64 eager launches, best of 4 grids; copy: torch copy_ of 1 GiB, "
                  "(read + written) bytes / time, best of 10")
    return out


# ----------------------------------------------------------------------------
# Decode layer (8B-shaped), the headline workload
# ----------------------------------------------------------------------------
class DecodeLayer:
    CHAIN = [("qkv", ["wq", "wk", "wv"]), ("o", ["wo"]), ("gate_up", ["wg", "wu"]), ("down", ["wd"])]
    ONE = [("all", ["wq", "wk", "wv", "wo", "wg", "wu", "wd"])]

    def __init__(self, q, torch, synth, M: int, copies: int):
        self.q, self.torch, self.M = q, torch, M
        dev = torch.device("cuda:0")
        ws, xs = synth.layer_8b(M)
        self.shapes = {n: (w.N, w.K) for n, w in ws.items()}
        self.input_of = dict(synth.LAYER_8B_INPUT)
        base = {}
        for n, w in ws.items():
            canon = torch.from_numpy(w.canon).to(dev)
            base[n] = q.repack(w.fmt, canon, w.N, w.K)
            del canon
        self.copies = [base] + [{n: t.clone() for n, t in base.items()} for _ in range(copies - 1)]
        self.x = {}
        for xn, a in xs.items():
            t = torch.from_numpy(a.bits.view("int16")).view(torch.float16).to(dev)
            self.x[xn] = t
        self.y = {n: torch.empty((M, N), dtype=torch.float32, device=dev) for n, (N, K) in self.shapes.items()}
        self.descs = {}
        for mode, groups in (("one", self.ONE), ("chain", self.CHAIN)):
            per_copy = []
            for c in self.copies:
                per = []
                for g, names in groups:
                    probs = [(c[n], self.shapes[n][0], self.shapes[n][1], self.x[synth.LAYER_8B_INPUT[n]],
                              self.y[n]) for n in names]
                    per.append((g, probs, q.gemv_descs(probs)))
                per_copy.append(per)
            self.descs[mode] = per_copy
        self.mode = "one"
        torch.cuda.synchronize()

    def bytes_of(self, names) -> int:
        """Algorithmic bytes of one launch over `names`: weights + outputs + each
        distinct activation row block once."""
        M = self.M
        total = sum(self.q.repacked_bytes(1, *self.shapes[n]) + M * self.shapes[n][0] * 4 for n in names)
        inputs = {self.input_of[n]: self.shapes[n][1] for n in names}
        return total + sum(M * K * 2 for K in inputs.values())

    def step_bytes(self) -> int:
        groups = self.ONE if self.mode == "one" else self.CHAIN
        return sum(self.bytes_of(names) for _, names in groups)

    def step(self, copy: int, timed_group=None, events=None):
        for g, probs, descs in self.descs[self.mode][copy]:
            ev = events if g == timed_group else None
            self.q.qgemv_grouped(1, probs, self.M, descs=descs, events=ev)


def _gate_cycles(torch, gate_us: float = 300.0) -> int:
    """Cycles of torch's bounded spin kernel (torch.cuda._sleep) that hold a
    stream for about gate_us microseconds, from one timed calibration run."""
    n = 1 << 20
    torch.cuda._sleep(n)                 # first launch loads the kernel
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    torch.cuda._sleep(n)
    e1.record()
    torch.cuda.synchronize()
    us = max(e0.elapsed_time(e1) * 1e3, 1.0)
    return max(1, min(int(n * gate_us / us), 1 << 28))


def time_graph_steps(torch, layer: DecodeLayer, steps: int, warmup: int):
    """Time `steps` decode steps replayed from one HIP graph.

    Returns (GPU seconds of the `steps` timed steps, host seconds around
    them).  The W warm-up steps and the K timed steps are each captured as
    one graph (consecutive steps on consecutive weight copies, as the layers
    of a model's decode graph), so the timed span holds one graph launch.
    That span sits between two events on the stream that runs it; before the
    first event the stream is held by a bounded spin kernel (~300 us) while
    the host submits the graph, so the host's launch latency stays outside
    it; the host clock around spin + steps is returned beside it.  Before the
    warm-up steps an 8-step graph is replayed, untimed, for SETTLE_MS."""
    L = len(layer.copies)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for c in range(L):               # eager warm-up on the capture stream
            layer.step(c)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()

    def capture(n, start):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                layer.step((start + i) % L)
        return g

    g_all = capture(L, 0)
    g_warm = capture(warmup, 0) if warmup > 0 else None
    g_timed = capture(steps, warmup % L)
    torch.cuda.synchronize()
    gate = _gate_cycles(torch)

    settle(torch, lambda i: g_all.replay())
    if g_warm is not None:
        g_warm.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    torch.cuda._sleep(gate)
    e0.record()
    g_timed.replay()
    e1.record()
    torch.cuda.synchronize()
    host = time.perf_counter() - t0
    del g_all, g_warm, g_timed
    return e0.elapsed_time(e1) * 1e-3, host


def time_dominant_kernel(q, layer: DecodeLayer, ev: HipEvents, reps: int, group: str):
    """Mean duration (s) of one launch group, from dispatch-recorded events."""
    pairs = [(ev.create(), ev.create()) for _ in range(reps)]
    L = len(layer.copies)
    n = settle(layer.torch, lambda i: layer.step(i % L))
    log(f"{group}: {n} untimed launches, then {reps} timed")
    for i in range(reps):
        layer.step(i % L, timed_group=group, events=pairs[i])
    durs = [ev.elapsed_ms(a, b) * 1e-3 for a, b in pairs]
    for a, b in pairs:
        ev.destroy(a)
        ev.destroy(b)
    return sum(durs) / len(durs), durs


def _profile_traffic(source_hash: str):
    path = os.path.join(ROOT, "profiles", "qgemv_layer_8b_m1_one_launch_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    if rec.get("kernel_source_hash") != source_hash:
        return None
    return rec.get("traffic_bytes_per_launch")


# ----------------------------------------------------------------------------
# CPU baseline: the oracle itself on one decode step of the layer
# ----------------------------------------------------------------------------
def cpu_baseline(synth, budget_s: float = 25.0):
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        blas_threads = 1
    ws, xs = synth.layer_8b(1)
    total_bytes = 0
    t0 = time.perf_counter()
    steps = 0
    while True:
        for n, w in ws.items():
            x = xs[synth.LAYER_8B_INPUT[n]]
            oracle.qgemv(w.fmt, w.canon, w.N, w.K, x.values)
            total_bytes += w.canon.size + 2 * w.K + 4 * w.N
        steps += 1
        if time.perf_counter() - t0 > budget_s / 2 or steps >= 24:
            break
    dt = time.perf_counter() - t0
    del np
    flops = steps * sum(2.0 * w.N * w.K for w in ws.values())
    return {"value": total_bytes / dt / 1e9, "unit": "GB/s", "cores": blas_threads, "kind": "oracle",
            "wall_s": round(dt, 2), "GFLOP/s": round(flops / dt / 1e9, 3), "cpu_count": os.cpu_count(),
            "sample": f"{steps} decode step(s) of the 8B-shaped layer at M=1 (7 matrices, "
                      f"{total_bytes // steps} algorithmic bytes each) through the fp64 NumPy oracle "
                      f"(dequantise then matmul), {dt:.1f} s; elementwise NumPy is single-threaded, "
                      f"BLAS used {blas_threads} thread(s)"}


# ----------------------------------------------------------------------------
# Other workloads
# ----------------------------------------------------------------------------
def _time_launches(torch, fn, reps: int, warmup: int = 3):
    settle(torch, fn)
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        fn(i)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e-3 / reps


EXTRA_GROUPS = ("layer", "gemv2048", "q8_3b", "fp16", "ffn", "prefill", "moe", "moe_decode", "attn")


def extra_workloads(q, torch, synth, ev: HipEvents, quick: bool, only=None):
    """Every other workload, or only the groups named in `only`."""
    def want(name):
        return only is None or name in only

    out = []
    dev = torch.device("cuda:0")
    # The M = 1 step in dependency order, and both forms at other M (graph replays as for the headline).
    for M in ([1] if quick else [1, 2, 4, 8]) if want("layer") else []:
        lay = DecodeLayer(q, torch, synth, M, LAYER_COPIES)
        for mode in (["chain"] if M == 1 else ["one", "chain"]):
            lay.mode = mode
            dt, _ = time_graph_steps(torch, lay, 2000, 200)   # settled step time, as for the headline
            rec = {"workload": f"8B layer decode step M={M}, " + (
                "one grouped launch" if mode == "one" else "dependency order (4 launches)"),
                "GB/s": round(lay.step_bytes() * 2000 / dt / 1e9, 1), "us_per_step": round(dt / 2000 * 1e6, 2)}
            if mode == "chain":
                mean_k, _ = time_dominant_kernel(q, lay, ev, 32, "gate_up")
                rec["gate_up_kernel_us"] = round(mean_k * 1e6, 2)
                rec["gate_up_kernel_GB/s"] = round(lay.bytes_of(["wg", "wu"]) / mean_k / 1e9, 1)
            out.append(rec)
        del lay
        torch.cuda.empty_cache()
    if want("gemv2048"):
        out.append(gemv2048_workload(q, torch, synth, ev))
    if want("q8_3b"):
        out += q8_3b_workloads(q, torch, synth, ev, quick)
    if want("fp16"):
        out.append(fp16_layer_workload(q, torch, synth, ev))
    if want("ffn"):
        out += ffn_workloads(q, torch, synth, ev, quick)
    if want("prefill"):
        out += prefill_workloads(q, torch, synth, ev, quick)
    if want("moe"):
        out += moe_workload(q, torch, synth)
        if not quick:
            out += moe_workload(q, torch, synth, fmt=2)
    if want("moe_decode"):
        out += moe_decode_workloads(q, torch, synth, quick)
    if want("attn"):
        out += attn_workloads(q, torch, synth, ev, quick)
    return out


def gemv2048_workload(q, torch, synth, ev: HipEvents):
    """Single 2048x2048 GEMV (latency-bound: 2.37 MB)."""
    dev = torch.device("cuda:0")
    w, x = synth.gemv_problem(1, 2048, 2048, 1, synth.F16, synth.GEMV_2048["seed"])
    W0 = q.repack(1, torch.from_numpy(w.canon).to(dev), 2048, 2048)
    Ws = [W0] + [W0.clone() for _ in range(127)]          # 302 MB: more than the Infinity Cache
    xt = torch.from_numpy(x.bits.view("int16")).view(torch.float16).to(dev)
    y = torch.empty((1, 2048), dtype=torch.float32, device=dev)
    probs = [[(Wi, 2048, 2048, xt, y)] for Wi in Ws]
    descs = [q.gemv_descs(p) for p in probs]
    pairs = [(ev.create(), ev.create()) for _ in range(64)]
    settle(torch, lambda i: q.qgemv_grouped(1, probs[i % 128], 1, descs=descs[i % 128]))
    for i in range(64):
        q.qgemv_grouped(1, probs[i], 1, descs=descs[i], events=pairs[i])
    kd = sum(ev.elapsed_ms(a, b) for a, b in pairs) / 64 * 1e-3
    nb = q.repacked_bytes(1, 2048, 2048) + 2048 * 2 + 2048 * 4
    b2b = _time_launches(torch, lambda i: q.qgemv_grouped(1, probs[i % 128], 1, descs=descs[i % 128]), 256)
    rec = {"workload": "q4_0 gemv 2048x2048 M=1", "kernel_us": round(kd * 1e6, 2),
           "kernel_GB/s": round(nb / kd / 1e9, 1), "back_to_back_us": round(b2b * 1e6, 2),
           "back_to_back_GB/s": round(nb / b2b / 1e9, 1)}
    del Ws, probs, descs
    torch.cuda.empty_cache()
    return rec


def q8_3b_workloads(q, torch, synth, ev: HipEvents, quick: bool):
    """Q8_0 3B-shaped matrices, M = 1 and 8: one launch each, and one grouped launch."""
    out = []
    dev = torch.device("cuda:0")
    for M in ([1, 8] if not quick else [1]):
        ws, xs = synth.q8_3b(M)
        tot_b, tot_t = 0, 0.0
        for name, w in ws.items():
            W0 = q.repack(2, torch.from_numpy(w.canon).to(dev), w.N, w.K)
            copies = [W0] + [W0.clone() for _ in range(max(1, 300_000_000 // W0.numel()))]
            xt = torch.from_numpy(xs[name].bits.view("int16")).view(torch.bfloat16).to(dev)
            yq = torch.empty((M, w.N), dtype=torch.float32, device=dev)
            probs = [[(c, w.N, w.K, xt, yq)] for c in copies]
            descs = [q.gemv_descs(p) for p in probs]
            pairs = [(ev.create(), ev.create()) for _ in range(32)]
            settle(torch, lambda i: q.qgemv_grouped(2, probs[i % len(probs)], M, descs=descs[i % len(probs)]))
            for i in range(32):
                q.qgemv_grouped(2, probs[i % len(probs)], M, descs=descs[i % len(probs)], events=pairs[i])
            kd = sum(ev.elapsed_ms(a, b) for a, b in pairs) / 32 * 1e-3
            tot_t += kd
            tot_b += q.repacked_bytes(2, w.N, w.K) + M * w.K * 2 + M * w.N * 4
            del copies, probs, descs
        torch.cuda.empty_cache()
        out.append({"workload": f"q8_0 3B-shape 4 matrices M={M}, one launch each", "sum_kernel_us": round(tot_t * 1e6, 2),
                    "GB/s": round(tot_b / tot_t / 1e9, 1)})
        # The four matrices in one grouped launch (independent inputs).
        names = list(ws)
        Ws = {n: q.repack(2, torch.from_numpy(ws[n].canon).to(dev), ws[n].N, ws[n].K) for n in names}
        copies = [Ws] + [{n: t.clone() for n, t in Ws.items()} for _ in range(4)]   # 334 MB
        xts = {n: torch.from_numpy(xs[n].bits.view("int16")).view(torch.bfloat16).to(dev) for n in names}
        yq = {n: torch.empty((M, ws[n].N), dtype=torch.float32, device=dev) for n in names}
        probs = [[(c[n], ws[n].N, ws[n].K, xts[n], yq[n]) for n in names] for c in copies]
        descs = [q.gemv_descs(p) for p in probs]
        pairs = [(ev.create(), ev.create()) for _ in range(32)]
        settle(torch, lambda i: q.qgemv_grouped(2, probs[i % 5], M, descs=descs[i % 5]))
        for i in range(32):
            q.qgemv_grouped(2, probs[i % 5], M, descs=descs[i % 5], events=pairs[i])
        kd = sum(ev.elapsed_ms(a, b) for a, b in pairs[4:]) / 28 * 1e-3
        out.append({"workload": f"q8_0 3B-shape 4 matrices M={M}, one grouped launch", "kernel_us": round(kd * 1e6, 2),
                    "GB/s": round(tot_b / kd / 1e9, 1)})
        del Ws, copies, probs, descs
        torch.cuda.empty_cache()
    return out


def attn_workloads(q, torch, synth, ev: HipEvents, quick: bool):
    """Prefill attention, 8B-shaped heads (Hq 32, Hkv 8, D 128), bf16: causal
    S = 512, 2048 and 4096, non-causal S = 2048.  Flops = 4 D Hq B x the
    visible (query, key) pairs (S (S + 1) / 2 causal, S^2 otherwise): QK^T and
    PV; time from dispatch events."""
    out = []
    dev = torch.device("cuda:0")
    c = synth.ATTN
    cases = [(2048, True)] if quick else [(512, True), (2048, True), (4096, True), (2048, False)]
    for S, causal in cases:
        qa, ka, va = synth.attention_inputs(c["B"], S, c["Hq"], c["Hkv"], c["D"], c["dt"], c["seed"])
        t = [torch.from_numpy(a.bits.view("int16")).view(torch.bfloat16).to(dev) for a in (qa, ka, va)]
        o = torch.empty_like(t[0])
        reps, warm = 200, 40   # back to back: the settled time
        pairs = [(ev.create(), ev.create()) for _ in range(reps + warm)]
        settle(torch, lambda i: q.attn_prefill(*t, causal=causal, out=o))
        for pr in pairs:
            q.attn_prefill(*t, causal=causal, out=o, events=pr)
        d = sorted(ev.elapsed_ms(a, b) * 1e-3 for a, b in pairs[warm:])
        for a, b in pairs:
            ev.destroy(a)
            ev.destroy(b)
        mean = sum(d) / len(d)
        fl = 4.0 * c["D"] * c["Hq"] * c["B"] * (S * (S + 1) / 2 if causal else S * S)
        kind = "causal" if causal else "non-causal"
        # The MFMA peak assumes 2.4 GHz: sample the clock over ~0.25 s of back-to-back calls.
        with ClockSampler(ev.hip) as clk:
            for _ in range(max(1, int(0.25 / max(mean, 1e-6)))):
                q.attn_prefill(*t, causal=causal, out=o)
            torch.cuda.synchronize()
        out.append({"workload": f"prefill attention S={S} Hq={c['Hq']} Hkv={c['Hkv']} D={c['D']} {kind} bf16",
                    "kernel_us_mean": round(mean * 1e6, 2), "kernel_us_median": round(d[len(d) // 2] * 1e6, 2),
                    "kernel_us_min": round(d[0] * 1e6, 2),
                    "TFLOP/s": round(fl / mean / 1e12, 1),
                    "mfma_frac": round(fl / mean / 1e12 / F16_MFMA_PEAK_TFLOPS, 4),
                    "sclk_during_calls": clk.summary()})
    return out


def fp16_layer_workload(q, torch, synth, ev: HipEvents):
    """Plain fp16 weights of the 8B-shaped layer (434 MB), M = 1 bf16
    activations, the seven projections in one grouped launch; two weight
    copies alternate (868 MB)."""
    dev = torch.device("cuda:0")
    mats = synth.LAYER_8B["mats"]
    base = [q.repack(synth.FP16, torch.from_numpy(synth.fp16_weight(synth.rng_for(59, i), N, K).canon).to(dev), N, K)
            for i, (n, N, K) in enumerate(mats)]
    copies = [base, [t.clone() for t in base]]
    xs = {K: torch.randn((1, K), device=dev).to(torch.bfloat16) for _, _, K in mats}
    ys = [torch.empty((1, N), dtype=torch.float32, device=dev) for _, N, _ in mats]
    probs = [[(c[i], N, K, xs[K], ys[i]) for i, (_, N, K) in enumerate(mats)] for c in copies]
    descs = [q.gemv_descs(p) for p in probs]
    pairs = [(ev.create(), ev.create()) for _ in range(36)]
    settle(torch, lambda i: q.qgemv_grouped(synth.FP16, probs[i % 2], 1, descs=descs[i % 2]))
    for i, pr in enumerate(pairs):
        q.qgemv_grouped(synth.FP16, probs[i % 2], 1, descs=descs[i % 2], events=pr)
    kd = sum(ev.elapsed_ms(a, b) for a, b in pairs[4:]) / 32 * 1e-3
    for a, b in pairs:
        ev.destroy(a)
        ev.destroy(b)
    nb = sum(q.repacked_bytes(synth.FP16, N, K) + N * 4 for _, N, K in mats) + 3 * 4096 * 2 + 12288 * 2
    del base, copies
    torch.cuda.empty_cache()
    return {"workload": "fp16 weights, 8B-shape layer 7 matrices M=1 (bf16 x), one grouped launch",
            "kernel_us": round(kd * 1e6, 2), "GB/s": round(nb / kd / 1e9, 1),
            "hbm_frac": round(nb / kd / 1e9 / HBM_PEAK_GBS, 4)}


def ffn_workloads(q, torch, synth, ev: HipEvents, quick: bool):
    """Decode FFN of the 8B-shaped layer (H 4096, F 12288, Q4_0): the fused
    gate/up SwiGLU GEMV (h as bf16, never zg/zu) then the down GEMV.
    Algorithmic bytes = the three matrices + x + h written and read back +
    y.  Timed as graph replays over 8 weight copies (step time) and with
    dispatch events around the two kernels of one call."""
    out = []
    dev = torch.device("cuda:0")
    H, F = 4096, 12288
    for M in ([1] if quick else [1, 8]):
        ws, xs = synth.layer_8b(M, mats=["wg", "wu", "wd"])
        base = {n: q.repack(1, torch.from_numpy(ws[n].canon).to(dev), ws[n].N, ws[n].K) for n in ws}
        copies = [base] + [{n: t.clone() for n, t in base.items()} for _ in range(LAYER_COPIES - 1)]
        x = torch.from_numpy(xs["x_ffn"].bits.view("int16")).view(torch.float16).to(dev)
        y = torch.empty((M, H), dtype=torch.float32, device=dev)
        h = torch.empty((M, F), dtype=torch.bfloat16, device=dev)
        wsp = torch.empty(q.ffn_decode_workspace(M, F), dtype=torch.uint8, device=dev)
        wbytes = 3 * q.repacked_bytes(1, F, H)
        nb = wbytes + M * H * 2 + 2 * M * F * 2 + M * H * 4
        nb_gu = 2 * q.repacked_bytes(1, F, H) + M * H * 2 + M * F * 2

        def step(i):
            c = copies[i % LAYER_COPIES]
            q.ffn_decode(1, c["wg"], c["wu"], c["wd"], H, F, x, out=y, ws=wsp)

        for i in range(LAYER_COPIES):
            step(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(LAYER_COPIES):
                step(i)
        settle(torch, lambda i: g.replay())
        for _ in range(25):
            g.replay()
        torch.cuda.synchronize()
        reps = 250   # 2000 steps: the settled step time
        t0 = time.perf_counter()
        for _ in range(reps):
            g.replay()
        torch.cuda.synchronize()
        dt = (time.perf_counter() - t0) / (reps * LAYER_COPIES)
        pairs = [(ev.create(), ev.create()) for _ in range(36)]
        settle(torch, lambda i: g.replay())
        for i, pr in enumerate(pairs):
            c = copies[i % LAYER_COPIES]
            q.ffn_decode(1, c["wg"], c["wu"], c["wd"], H, F, x, out=y, ws=wsp, events=pr)
        kd = sum(ev.elapsed_ms(a, b) for a, b in pairs[4:]) / 32 * 1e-3
        for i, pr in enumerate(pairs):
            c = copies[i % LAYER_COPIES]
            q.qgemv_swiglu(1, c["wg"], c["wu"], F, H, x, out=h, events=pr)
        kg = sum(ev.elapsed_ms(a, b) for a, b in pairs[4:]) / 32 * 1e-3
        for a, b in pairs:
            ev.destroy(a)
            ev.destroy(b)
        out.append({"workload": f"8B-shape decode FFN M={M}: fused gate/up SwiGLU GEMV + down GEMV (2 launches)",
                    "step_us": round(dt * 1e6, 2), "GB/s": round(nb / dt / 1e9, 1),
                    "call_kernels_us": round(kd * 1e6, 2), "call_kernels_GB/s": round(nb / kd / 1e9, 1),
                    "swiglu_kernel_us": round(kg * 1e6, 2), "swiglu_kernel_GB/s": round(nb_gu / kg / 1e9, 1)})
        del base, copies, g
        torch.cuda.empty_cache()
    return out


def prefill_workloads(q, torch, synth, ev: HipEvents, quick: bool):
    """Prefill GEMM Y[M, 12288] = X[M, 4096] W^T, Q4_0 at M = 128, 256, 512
    and 2048 (short and long prompts; Q8_0 and plain fp16 weights at
    M = 512), bf16 in and out.  The timed span of one call covers both of its kernels
    (bf16 -> fp16 pre-pass and the GEMM), from the first dispatch's start to
    the last one's end."""
    out = []
    dev = torch.device("cuda:0")
    for fmt, M in ([(1, 512)] if quick else [(1, 128), (1, 256), (1, 512), (1, 2048), (2, 512), (3, 512)]):
        w, x = synth.prefill(M)
        if fmt != 1:
            w = synth.weight(synth.rng_for(synth.PREFILL["seed"], 50), fmt, w.N, w.K)
        W0 = q.repack(fmt, torch.from_numpy(w.canon).to(dev), w.N, w.K)
        Ws = [W0] + [W0.clone() for _ in range(3)]
        X = torch.from_numpy(x.bits.view("int16")).view(torch.bfloat16).to(dev)
        Y = torch.empty((M, w.N), dtype=torch.bfloat16, device=dev)
        wsp = torch.empty(q.qgemm_workspace(synth.BF16, M, w.K), dtype=torch.uint8, device=dev)
        reps, warm = 200, 40   # back to back: the settled time
        pairs = [(ev.create(), ev.create()) for _ in range(reps + warm)]
        settle(torch, lambda i: q.qgemm(fmt, Ws[i % 4], w.N, w.K, X, out=Y, ws=wsp))
        for i in range(reps + warm):
            q.qgemm(fmt, Ws[i % 4], w.N, w.K, X, out=Y, ws=wsp, events=pairs[i])
        d = sorted(ev.elapsed_ms(a, b) * 1e-3 for a, b in pairs[warm:])
        for a, b in pairs:
            ev.destroy(a)
            ev.destroy(b)
        mean = sum(d) / len(d)
        fl = 2.0 * M * w.N * w.K
        # The MFMA peak assumes 2.4 GHz: sample the clock over ~0.25 s of back-to-back calls.
        with ClockSampler(ev.hip) as clk:
            n_sus = max(1, int(0.25 / max(mean, 1e-6)))
            for i in range(n_sus):
                q.qgemm(fmt, Ws[i % 4], w.N, w.K, X, out=Y, ws=wsp)
            torch.cuda.synchronize()
        out.append({"workload": f"{synth.FORMAT_NAME[fmt]} prefill gemm M={M} K={w.K} N={w.N} (bf16 in/out)",
                    "call_us_mean": round(mean * 1e6, 2), "call_us_median": round(d[len(d) // 2] * 1e6, 2),
                    "call_us_min": round(d[0] * 1e6, 2),
                    "TFLOP/s": round(fl / mean / 1e12, 1),
                    "mfma_frac": round(fl / mean / 1e12 / F16_MFMA_PEAK_TFLOPS, 4),
                    "sclk_during_calls": clk.summary()})
        del Ws, W0, X, Y, wsp
        torch.cuda.empty_cache()
    return out


def moe_workload(q, torch, synth, fmt: int = 1):
    """MoE layer: 512 bf16 tokens, 128 Q4_0 (or Q8_0) experts (gate/up
    768x2048, down 2048x768), top-8.  One step = route + sort + expert GEMMs
    + combine, timed with stream events (launch gaps included).  Expert
    weights are 340 MB at Q4_0 (642 MB at Q8_0), more than the Infinity
    Cache: the layer is HBM-bound, so the roofline is max(weight bytes /
    8 TB/s, flops / 2.5 PFLOP/s)."""
    dev = torch.device("cuda:0")
    cfg = synth.MOE
    T, E, k, H, F = cfg["T"], cfg["E"], cfg["topk"], cfg["H"], cfg["F"]
    logits, x, wg, wu, wd = synth.moe(fmt=fmt)

    def stack(ws, n, kk):
        return torch.cat([q.repack(fmt, torch.from_numpy(w.canon).to(dev), n, kk) for w in ws])

    Wg, Wu, Wd = stack(wg, F, H), stack(wu, F, H), stack(wd, H, F)
    L = torch.from_numpy(logits).to(dev)
    X = torch.from_numpy(x.bits.view("int16")).view(torch.bfloat16).to(dev)
    out = torch.empty((T, H), dtype=torch.float32, device=dev)
    wsp = torch.empty(q.moe_workspace(fmt, T, E, k, H, F), dtype=torch.uint8, device=dev)

    route = (torch.empty((T, k), dtype=torch.int32, device=dev), torch.empty((T, k), dtype=torch.float32, device=dev),
             torch.empty(E, dtype=torch.int32, device=dev), torch.empty(E + 1, dtype=torch.int32, device=dev),
             torch.empty(T * k, dtype=torch.int32, device=dev))

    def step_two(_):     # q4q8_moe_route, then q4q8_moe_qgemm
        ids, gates, counts, offsets, sp = q.moe_route(L, k, out=route)
        q.moe_qgemm(fmt, Wg, Wu, Wd, E, H, F, X, k, gates, offsets, sp, out=out, ws=wsp)

    def step_one(_):     # q4q8_moe_forward: the sort formed inside the gate+up kernel
        q.moe_forward(fmt, Wg, Wu, Wd, E, H, F, L, X, k, route=route, out=out, ws=wsp)

    fl = 2.0 * T * k * 3 * F * H
    wbytes = 3 * E * q.repacked_bytes(fmt, F, H)
    roof = max(wbytes / (HBM_PEAK_GBS * 1e9), fl / (F16_MFMA_PEAK_TFLOPS * 1e12))
    res = []
    for name, step in (("one call, moe_forward", step_one), ("moe_route + moe_qgemm", step_two)):
        dt = _time_launches(torch, step, 300, warmup=30)   # ~40 ms: the settled step time
        res.append({"workload": f"{synth.FORMAT_NAME[fmt]} moe T={T} E={E} top{k} H={H} F={F} (bf16 tokens; {name})",
                    "step_us": round(dt * 1e6, 2),
                    "TFLOP/s": round(fl / dt / 1e12, 1),
                    "mfma_frac": round(fl / dt / 1e12 / F16_MFMA_PEAK_TFLOPS, 4),
                    "weight_GB/s": round(wbytes / dt / 1e9, 1), "roofline_us": round(roof * 1e6, 2),
                    "roofline_frac": round(roof / dt, 4)})
    del Wg, Wu, Wd, wsp
    torch.cuda.empty_cache()
    return res


def moe_decode_workloads(q, torch, synth, quick: bool):
    """MoE decode: T = 1 and 8 tokens over the MoE layer's experts (E 128,
    top-8, H 2048, F 768, Q4_0).  One step = route + expert GEMVs (gate/up
    SwiGLU, down) + combine, captured in a HIP graph, in both forms: the
    routing call and the expert call, and the one-call entry point.  Steps cycle through 16
    token sets and two copies of the expert weights (680 MB, more than the
    Infinity Cache).  Algorithmic bytes = the distinct selected experts'
    three matrices + x + out."""
    out = []
    dev = torch.device("cuda:0")
    cfg = synth.MOE
    E, k, H, F = cfg["E"], cfg["topk"], cfg["H"], cfg["F"]
    _, _, wg, wu, wd = synth.moe(T=1)

    def stack(ws, n, kk):
        return torch.cat([q.repack(1, torch.from_numpy(w.canon).to(dev), n, kk) for w in ws])

    base = (stack(wg, F, H), stack(wu, F, H), stack(wd, H, F))
    copies = [base, tuple(t.clone() for t in base)]
    mat = q.repacked_bytes(1, F, H)
    for T in ([1] if quick else [1, 8]):
        sets = 16
        Ls = [torch.from_numpy(synth.router_logits(synth.rng_for(140, 100 * T + i), T, E)).to(dev)
              for i in range(sets)]
        X = torch.from_numpy(synth.activation(synth.rng_for(141, T), (T, H), synth.BF16).bits.view("int16")
                             ).view(torch.bfloat16).to(dev)
        o = torch.empty((T, H), dtype=torch.float32, device=dev)
        rt = (torch.empty((T, k), dtype=torch.int32, device=dev), torch.empty((T, k), dtype=torch.float32, device=dev),
              torch.empty(E, dtype=torch.int32, device=dev), torch.empty(E + 1, dtype=torch.int32, device=dev),
              torch.empty(T * k, dtype=torch.int32, device=dev))
        wsp = torch.empty(q.moe_workspace(1, T, E, k, H, F), dtype=torch.uint8, device=dev)

        def step_two(i):      # q4q8_moe_route, then q4q8_moe_qgemm
            Wg, Wu, Wd = copies[i % 2]
            ids, gates, counts, offsets, sp = q.moe_route(Ls[i % sets], k, out=rt)
            q.moe_qgemm(1, Wg, Wu, Wd, E, H, F, X, k, gates, offsets, sp, out=o, ws=wsp)

        def step_one(i):      # q4q8_moe_decode: routing inside the first expert kernel
            Wg, Wu, Wd = copies[i % 2]
            q.moe_decode(1, Wg, Wu, Wd, E, H, F, Ls[i % sets], X, k, route=rt, out=o, ws=wsp)

        nbytes = 0
        for i in range(sets):
            step_two(i)
            torch.cuda.synchronize()
            nbytes += int((rt[2] > 0).sum().item()) * 3 * mat + T * H * 2 + T * H * 4
        per = nbytes / sets
        for name, step in (("route + moe_qgemm: route, GEMV path, combine", step_two),
                           ("one call, moe_decode: routing inside the gate/up kernel up to 4 tokens", step_one)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(sets):
                    step(i)
            settle(torch, lambda i: g.replay())
            for _ in range(12):
                g.replay()
            torch.cuda.synchronize()
            reps = 125   # 2000 steps: the settled step time
            t0 = time.perf_counter()
            for _ in range(reps):
                g.replay()
            torch.cuda.synchronize()
            dt = (time.perf_counter() - t0) / (reps * sets)
            out.append({"workload": f"q4_0 moe decode T={T} E={E} top{k} H={H} F={F} ({name})",
                        "step_us": round(dt * 1e6, 2), "bytes_per_step": int(per), "GB/s": round(per / dt / 1e9, 1),
                        "hbm_frac": round(per / dt / 1e9 / HBM_PEAK_GBS, 4)})
            del g
    del base, copies
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    # 4000 steps after 400 warm-up ones take ~0.1 s of GPU time (the
    # driver's own runs use other K / W; every run first settles the GPU for
    # SETTLE_MS with untimed replays of the step).
    ap.add_argument("--steps", type=int, default=4000)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--kernel-reps", type=int, default=64)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--quick-extra", action="store_true")
    ap.add_argument("--only", nargs="+", choices=EXTRA_GROUPS, default=None,
                    help="run only these groups of the other workloads (e.g. for a profiled run)")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the measured HBM stream ceiling")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run a 256 MiB device copy (known HBM bytes) for counter calibration")
    args = ap.parse_args()

    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the quantised products are "
                          "single-device kernels; --gpus must be 1"}))
        sys.exit(2)

    import torch
    import gemm_q4_q8_amd as q
    import synth

    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)
    q.lib()
    ev = HipEvents()

    log("building the 8B-shaped layer (8 weight copies)...")
    layer = DecodeLayer(q, torch, synth, 1, LAYER_COPIES)
    step_bytes = layer.step_bytes()
    # The measured read ceiling and the step's launch timed alone (eager,
    # dispatch-recorded events) come first; each timed part is preceded by
    # SETTLE_MS of its own work, untimed.
    ceiling = None
    if not args.no_ceiling:
        ceiling = stream_ceiling(q, torch, ev, step_bytes)
    k_bytes = step_bytes
    mean_k, durs = time_dominant_kernel(q, layer, ev, args.kernel_reps, "all")
    achieved = k_bytes / mean_k / 1e9
    sd = sorted(durs)
    log(f"step kernel mean {mean_k * 1e6:.2f} us (min {sd[0] * 1e6:.2f}, median {sd[len(sd) // 2] * 1e6:.2f}, "
        f"max {sd[-1] * 1e6:.2f}) -> {achieved:.1f} GB/s")
    if ceiling is not None:
        ceiling["headline_kernel_frac_of_read"] = round(achieved / ceiling["read_GB/s"], 4)
        ceiling["headline_kernel_vs_read_launch"] = round(achieved / ceiling["read_launch_GB/s"], 4)
        log(f"measured stream ceiling {json.dumps(ceiling)}")

    log(f"step bytes {step_bytes}; timing {args.steps} steps after {args.warmup} warm-up steps")
    dt, host_dt = time_graph_steps(torch, layer, args.steps, args.warmup)
    value = step_bytes * args.steps / dt / 1e9
    ms_per_step = dt / args.steps * 1e3
    log(f"value {value:.1f} GB/s, {ms_per_step * 1e3:.2f} us/step (host clock around gate + steps: "
        f"{host_dt * 1e3:.3f} ms)")

    src_hash = _kernel_source_hash()
    traffic = _profile_traffic(src_hash)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "qgemv grouped launch of the 8B layer's seven Q4_0 projections, M=1",
                "algorithmic_bytes_per_launch": k_bytes, "mean_kernel_us": round(mean_k * 1e6, 3),
                "kernel_us_min_median_max": [round(sd[0] * 1e6, 2), round(sd[len(sd) // 2] * 1e6, 2),
                                             round(sd[-1] * 1e6, 2)],
                "launches_timed": len(durs), "kernel_source_hash": src_hash,
                # the same launch replayed from a HIP graph, one per step, gaps included
                "graph_step_us": round(ms_per_step * 1e3, 3),
                "graph_step_frac": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)}
    if ceiling is not None:
        roofline["measured_ceiling"] = ceiling

    if args.calibrate_copy:
        a = torch.empty(1 << 28, dtype=torch.uint8, device="cuda:0")
        b = torch.empty_like(a)
        for _ in range(4):
            b.copy_(a)
        torch.cuda.synchronize()
        del a, b

    del layer
    torch.cuda.empty_cache()
    workloads = []
    if not args.no_extra:
        workloads = extra_workloads(q, torch, synth, ev, args.quick_extra, args.only)
        for w in workloads:
            log(json.dumps(w))

    cpu = None
    if not args.no_cpu:
        log("timing the CPU oracle...")
        cpu = cpu_baseline(synth)
        log(json.dumps(cpu))

    line = {
        "metric": "decode qGEMV GB/s (% HBM peak); prefill/MoE qGEMM TFLOP/s (% MFMA peak)",
        "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f16", "data": "synthetic",
        "config": {"workload": "decode step of one 8B-shaped layer's seven projections (q, k, v, o, gate, up, "
                               "down; hidden 4096, ffn 12288), Q4_0 weights, M=1 fp16 activations (four "
                               "independent inputs), one grouped launch",
                   "M": 1, "weight_copies": LAYER_COPIES, "launches_per_step": 1, "step_bytes": step_bytes,
                   "timing": "the W warm-up steps and the K timed steps each captured as one HIP graph "
                             "(one launch per step, consecutive steps on consecutive weight copies); GPU "
                             "events around the timed graph, queued behind a bounded spin kernel; before "
                             f"the W steps an 8-step graph is replayed untimed for {SETTLE_MS:g} ms so the GPU "
                             "leaves its idle clock state",
                   "host_ms_gate_and_steps": round(host_dt * 1e3, 4),
                   "hbm_frac": round(value / HBM_PEAK_GBS, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "workloads": workloads,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
