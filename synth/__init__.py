"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module only draws random numbers and lays them out in the interchange
formats; it holds none of the arithmetic of the quantised products (no
dequantisation, no dot product, no routing).  Both the CPU oracle and the GPU
path consume what it returns, and nothing else is shared between them.

Interchange formats (the plain GGUF-style block layout):

* Q4_0 block, 18 bytes: fp16 scale (little-endian), then 16 bytes where byte i
  carries code i in its low nibble and code i+16 in its high nibble.
* Q8_0 block, 34 bytes: fp16 scale, then 32 two's-complement int8 codes.

Blocks run along K (32 weights each); rows n = 0..N-1 follow one another.

Activations are drawn in fp64 from N(0, 1) and rounded to nearest-even fp16 or
bf16; the rounded tensor is the input of both sides.  bf16 is carried as its
raw 16-bit pattern (uint16), rounded from the fp32 value.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

Q4_0 = 1
Q8_0 = 2
FP16 = 3            # plain fp16 weights (no quantisation)
F16 = 1
BF16 = 2
F32 = 3

BLOCK = 32
BLOCK_BYTES = {Q4_0: 18, Q8_0: 34, FP16: 64}
FORMAT_NAME = {Q4_0: "q4_0", Q8_0: "q8_0", FP16: "fp16"}
DTYPE_NAME = {F16: "f16", BF16: "bf16", F32: "f32"}

# Scale / code distributions of the workloads.
Q4_SCALE = (0.002, 0.02)
Q8_SCALE = (0.0002, 0.002)


@dataclass
class QWeight:
    """One block-quantised matrix: canonical bytes plus the logical draw."""

    fmt: int
    N: int
    K: int
    canon: np.ndarray       # uint8 [N * K/32 * block_bytes]
    scales: np.ndarray      # float16 [N, K/32] (None for FP16)
    codes: np.ndarray       # uint8 (Q4_0, 0..15), int8 (Q8_0) or float16 (FP16: the weights) [N, K]


@dataclass
class Act:
    """An activation tensor: its raw 16-bit storage and its exact value."""

    dtype: int
    bits: np.ndarray        # uint16, the stored fp16 / bf16 pattern
    values: np.ndarray      # float64, exactly the stored value


def rng_for(seed: int, index: int) -> np.random.Generator:
    """Generator for tensor number `index` of the workload seeded `seed`."""
    # Same stream as SeedSequence(seed).spawn(index + 1)[index], built directly.
    ss = np.random.SeedSequence(seed, spawn_key=(index,))
    return np.random.Generator(np.random.PCG64(ss))


def pack_blocks(fmt: int, scales: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """Lay out scales [N, K/32] (fp16) and codes [N, K] as canonical blocks."""
    N, K = codes.shape
    nb = K // BLOCK
    sc = np.ascontiguousarray(scales.astype(np.float16)).view(np.uint8).reshape(N, nb, 2)
    if fmt == Q4_0:
        c = codes.astype(np.uint8).reshape(N, nb, BLOCK)
        body = (c[:, :, :16] & 0xF) | ((c[:, :, 16:] & 0xF) << 4)
    elif fmt == Q8_0:
        body = codes.astype(np.int8).view(np.uint8).reshape(N, nb, BLOCK)
    else:
        raise ValueError(f"unknown format {fmt}")
    return np.concatenate([sc, body.astype(np.uint8)], axis=2).reshape(-1)


def q_weight(rng: np.random.Generator, fmt: int, N: int, K: int,
             scale_range=None, code_range=None) -> QWeight:
    """Uniform fp16 scales (drawn in fp64, rounded to fp16) and uniform codes."""
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    if scale_range is None:
        scale_range = Q4_SCALE if fmt == Q4_0 else Q8_SCALE
    if code_range is None:
        code_range = (0, 15) if fmt == Q4_0 else (-127, 127)
    lo, hi = scale_range
    scales = rng.uniform(lo, hi, size=(N, K // BLOCK)).astype(np.float16)
    c = rng.integers(code_range[0], code_range[1] + 1, size=(N, K), dtype=np.int16)
    codes = c.astype(np.uint8) if fmt == Q4_0 else c.astype(np.int8)
    return QWeight(fmt, N, K, pack_blocks(fmt, scales, codes), scales, codes)


def fp16_weight(rng: np.random.Generator, N: int, K: int, sigma: float = 0.02) -> QWeight:
    """Plain fp16 weights N(0, sigma^2) rounded to fp16; canonical = row-major
    little-endian fp16 [N, K]."""
    if K % BLOCK:
        raise ValueError("K must be a multiple of 32")
    w = (rng.standard_normal(size=(N, K)) * sigma).astype(np.float16)
    return QWeight(FP16, N, K, np.ascontiguousarray(w).view(np.uint8).reshape(-1).copy(), None, w)


def weight(rng: np.random.Generator, fmt: int, N: int, K: int) -> QWeight:
    """A matrix of any format with the workloads' distributions."""
    return fp16_weight(rng, N, K) if fmt == FP16 else q_weight(rng, fmt, N, K)


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to nearest-even bf16; returns the uint16 patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(np.asarray(a, dtype=np.float32))
    r[nan] = 0x7FC0
    return r


def bits_to_values(dtype: int, bits: np.ndarray) -> np.ndarray:
    if dtype == F16:
        return bits.view(np.float16).astype(np.float64)
    if dtype == BF16:
        return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    raise ValueError(dtype)


def activation(rng: np.random.Generator, shape, dtype: int) -> Act:
    """fp64 N(0,1) rounded to the storage type."""
    v = rng.standard_normal(size=shape)
    if dtype == F16:
        bits = v.astype(np.float16).view(np.uint16)
    elif dtype == BF16:
        bits = f32_to_bf16_bits(v.astype(np.float32))
    else:
        raise ValueError(dtype)
    return Act(dtype, bits, bits_to_values(dtype, bits))


def act_from_values(values: np.ndarray, dtype: int) -> Act:
    """Store given values (rounded) as an activation tensor."""
    v = np.asarray(values, dtype=np.float64)
    if dtype == F16:
        bits = v.astype(np.float16).view(np.uint16)
    else:
        bits = f32_to_bf16_bits(v.astype(np.float32))
    return Act(dtype, bits, bits_to_values(dtype, bits))


def router_logits(rng: np.random.Generator, T: int, E: int) -> np.ndarray:
    return rng.standard_normal(size=(T, E)).astype(np.float32)


# ----------------------------------------------------------------------------
# The five workloads.  Seeds are fixed per workload; tensors are drawn from
# spawned streams in the order listed.
# ----------------------------------------------------------------------------
SEED_BASE = 20260701

GEMV_2048 = dict(name="q4_0 gemv 2048x2048 m1", fmt=Q4_0, xdt=F16,
                 mats=[("w", 2048, 2048)], ms=[1], seed=SEED_BASE + 0)

LAYER_8B = dict(name="q4_0 decode layer 8B-shape (hidden 4096, ffn 12288)", fmt=Q4_0, xdt=F16,
                mats=[("wq", 4096, 4096), ("wk", 1024, 4096), ("wv", 1024, 4096),
                      ("wo", 4096, 4096), ("wg", 12288, 4096), ("wu", 12288, 4096),
                      ("wd", 4096, 12288)],
                ms=[1, 2, 4, 8], seed=SEED_BASE + 1)

# Inputs of the 8B layer: x_attn feeds q/k/v, x_o feeds o, x_ffn feeds gate/up,
# x_dn feeds down.
LAYER_8B_INPUT = {"wq": "x_attn", "wk": "x_attn", "wv": "x_attn", "wo": "x_o",
                  "wg": "x_ffn", "wu": "x_ffn", "wd": "x_dn"}

Q8_3B = dict(name="q8_0 decode gemv 3B-shape (hidden 3072, ffn 8192)", fmt=Q8_0, xdt=BF16,
             mats=[("w3072x3072", 3072, 3072), ("w1024x3072", 1024, 3072),
                   ("w8192x3072", 8192, 3072), ("w3072x8192", 3072, 8192)],
             ms=[1, 2, 3, 4, 5, 6, 7, 8], seed=SEED_BASE + 2)

PREFILL = dict(name="q4_0 prefill gemm K4096 N12288", fmt=Q4_0, xdt=BF16, ydt=BF16,
               N=12288, K=4096, ms=[512, 2048], seed=SEED_BASE + 3)

MOE = dict(name="q4_0 moe prefill E128 top8 H2048 F768 T512", fmt=Q4_0, xdt=BF16,
           E=128, topk=8, H=2048, F=768, T=512, seed=SEED_BASE + 4)


ATTN = dict(name="prefill attention 8B-shape (Hq 32, Hkv 8, D 128), causal", B=1, S=2048, Hq=32, Hkv=8, D=128,
            dt=BF16, seed=SEED_BASE + 5)


def attention_inputs(B: int, S: int, Hq: int, Hkv: int, D: int, dtype: int, seed: int):
    """q [B, S, Hq, D], k and v [B, S, Hkv, D]: N(0,1) rounded to dtype."""
    return (activation(rng_for(seed, 0), (B, S, Hq, D), dtype), activation(rng_for(seed, 1), (B, S, Hkv, D), dtype),
            activation(rng_for(seed, 2), (B, S, Hkv, D), dtype))


def gemv_problem(fmt: int, N: int, K: int, M: int, xdt: int, seed: int):
    """One matrix and one activation block, for parity cases of any size."""
    w = q_weight(rng_for(seed, 0), fmt, N, K)
    x = activation(rng_for(seed, 1), (M, K), xdt)
    return w, x


def layer_8b(M: int, seed: int = LAYER_8B["seed"], mats=None):
    """The seven projection matrices and four inputs of the 8B-shaped layer."""
    out_w = {}
    for i, (name, N, K) in enumerate(LAYER_8B["mats"]):
        if mats is not None and name not in mats:
            continue
        out_w[name] = q_weight(rng_for(seed, i), Q4_0, N, K)
    xs = {}
    for j, (xname, K) in enumerate([("x_attn", 4096), ("x_o", 4096), ("x_ffn", 4096),
                                    ("x_dn", 12288)]):
        xs[xname] = activation(rng_for(seed, 100 + 10 * M + j), (M, K), F16)
    return out_w, xs


def q8_3b(M: int, seed: int = Q8_3B["seed"]):
    ws, xs = {}, {}
    for i, (name, N, K) in enumerate(Q8_3B["mats"]):
        ws[name] = q_weight(rng_for(seed, i), Q8_0, N, K)
        xs[name] = activation(rng_for(seed, 100 + 10 * M + i), (M, K), BF16)
    return ws, xs


def prefill(M: int, seed: int = PREFILL["seed"], N: int = PREFILL["N"], K: int = PREFILL["K"]):
    w = q_weight(rng_for(seed, 0), Q4_0, N, K)
    x = activation(rng_for(seed, 1 + M), (M, K), BF16)
    return w, x


def moe(seed: int = MOE["seed"], T: int = MOE["T"], E: int = MOE["E"], H: int = MOE["H"],
        F: int = MOE["F"], fmt: int = Q4_0):
    """Router logits, tokens and the stacked expert weights.

    Returns (logits fp32 [T,E], x Act [T,H], wg, wu, wd) where each w is a list
    of E QWeight: gate and up are [F, H], down is [H, F].
    """
    logits = router_logits(rng_for(seed, 0), T, E)
    x = activation(rng_for(seed, 1), (T, H), BF16)
    wg = [q_weight(rng_for(seed, 1000 + e), fmt, F, H) for e in range(E)]
    wu = [q_weight(rng_for(seed, 2000 + e), fmt, F, H) for e in range(E)]
    wd = [q_weight(rng_for(seed, 3000 + e), fmt, H, F) for e in range(E)]
    return logits, x, wg, wu, wd
