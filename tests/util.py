"""Test helpers: device upload of the seeded inputs and the acceptance rule."""
import numpy as np
import torch

import synth

REL = 2e-3
ABS = 1e-5


def dev():
    return torch.device("cuda:0")


def act_tensor(a: synth.Act) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a.bits).view(np.int16))
    dt = torch.float16 if a.dtype == synth.F16 else torch.bfloat16
    return t.view(dt).to(dev())


def bytes_tensor(b: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint8)).to(dev())


def repacked_weight(lib, w: synth.QWeight) -> torch.Tensor:
    """Upload canonical blocks and convert them with the library's repack kernel."""
    return lib.repack(w.fmt, bytes_tensor(w.canon), w.N, w.K)


def tolerance(bound):
    return REL * np.asarray(bound) + ABS


def check(got, ref, bound, what=""):
    """|got - ref| <= 2e-3 * sum|w*x| + 1e-5 elementwise; returns max err/tol."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    tol = tolerance(bound)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    err = np.abs(got - ref)
    ratio = err / tol
    worst = np.unravel_index(np.argmax(ratio), ratio.shape)
    assert np.all(err <= tol), (f"{what}: max err/tol {ratio.max():.3g} at {worst}: got {got[worst]!r} "
                                f"ref {ref[worst]!r} tol {tol[worst]!r}")
    return float(ratio.max())


def bf16_values(t: torch.Tensor) -> np.ndarray:
    bits = t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    return synth.bits_to_values(synth.BF16, bits)


def check_rounded(got_bf16: np.ndarray, ref, bound, what=""):
    """A bf16 output passes if it is the nearest-even bf16 of some value v with
    |v - ref| <= 2e-3 * sum|w*x| + 1e-5 (the output format's own rounding is
    allowed on top of the tolerance)."""
    ref = np.asarray(ref, dtype=np.float64)
    tol = tolerance(bound)
    lo = synth.bits_to_values(synth.BF16, synth.f32_to_bf16_bits((ref - tol).astype(np.float32)))
    hi = synth.bits_to_values(synth.BF16, synth.f32_to_bf16_bits((ref + tol).astype(np.float32)))
    # fp32 rounding of ref +- tol may move the ends by one fp32 ulp; widen by it.
    lo = np.minimum(lo, synth.bits_to_values(synth.BF16, synth.f32_to_bf16_bits(
        np.nextafter((ref - tol).astype(np.float32), np.float32(-np.inf)))))
    hi = np.maximum(hi, synth.bits_to_values(synth.BF16, synth.f32_to_bf16_bits(
        np.nextafter((ref + tol).astype(np.float32), np.float32(np.inf)))))
    got = np.asarray(got_bf16, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    ok = (got >= lo) & (got <= hi)
    if not np.all(ok):
        i = np.unravel_index(np.argmin(ok), ok.shape)
        raise AssertionError(f"{what}: {got[i]!r} outside [{lo[i]!r}, {hi[i]!r}] (ref {ref[i]!r}, tol {tol[i]!r})")
    return float((np.abs(got - ref) / tol).max())
