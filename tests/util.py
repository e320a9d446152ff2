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


def values(t: torch.Tensor) -> np.ndarray:
    """Exact fp64 values of a bf16 / fp16 / fp32 GPU tensor."""
    if t.dtype == torch.bfloat16:
        return bf16_values(t)
    return t.detach().cpu().to(torch.float64).numpy()


def _round_to(dtype, v64):
    """Nearest-even rounding of fp64 values to bf16 / fp16 (via fp32 for bf16)."""
    if dtype == "bf16":
        v32 = v64.astype(np.float32)
        return synth.bits_to_values(synth.BF16, synth.f32_to_bf16_bits(v32))
    return v64.astype(np.float16).astype(np.float64)


def check_rounded(got_bf16: np.ndarray, ref, bound, what="", dtype="bf16"):
    """A bf16 (or fp16) output passes if it is the nearest-even rounding of some
    value v with |v - ref| <= 2e-3 * sum|w*x| + 1e-5: the output format's own
    rounding is allowed on top of the tolerance.  Rounding is monotone, so
    that is: got in [round(ref - tol), round(ref + tol)]."""
    ref = np.asarray(ref, dtype=np.float64)
    tol = tolerance(bound)
    lo = _round_to(dtype, ref - tol)
    hi = _round_to(dtype, ref + tol)
    if dtype == "bf16":
        # the fp32 step before bf16 may move the ends by one fp32 ulp; widen by it
        lo = np.minimum(lo, _round_to(dtype, np.nextafter((ref - tol).astype(np.float32), np.float32(-np.inf))
                                      .astype(np.float64)))
        hi = np.maximum(hi, _round_to(dtype, np.nextafter((ref + tol).astype(np.float32), np.float32(np.inf))
                                      .astype(np.float64)))
    got = np.asarray(got_bf16, dtype=np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    ok = (got >= lo) & (got <= hi)
    if not np.all(ok):
        i = np.unravel_index(np.argmin(ok), ok.shape)
        raise AssertionError(f"{what}: {got[i]!r} outside [{lo[i]!r}, {hi[i]!r}] (ref {ref[i]!r}, tol {tol[i]!r})")
    return float((np.abs(got - ref) / tol).max())
