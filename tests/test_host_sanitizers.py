"""Host code under AddressSanitizer + UndefinedBehaviorSanitizer (CPU only).

Builds the library with the sanitizers on its host pass only
(gemm_q4_q8_amd/build.py, build_sanitized; about 40 s), then runs
tests/san_driver.py in a child process with the clang ASan runtime preloaded:
argument validation of every entry point, workspace queries at extreme
sizes, the host repack, and -- with no GPU present -- valid calls that must
return Q4Q8_ERR_HIP instead of crashing.
"""
import importlib.util
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location("q4q8_build", os.path.join(ROOT, "gemm_q4_q8_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    return b


def _gpu_present() -> bool:
    import torch
    return torch.cuda.is_available()


def test_valid_call_without_gpu_returns_hip_error():
    """A valid call with no GPU in the machine reports Q4Q8_ERR_HIP (the
    validation passes, the HIP runtime finds no device) and does not crash."""
    if _gpu_present():
        pytest.skip("a GPU is present: this checks the no-device path")
    import ctypes
    import gemm_q4_q8_amd as q
    L = q.lib()
    vp = ctypes.c_void_p
    assert L.q4q8_repack(1, vp(0x10000), 16, 128, vp(0x20000), 1152, None) == -5
    assert "device" in q.last_error()
    assert L.q4q8_qgemv(1, vp(0x10000), 64, 256, vp(0x20000), 1, 256, 1, vp(0x30000), 64, None) == -5


def test_host_code_under_asan_ubsan():
    b = _build_module()
    lib = b.build_sanitized(verbose=False)
    env = dict(os.environ)
    env["LD_PRELOAD"] = b.asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    args = [sys.executable, os.path.join(ROOT, "tests", "san_driver.py"), lib]
    if not _gpu_present():
        args.append("nogpu")
    r = subprocess.run(args, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    assert "sanitized host checks ok" in r.stdout
    assert "runtime error" not in out and "AddressSanitizer" not in out, out[-4000:]
