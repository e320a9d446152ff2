"""Build the HIP library libq4q8.so in-tree for gfx950.

Compiles every gemm_q4_q8_amd/csrc/*.hip with hipcc (one object per source,
in parallel) and links them into gemm_q4_q8_amd/libq4q8.so.  Always rebuilds.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "libq4q8.so")
BUILD = os.path.join(HERE, "_build")
ARCH = "gfx950"

CFLAGS = [
    "-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
    # Packed fp32 ops are kept out of the generated code on purpose.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found")


# Kernels whose pipelines wait on hand-counted outstanding loads
# (s_waitcnt vmcnt(N) in qgemm_core.h): a register spill would add scratch
# loads and stores to those counts and break the waits silently, so the
# build fails if any of them uses scratch.
NO_SCRATCH = ("qgemm_kernel",)


def _scratch_users(remarks: str):
    """(kernel, bytes/lane) of every kernel the compiler reports with scratch."""
    out, name = [], None
    for line in remarks.splitlines():
        if "Function Name:" in line:
            name = line.split("Function Name:", 1)[1].strip()
        elif name and "ScratchSize [bytes/lane]:" in line:
            n = int(line.split("ScratchSize [bytes/lane]:", 1)[1].split()[0])
            if n:
                out.append((name, n))
    return out


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [_hipcc(), *CFLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stderr}")
    bad = [(k, n) for k, n in _scratch_users(r.stderr) if any(s in k for s in NO_SCRATCH)]
    if bad:
        raise RuntimeError(f"{src}: kernels with hand-counted load waits use scratch (register spills): {bad}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = OUT + ".tmp"
    cmd = [_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


# Host-side AddressSanitizer + UndefinedBehaviorSanitizer build, for CPU tests
# of the host code (argument validation, the host repack): every -fsanitize=
# applies to the host pass only; the device code is built as usual.
SAN_DIR = os.path.join(BUILD, "san")
SAN_OUT = os.path.join(SAN_DIR, "libq4q8_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-omit-frame-pointer", "-g"]


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime to preload into an uninstrumented python."""
    hits = sorted(glob.glob(os.path.join(os.path.dirname(os.path.dirname(os.path.realpath(_hipcc()))),
                                         "llvm", "lib", "clang", "*", "lib", "linux", "libclang_rt.asan-x86_64.so")))
    if not hits:
        raise RuntimeError("libclang_rt.asan-x86_64.so not found next to hipcc")
    return hits[-1]


def build_sanitized(verbose: bool = True) -> str:
    os.makedirs(SAN_DIR, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))

    def one(src):
        obj = os.path.join(SAN_DIR, os.path.basename(src) + ".o")
        r = subprocess.run([_hipcc(), *CFLAGS, *SAN_FLAGS, "-c", src, "-o", obj], capture_output=True, text=True)
        if r.returncode:
            raise RuntimeError(f"hipcc (sanitized) failed on {src}:\n{r.stderr}")
        return obj

    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(one, srcs))
    r = subprocess.run([_hipcc(), "-shared", "-fPIC", f"--offload-arch={ARCH}", *SAN_FLAGS, "-shared-libsan", *objs,
                        "-o", SAN_OUT], capture_output=True, text=True)
    if r.returncode:
        raise RuntimeError(f"link (sanitized) failed:\n{r.stderr}")
    if verbose:
        print(f"built {SAN_OUT}")
    return SAN_OUT


if __name__ == "__main__":
    build()
    sys.exit(0)
