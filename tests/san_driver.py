"""Host code of the library under AddressSanitizer + UndefinedBehaviorSanitizer.

Run by tests/test_host_sanitizers.py in a child process with the clang ASan
runtime preloaded and the host-sanitized library (gemm_q4_q8_amd/build.py,
build_sanitized) in place of the product one.  Exercises what runs on the
host: argument validation of every entry point (valid and invalid shapes,
sizes near the limits), workspace-size queries, the host repack (checked
byte for byte against an independent un-repack), status strings.  With no
GPU, valid calls reach the HIP runtime and must return Q4Q8_ERR_HIP.
Exits non-zero on any mismatch; the sanitizers abort on any error they find.
"""
import ctypes
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

import gemm_q4_q8_amd as q  # noqa: E402
import synth  # noqa: E402

q.LIB_PATH = sys.argv[1]
q._lib = None
L = q.lib()
vp = ctypes.c_void_p
no_gpu = len(sys.argv) > 2 and sys.argv[2] == "nogpu"


def expect(st, want, what):
    if st != want:
        print(f"FAIL {what}: status {st}, want {want}: {q.last_error()}", flush=True)
        sys.exit(1)


# Status strings and sizes.
for s in (0, -1, -2, -3, -4, -5, -99, 7):
    assert isinstance(q.status_string(s), str)
for fmt in (1, 2, 3, 0, 9):
    for N, K in ((1, 32), (17, 96), (4096, 4096), (0, 32), (16, -32), (1 << 31, 1 << 20), (1 << 62, 1 << 62)):
        q.canonical_bytes(fmt, N, K)
        q.repacked_bytes(fmt, N, K)
for args in ((2, 17, 256), (1, 17, 256), (2, 1 << 40, 1 << 20), (2, -1, 128), (5, 3, 128)):
    q.qgemm_workspace(*args)
for args in ((1, 512, 128, 8, 2048, 768), (2, 1 << 30, 1024, 16, 1 << 20, 1 << 20), (1, 0, 1, 1, 128, 128),
             (1, 8, 1024, 16, -128, 128)):
    q.moe_workspace(*args)
for M, F in ((1, 128), (8, 14336), (0, 128), (9, 128), (3, 1 << 40)):
    q.ffn_decode_workspace(M, F)

# Host repack, checked against a test-side read of the documented layout.
from test_abi import _unrepack  # noqa: E402

rng = np.random.default_rng(5)
for fmt in (synth.Q4_0, synth.Q8_0):
    for N, K in ((16, 128), (33, 96), (5, 32), (70, 416)):
        w = synth.q_weight(rng, fmt, N, K)
        canon = np.ascontiguousarray(w.canon)
        out = np.zeros(q.repacked_bytes(fmt, N, K), dtype=np.uint8)
        expect(L.q4q8_repack_host(fmt, canon.ctypes.data, N, K, out.ctypes.data, out.nbytes), 0, "repack_host")
        scales, codes = _unrepack(fmt, out, N, K)
        if not (np.array_equal(scales[:N, :K // 32], w.scales.astype(np.float64))
                and np.array_equal(codes[:N, :K], w.codes.astype(np.int64))):
            print(f"FAIL repack_host round trip fmt {fmt} N {N} K {K}", flush=True)
            sys.exit(1)
        expect(L.q4q8_repack_host(fmt, canon.ctypes.data, N, K, out.ctypes.data, out.nbytes - 1), -1,
               "repack_host short destination")

# Validation of every entry point with bad arguments (nothing may be enqueued).
p = vp(0x10000)
expect(L.q4q8_qgemv(1, None, 64, 256, p, 1, 256, 1, p, 64, None), -1, "qgemv null W")
expect(L.q4q8_qgemv(1, p, 64, 100, p, 1, 256, 1, p, 64, None), -1, "qgemv K % 32")
expect(L.q4q8_qgemv(1, p, 64, 256, p, 1, 256, 9, p, 64, None), -1, "qgemv M 9")
expect(L.q4q8_qgemm(1, p, 64, 256, p, 2, 256, 17, p, 7, 64, p, 1 << 20, None), -2, "qgemm ydt")
expect(L.q4q8_qgemm(1, p, 64, 256, p, 2, 256, 17, p, 2, 64, None, 0, None), -3, "qgemm ws")
expect(L.q4q8_qgemm(1, p, 1 << 31, 1 << 25, p, 2, 1 << 25, 17, p, 2, 1 << 31, p, 1 << 20, None), -2, "qgemm huge")
expect(L.q4q8_moe_route(None, 4, 8, 2, p, p, p, p, p, None), -1, "route null")
expect(L.q4q8_moe_route(p, 4, 8, 9, p, p, p, p, p, None), -1, "route topk > E")
expect(L.q4q8_moe_route(p, 4, 2000, 8, p, p, p, p, p, None), -2, "route E > 1024")
expect(L.q4q8_moe_qgemm(1, p, p, p, 8, 256, 100, p, 2, 4, 2, p, p, p, p, None, p, 1 << 20, None), -1, "moe F")
expect(L.q4q8_moe_qgemm(1, p, p, p, 8, 256, 128, p, 2, 4, 2, p, p, p, p, None, p, 10, None), -3, "moe ws")
expect(L.q4q8_moe_qgemm(1, p, p, p, 32, 256, 128, p, 2, 1 << 30, 16, p, p, p, p, None, p, 1 << 40, None), -2, "moe huge")
expect(L.q4q8_moe_decode(1, p, p, p, 8, 256, 128, p, p, 2, 9, 2, p, p, p, p, p, p, None, p, 1 << 20, None), -2,
       "moe_decode T 9")
expect(L.q4q8_moe_forward(3, p, p, p, 8, 256, 128, p, p, 2, 9, 2, p, p, p, p, p, p, None, p, 1 << 20, None), -2,
       "moe_forward fp16 weights")
expect(L.q4q8_moe_decode_noalloc(1, p, p, p, 32, 3200, 3200, p, p, 2, 8, 16, p, p, p, p, p, p, None, None), -2,
       "moe_decode_noalloc beyond scratch")
expect(L.q4q8_attn_prefill(2, p, p, p, p, 1, 64, 32, 8, 64, 1, ctypes.c_float(0.1), None), -2, "attn D 64")
expect(L.q4q8_attn_prefill(2, p, p, p, p, 1, 64, 30, 8, 128, 1, ctypes.c_float(0.1), None), -1, "attn GQA")
expect(L.q4q8_ffn_decode(1, p, p, p, 256, 128, p, 1, 256, 2, p, 256, None, 0, None), -3, "ffn ws")

if no_gpu:
    # Valid calls: validation passes, the HIP runtime finds no device.
    expect(L.q4q8_repack(1, p, 16, 128, vp(0x20000), 1152, None), -5, "repack without a GPU")
    expect(L.q4q8_qgemm(1, p, 64, 256, vp(0x20000), 1, 256, 16, vp(0x30000), 3, 64, None, 0, None), -5,
           "qgemm without a GPU")
    expect(L.q4q8_moe_decode_noalloc(1, p, p, p, 8, 256, 128, vp(0x1000), vp(0x2000), 2, 2, 2, vp(0x3000),
                                     vp(0x4000), vp(0x5000), vp(0x6000), vp(0x7000), vp(0x8000), None, None), -5,
           "moe_decode_noalloc without a GPU")
print("sanitized host checks ok", flush=True)
