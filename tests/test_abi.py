"""Host-side checks of the C ABI: symbols, validation, host repack (no GPU)."""
import ctypes
import glob
import os
import re

import numpy as np
import pytest

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


@pytest.fixture(scope="module")
def q():
    import gemm_q4_q8_amd as q
    q.lib()
    return q


def _declared_functions():
    text = "\n".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(q4q8_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for need in ["q4q8_repack", "q4q8_repack_host", "q4q8_qgemv", "q4q8_qgemv_grouped", "q4q8_qgemm",
                 "q4q8_moe_route", "q4q8_moe_qgemm", "q4q8_moe_workspace", "q4q8_last_error", "q4q8_qgemv_swiglu",
                 "q4q8_ffn_decode", "q4q8_attn_prefill"]:
        assert need in names


def test_library_exports_every_declared_symbol(q):
    raw = ctypes.CDLL(q.LIB_PATH)
    missing = [n for n in _declared_functions() if not hasattr(raw, n)]
    assert not missing, missing
    assert q.lib().q4q8_abi_version() == 1


def test_status_strings(q):
    assert q.status_string(0) == "ok"
    for s in (-1, -2, -3, -4, -5):
        assert q.status_string(s) not in ("ok", "unknown status")


def test_fp16_sizes(q):
    assert q.canonical_bytes(synth.FP16, 100, 96) == 100 * 96 * 2
    assert q.repacked_bytes(synth.FP16, 100, 96) == 7 * 1 * 4096
    assert q.repacked_bytes(synth.FP16, 4096, 4096) == 4096 * 4096 * 2
    L = q.lib()
    st = L.q4q8_qgemm(synth.FP16, None, 64, 256, _vp(0x2000), 1, 256, 16, _vp(0x3000), 1, 64, None, 0, None)
    assert st == -1     # the format is accepted; the null weight pointer is not
    st = L.q4q8_qgemm(4, _vp(0x1000), 64, 256, _vp(0x2000), 1, 256, 16, _vp(0x3000), 1, 64, None, 0, None)
    assert st == -2
    nws = q.moe_workspace(1, 4, 8, 2, 256, 256)
    assert q.moe_workspace(synth.FP16, 4, 8, 2, 256, 256) == 0 and nws > 0


@pytest.mark.parametrize("N,K", [(16, 128), (17, 160), (33, 256), (1, 32)])
def test_host_repack_fp16(q, N, K):
    """Plain fp16 records: block j's slot l (= 16 g + r) at j * 1024 + 16 l holds
    row r's weights 8 g .. 8 g + 7 of the block; padding is zero."""
    w = synth.fp16_weight(synth.rng_for(43, N + K), N, K)
    rep = q.repack_host(synth.FP16, w.canon, N, K)
    tiles, chunks = (N + 15) // 16, (K + 127) // 128
    assert rep.size == tiles * chunks * 4096
    recs = rep.view(np.float16).reshape(tiles, chunks, 4, 64, 8)
    full = np.zeros((tiles * 16, chunks * 128), dtype=np.float16)
    full[:N, :K] = w.codes
    for j in range(4):
        for l in range(64):
            r, g = l % 16, l // 16
            k0 = 32 * j + 8 * g
            want = full[r::16, :].reshape(tiles, chunks, 128)[:, :, k0:k0 + 8]
            assert np.array_equal(recs[:, :, j, l, :].view(np.uint16), want.view(np.uint16))


@pytest.mark.parametrize("fmt,bb", [(synth.Q4_0, 18), (synth.Q8_0, 34)])
def test_sizes(q, fmt, bb):
    assert q.canonical_bytes(fmt, 4096, 4096) == 4096 * 128 * bb
    assert q.repacked_bytes(fmt, 4096, 4096) == 4096 * 128 * bb      # aligned: no padding
    assert q.repacked_bytes(fmt, 17, 160) == 2 * 2 * (64 * 16 * (bb - 2) // 16 + 128)
    assert q.canonical_bytes(fmt, 4, 33) == 0
    assert q.repacked_bytes(4, 4, 32) == 0


def _unrepack(fmt, rep, N, K):
    """Read scales/codes back out of the documented tile layout (test-side)."""
    tiles, chunks = (N + 15) // 16, (K + 127) // 128
    rb = 1152 if fmt == synth.Q4_0 else 2176
    cb = rb - 128
    recs = rep.reshape(tiles, chunks, rb)
    codes = np.zeros((tiles * 16, chunks * 128), dtype=np.int64)
    scales = np.zeros((tiles * 16, chunks * 4), dtype=np.float64)
    for g in range(4):
        for r in range(16):
            slot = 16 * g + r
            for j in range(4):
                for e in range(8):
                    k = 32 * j + 8 * g + e
                    if fmt == synth.Q4_0:
                        word = recs[:, :, slot * 16 + 4 * j: slot * 16 + 4 * j + 4].astype(np.uint32)
                        word = word[..., 0] | (word[..., 1] << 8) | (word[..., 2] << 16) | (word[..., 3] << 24)
                        sh = 4 * ((e & 1) * 4 + (e >> 1))
                        codes[r::16, k::128][:tiles, :chunks] = ((word >> sh) & 0xF)
                    else:
                        off = (j >> 1) * 1024 + slot * 16 + (j & 1) * 8 + e
                        codes[r::16, k::128][:tiles, :chunks] = recs[:, :, off].view(np.int8)
    sc = recs[:, :, cb:].reshape(tiles, chunks, 16, 4, 2)
    sbits = sc[..., 0].astype(np.uint16) | (sc[..., 1].astype(np.uint16) << 8)
    scales = sbits.view(np.float16).astype(np.float64).transpose(0, 2, 1, 3).reshape(tiles * 16, chunks * 4)
    return scales, codes


@pytest.mark.parametrize("fmt", [synth.Q4_0, synth.Q8_0])
@pytest.mark.parametrize("N,K", [(16, 128), (17, 160), (33, 256), (1, 32)])
def test_host_repack_roundtrip(q, fmt, N, K):
    w = synth.q_weight(synth.rng_for(41, N * K + fmt), fmt, N, K)
    rep = q.repack_host(fmt, w.canon, N, K)
    assert rep.size == q.repacked_bytes(fmt, N, K)
    scales, codes = _unrepack(fmt, rep, N, K)
    assert np.array_equal(scales[:N, :K // 32], w.scales.astype(np.float64))
    assert np.array_equal(codes[:N, :K], w.codes.astype(np.int64))
    # padding rows / blocks carry scale 0 and code 0
    assert np.all(scales[N:] == 0) and np.all(scales[:, K // 32:] == 0)
    assert np.all(codes[N:] == 0) and np.all(codes[:, K:] == 0)


def test_host_repack_preserves_bytes(q):
    w = synth.q_weight(synth.rng_for(42, 0), synth.Q8_0, 32, 256)
    rep = q.repack_host(synth.Q8_0, w.canon, 32, 256)
    assert rep.size == w.canon.size
    assert np.array_equal(np.sort(rep), np.sort(w.canon))


# --- validation: every bad call returns its status before touching the GPU ---
def _vp(v=0x1000):
    return ctypes.c_void_p(v)


def test_qgemv_validation(q):
    L = q.lib()
    Q4, F16 = synth.Q4_0, synth.F16
    cases = [
        (dict(fmt=4), -2), (dict(N=0), -1), (dict(K=48), -1), (dict(K=0), -1), (dict(M=0), -1), (dict(M=9), -1),
        (dict(xdt=3), -2), (dict(W=None), -1), (dict(x=None), -1), (dict(y=None), -1),
        (dict(W=0x1008), -4), (dict(x=0x1004), -4), (dict(M=2, ldx=4100), -4), (dict(M=2, ldx=100), -1),
        (dict(M=2, ldy=10), -1),
    ]
    for over, want in cases:
        a = dict(fmt=Q4, W=0x1000, N=64, K=4096, x=0x2000, xdt=F16, ldx=4096, M=1, y=0x3000, ldy=64)
        a.update(over)
        st = L.q4q8_qgemv(a["fmt"], _vp(a["W"]) if a["W"] else None, a["N"], a["K"],
                          _vp(a["x"]) if a["x"] else None, a["xdt"], a["ldx"], a["M"],
                          _vp(a["y"]) if a["y"] else None, a["ldy"], None)
        assert st == want, (over, st, q.last_error())
        assert q.last_error()


def test_grouped_validation(q):
    L = q.lib()
    arr = (q.GemvDesc * 9)()
    for i in range(9):
        arr[i] = q.GemvDesc(0x1000, 0x2000, 0x3000, 64, 256, 256, 64)
    assert L.q4q8_qgemv_grouped(1, arr, 9, 1, 1, None) == -1
    assert L.q4q8_qgemv_grouped(1, arr, 0, 1, 1, None) == -1
    arr[3].K = 100
    assert L.q4q8_qgemv_grouped(1, arr, 4, 1, 1, None) == -1
    assert "qgemv" in q.last_error() or "K=" in q.last_error()


def test_swiglu_validation(q):
    L = q.lib()
    ok = dict(fmt=1, Wg=0x1000, Wu=0x5000, F=64, K=256, x=0x2000, xdt=2, ldx=256, M=3, h=0x3000, hdt=2, ldh=64)
    for over, want in [(dict(Wu=None), -1), (dict(Wu=0x5008), -4), (dict(hdt=0), -2),
                       (dict(hdt=3, h=0x3002), -4), (dict(h=0x3001), -4), (dict(ldh=32), -1), (dict(M=9), -1),
                       (dict(K=100), -1), (dict(xdt=3), -2)]:
        a = dict(ok)
        a.update(over)
        st = L.q4q8_qgemv_swiglu(a["fmt"], _vp(a["Wg"]), _vp(a["Wu"]) if a["Wu"] else None, a["F"], a["K"],
                                 _vp(a["x"]), a["xdt"], a["ldx"], a["M"], _vp(a["h"]), a["hdt"], a["ldh"], None)
        assert st == want, (over, st, q.last_error())


def test_ffn_decode_validation(q):
    L = q.lib()
    assert q.ffn_decode_workspace(3, 14336) == (3 * 14336 * 2 + 255) // 256 * 256
    assert q.ffn_decode_workspace(0, 128) == 0 and q.ffn_decode_workspace(9, 128) == 0
    assert q.ffn_decode_workspace(1, 100) == 0
    nws = q.ffn_decode_workspace(2, 256)
    ok = dict(fmt=2, Wg=0x1000, Wu=0x2000, Wd=0x3000, H=512, F=256, x=0x4000, xdt=1, ldx=512, M=2, y=0x5000,
              ldy=512, ws=0x100000, nws=nws)
    for over, want in [(dict(ws=0), -3), (dict(nws=nws - 1), -3), (dict(ws=0x100010), -4), (dict(F=100), -1),
                       (dict(F=0), -1), (dict(H=0), -1),
                       (dict(Wd=None), -1), (dict(Wd=0x3008), -4), (dict(ldy=100), -1), (dict(y=0x5002), -4),
                       (dict(M=0), -1), (dict(fmt=0), -2)]:
        a = dict(ok)
        a.update(over)
        st = L.q4q8_ffn_decode(a["fmt"], _vp(a["Wg"]), _vp(a["Wu"]), _vp(a["Wd"]) if a["Wd"] else None, a["H"],
                               a["F"], _vp(a["x"]), a["xdt"], a["ldx"], a["M"], _vp(a["y"]), a["ldy"],
                               _vp(a["ws"]) if a["ws"] else None, a["nws"], None)
        assert st == want, (over, st, q.last_error())


def test_attn_validation(q):
    L = q.lib()
    ok = dict(dt=2, Q=0x1000, K=0x2000, V=0x3000, O=0x4000, B=1, S=64, Hq=8, Hkv=2, D=128, causal=1, scale=0.088)
    for over, want in [(dict(dt=3), -2), (dict(D=64), -2), (dict(Q=None), -1), (dict(Hkv=3), -1), (dict(S=0), -1),
                       (dict(scale=0.0), -1), (dict(scale=-1.0), -1), (dict(K=0x2008), -4), (dict(O=0x4004), -4),
                       (dict(B=0), -1)]:
        a = dict(ok)
        a.update(over)
        st = L.q4q8_attn_prefill(a["dt"], _vp(a["Q"]) if a["Q"] else None, _vp(a["K"]), _vp(a["V"]), _vp(a["O"]),
                                 a["B"], a["S"], a["Hq"], a["Hkv"], a["D"], a["causal"], a["scale"], None)
        assert st == want, (over, st, q.last_error())


def test_qgemm_validation(q):
    L = q.lib()
    ok = dict(fmt=1, W=0x1000, N=64, K=256, X=0x2000, xdt=2, ldx=256, M=17, Y=0x3000, ydt=2, ldy=64)
    ok["ws"], ok["nws"] = 0x100000, q.qgemm_workspace(2, 17, 256)
    # the row-scaled fp16 copy (M x Kp halfs) and the rows' int32 exponents, each rounded up to 256 bytes
    assert ok["nws"] == -(-17 * 256 * 2 // 256) * 256 + -(-17 * 4 // 256) * 256
    assert q.qgemm_workspace(1, 17, 256) == 0 and q.qgemm_workspace(5, 17, 256) == 0
    for over, want in [(dict(ydt=7), -2), (dict(xdt=3), -2), (dict(M=0), -1), (dict(ldx=128), -1),
                       (dict(ldy=32), -1), (dict(Y=0x3001), -4), (dict(ydt=3, Y=0x3002), -4), (dict(ldx=260), -4), (dict(K=100), -1),
                       (dict(ws=0), -3), (dict(nws=ok["nws"] - 1), -3), (dict(ws=0x100010), -4)]:
        a = dict(ok)
        a.update(over)
        st = L.q4q8_qgemm(a["fmt"], _vp(a["W"]), a["N"], a["K"], _vp(a["X"]), a["xdt"], a["ldx"], a["M"],
                          _vp(a["Y"]), a["ydt"], a["ldy"], _vp(a["ws"]), a["nws"], None)
        assert st == want, (over, st, q.last_error())


def test_moe_validation(q):
    L = q.lib()
    p = [_vp(0x1000 * (i + 1)) for i in range(6)]
    assert L.q4q8_moe_route(p[0], 512, 128, 0, *p[1:], None) == -1
    assert L.q4q8_moe_route(p[0], 512, 128, 129, *p[1:], None) == -1
    assert L.q4q8_moe_route(p[0], 512, 2048, 8, *p[1:], None) == -2
    assert L.q4q8_moe_route(None, 512, 128, 8, *p[1:], None) == -1
    assert L.q4q8_moe_route(p[0], 0, 128, 8, *p[1:], None) == -1          # no tokens
    assert L.q4q8_moe_route(p[0], 512, 0, 1, *p[1:], None) == -1          # no experts
    assert q.moe_workspace(1, 0, 128, 8, 2048, 768) == 0
    nws = q.moe_workspace(1, 512, 128, 8, 2048, 768)
    assert nws > 0
    args = [1, _vp(0x1000), _vp(0x2000), _vp(0x3000), 128, 2048, 768, _vp(0x4000), 2, 512, 8,
            _vp(0x5000), _vp(0x6000), _vp(0x7000), _vp(0x8000), None, _vp(0x10000), nws, None]
    a = list(args)
    a[16] = None
    assert L.q4q8_moe_qgemm(*a) == -3
    a = list(args)
    a[17] = nws - 1
    assert L.q4q8_moe_qgemm(*a) == -3
    a = list(args)
    a[5] = 2000
    assert L.q4q8_moe_qgemm(*a) == -1
    a = list(args)
    a[9] = 0                       # T = 0
    assert L.q4q8_moe_qgemm(*a) == -1
    a = list(args)
    a[16] = _vp(0x10010)
    assert L.q4q8_moe_qgemm(*a) == -4


def test_moe_decode_validation(q):
    L = q.lib()
    nws = q.moe_workspace(1, 4, 128, 8, 2048, 768)
    v = lambda i: _vp(0x1000 * (i + 1))
    # fmt, Wg, Wu, Wd, E, H, F, logits, X, xdt, T, topk, ids, gates, counts, offsets, sorted, out, h_out, ws, bytes, s
    args = [1, v(0), v(1), v(2), 128, 2048, 768, v(3), v(4), 2, 4, 8, v(5), v(6), v(7), v(8), v(9), v(10), None,
            _vp(0x100000), nws, None]
    for i, val, want in [(0, 3, -2), (9, 3, -2), (1, None, -1), (7, None, -1), (12, None, -1), (10, 0, -1),
                         (11, 129, -1), (11, 17, -1), (4, 2048, -1), (5, 2000, -1), (10, 9, -2),
                         (19, None, -3), (20, nws - 1, -3), (19, _vp(0x100010), -4), (13, _vp(0x6002), -4)]:
        a = list(args)
        a[i] = val
        assert L.q4q8_moe_decode(*a) == want, (i, val)
    a = list(args)
    a[5], a[6] = 8192, 8192          # 4 rows of 8192 halfs exceed the decode path's LDS buffer
    a[20] = q.moe_workspace(1, 4, 128, 8, 8192, 8192)
    assert L.q4q8_moe_decode(*a) == -2


def test_repack_validation(q):
    L = q.lib()
    assert L.q4q8_repack(1, _vp(), 16, 128, _vp(0x2000), 10, None) == -1
    assert L.q4q8_repack(1, _vp(), 16, 128, _vp(0x2008), 1 << 20, None) == -4
    assert L.q4q8_repack(5, _vp(), 16, 128, _vp(0x2000), 1 << 20, None) == -2
    assert L.q4q8_repack_host(1, None, 16, 128, _vp(0x2000), 1 << 20) == -1


def test_stream_read_validation(q):
    """The read-ceiling probe rejects bad arguments before any launch."""
    L = q.lib()
    n = L.q4q8_stream_read_digest_bytes()
    assert n > 0 and n % 4 == 0
    ok = dict(buf=0x10000, bytes=1 << 20, digest=0x20000, dbytes=n)
    for over, want in [(dict(buf=None), -1), (dict(digest=None), -1), (dict(bytes=0), -1), (dict(bytes=24), -1),
                       (dict(dbytes=n - 4), -1), (dict(buf=0x10008), -4), (dict(digest=0x20002), -4)]:
        a = dict(ok)
        a.update(over)
        st = L.q4q8_stream_read_timed(_vp(a["buf"]) if a["buf"] else None, a["bytes"],
                                      _vp(a["digest"]) if a["digest"] else None, a["dbytes"], None, None, None)
        assert st == want, (over, st, q.last_error())
    for wgs in (0, -1, 16385):   # the grid form: workgroups outside 1 .. 16384
        st = L.q4q8_stream_read_grid_timed(_vp(ok["buf"]), ok["bytes"], wgs, _vp(ok["digest"]), ok["dbytes"],
                                           None, None, None)
        assert st == -1, (wgs, st, q.last_error())


def test_build_scratch_guard_parses_remarks():
    """build.py refuses spills in the kernels whose waits are hand-counted;
    its parser of the compiler's resource remarks finds scratch users."""
    import importlib.util
    spec = importlib.util.spec_from_file_location("q4q8_build", os.path.join(ROOT, "gemm_q4_q8_amd", "build.py"))
    b = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(b)
    text = ("x.hip:1:1: remark: Function Name: _ZN4q4q812qgemm_kernelILi1E [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:1:1: remark:     VGPRs: 250 [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:1:1: remark:     ScratchSize [bytes/lane]: 16 [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:2:1: remark: Function Name: _ZN4q4q88other_kernel [-Rpass-analysis=kernel-resource-usage]\n"
            "x.hip:2:1: remark:     ScratchSize [bytes/lane]: 0 [-Rpass-analysis=kernel-resource-usage]\n")
    assert b._scratch_users(text) == [("_ZN4q4q812qgemm_kernelILi1E [-Rpass-analysis=kernel-resource-usage]", 16)]
    assert "qgemm_kernel" in b.NO_SCRATCH


def test_measurement_calls_live_in_their_own_header():
    """The product header declares no measurement call; q4q8_measure.h holds
    them (the library exports both sets)."""
    prod = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "q4q8.h")).read(), flags=re.S)
    meas = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "q4q8_measure.h")).read(), flags=re.S)
    prod_names = set(re.findall(r"\b(q4q8_[a-z0-9_]+)\s*\(", prod))
    meas_names = set(re.findall(r"\b(q4q8_[a-z0-9_]+)\s*\(", meas))
    assert not [n for n in prod_names if n.endswith("_timed") or "stream_read" in n]
    assert {"q4q8_qgemv_grouped_timed", "q4q8_qgemm_timed", "q4q8_stream_read_timed",
            "q4q8_stream_read_digest_bytes"} <= meas_names


@pytest.mark.parametrize("name", ["q4q8.h", "q4q8_measure.h"])
def test_headers_compile_as_c_and_cxx(name, tmp_path):
    """Each public header is self-contained C99 and C++ (extern "C")."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    src = tmp_path / "use.c"
    src.write_text(f'#include "{name}"\nint main(void) {{ return Q4Q8_OK; }}\n')
    inc = os.path.join(ROOT, "include")
    for lang, std in (("c", "-std=c99"), ("c++", "-std=c++17")):
        r = subprocess.run([gcc, "-x", lang, std, "-Wall", "-Werror", "-fsyntax-only", "-I", inc, str(src)],
                           capture_output=True, text=True)
        assert r.returncode == 0, r.stderr
