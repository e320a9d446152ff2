"""The HBM read-ceiling probe reads every byte of its buffer exactly once:
the XOR of its per-wave digests equals the XOR of the buffer's 32-bit words."""
import numpy as np
import pytest
import torch

from util import dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def q():
    import gemm_q4_q8_amd as q
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    q.lib()
    return q


@pytest.mark.parametrize("n16", [1, 1000003, 4 * 1024 * 1024])
def test_stream_read_digest(q, n16):
    rng = np.random.default_rng(77 + n16)
    host = rng.integers(0, 2**32, size=4 * n16, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(dev())
    digest = q.stream_read(buf)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(digest.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)
    # Twice in a row on the same digest buffer: fully overwritten.
    digest2 = q.stream_read(buf, digest=digest)
    torch.cuda.synchronize()
    assert np.bitwise_xor.reduce(digest2.cpu().numpy().view(np.uint32)) == np.bitwise_xor.reduce(host)


@pytest.mark.parametrize("wgs", [1, 2048, 8192])
def test_stream_read_grid_digest(q, wgs):
    """The grid form (a caller-chosen number of workgroups) also reads every
    byte once: the XOR of the digest words of its wgs * 8 waves equals the
    buffer's."""
    n16 = 1000003
    rng = np.random.default_rng(91 + wgs)
    host = rng.integers(0, 2**32, size=4 * n16, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).to(dev())
    digest = q.stream_read(buf, workgroups=wgs)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(digest.cpu().numpy().view(np.uint32)[: wgs * 8])
    assert got == np.bitwise_xor.reduce(host)
