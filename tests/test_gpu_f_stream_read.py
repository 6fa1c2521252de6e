"""GPU: the streaming-read measurement kernel reads every 16-byte word once: the XOR of the
per-block folds it writes equals the XOR of all 32-bit words of the buffer (numpy), for
sizes that leave a ragged tail against the launch's grid stride and unroll."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    from decode_linear_amd import build
    build.ensure_built()


@pytest.mark.parametrize("words16", [1, 7, 512 * 256 - 3, 512 * 256 * 4 + 5, 4128768])
def test_stream_read_folds_every_word(words16):
    from decode_linear_amd import qlin_dispatch_count, qlin_stream_read
    rng = np.random.default_rng(words16)
    host = rng.integers(0, 2 ** 32, size=words16 * 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    before = qlin_dispatch_count(5)
    part = torch.zeros(1024, dtype=torch.int32, device="cuda")
    qlin_stream_read(buf, part)
    torch.cuda.synchronize()
    assert qlin_dispatch_count(5) == before + 1
    got = np.bitwise_xor.reduce(part.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


@pytest.mark.parametrize("blocks,unroll,nt", [(1, 1, 0), (256, 4, 1), (512, 16, 0), (1024, 8, 1), (7, 2, 0)])
def test_stream_read_config_folds_every_word(blocks, unroll, nt):
    from decode_linear_amd import qlin_stream_read_config
    for words16 in (3, 512 * 256 * 4 + 5):
        rng = np.random.default_rng(words16 + blocks)
        host = rng.integers(0, 2 ** 32, size=words16 * 4, dtype=np.uint64).astype(np.uint32)
        buf = torch.from_numpy(host.view(np.int32)).cuda()
        part = torch.zeros(1024, dtype=torch.int32, device="cuda")
        qlin_stream_read_config(buf, blocks, unroll, bool(nt), part)
        torch.cuda.synchronize()
        got = np.bitwise_xor.reduce(part.cpu().numpy().view(np.uint32)[:blocks])
        assert got == np.bitwise_xor.reduce(host)
