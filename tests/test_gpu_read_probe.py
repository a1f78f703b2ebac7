"""The streaming-read probe (measurement support) reads every 16-byte word of
its buffer exactly once: the XOR of its per-workgroup sink words equals the
XOR of the buffer's 32-bit words, for sizes that end mid-stride."""
import numpy as np
import pytest

from tests import gpu_util as gu

pytestmark = pytest.mark.gpu
torch = gu.torch
import paged_kv_cache_135_amd as pkv  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    gu.need_gpu()


@pytest.mark.parametrize("words", [4, 4 * 1000 + 4, 4 * (1 << 20) + 12, 4 * 3_000_001])
def test_probe_reads_every_word_once(words):
    rng = np.random.default_rng(words)
    host = rng.integers(0, 2**32, size=words, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = pkv.read_probe(buf)
    got = np.bitwise_xor.reduce(gu.host(sink).view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


def test_probe_on_an_empty_buffer_leaves_the_sink_alone():
    buf = torch.empty(0, dtype=torch.int32, device="cuda")
    sink = torch.full((pkv.load().pkv_read_probe_blocks(),), 7, dtype=torch.int32, device="cuda")
    pkv.read_probe(buf, sink)
    assert np.all(gu.host(sink) == 7)


@pytest.mark.parametrize("workers", [1, 7, 64, 1024])
@pytest.mark.parametrize("mode", [0, 1])
def test_tile_gather_probe_reads_every_listed_tile_once(mode, workers):
    """The gather probe (direct to registers, or staged through LDS) folds
    every 16-byte word of every listed K and V tile exactly once: the XOR of
    its sink equals the XOR of those tiles' words, computed on the host.  A
    tile listed twice cancels out, as XOR does."""
    rng = np.random.default_rng(workers + 10 * mode)
    nrows = 16 * 300
    kh = rng.integers(0, 2**32, size=(nrows, 64), dtype=np.uint64).astype(np.uint32)
    vh = rng.integers(0, 2**32, size=(nrows, 64), dtype=np.uint64).astype(np.uint32)
    kc = torch.from_numpy(kh.view(np.int16)).cuda().view(torch.bfloat16).view(nrows, 128)
    vc = torch.from_numpy(vh.view(np.int16)).cuda().view(torch.bfloat16).view(nrows, 128)
    tiles = rng.integers(0, nrows - 16, size=977).astype(np.int32)  # any row, not only block starts
    sink = pkv.tile_gather_probe(kc, vc, gu.dev(tiles), workers, mode)
    want = np.uint32(0)
    for r in tiles:
        want ^= np.bitwise_xor.reduce(kh[r:r + 16].ravel()) ^ np.bitwise_xor.reduce(vh[r:r + 16].ravel())
    got = np.bitwise_xor.reduce(gu.host(sink).view(np.uint32))
    assert got == want


def test_tile_gather_probe_refusals():
    kc = torch.zeros(64, 128, dtype=torch.bfloat16, device="cuda")
    rows = torch.zeros(4, dtype=torch.int32, device="cuda")
    with pytest.raises(pkv.PagedKVError):
        pkv.tile_gather_probe(kc, kc.clone(), rows, 0, 0)   # no workers
    with pytest.raises(pkv.PagedKVError):
        pkv.tile_gather_probe(kc, kc.clone(), rows, 4, 2)   # no such mode
    with pytest.raises(ValueError):
        pkv.tile_gather_probe(kc.float(), kc.float(), rows, 4, 0)
