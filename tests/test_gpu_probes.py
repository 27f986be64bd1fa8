"""The ceiling probes behind bench.py's measured ceilings do the work they claim: every MFMA
result and every byte read is checked on the host."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def x():
    from sparse_depth_token_amd import xmod
    return xmod


def test_probe_mfma_results(x):
    out = torch.full((x.PROBE_THREADS,), -1.0, dtype=torch.float32, device="cuda")
    x.probe_mfma(out, 1000)
    torch.cuda.synchronize()
    assert torch.all(out == 64.0 * 1000).item()


@pytest.mark.parametrize("depth", [4, 8, 16])
@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 1 << 24, (1 << 26) + 16 * 7])
def test_probe_read_sums_every_word(x, nbytes, depth):
    rng = np.random.default_rng(31)
    words = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    out = torch.zeros(x.PROBE_THREADS, dtype=torch.int32, device="cuda")
    x.probe_read(src, out, depth)
    torch.cuda.synchronize()
    got = int(out.cpu().numpy().view(np.uint32).astype(np.uint64).sum()) % (1 << 32)
    assert got == int(words.astype(np.uint64).sum()) % (1 << 32)


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, 1 << 24, (1 << 26) + 16 * 7])
def test_probe_read_chunked_sums_every_word(x, nbytes):
    rng = np.random.default_rng(37)
    words = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    src = torch.from_numpy(words.view(np.int32)).cuda()
    out = torch.zeros(x.PROBE_THREADS, dtype=torch.int32, device="cuda")
    x.probe_read_chunked(src, out)
    torch.cuda.synchronize()
    got = int(out.cpu().numpy().view(np.uint32).astype(np.uint64).sum()) % (1 << 32)
    assert got == int(words.astype(np.uint64).sum()) % (1 << 32)
