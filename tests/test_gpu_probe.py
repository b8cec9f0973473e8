"""The measurement helpers on the GPU (bench.py's read ceiling and launch
cost): every read mode and depth completes, and the loads really read the
buffer (a 16-byte buffer whose four words fold to the sink value makes the
reading thread write it)."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

MAGIC = 0x9E3779B9


@pytest.fixture(scope="module")
def q4k():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from quantized_decode_q4_amd import q4k as mod
    return mod


@pytest.mark.parametrize("contiguous", [False, True])
@pytest.mark.parametrize("depth", [1, 2, 4, 8, 16])
def test_probe_read_reads_the_data(q4k, depth, contiguous):
    words = np.array([MAGIC, 0, 0, 0], np.uint32)
    buf = torch.from_numpy(words.view(np.uint8).copy()).cuda()
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    q4k.q4k_probe_read(buf, 16, 1, 64, depth, contiguous, sink)
    torch.cuda.synchronize()
    assert int(sink.cpu().numpy().view(np.uint32)[0]) == MAGIC


@pytest.mark.parametrize("contiguous", [False, True])
@pytest.mark.parametrize("grid,threads,depth", [(256, 512, 8), (2048, 1024, 16), (7, 64, 1)])
def test_probe_read_large_buffers_complete(q4k, grid, threads, depth, contiguous):
    nbytes = 64 << 20
    buf = torch.ones(nbytes, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda")
    q4k.q4k_probe_read(buf, nbytes, grid, threads, depth, contiguous, sink)
    q4k.q4k_probe_empty(grid, 256, sink)
    torch.cuda.synchronize()
    assert int(sink.cpu()[0]) == 0      # the fold of all-ones words is never the magic value
