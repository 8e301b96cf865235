"""The machine-ceiling probes (bit_quantized_routed_amd/csrc/moe_probe.h) run and read what they
claim to read.  They compute nothing of the layer; the benchmark uses them to
report rates against what this machine sustains."""
import numpy as np
import pytest
import torch

import bit_quantized_routed_amd as M
from gpu_common import need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def test_stream_probe_reads_every_word():
    n = (1 << 20) + 4096                       # not a multiple of the launch's stride
    host = np.random.default_rng(5).integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.uint8)).cuda()
    for grid in (1, 7, 256):
        for nt in (False, True):
            sink = torch.zeros(grid * 512 * 4, dtype=torch.int32, device="cuda")
            M.probe_stream_read(buf, grid, sink, nt)
            torch.cuda.synchronize()
            got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32).reshape(-1, 4), axis=0)
            want = np.bitwise_xor.reduce(host.reshape(-1, 4), axis=0)
            assert np.array_equal(got, want), (grid, nt)


@pytest.mark.parametrize("shape,elems,kdim", [(0, 4, 32), (1, 16, 16)])
def test_mfma_probe_runs(shape, elems, kdim):
    sink = torch.zeros(8 * 256, dtype=torch.float32, device="cuda")
    M.probe_mfma_loop(shape, 8, 3, sink)
    torch.cuda.synchronize()
    s = sink.cpu().numpy()
    # every lane sums 8 accumulators x `elems` elements of 3 rounds of `kdim` products of ~1
    want = 8 * elems * 3 * kdim
    assert np.all(np.isfinite(s)) and np.all(s > 0.9 * want) and np.all(s < 1.1 * want)
