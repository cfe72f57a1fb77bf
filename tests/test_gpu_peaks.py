"""The measurement helpers on the GPU: the read stream reads every 16-byte
word exactly once (the xor of its per-thread results equals the xor of the
buffer, also for a size that leaves the last block short), and the MFMA loop
runs and writes finite sums."""
import numpy as np
import pytest
import torch

from mixture_experts_layer_14_amd import binding as B

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("words,blocks", [(1, 1), (4096, 8), (1000003, 97), (1 << 22, 1024)])
def test_read_stream_reads_each_word_once(words, blocks):
    rng = np.random.default_rng(words)
    host = rng.integers(0, 2 ** 32, size=words * 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(blocks * 256, dtype=torch.int32, device="cuda")
    B.moe_peak_read(buf, blocks, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(host)


def test_mfma_loop_runs():
    sink = torch.full((8 * 256,), float("nan"), dtype=torch.float32, device="cuda")
    B.moe_peak_mfma_bf16(16, 8, sink)
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all()
