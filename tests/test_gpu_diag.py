"""The HBM-ceiling diagnostic (pact_debug_stream) moves exactly the bytes it
is asked to: chunk c of the output is the xor of the source chunks its thread
read up to c, which a numpy model of the launch (one iteration per thread at
these sizes: workgroups of 256 threads, 4 chunks of 16 bytes each, 256 apart)
reproduces.  This is a measurement tool, not part of the data flow, so there
is no oracle function for it."""
import numpy as np
import pytest
import torch

from nvfp4_gemm_amd import pact as pb

pytestmark = pytest.mark.gpu


def _model(src_words: np.ndarray, nr: int, nw: int) -> np.ndarray:
    n = max(nr, nw)
    blocks = -(-n // 1024)
    s = np.zeros((blocks * 1024, 4), dtype=np.uint32)
    s[:nr] = src_words.reshape(-1, 4)[:nr]
    acc = np.bitwise_xor.accumulate(s.reshape(blocks, 4, 256, 4), axis=1)
    return acc.reshape(-1, 4)[:nw]


@pytest.mark.parametrize("nr,nw", [(64 * 1024, 64 * 1024), (1000, 1500), (1500, 1000), (0, 4096)])
def test_stream_writes_thread_xor(nr, nw):
    rng = np.random.default_rng(nr + 7 * nw)
    words = rng.integers(0, 2**32, size=max(nr, 1) * 4, dtype=np.uint32)
    src = torch.from_numpy(words.view(np.int32).copy()).cuda()
    dst = torch.full((max(nw, 1) * 4,), -1, dtype=torch.int32, device="cuda")
    pb.pact_debug_stream(src if nr else None, 16 * nr, dst, 16 * nw)
    torch.cuda.synchronize()
    got = dst.cpu().numpy().view(np.uint32).reshape(-1, 4)[:nw]
    np.testing.assert_array_equal(got, _model(words, nr, nw))


def test_stream_read_only_leaves_dst():
    src = torch.zeros(1 << 18, dtype=torch.int32, device="cuda")
    dst = torch.full((4,), 123, dtype=torch.int32, device="cuda")
    pb.pact_debug_stream(src, src.numel() * 4, dst, 0)
    torch.cuda.synchronize()
    assert dst.cpu().tolist() == [123] * 4
