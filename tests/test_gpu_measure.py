"""The plain streaming-read helper (tq_stream_read) reads every byte it is given: the XOR of its
per-wavefront folds equals the XOR of all 32-bit words of the buffer (exact, integer)."""

import numpy as np
import pytest
import torch

import dequant_gemv_tq_amd as tqa

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096, 1 << 20, (37 << 20) + 48])
def test_stream_read_folds_every_word(nbytes):
    g = torch.Generator(device="cuda")
    g.manual_seed(nbytes)
    buf = torch.randint(-(1 << 31), (1 << 31) - 1, (nbytes // 4 + 64,), dtype=torch.int32, device="cuda", generator=g)
    sink = torch.zeros(tqa.STREAM_READ_SINK_WORDS, dtype=torch.int32, device="cuda")
    tqa.stream_read(buf, nbytes, sink=sink)
    torch.cuda.synchronize()
    words = buf[: nbytes // 4].cpu().numpy().view(np.uint32)
    want = np.bitwise_xor.reduce(words)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32))
    assert got == want
