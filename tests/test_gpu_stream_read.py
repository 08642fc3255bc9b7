"""The streaming reader that bench.py measures the weight streams against
(q8s_stream_read): it reads every byte it is given once, so the xor of the
words it writes equals the xor of the buffer's 32-bit words, for sizes that
fill whole rounds of its loads and for ragged ones."""
import numpy as np
import pytest
import torch

import q8_gemv_sparse_amd as q8

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 3 << 20, (64 << 20) + 48])
def test_stream_read_reads_every_word_once(nbytes):
    print("[case] q8s_stream_read %d bytes" % nbytes, flush=True)
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).cuda()
    out = q8.q8s_stream_read(buf)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    assert got == np.bitwise_xor.reduce(words)
    # a prefix only
    half = (nbytes // 32) * 16
    if half:
        out = q8.q8s_stream_read(buf, nbytes=half)
        torch.cuda.synchronize()
        assert np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32)) == np.bitwise_xor.reduce(words[:half // 4])
