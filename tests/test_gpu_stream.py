"""GPU check of tq_stream_read (the read-ceiling measurement helper): the
XOR of the sink words equals the XOR of every 16-byte word of the buffer,
for sizes below one block's share, ragged against the grid, and large ones;
sink words past the launched blocks are left untouched."""
import sys

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def env():
    import torch
    import bit_gemv_tq_amd as tq
    return torch, tq


@pytest.mark.parametrize("nbytes", [16, 4096 + 16, 32768 * 3 + 48, 3 << 20, 64 << 20])
def test_stream_read_xor(env, nbytes):
    torch, tq = env
    print(f"stream_read bytes={nbytes}", flush=True)
    sys.stdout.flush()
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.full((4096, 4), 0, dtype=torch.int32, device="cuda")
    tq.tq_stream_read(buf, sink)
    torch.cuda.synchronize()
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32), axis=0)
    want = np.bitwise_xor.reduce(host.reshape(-1, 4), axis=0)
    np.testing.assert_array_equal(got, want)


def test_stream_read_small_sink(env):
    # two sink words: the grid shrinks to two blocks, the rest is untouched
    torch, tq = env
    host = np.arange((1 << 20) // 4, dtype=np.uint32) * np.uint32(2654435761)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.full((5, 4), 7, dtype=torch.int32, device="cuda")
    tq.tq_stream_read(buf, sink[:2])
    torch.cuda.synchronize()
    s = sink.cpu().numpy().view(np.uint32)
    np.testing.assert_array_equal(np.bitwise_xor.reduce(s[:2], axis=0),
                                  np.bitwise_xor.reduce(host.reshape(-1, 4), axis=0))
    assert np.all(s[2:] == 7)
