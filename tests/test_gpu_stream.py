"""The plain streaming read behind the one-token kernel's measured ceiling
(ttq_stream_read): it must read every byte once, which its per-workgroup XOR
words show bit for bit against a host computation."""
import numpy as np
import pytest

pytestmark = pytest.mark.gpu

BLOCK = 128 * 1024


@pytest.mark.parametrize("nbytes", [16, 4096, BLOCK, 3 * BLOCK + 4096 + 16,
                                    32 * 1024 * 1024])
def test_stream_read_touches_every_word(nbytes):
    import torch
    import online_activation_aware_ttq_amd as ttq
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint32)
    print(f"[case] stream_read bytes={nbytes}", flush=True)
    src = torch.from_numpy(host.view(np.int32)).cuda()
    sink = ttq.stream_read(src)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    nblk = -(-nbytes // BLOCK)
    words = BLOCK // 4
    want = np.array([np.bitwise_xor.reduce(host[b * words:(b + 1) * words])
                     for b in range(nblk)], dtype=np.uint32)
    assert got.shape[0] == nblk
    assert np.array_equal(got, want)
