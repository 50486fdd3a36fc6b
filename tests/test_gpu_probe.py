"""The read-bandwidth probe reads every byte once: its per-workgroup word sums add up (mod 2^32)
to the buffer's word sum."""

import numpy as np
import pytest

from gpu_util import announce

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.mark.parametrize("words,groups", [(4, 1), (1000, 7), (1 << 20, 256), ((64 << 20) + 12, 1024)])
def test_probe_reads_every_word(words, groups):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import activation_sparse_decode_relu_amd as pi
    announce(f"read probe: {words} words, {groups} workgroups")
    rng = np.random.default_rng(words)
    host = rng.integers(0, 2 ** 32, size=words, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sums = torch.zeros(groups, dtype=torch.int32, device="cuda")
    pi.probe_read(buf, sums)
    torch.cuda.synchronize()
    got = int(sums.cpu().numpy().view(np.uint32).astype(np.uint64).sum() % (1 << 32))
    assert got == int(host.astype(np.uint64).sum() % (1 << 32))
