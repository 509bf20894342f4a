"""The read-bandwidth probe reads every word it is given: the XOR of its
per-workgroup folds equals the XOR of all 32-bit words of the buffer
(NumPy), for an empty buffer, one piece, a size with a ragged tail beyond the
unrolled loop, and 64 MiB."""
import numpy as np
import pytest
import torch

from medusa_tree_verification_amd import api
from helpers import announce

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("nbytes", [0, 16, 4096 * 16 * 9 + 48, 64 << 20])
def test_read_probe_reads_every_word(nbytes):
    rng = np.random.default_rng(nbytes)
    words = rng.integers(0, 2 ** 32, size=nbytes // 4, dtype=np.uint64).astype(np.uint32)
    buf = torch.from_numpy(words.view(np.int32)).to(DEV)
    announce("read probe", nbytes)
    parts = api.read_probe(buf)
    torch.cuda.synchronize()
    got = int(np.bitwise_xor.reduce(parts.cpu().numpy().view(np.uint32)))
    expect = int(np.bitwise_xor.reduce(words)) if words.size else 0
    assert got == expect
