"""The streaming-read probe reads every byte of its buffer exactly once.

Its digest is recomputed on the host from the definition in the header:
16-byte element e is loaded by lane e mod 256 of workgroup (e / 1024) mod
256, which XORs the element's four 32-bit words into its digest word.  A
skipped, repeated or misplaced load changes some word.
"""

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import sparse_draft_speculative_amd as sd
    sd.load()
    return sd


def expected_digest(words):
    """words: uint32 [n16 * 4] host copy of the buffer."""
    w = words.reshape(-1, 4)
    elem = w[:, 0] ^ w[:, 1] ^ w[:, 2] ^ w[:, 3]
    e = np.arange(elem.size, dtype=np.int64)
    slot = 256 * ((e // 1024) % 256) + (e % 256)
    out = np.zeros(65536, dtype=np.uint32)
    np.bitwise_xor.at(out, slot, elem)
    return out


@pytest.mark.parametrize("n16", [1, 1024, 1024 * 256, 1024 * 256 * 3 + 1024 * 5 + 3,
                                 1024 * 700 + 777])
def test_probe_digest(lib, n16):
    g = torch.Generator().manual_seed(n16)
    host = torch.randint(-2 ** 31, 2 ** 31 - 1, (n16 * 4,), dtype=torch.int32, generator=g)
    print(f"probe n16={n16}", flush=True)
    sink = lib.std_hbm_read_probe(host.cuda())
    torch.cuda.synchronize()
    got = sink.cpu().numpy().view(np.uint32)
    ref = expected_digest(host.numpy().view(np.uint32))
    assert np.array_equal(got, ref)
