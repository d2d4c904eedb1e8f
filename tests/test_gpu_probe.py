"""The measurement aids: the read probe reads every 16-byte piece of its buffer exactly once (the
XOR of its per-workgroup results equals the XOR of all words, computed on the host), and the
flush writes every byte of its buffer."""
import numpy as np
import pytest
import torch

from draft_attention_amd import binding as W
from gpu_common import DEV, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (64 << 20) + 16 * 12345])
def test_probe_reads_every_word_once(nbytes):
    say(f"read probe {nbytes} bytes")
    g = torch.Generator().manual_seed(nbytes)
    host = torch.randint(-(1 << 31), (1 << 31) - 1, (nbytes // 4 + 64,), dtype=torch.int64,
                         generator=g).to(torch.int32)
    buf = host.to(DEV)
    out = torch.full((W.WMTP_PROBE_BLOCKS,), -1, dtype=torch.int32, device=DEV)
    W.wmtp_probe_read(buf, out, nbytes)
    got = np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
    want = np.bitwise_xor.reduce(host[:nbytes // 4].numpy().view(np.uint32))
    assert got == want


def test_flush_writes_every_byte():
    say("llc flush 8 MiB + 16")
    buf = torch.zeros((8 << 20) + 16, dtype=torch.uint8, device=DEV)
    W.wmtp_llc_flush(buf, 0xA5)
    assert bool((buf == 0xA5).all())
