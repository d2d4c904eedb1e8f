"""The measurement aids: the read probe reads every 16-byte piece of its buffer exactly once (the
XOR of its per-workgroup results equals the XOR of all words, computed on the host); the hand-off
skeleton writes every partial word as its header defines it and reads every partial back; and the
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


@pytest.mark.parametrize("nbytes,n_groups,part_bytes",
                         [(16, 1, 16), (4096 + 48, 130, 16384),
                          ((8 << 20) + 16 * 777, 257, 16384 + 128)])
def test_handoff_writes_and_reads_every_partial(nbytes, n_groups, part_bytes):
    say(f"hand-off skeleton {nbytes} bytes, {n_groups} groups, {part_bytes}-byte partials")
    g = torch.Generator().manual_seed(nbytes + n_groups)
    host = torch.randint(-(1 << 31), (1 << 31) - 1, (nbytes // 4,), dtype=torch.int64,
                         generator=g).to(torch.int32)
    buf = host.to(DEV)
    parts = torch.zeros(n_groups * part_bytes // 4, dtype=torch.int32, device=DEV)
    out = torch.full((W.WMTP_PROBE_HANDOFF_BLOCKS,), -1, dtype=torch.int32, device=DEV)
    W.wmtp_probe_handoff(buf, n_groups, parts, part_bytes, out)
    # expected partials: group g folds its share of 16-byte words into c_g, word i = (c_g+i, g, i, 0)
    words = host.numpy().view(np.uint32)
    n16, part16 = nbytes // 16, part_bytes // 16
    chunk = -(-n16 // n_groups)
    i = np.arange(part16, dtype=np.uint64)
    want = np.zeros((n_groups, part16, 4), dtype=np.uint32)
    for grp in range(n_groups):
        beg = min(grp * chunk, n16)
        end = min(beg + chunk, n16)
        c = int(np.bitwise_xor.reduce(words[4 * beg:4 * end])) if end > beg else 0
        want[grp, :, 0] = ((c + i) & 0xFFFFFFFF).astype(np.uint32)
        want[grp, :, 1] = grp
        want[grp, :, 2] = (i & 0xFFFFFFFF).astype(np.uint32)
    got = parts.cpu().numpy().view(np.uint32).reshape(n_groups, part16, 4)
    assert np.array_equal(got, want)
    assert (np.bitwise_xor.reduce(out.cpu().numpy().view(np.uint32))
            == np.bitwise_xor.reduce(want.reshape(-1)))


def test_flush_writes_every_byte():
    say("llc flush 8 MiB + 16")
    buf = torch.zeros((8 << 20) + 16, dtype=torch.uint8, device=DEV)
    W.wmtp_llc_flush(buf, 0xA5)
    assert bool((buf == 0xA5).all())
