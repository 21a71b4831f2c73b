"""kvq_issue_probe runs every instruction mix through the C ABI and writes
exactly its n_blocks x 256 words (measurement kernel; bench.py --issue-probe
times it)."""
import pytest
import torch

from decode_attention_select_amd import kvq

pytestmark = pytest.mark.gpu

SENTINEL = 0x5A5A5A5A


@pytest.mark.parametrize("kind", range(7))
def test_issue_probe_writes_its_words_only(kind):
    nb = 4
    print("issue probe kind %d, %d blocks" % (kind, nb), flush=True)
    out = torch.full((nb * 256 + 1024,), SENTINEL, dtype=torch.int32, device="cuda")
    kvq.kvq_issue_probe(kind, nb, out)
    torch.cuda.synchronize()
    o = out.cpu()
    assert (o[nb * 256:] == SENTINEL).all(), "words past the launch were written"
    # each thread stores a word folded from its registers: (almost) none is the fill
    assert (o[:nb * 256] != SENTINEL).sum() >= nb * 256 - 4
