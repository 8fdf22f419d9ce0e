"""The benchmark's streaming probe (ssd_stream_probe) on the GPU: every mix writes the sum of
its source arrays to each destination array, with cached and non-temporal accesses."""
import os
import sys

import pytest
import torch

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

from mamba_ssd_chunked_amd import ssd  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("nt", [False, True])
@pytest.mark.parametrize("nr,nw", [(6, 1), (4, 1), (3, 1), (2, 1), (1, 1), (0, 1), (1, 0)])
def test_stream_probe_moves_the_sums(nr, nw, nt):
    n16 = 70000  # more than one grid-stride pass at the largest grid, with a ragged tail
    g = torch.Generator().manual_seed(5 + nr)
    src = torch.randint(-8, 8, (max(nr, 1), n16, 4), generator=g).float().cuda()
    dst = torch.full((max(nw, 1), n16, 4), 7.0, device="cuda")
    rc = ssd.ssd_stream_probe(nr, nw, nt, src[:nr].reshape(-1) if nr else None, dst.reshape(-1), n16)
    assert rc == 0, ssd.ssd_last_error()
    torch.cuda.synchronize()
    want = src[:nr].sum(0) if nr else torch.zeros(n16, 4, device="cuda")
    if nw == 0:
        assert torch.all(dst == 7.0)  # nothing written (the sums of small integers are never 1e30)
    else:
        for a in range(nw):
            assert torch.equal(dst[a], want)
