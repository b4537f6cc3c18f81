"""GPU checks of the peak probes (sffn_probe_hbm, sffn_probe_mfma): the copy
moves every byte, including a ragged tail past the four-chunk unroll, the
read-only pass runs, and every MFMA of the compute probe ran (each lane's sum
is 2048 * iters exactly)."""
from __future__ import annotations

import pytest
import torch

pytestmark = pytest.mark.gpu


def _sffn():
    from activation_sparse_feed_amd import sffn
    return sffn


@pytest.mark.parametrize("n16,wgs", [(1, 1), (4 * 256 * 3 + 17, 3), (1 << 20, 64)])
def test_probe_hbm_copies_every_byte(n16, wgs):
    sffn = _sffn()
    g = torch.Generator(device="cuda").manual_seed(n16)
    src = torch.randint(-2**31, 2**31 - 1, (n16 * 4,), dtype=torch.int32, device="cuda", generator=g)
    dst = torch.zeros_like(src)
    sffn.probe_hbm(src, dst, workgroups=wgs)
    sffn.probe_hbm(src, None, workgroups=wgs)  # read-only pass
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_probe_mfma_counts_every_instruction():
    sffn = _sffn()
    out = torch.full((8 * 256,), -1.0, dtype=torch.float32, device="cuda")
    sffn.probe_mfma(out, iters=100)
    torch.cuda.synchronize()
    assert torch.all(out == 2048.0 * 100)
