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


def test_bf16_rounding_is_nearest_even():
    """The library's float32 -> bfloat16 store rounding against a host
    round-to-nearest-even of the same bit patterns: random normals over the
    whole exponent range, subnormals, exact ties (both parities), values that
    round up into the next binade or to infinity, signed zeros and infinities;
    NaN must stay NaN."""
    import numpy as np
    from activation_sparse_feed_amd import workloads as wl
    sffn = _sffn()
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 2**32, size=1 << 18, dtype=np.uint64).astype(np.uint32)
    ties = (rng.integers(0, 2**16, size=4096, dtype=np.uint64).astype(np.uint32) << 16) | 0x8000
    special = np.array([0x00000000, 0x80000000, 0x00000001, 0x807FFFFF, 0x00008000, 0x00018000,
                        0x3F7FFFFF, 0x3F808000, 0x3F818000, 0x7F7FFFFF, 0x7F7F8000, 0xFF7F8000,
                        0x7F800000, 0xFF800000], dtype=np.uint32)
    u = np.concatenate([bits, ties, special])
    u = u[(u & 0x7FFFFFFF) <= 0x7F800000]  # finite and infinite inputs
    x = torch.from_numpy(u.view(np.float32).copy()).cuda()
    out = torch.empty(x.numel(), dtype=torch.int16, device="cuda")
    sffn.probe_bf16_round(x, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    # the host reference handles finite inputs; infinities map to themselves
    fin = (u & 0x7FFFFFFF) < 0x7F800000
    want = np.where(fin, wl.f32_to_bf16_bits(np.where(fin, u, 0).view(np.float32)),
                    (u >> 16).astype(np.uint16))
    bad = np.nonzero(got != want)[0]
    assert len(bad) == 0, [(hex(u[i]), hex(got[i]), hex(want[i])) for i in bad[:8]]
    nan = torch.tensor([float("nan"), -float("nan")], dtype=torch.float32, device="cuda")
    nout = torch.empty(2, dtype=torch.int16, device="cuda")
    sffn.probe_bf16_round(nan, nout)
    torch.cuda.synchronize()
    nb = nout.cpu().numpy().view(np.uint16)
    assert np.all((nb & 0x7F80) == 0x7F80) and np.all((nb & 0x7F) != 0)
