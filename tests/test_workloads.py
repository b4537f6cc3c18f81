"""The seeded input generator: determinism, bf16 rounding, row recipes."""
import numpy as np
import torch

from activation_sparse_feed_amd import workloads as wl


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.00390625, 1.01171875, -1.00390625, 3e-39, 65504.0,
                                  0.0, -0.0], np.float32)])
    ours = wl.f32_to_bf16_bits(a)
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = wl.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(a).to(torch.bfloat16).float().numpy())


def test_generation_is_deterministic_and_seeded_per_tensor():
    w = wl.WORKLOADS["tiny_f32"]
    a, b = wl.generate(w), wl.generate(w)
    for n in ("x", "wg_t", "wu_t", "wd", "b_g"):
        assert np.array_equal(getattr(a, n), getattr(b, n))
    assert not np.array_equal(a.wg_t, a.wu_t)
    assert a.x.dtype == np.float32 and a.x.shape == (64, 256)
    assert a.wg_t.shape == (1024, 256) and a.wd.shape == (1024, 256)
    assert np.all(a.b_g == np.float32(-2.054))


def test_variances_follow_fan_in():
    w = wl.WORKLOADS["prefill_1pct"].replace(T=256)
    inp = wl.generate(w)
    assert inp.x.dtype == np.uint16
    assert abs(inp.as_f64("x").var() - 1.0) < 0.02
    assert abs(inp.as_f64("wg_t").var() * 2048 - 1.0) < 0.02
    assert abs(inp.as_f64("wd").var() * 5632 - 1.0) < 0.02


def test_row_recipes():
    mix = wl.WORKLOADS["hybrid_mix"]
    s = wl.row_scales(mix)
    assert (s > 1).sum() == 41 and np.all(s[s > 1] == np.float32(3.8))
    ln = wl.WORKLOADS["large_lognormal"].replace(T=20000)
    s = wl.row_scales(ln)
    assert abs(np.log(s).std() - 0.35) < 0.01 and abs(np.median(s) - 1) < 0.01
