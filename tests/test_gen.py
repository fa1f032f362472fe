"""The seeded generator: host properties, and host/device bit-identity."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from looped_transformer_latent_amd import gen


def test_host_generator_is_deterministic_and_counter_based():
    a = gen.normal_f32(5, 7, 1000)
    b = gen.normal_f32(5, 7, np.arange(1000, dtype=np.uint64))
    assert np.array_equal(a, b)
    c = gen.normal_f32(5, 7, np.array([999, 3], dtype=np.uint64))
    assert c[0] == a[999] and c[1] == a[3]
    assert not np.array_equal(a, gen.normal_f32(5, 8, 1000))
    assert not np.array_equal(a, gen.normal_f32(6, 7, 1000))


def test_host_generator_distribution():
    v = gen.normal_f32(1, 1, 400000, scale=2.0).astype(np.float64)
    assert abs(v.mean()) < 0.02 and abs(v.std() - 2.0) < 0.02
    assert np.abs(v).max() <= 2.0 * 3.4642
    k = ((v / 2.0) ** 4).mean()
    assert 2.6 < k < 3.0  # Irwin-Hall(4): kurtosis 2.7 (a normal has 3)


def test_bf16_rounding_matches_torch():
    v = gen.normal_f32(2, 3, 100000, scale=7.0)
    v = np.concatenate([v, np.float32([0.0, -0.0, np.inf, -np.inf, 3.4e38])])
    want = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(gen.f32_to_bf16_bits(v), want)


@pytest.mark.gpu
@pytest.mark.parametrize("bf16", [False, True])
def test_device_generator_matches_host_bits(bf16):
    from looped_transformer_latent_amd import lla
    n = 3_000_001
    t = torch.empty(n, dtype=torch.bfloat16 if bf16 else torch.float32, device="cuda")
    lla.gen_normal_(t, 1234, 77, scale=0.37, offset=5)
    torch.cuda.synchronize()
    got = (t.view(torch.int16).cpu().numpy().view(np.uint16) if bf16 else t.cpu().numpy())
    idx = np.concatenate([np.arange(1000), np.random.default_rng(0).integers(0, n, 5000), [n - 1]])
    want = gen.normal_f32(1234, 77, (idx + 5).astype(np.uint64), scale=0.37)
    if bf16:
        want = gen.f32_to_bf16_bits(want)
        assert np.array_equal(got[idx], want)
    else:
        assert np.array_equal(got[idx].view(np.uint32), want.view(np.uint32))
