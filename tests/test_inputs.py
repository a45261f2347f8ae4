"""Seeded input generator: determinism, bf16 rounding, distributions."""

import numpy as np
import pytest
import torch

from synth import CONFIGS, bf16_bits, bf16_round, bits_to_f32, get_config, make_inputs


def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(1000) * 1e-30).astype(np.float32),
        (rng.standard_normal(1000) * 1e30).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 1.00390625, 1.01171875, 3.0e38], dtype=np.float32),
    ])
    # values exactly half-way between two bf16 neighbours (ties to even)
    base = bits_to_f32(np.arange(0x3F80, 0x3F90, dtype=np.uint16))
    half = (base.view(np.uint32) + 0x8000).view(np.float32)
    x = np.concatenate([x, half])
    ours = bf16_bits(x)
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)
    assert np.array_equal(bf16_round(x), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generator_is_deterministic_and_ordered():
    c = CONFIGS["pages_check_t129"]
    x1 = make_inputs(c)
    x2 = make_inputs(c)
    for n in ("q", "k", "v", "do", "a", "r"):
        assert np.array_equal(getattr(x1, n), getattr(x2, n))
    # draw order: Q, K, V, dO, then a, then r noise (float32 standard normals)
    rng = np.random.default_rng(c.seed)
    q = bf16_round(rng.standard_normal((c.B, c.H, c.T, c.D), dtype=np.float32))
    assert np.array_equal(q.reshape(x1.q.shape), x1.q)
    for _ in range(3):
        rng.standard_normal((c.B, c.H, c.T, c.D), dtype=np.float32)
    a = rng.standard_normal((c.H, c.Tp), dtype=np.float32)
    assert np.array_equal(a, x1.a)
    assert x1.a.shape == (c.H, 192) and x1.r.dtype == np.float32
    assert list(x1.frozen) == [0, 1, 0, 1]


def test_distributions_tiny_and_headline():
    x = make_inputs(get_config(0))
    assert x.q.dtype == np.float32 and x.do is not None
    d = np.arange(x.cfg.Tp)
    resid = x.r + 0.05 * d
    assert abs(resid.std() - 0.5) < 0.05
    c1 = get_config(1)
    assert (c1.B, c1.H, c1.T, c1.D, c1.frozen) == (8, 12, 4096, 64, (9, 10, 11))
    small = c1.with_(B=1, H=12, T=256)
    x1 = make_inputs(small)
    assert abs(x1.q.std() - 0.125) < 0.01
    assert np.array_equal(bf16_round(x1.q), x1.q)


def test_peaked_r_is_deterministic():
    c = get_config(4).with_(T=64)
    x = make_inputs(c)
    assert x.do is None
    expect = np.where(np.arange(64) < 8, 3.0, -0.01 * np.arange(64)).astype(np.float32)
    for h in range(c.H):
        assert np.array_equal(x.r[h], expect)
