"""Pins for the oracle's numeric building blocks (CPU only).

Each check compares against something other than the oracle itself: a
library routine, a textbook special case, a closed form or an exhaustive
enumeration.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import (logsumexp, rms_norm, rope, rope_angles, round_bf16, silu,
                    softmax)


def _bf16_bits_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint32) << 16).view(np.float32).astype(
        np.float64)


def test_round_bf16_matches_torch_on_f32_inputs():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(200000) * 10.0 ** rng.integers(-40, 38, 200000),
        rng.standard_normal(1000),
        np.array([0.0, -0.0, 1e-45, -1e-45, 3.4e38, 1.0 + 2.0 ** -8]),
    ]).astype(np.float32)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    got = round_bf16(x.astype(np.float64))
    np.testing.assert_array_equal(got, want)


def test_round_bf16_exhaustive_midpoints():
    # Every pair of adjacent positive finite bf16 values: the exact midpoint
    # rounds to the even neighbour, anything strictly inside rounds to the
    # nearer one.  Negative values mirror.
    bits = np.arange(0, 0x7F7F, dtype=np.uint32)
    lo, hi = _bf16_bits_to_f64(bits), _bf16_bits_to_f64(bits + 1)
    mid = (lo + hi) / 2.0                         # exact in float64
    even = np.where(bits % 2 == 0, lo, hi)
    np.testing.assert_array_equal(round_bf16(mid), even)
    below = np.nextafter(mid, -np.inf)
    above = np.nextafter(mid, np.inf)
    np.testing.assert_array_equal(round_bf16(below), lo)
    np.testing.assert_array_equal(round_bf16(above), hi)
    np.testing.assert_array_equal(round_bf16(-mid), -even)
    np.testing.assert_array_equal(round_bf16(lo), lo)


def test_round_bf16_double_rounding_case():
    # 1 + 2^-8 + 2^-40: nearest-even to f32 alone gives 1 + 2^-8 (a bf16
    # tie that would round down to 1.0); the true nearest bf16 is 1 + 2^-7.
    x = 1.0 + 2.0 ** -8 + 2.0 ** -40
    assert round_bf16(np.array([x]))[0] == 1.0 + 2.0 ** -7


@pytest.mark.parametrize("gain", ["ones", "random"])
def test_rms_norm_matches_torch(gain):
    rng = np.random.default_rng(1)
    x = rng.standard_normal((7, 96)) * 3.0
    g = np.ones(96) if gain == "ones" else rng.uniform(0.5, 1.5, 96)
    want = F.rms_norm(torch.from_numpy(x), (96,), weight=torch.from_numpy(g),
                      eps=1e-6).numpy()
    np.testing.assert_allclose(rms_norm(x, g, 1e-6), want, rtol=1e-13,
                               atol=1e-13)


def test_silu_softmax_logsumexp_match_torch():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 333)) * 6.0
    t = torch.from_numpy(x)
    np.testing.assert_allclose(silu(x), F.silu(t).numpy(), rtol=1e-14,
                               atol=1e-15)
    np.testing.assert_allclose(softmax(x), torch.softmax(t, -1).numpy(),
                               rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(logsumexp(x), torch.logsumexp(t, -1).numpy(),
                               rtol=1e-14)


def test_rope_two_dims_is_plane_rotation():
    # d = 2: one pair with inverse frequency theta^0 = 1, so position p is a
    # rotation of the plane by p radians (counter-clockwise).
    x = np.array([[[0.3, -1.7]]])
    for p in [0, 1, 5, 1000]:
        got = rope(x, np.array([p]), 1e6)[0, 0]
        c, s = np.cos(p), np.sin(p)
        rot = np.array([[c, -s], [s, c]])
        np.testing.assert_allclose(got, rot @ x[0, 0], rtol=1e-13, atol=1e-15)


def test_rope_equals_complex_multiplication():
    # Rotate-half RoPE is multiplication of z_i = x_i + 1j * x_{i+d/2}
    # by exp(1j * p * theta^(-2i/d)).
    rng = np.random.default_rng(3)
    d, theta = 64, 1e6
    x = rng.standard_normal((9, 3, d))
    pos = rng.integers(0, 40000, 9)
    z = x[..., : d // 2] + 1j * x[..., d // 2:]
    inv = theta ** (-np.arange(0, d, 2) / d)
    zr = z * np.exp(1j * pos[:, None, None] * inv[None, None, :])
    want = np.concatenate([zr.real, zr.imag], axis=-1)
    np.testing.assert_allclose(rope(x, pos, theta), want, rtol=1e-12,
                               atol=1e-12)


def test_rope_identities():
    rng = np.random.default_rng(4)
    d, theta = 128, 1e6
    q = rng.standard_normal((1, 1, d))
    k = rng.standard_normal((1, 1, d))
    # R(0) = I
    np.testing.assert_array_equal(rope(q, np.array([0]), theta), q)
    # norm preserved
    for p in [1, 77, 32783]:
        assert np.isclose(np.linalg.norm(rope(q, np.array([p]), theta)),
                          np.linalg.norm(q), rtol=1e-13)
    # <R(p) q, R(p') k> depends only on p - p'
    dots = []
    for p in [10, 500, 20000]:
        a = rope(q, np.array([p]), theta).ravel()
        b = rope(k, np.array([p - 7]), theta).ravel()
        dots.append(a @ b)
    np.testing.assert_allclose(dots, dots[0], rtol=1e-10)
    ang = rope_angles(np.array([3]), d, theta)
    assert ang.shape == (1, d // 2) and ang[0, 0] == 3.0
