"""Scalar building blocks of the oracle, in float64.

The pages fix none of these details; the readings taken are: RMSNorm with a gain, rotate-half RoPE with inverse frequencies
theta^(-2i/d), SiLU-gated MLP, softmax in float64, and bf16 storage rounding
to nearest-even at the points where the drafter stores bf16 tensors.
"""
from __future__ import annotations

import numpy as np


def identity_round(x):
    """Storage rounding of an f32 drafter: none (the oracle keeps float64)."""
    return np.asarray(x, dtype=np.float64)


def round_bf16(x):
    """Round float64 values to the nearest bf16 value, ties to even.

    Done in two steps that together are exact: float64 -> float32 with
    round-to-odd (truncate toward zero, then force the last bit to 1 if any
    discarded bit was set), then float32 -> bf16 with round-to-nearest-even
    on the upper 16 bits.  Round-to-odd into a format with at least two more
    bits than the target makes the second rounding equal to a direct one.
    """
    x = np.asarray(x, dtype=np.float64)
    f = x.astype(np.float32)                       # nearest-even
    back = f.astype(np.float64)
    over = np.abs(back) > np.abs(x)                # rounded away from zero
    f = np.where(over, np.nextafter(f, np.float32(0.0)), f)
    bits = np.ascontiguousarray(f).view(np.uint32).astype(np.uint64)
    inexact = f.astype(np.float64) != x
    bits = np.where(inexact, bits | np.uint64(1), bits)
    lsb = (bits >> np.uint64(16)) & np.uint64(1)
    bits = (bits + np.uint64(0x7FFF) + lsb) & np.uint64(0xFFFF0000)
    out = bits.astype(np.uint32).view(np.float32).astype(np.float64)
    return out.reshape(x.shape)


def rms_norm(x, g, eps):
    """x / sqrt(mean(x^2) + eps) * g over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(g, dtype=np.float64)


def silu(x):
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))


def rope_angles(pos, head_dim, theta):
    """Rotation angle pos * theta^(-2i/d) for i in [0, d/2): shape [..., d/2]."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    inv_freq = theta ** (-2.0 * i / head_dim)
    return np.asarray(pos, dtype=np.float64)[..., None] * inv_freq


def rope(x, pos, theta):
    """Rotary position embedding, rotate-half pairing (i, i + d/2).

    x: [..., n_pos, heads, d] with pos: [n_pos]; each pair
    (x_i, x_{i+d/2}) is rotated by the angle of position pos and index i.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = rope_angles(pos, d, theta)[..., None, :]       # [n_pos, 1, d/2]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def logsumexp(z, axis=-1):
    z = np.asarray(z, dtype=np.float64)
    m = np.max(z, axis=axis, keepdims=True)
    return (m + np.log(np.sum(np.exp(z - m), axis=axis, keepdims=True))
            ).squeeze(axis)


def softmax(z, axis=-1):
    z = np.asarray(z, dtype=np.float64)
    m = np.max(z, axis=axis, keepdims=True)
    e = np.exp(z - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def decode_e4m3(codes):
    """Values of FP8 E4M3 codes (the OCP 8-bit float: 1 sign bit, 4 exponent
    bits with bias 7, 3 mantissa bits, no infinities, S.1111.111 is NaN).

    exponent field e > 0: (-1)^s * (1 + m/8) * 2^(e - 7)
    exponent field e = 0: (-1)^s * (m/8) * 2^(-6)   (subnormal)
    """
    c = np.asarray(codes).astype(np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e > 0, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0),
                   (m / 8.0) * 2.0 ** -6)
    val = sign * val
    return np.where((c & 0x7F) == 0x7F, np.nan, val)


def dequant_rows(codes, scale):
    """Weights stored as E4M3 codes with one float32 scale per output row
    (row-major [out, in]): w[j, k] = scale[j] * value(codes[j, k])."""
    return decode_e4m3(codes) * np.asarray(scale, dtype=np.float64)[:, None]
