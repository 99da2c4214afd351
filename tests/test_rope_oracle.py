"""Pins of the bias + rotary epilogue oracle (CPU): the rotation is a rotation
(norms kept, position 0 with a unit table is the identity), composes by adding
angles, matches the complex-number form, and leaves v alone; bias is additive."""
from __future__ import annotations

import numpy as np

from oracle.rope import qkv_bias_rope
from gqa_attention_head_amd import workloads as W


def plain_table(rows, d, theta=10000.0):
    inv = theta ** (-np.arange(0, d // 2) * 2.0 / d)
    ang = np.arange(rows)[:, None] * inv[None, :]
    return np.concatenate([np.cos(ang), np.sin(ang)], axis=1)


def test_identity_at_position_zero_and_bias_additive():
    rng = np.random.default_rng(0)
    qkv = rng.standard_normal((5, (4 + 2 * 2) * 64))
    bias = rng.standard_normal((4 + 2 * 2) * 64)
    tab = plain_table(8, 64)
    q, k, v = qkv_bias_rope(qkv, bias, np.zeros(5, int), tab, 4, 2)
    x = (qkv + bias).reshape(5, 8, 64)
    assert np.array_equal(q, x[:, :4]) and np.array_equal(k, x[:, 4:6]) and np.array_equal(v, x[:, 6:])


def test_rotation_keeps_pair_norms_and_matches_complex_form():
    rng = np.random.default_rng(1)
    qkv = rng.standard_normal((7, (2 + 2 * 1) * 64))
    pos = rng.integers(0, 100, 7)
    tab = plain_table(100, 64)
    q, k, v = qkv_bias_rope(qkv, np.zeros(4 * 64), pos, tab, 2, 1)
    x = qkv.reshape(7, 4, 64)
    z = x[:, :3, :32] + 1j * x[:, :3, 32:]
    ang = pos[:, None] * (10000.0 ** (-np.arange(32) * 2.0 / 64))[None, :]
    zr = z * np.exp(1j * ang)[:, None, :]
    got = np.concatenate([q, k], axis=1)
    assert np.abs(got[..., :32] - zr.real).max() <= 1e-12
    assert np.abs(got[..., 32:] - zr.imag).max() <= 1e-12
    assert np.allclose(np.abs(got[..., :32] + 1j * got[..., 32:]), np.abs(z), rtol=1e-13, atol=0)
    assert np.array_equal(v, x[:, 3:])


def test_angles_compose():
    """Rotating by p then by p' equals rotating by p + p' (a table with linear angles)."""
    rng = np.random.default_rng(2)
    qkv = rng.standard_normal((3, 3 * 64))
    tab = plain_table(64, 64)
    q1, k1, _ = qkv_bias_rope(qkv, np.zeros(3 * 64), np.full(3, 5), tab, 1, 1)
    again = np.concatenate([q1.reshape(3, 64), k1.reshape(3, 64), np.zeros((3, 64))], axis=1)
    q2, k2, _ = qkv_bias_rope(again, np.zeros(3 * 64), np.full(3, 7), tab, 1, 1)
    q3, k3, _ = qkv_bias_rope(qkv, np.zeros(3 * 64), np.full(3, 12), tab, 1, 1)
    assert np.abs(q2 - q3).max() <= 1e-12 and np.abs(k2 - k3).max() <= 1e-12


def test_positions_clamped_to_table():
    rng = np.random.default_rng(3)
    qkv = rng.standard_normal((2, 3 * 64))
    tab = plain_table(10, 64)
    a = qkv_bias_rope(qkv, np.zeros(3 * 64), np.array([-4, 99]), tab, 1, 1)
    b = qkv_bias_rope(qkv, np.zeros(3 * 64), np.array([0, 9]), tab, 1, 1)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_yarn_table_reduces_to_plain_rope_without_scaling():
    """The seeded YaRN table builder with factor 1 is the plain rotary table."""
    tab = W.yarn_table(64, 64, theta=150000.0, factor=1.0, original_max=4096, beta_fast=32.0,
                       beta_slow=1.0)
    assert np.abs(tab - plain_table(64, 64, 150000.0)).max() <= 1e-6
