"""Pins of the oracle's elementary layers against closed forms, hand values
and independent routines (CPU only)."""
import math

import numpy as np
import pytest
import torch

from oracle.layers import attend, attend_bruteforce, rmsnorm, rope, silu, swiglu_mlp

pytestmark = pytest.mark.cpu


def test_rmsnorm_hand_value_and_gain():
    x = np.array([[3.0, 4.0, 0.0]])
    g = np.array([1.0, 2.0, 3.0])
    rms = math.sqrt(25.0 / 3.0)
    y = rmsnorm(x, g, 0.0)
    np.testing.assert_allclose(y[0], [3.0 / rms, 8.0 / rms, 0.0], rtol=1e-15)


def test_rmsnorm_scale_invariance_and_eps():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((5, 64))
    g = rng.standard_normal(64)
    np.testing.assert_allclose(rmsnorm(7.5 * x, g, 0.0), rmsnorm(x, g, 0.0), rtol=1e-12)
    # eps enters under the root: a zero vector stays zero, a constant vector c
    # maps to g * c / sqrt(c^2 + eps)
    c = np.full((1, 8), 1e-3)
    np.testing.assert_allclose(rmsnorm(c, np.ones(8), 1e-6)[0], 1e-3 / math.sqrt(1e-6 + 1e-6), rtol=1e-12)


def test_rope_identity_at_zero_and_hand_rotation():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((1, 8))
    np.testing.assert_allclose(rope(x, np.array([0]), 8, 10000.0), x, rtol=0, atol=0)
    # head_dim 4, theta 100: frequencies 1 and 100^(-1/2) = 0.1; pairs (0,2), (1,3)
    e0 = np.array([[1.0, 0.0, 0.0, 0.0]])
    y = rope(e0, np.array([2]), 4, 100.0)
    np.testing.assert_allclose(y[0], [math.cos(2.0), 0.0, math.sin(2.0), 0.0], atol=1e-15)
    e1 = np.array([[0.0, 1.0, 0.0, 0.0]])
    y = rope(e1, np.array([3]), 4, 100.0)
    np.testing.assert_allclose(y[0], [0.0, math.cos(0.3), 0.0, math.sin(0.3)], atol=1e-15)


def test_rope_relative_position_property():
    rng = np.random.default_rng(2)
    hd, nh = 16, 2
    q = rng.standard_normal((1, nh * hd))
    k = rng.standard_normal((1, nh * hd))
    def dot(m, n):
        a = rope(q, np.array([m]), hd, 10000.0).reshape(nh, hd)
        b = rope(k, np.array([n]), hd, 10000.0).reshape(nh, hd)
        return (a * b).sum(-1)
    np.testing.assert_allclose(dot(5, 2), dot(105, 102), rtol=1e-10)
    # rotation preserves the norm of each head
    y = rope(q, np.array([12345]), hd, 10000.0).reshape(nh, hd)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), np.linalg.norm(q.reshape(nh, hd), axis=-1), rtol=1e-12)


def test_silu_values():
    z = np.array([0.0, 1.0, -1.0, 30.0, -30.0])
    y = silu(z)
    np.testing.assert_allclose(y[:3], [0.0, 1 / (1 + math.e ** -1), -1 / (1 + math.e)], rtol=1e-15)
    assert abs(y[3] - 30.0) < 1e-9 and abs(y[4]) < 1e-9


def test_swiglu_matches_explicit_loops():
    rng = np.random.default_rng(3)
    H, F = 6, 5
    x = rng.standard_normal((2, H))
    wg, wu, wd = rng.standard_normal((F, H)), rng.standard_normal((F, H)), rng.standard_normal((H, F))
    out = swiglu_mlp(x, wg, wu, wd)
    for r in range(2):
        a = []
        for f in range(F):
            g = sum(x[r, i] * wg[f, i] for i in range(H))
            u = sum(x[r, i] * wu[f, i] for i in range(H))
            a.append(g / (1 + math.exp(-g)) * u)
        for o in range(H):
            assert abs(out[r, o] - sum(a[f] * wd[o, f] for f in range(F))) < 1e-12


def test_attend_vs_bruteforce():
    rng = np.random.default_rng(4)
    nh, hd, n = 3, 5, 7
    q = rng.standard_normal((nh, hd))
    K = rng.standard_normal((n, nh, hd))
    V = rng.standard_normal((n, nh, hd))
    np.testing.assert_allclose(attend(q, K, V), np.array(attend_bruteforce(q.tolist(), K.tolist(), V.tolist())), rtol=1e-12)


def test_attend_special_cases():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((2, 4))
    K = rng.standard_normal((1, 2, 4))
    V = rng.standard_normal((1, 2, 4))
    np.testing.assert_allclose(attend(q, K, V), V[0], rtol=1e-15)       # one position: output = V
    K = np.repeat(rng.standard_normal((1, 2, 4)), 6, axis=0)             # equal keys: mean of V
    V = rng.standard_normal((6, 2, 4))
    np.testing.assert_allclose(attend(q, K, V), V.mean(axis=0), rtol=1e-12)


def test_attend_matches_torch_causal_sdpa():
    rng = np.random.default_rng(6)
    nh, hd, T = 2, 8, 9
    Q = rng.standard_normal((T, nh, hd))
    K = rng.standard_normal((T, nh, hd))
    V = rng.standard_normal((T, nh, hd))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(Q).transpose(0, 1), torch.from_numpy(K).transpose(0, 1),
        torch.from_numpy(V).transpose(0, 1), is_causal=True).transpose(0, 1).numpy()
    for i in range(T):
        np.testing.assert_allclose(attend(Q[i], K[: i + 1], V[: i + 1]), ref[i], rtol=1e-12, atol=1e-14)
