"""Pins of the closed forms (CPU only): Eq. 1, Eq. 2, Eq. 3/4 fits and the
App. E.1 KV footprint against Table 4's printed values."""
import numpy as np
import pytest

from oracle.bounds import (fit_depth_linear, fit_latency, kv_bytes_per_token, s_dec,
                           s_dec_tokens, s_e2e, saturation_batch)
from tests.conftest import read_tsv

pytestmark = pytest.mark.cpu


def test_table4_kv_footprint():
    for model, layout, slots, kib, gib, l0, lr, kv_dim in read_tsv("table4_kv_footprint.tsv"):
        b = kv_bytes_per_token(int(l0), int(lr), int(slots), int(kv_dim))
        # the table prints KiB rounded to an integer and GiB to two decimals
        assert abs(b / 1024 - float(kib)) <= 0.5, (model, layout, b / 1024)
        assert abs(b * 4096 / 2 ** 30 - float(gib)) <= 0.005, (model, layout, b * 4096 / 2 ** 30)


def test_sharing_factor_of_e1():
    # single-slot shrinks the cache 4x for Ouro and 8.5x for Huginn (App. E.1)
    assert kv_bytes_per_token(0, 24, 4, 2048) / kv_bytes_per_token(0, 24, 1, 2048) == 4.0
    assert kv_bytes_per_token(4, 4, 16, 5280) / kv_bytes_per_token(4, 4, 1, 5280) == 8.5


def test_eq1_bound_properties():
    assert s_dec(0.0, 1.0, 4, 2.5) == pytest.approx(4 / 2.5)           # F0 = 0 reaches r_max/d
    for F0 in (0.1, 1.0, 10.0):
        assert s_dec(F0, 1.0, 4, 2.5) < 4 / 2.5
    assert s_dec(3.0, 1.0, 4, 4.0) == 1.0                               # no exits, no speedup
    # per-token form reduces to Eq. 1 when costs are equal
    assert s_dec_tokens([2.0] * 5, [1.0] * 5, 4, [2, 3, 4, 2, 3]) == pytest.approx(s_dec(2.0, 1.0, 4, 2.8))


def test_eq2_limits():
    assert s_e2e(0.0, 1.7) == pytest.approx(1.7)
    assert s_e2e(1.0, 1.7) == pytest.approx(1.0)
    a, s = 0.3, 1.6
    assert s_e2e(a, s) == pytest.approx(1.0 / (0.3 + 0.7 / 1.6))
    assert 1.0 < s_e2e(a, s) < s


def test_latency_fits_recover_parameters():
    delta, gamma, alpha = 5.4e-3, 2.0e-5, 3.0e-8
    B = np.array([1, 2, 4, 8, 16, 32, 64, 1, 8, 64], dtype=float)
    L = np.array([128] * 7 + [8192] * 3, dtype=float)
    t = delta + gamma * B + alpha * B * L
    d2, g2, a2 = fit_latency(B, L, t)
    assert d2 == pytest.approx(delta) and g2 == pytest.approx(gamma) and a2 == pytest.approx(alpha)
    assert saturation_batch(delta, gamma, alpha, 128) == pytest.approx(delta / (gamma + alpha * 128))
    t0, tr, r2 = fit_depth_linear([1, 2, 3, 4], [0.4 + 1.5 * r for r in [1, 2, 3, 4]])
    assert t0 == pytest.approx(0.4) and tr == pytest.approx(1.5) and r2 == pytest.approx(1.0)
