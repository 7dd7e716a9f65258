"""Closed forms of the pages.  Test infrastructure only.

"Depth-adaptive Inference of Looped Language Models via Continuous Depth
Batching" (arXiv 2608.09444):

* Eq. 1 (§5): FLOP-based decode speedup bound of adaptive over fixed depth,
  S_dec = (F0 + r_max F_r) / (F0 + d_bar F_r) <= r_max / d_bar.
* Eq. 2 (§5): prefill-corrected bound S_e2e = 1 / (alpha + (1 - alpha)/S_dec)
  with alpha the measured prefill share of time.
* §5 latency model t(N_c, N_b) = delta + gamma N_b + alpha N_c and Eq. 4
  (App. B): at context L, t(B) = delta + (gamma + alpha L) B, saturation
  B* = delta / (gamma + alpha L).
* Eq. 3 (App. B): tau(r) = tau_0 + tau_r r.
* App. E.1 and Table 4: a cache with s KV slots per recurrent layer holds
  l_0 + l_r s KV entries per token; each entry is K and V of kv_dim values.
"""
from __future__ import annotations

from typing import Sequence, Tuple

import numpy as np


def s_dec(F0: float, Fr: float, r_max: float, d_bar: float) -> float:
    """Eq. 1."""
    return (F0 + r_max * Fr) / (F0 + d_bar * Fr)


def s_dec_tokens(F0: Sequence[float], Fr: Sequence[float], r_max: int, depths: Sequence[int]) -> float:
    """Eq. 1 summed over tokens whose per-token costs differ (each token t
    with boundary cost F0[t], per-loop cost Fr[t] and exit depth depths[t])."""
    F0 = np.asarray(F0, dtype=np.float64)
    Fr = np.asarray(Fr, dtype=np.float64)
    d = np.asarray(depths, dtype=np.float64)
    return float((F0 + r_max * Fr).sum() / (F0 + d * Fr).sum())


def s_e2e(alpha: float, sdec: float) -> float:
    """Eq. 2."""
    return 1.0 / (alpha + (1.0 - alpha) / sdec)


def fit_depth_linear(r: Sequence[float], tau: Sequence[float]) -> Tuple[float, float, float]:
    """Least-squares fit of Eq. 3; returns (tau_0, tau_r, R^2)."""
    r = np.asarray(r, dtype=np.float64)
    tau = np.asarray(tau, dtype=np.float64)
    A = np.stack([np.ones_like(r), r], axis=1)
    coef, *_ = np.linalg.lstsq(A, tau, rcond=None)
    pred = A @ coef
    ss_res = float(((tau - pred) ** 2).sum())
    ss_tot = float(((tau - tau.mean()) ** 2).sum())
    return float(coef[0]), float(coef[1]), 1.0 - ss_res / ss_tot if ss_tot > 0 else 1.0


def fit_latency(B: Sequence[float], L: Sequence[float], t: Sequence[float]) -> Tuple[float, float, float]:
    """Least-squares fit of t = delta + gamma B + alpha B L (Eq. 4 with N_b =
    B and N_c = B L); returns (delta, gamma, alpha)."""
    B = np.asarray(B, dtype=np.float64)
    L = np.asarray(L, dtype=np.float64)
    t = np.asarray(t, dtype=np.float64)
    A = np.stack([np.ones_like(B), B, B * L], axis=1)
    coef, *_ = np.linalg.lstsq(A, t, rcond=None)
    return float(coef[0]), float(coef[1]), float(coef[2])


def saturation_batch(delta: float, gamma: float, alpha: float, L: float) -> float:
    """B* = delta / (gamma + alpha L) (App. B)."""
    return delta / (gamma + alpha * L)


def kv_bytes_per_token(l0: int, lr: int, slots: int, kv_dim: int, bytes_per: int = 2) -> int:
    """(l_0 + l_r s) KV entries per token, each K and V of kv_dim values."""
    return (l0 + lr * slots) * 2 * kv_dim * bytes_per
