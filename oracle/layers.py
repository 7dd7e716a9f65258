"""Elementary transformer pieces of the looped LM, written plainly in numpy.

Test infrastructure only (see the package docstring).

The pages describe the architecture only at the level of stages and layers
("Depth-adaptive Inference of Looped Language Models via Continuous Depth
Batching", §2 Problem Setup); the layer internals below are the plainest
reading of a pre-norm Llama-style block with a SwiGLU MLP, RMSNorm with
epsilon 1e-6, rotary embedding with theta 10000 in rotate-half pairing, and
causal multi-head softmax attention scaled by 1/sqrt(head_dim).  Multi-head
(not grouped) K/V follows from the KV footprint of Table 4 (App. E.1), which
needs kv_dim equal to the hidden size.
"""
from __future__ import annotations

import numpy as np


def rmsnorm(x: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """y = g * x / sqrt(mean(x^2) + eps) over the last axis."""
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return (x / np.sqrt(ms + x.dtype.type(eps))) * g


def rope_cos_sin(positions: np.ndarray, head_dim: int, theta: float, dtype):
    """cos and sin of the rotary angles pos * theta^(-2i/head_dim) for
    i < head_dim/2.  Angles are formed and evaluated in float64 and then
    rounded once to the compute dtype, so large positions lose no accuracy
    to the product."""
    half = head_dim // 2
    inv = theta ** (-(2.0 * np.arange(half, dtype=np.float64)) / head_dim)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]
    return np.cos(ang).astype(dtype), np.sin(ang).astype(dtype)


def rope(x: np.ndarray, positions: np.ndarray, head_dim: int, theta: float) -> np.ndarray:
    """Rotate-half rotary embedding of x[T, n_heads*head_dim] at positions[T].

    Within each head the pair (x_i, x_{i+half}) is rotated by the angle of
    element i: (a, b) -> (a cos - b sin, b cos + a sin)."""
    T = x.shape[0]
    half = head_dim // 2
    xh = x.reshape(T, -1, head_dim)
    c, s = rope_cos_sin(positions, head_dim, theta, x.dtype)
    c = c[:, None, :]
    s = s[:, None, :]
    a = xh[..., :half]
    b = xh[..., half:]
    out = np.concatenate([a * c - b * s, b * c + a * s], axis=-1)
    return out.reshape(T, -1)


def silu(z: np.ndarray) -> np.ndarray:
    return z / (z.dtype.type(1.0) + np.exp(-z))


def swiglu_mlp(xn: np.ndarray, wg: np.ndarray, wu: np.ndarray, wd: np.ndarray) -> np.ndarray:
    """down( silu(x W_g^T) * (x W_u^T) ); weights are [out][in]."""
    return (silu(xn @ wg.T) * (xn @ wu.T)) @ wd.T


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Softmax attention of one query per head over n cached positions.

    q: [n_heads, hd]; K, V: [n, n_heads, hd].  Returns [n_heads, hd].
    Scores are scaled by 1/sqrt(hd); the softmax subtracts the row max."""
    hd = q.shape[-1]
    s = np.einsum("hd,nhd->hn", q, K) / q.dtype.type(np.sqrt(hd))
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    return np.einsum("hn,nhd->hd", p, V)


def attend_bruteforce(q, K, V):
    """The same attention as ``attend`` written as explicit loops in float64
    (for tiny inputs only)."""
    import math
    nh, hd = len(q), len(q[0])
    n = len(K)
    out = [[0.0] * hd for _ in range(nh)]
    for h in range(nh):
        scores = []
        for j in range(n):
            acc = 0.0
            for t in range(hd):
                acc += float(q[h][t]) * float(K[j][h][t])
            scores.append(acc / math.sqrt(hd))
        m = max(scores)
        ws = [math.exp(x - m) for x in scores]
        tot = sum(ws)
        for t in range(hd):
            acc = 0.0
            for j in range(n):
                acc += ws[j] * float(V[j][h][t])
            out[h][t] = acc / tot
    return out
