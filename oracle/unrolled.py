"""An independently written plain deep transformer used to pin the oracle.

Test infrastructure only (see the package docstring).

"Depth-adaptive Inference of Looped Language Models via Continuous Depth
Batching", §2 Problem Setup: a p-c-q looped model run for r loops executes
p + c*r + q transformer layers.  With the exit gate switched off (every token
at r_max), the looped LM is therefore exactly a plain (p + c*r_max + q)-layer
transformer whose core layers repeat with tied weights, where every unrolled
layer keeps its own KV — which is what the depth-indexed cache of §4.2 stores
(one slot per loop step).  This module computes that plain transformer over a
whole token sequence at once (teacher forcing, full causal attention), in
float64 with torch CPU ops and a complex-number form of the rotary embedding,
sharing no code with ``oracle.model``.  With additive injection (the
Huginn-like configuration) every core layer group adds the prelude output to
its input and the first group starts from zero.
"""
from __future__ import annotations

import numpy as np
import torch


def _norm(x, g, eps):
    return x * torch.rsqrt((x * x).mean(-1, keepdim=True) + eps) * g


def _rotary(x, n_heads, head_dim, theta):
    """x: [T, n_heads*head_dim].  Pairs (i, i + head_dim/2) form the complex
    number a + ib, multiplied by exp(i * pos * theta^(-2i/head_dim))."""
    T = x.shape[0]
    half = head_dim // 2
    xh = x.view(T, n_heads, 2, half)
    z = torch.complex(xh[:, :, 0, :], xh[:, :, 1, :])
    freq = theta ** (-(torch.arange(half, dtype=torch.float64) * 2.0) / head_dim)
    ang = torch.arange(T, dtype=torch.float64)[:, None] * freq[None, :]
    z = z * torch.polar(torch.ones_like(ang), ang)[:, None, :]
    return torch.stack([z.real, z.imag], dim=2).reshape(T, n_heads * head_dim)


def _layer(x, w, pre, d):
    T = x.shape[0]
    t = lambda n: torch.from_numpy(np.asarray(w[pre + n], dtype=np.float64))
    a = _norm(x, t(".attn_norm"), d.rms_eps)
    q = _rotary(a @ t(".wq").T, d.n_heads, d.head_dim, d.rope_theta)
    k = _rotary(a @ t(".wk").T, d.n_heads, d.head_dim, d.rope_theta)
    v = a @ t(".wv").T
    q = q.view(T, d.n_heads, d.head_dim).transpose(0, 1)
    k = k.view(T, d.n_heads, d.head_dim).transpose(0, 1)
    v = v.view(T, d.n_heads, d.head_dim).transpose(0, 1)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
    x = x + o.transpose(0, 1).reshape(T, -1) @ t(".wo").T
    m = _norm(x, t(".mlp_norm"), d.rms_eps)
    g = m @ t(".wg").T
    return x + ((g * torch.sigmoid(g)) * (m @ t(".wu").T)) @ t(".wd").T


def unrolled_forward(d, w, tokens, loops: int):
    """Hidden states after the last core layer (before any coda layer) and
    the logits, for every position of ``tokens``, with the core unrolled
    ``loops`` times.  Returns (core_out [T, H], logits [T, V]) as float64."""
    with torch.no_grad():
        ids = torch.as_tensor(np.asarray(tokens, dtype=np.int64))
        x = torch.from_numpy(np.asarray(w["embed"], dtype=np.float64))[ids]
        for i in range(d.n_prelude):
            x = _layer(x, w, f"prelude.{i}", d)
        inj = x if d.inject else None
        h = torch.zeros_like(x) if d.inject else x
        for _ in range(loops):
            if inj is not None:
                h = h + inj
            for i in range(d.n_core):
                h = _layer(h, w, f"core.{i}", d)
        core_out = h
        for i in range(d.n_coda):
            h = _layer(h, w, f"coda.{i}", d)
        gf = torch.from_numpy(np.asarray(w["final_norm"], dtype=np.float64))
        logits = _norm(h, gf, d.rms_eps) @ torch.from_numpy(np.asarray(w["lm_head"], dtype=np.float64)).T
        return core_out.numpy(), logits.numpy()


def unrolled_forward_exits(d, w, tokens, exits):
    """The same unrolled transformer with per-position exit depths: position
    j runs ``exits[j]`` loops, and in every later loop the other positions
    see it through the K/V it produced in its last loop ("Depth-adaptive
    Inference of Looped Language Models via Continuous Depth Batching",
    §4.2: the skipped depth slots of a token hold its last-exited KV).

    Teacher forcing over the whole sequence: loop r runs the core layers on
    all positions at once; in layer l of loop r a position with exits[j] < r
    contributes the K/V it produced in layer l of loop exits[j] (kept aside
    when it ran that loop); its own state stops at loop exits[j].  The coda
    layers (own single K/V per position) then run on the exit states.
    Depth-indexed layout only.  Returns (exit states [T, H], logits [T, V])
    as float64."""
    ex = torch.as_tensor(np.asarray(exits, dtype=np.int64))
    T = ex.shape[0]
    R = int(ex.max())
    with torch.no_grad():
        ids = torch.as_tensor(np.asarray(tokens, dtype=np.int64))
        x = torch.from_numpy(np.asarray(w["embed"], dtype=np.float64))[ids]
        for i in range(d.n_prelude):
            x = _layer(x, w, f"prelude.{i}", d)
        inj = x if d.inject else None
        h = torch.zeros_like(x) if d.inject else x
        out = torch.zeros_like(h)
        kept = {}                                  # (layer, loop) -> (K, V) of every position
        for r in range(1, R + 1):
            if inj is not None:
                h = h + inj
            for i in range(d.n_core):
                h = _layer_frozen(h, w, f"core.{i}", d, ex, r, i, kept)
            done = ex == r
            out[done] = h[done]
        h = out
        for i in range(d.n_coda):
            h = _layer(h, w, f"coda.{i}", d)
        gf = torch.from_numpy(np.asarray(w["final_norm"], dtype=np.float64))
        logits = _norm(h, gf, d.rms_eps) @ torch.from_numpy(np.asarray(w["lm_head"], dtype=np.float64)).T
        return out.numpy(), logits.numpy()


def _layer_frozen(x, w, pre, d, ex, r, li, kept):
    """_layer for loop r where positions that left before loop r attend as
    they were in their exit loop (their K/V from kept[(li, ex_j)])."""
    T = x.shape[0]
    t = lambda n: torch.from_numpy(np.asarray(w[pre + n], dtype=np.float64))
    a = _norm(x, t(".attn_norm"), d.rms_eps)
    q = _rotary(a @ t(".wq").T, d.n_heads, d.head_dim, d.rope_theta)
    k = _rotary(a @ t(".wk").T, d.n_heads, d.head_dim, d.rope_theta)
    v = a @ t(".wv").T
    kept[(li, r)] = (k.clone(), v.clone())
    for j in range(T):
        e = int(ex[j])
        if e < r:
            k[j], v[j] = kept[(li, e)][0][j], kept[(li, e)][1][j]
    q = q.view(T, d.n_heads, d.head_dim).transpose(0, 1)
    k = k.view(T, d.n_heads, d.head_dim).transpose(0, 1)
    v = v.view(T, d.n_heads, d.head_dim).transpose(0, 1)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
    x = x + o.transpose(0, 1).reshape(T, -1) @ t(".wo").T
    m = _norm(x, t(".mlp_norm"), d.rms_eps)
    g = m @ t(".wg").T
    return x + ((g * torch.sigmoid(g)) * (m @ t(".wu").T)) @ t(".wd").T
