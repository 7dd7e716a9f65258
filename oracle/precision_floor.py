"""How far bf16 storage alone moves the looped LM from its fp32 self.

Test infrastructure only (like the rest of this package).  Run as

    python -m oracle.precision_floor [huginn|ouro] [--each]

The pages run their models in bfloat16 ("Depth-adaptive Inference of Looped
Language Models via Continuous Depth Batching", §6.1 Setup).  A bf16 path
keeps weights, the KV cache and the inputs of every projection in bf16 and
accumulates in fp32.  This module subclasses the oracle so that it rounds
exactly those values to bf16 -- K and V as they enter the cache, the
normalised activations before the QKV and gate/up projections, the attention
output before the output projection, the SwiGLU product before the down
projection -- and otherwise computes as the fp32 oracle does.  It decodes
the same prompts under forced replay of the fp32 oracle's own tokens and
exits and reports the largest exit-state (relative, norm-wise) and logit
(absolute) departure.  That departure is the floor any bf16 implementation
of the path sits on, whatever its kernels do.
"""
from __future__ import annotations

import sys

import numpy as np

import cdb_synth as S
from .layers import attend, rmsnorm, rope
from .model import OracleLM


def _bf(x):
    return S.bf16_round(np.asarray(x, np.float32)).astype(np.float32)


POINTS = ("kv", "qkv_in", "o_in", "gu_in", "down_in", "lm_in")
# the bf16 matrix-core prefill attention additionally stores the scaled
# queries (pf_q) and the unnormalised probabilities before the P.V product
# (pf_p) in bf16; the softmax denominator keeps the fp32 probabilities
PREFILL_POINTS = ("pf_q", "pf_p")


def _attend_rounded(q, K, V, round_q, round_p):
    """Softmax attention of one query per head (as oracle.layers.attend) with
    the scaled query and the unnormalised probabilities of the numerator
    rounded to bf16."""
    hd = q.shape[-1]
    qs = q / q.dtype.type(np.sqrt(hd))
    if round_q:
        qs = _bf(qs)
    s = np.einsum("hd,nhd->hn", qs, K)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    num = _bf(p) if round_p else p
    return np.einsum("hn,nhd->hd", num, V) / p.sum(axis=-1, keepdims=True)


class Bf16StorageLM(OracleLM):
    """The oracle with bf16 rounding at the storage points of a bf16 path:
    K/V entering the cache (kv), the inputs of the QKV, output, gate/up and
    down projections (qkv_in, o_in, gu_in, down_in) and of the LM head
    (lm_in).  ``points`` selects which are rounded (default: all of them, as
    the bf16 path stores each in bf16)."""

    def __init__(self, *a, points=POINTS, **k):
        super().__init__(*a, **k)
        self.points = set(points)

    def _r(self, name, x):
        return _bf(x) if name in self.points else x

    def _block(self, x, positions, prefix, put_kv, get_kv):
        d, w, eps = self.d, self.w, self.d.rms_eps
        T = x.shape[0]
        xn = self._r("qkv_in", rmsnorm(x, w[prefix + ".attn_norm"], eps))
        q = rope(xn @ w[prefix + ".wq"].T, positions, d.head_dim, d.rope_theta)
        k = rope(xn @ w[prefix + ".wk"].T, positions, d.head_dim, d.rope_theta)
        v = xn @ w[prefix + ".wv"].T
        put_kv(self._r("kv", k).reshape(T, d.n_heads, d.head_dim), self._r("kv", v).reshape(T, d.n_heads, d.head_dim))
        o = np.empty((T, d.qdim), dtype=self.dt)
        qh = q.reshape(T, d.n_heads, d.head_dim)
        # prefill rows (a chunk of several positions) take the matrix-core
        # attention's extra rounding points when selected
        rq, rp = T > 1 and "pf_q" in self.points, T > 1 and "pf_p" in self.points
        for i in range(T):
            K, V = get_kv(i)
            o[i] = (_attend_rounded(qh[i], K, V, rq, rp) if (rq or rp) else attend(qh[i], K, V)).reshape(-1)
        x = x + self._r("o_in", o) @ w[prefix + ".wo"].T
        xn = self._r("gu_in", rmsnorm(x, w[prefix + ".mlp_norm"], eps))
        g = xn @ w[prefix + ".wg"].T
        u = xn @ w[prefix + ".wu"].T
        a = self._r("down_in", g / (1.0 + np.exp(-g)) * u)
        return x + a @ w[prefix + ".wd"].T

    def lm_head(self, x):
        xn = self._r("lm_in", rmsnorm(x, self.w["final_norm"], self.d.rms_eps))
        return xn @ self.w["lm_head"].T


CASES = {
    # Huginn-like widths, one prelude / core / coda layer, injection
    "huginn": (S.ModelDims("t", vocab=4096, hidden=5280, n_heads=55, head_dim=96, ffn=17920, n_prelude=1,
                           n_core=1, n_coda=1, r_max=3, dtype="bf16", inject=True, gate_bias=0.0), [300, 41]),
    # Ouro-like widths, one core layer
    "ouro": (S.ModelDims("t", vocab=512, hidden=2048, n_heads=16, head_dim=128, ffn=5632, n_prelude=0,
                         n_core=1, n_coda=0, r_max=3, dtype="bf16", gate_bias=0.0), [300, 41]),
    # the full Ouro-like model (24 core layers, r_max 4, calibrated gate) on
    # the shortest prompt of the C2 mix (139 tokens), 6 outputs
    "c2short": (S.CONFIGS["c2"], [139], 6),
}


def floor(d, prompt_lens, n_out=4, seed=0, points=POINTS):
    w = S.make_weights(d, seed=seed)
    prompts = S.make_prompts(d.vocab, prompt_lens, seed=seed + 1)
    ref = OracleLM(d, w, dtype=np.float32, keep_logits=True)
    low = Bf16StorageLM(d, w, dtype=np.float32, keep_logits=True, points=points)
    ws = wl = sd = 0.0
    for p in prompts:
        t, e, r0 = ref.decode_sequential(p, n_out, keep_state=True)
        _, _, r1 = low.decode_sequential(p, n_out, keep_state=True, forced_tokens=t[:-1], forced_exits=e)
        for g in range(1, n_out):
            a, b = r1[g].exit_state, r0[g].exit_state
            ws = max(ws, float(np.linalg.norm(a - b) / np.linalg.norm(b)))
            wl = max(wl, float(np.abs(r1[g].logits - r0[g].logits).max()))
            sd = max(sd, float(np.std(r0[g].logits)))
    return dict(state_rel=ws, logit_abs=wl, logit_std=sd)


if __name__ == "__main__":
    # python -m oracle.precision_floor [huginn|ouro|c2short] [--each]: all
    # points (with and without the prefill attention's), or (--each) every
    # storage point alone, then all of them
    args = [x for x in sys.argv[1:] if not x.startswith("--")]
    each = "--each" in sys.argv
    for name in (args or ["huginn", "ouro"]):
        d, lens, n_out = (CASES[name] + (4,))[:3]
        sets = [(p,) for p in POINTS + PREFILL_POINTS] if each else []
        sets += [POINTS, POINTS + PREFILL_POINTS]
        for pts in sets:
            print(name, ",".join(pts), floor(d, lens, n_out=n_out, points=pts), flush=True)
