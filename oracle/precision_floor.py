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
        for i in range(T):
            K, V = get_kv(i)
            o[i] = attend(qh[i], K, V).reshape(-1)
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
    # python -m oracle.precision_floor [huginn|ouro] [--each]: all points, or
    # (--each) every storage point alone, then all of them
    args = [x for x in sys.argv[1:] if not x.startswith("--")]
    each = "--each" in sys.argv
    for name in (args or ["huginn", "ouro"]):
        d, lens = CASES[name]
        for pts in ([(p,) for p in POINTS] + [POINTS]) if each else [POINTS]:
            print(name, ",".join(pts), floor(d, lens, points=pts), flush=True)
