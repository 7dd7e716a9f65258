"""Seeded synthetic inputs shared by the oracle and the HIP path.

This module holds *inputs only*: model shapes, seeded weight tensors, prompt
token ids, request-length mixes, synthetic KV contents and exit-depth maps.
It contains none of the method's arithmetic (no norm, attention, gate or
scheduling logic), so that the oracle under ``oracle/`` and the product
under ``continuous_depth_batching_amd/`` share nothing beyond their inputs.

Shapes follow the looped-LM split of "Depth-adaptive Inference of Looped
Language Models via Continuous Depth Batching" (arXiv 2608.09444, §2 Problem
Setup): a prelude of ``n_prelude`` layers, a shared core of ``n_core`` layers
looped up to ``r_max`` times, and a coda of ``n_coda`` layers.  A 0-N-0 model
has only the embedding before and the LM head after the core.

Weight layout (both sides): every projection matrix is ``[out][in]``
row-major; norm gains and the gate vector are length-``hidden`` vectors.
In bf16 mode every tensor is rounded to bfloat16 (round to nearest, ties to
even) and both sides receive exactly those values.
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field
from typing import Dict, List, Optional

import numpy as np

__all__ = [
    "ModelDims", "Workload", "CONFIGS", "WORKLOADS", "bf16_round", "bf16_bits",
    "bits_to_f32", "tensor_order", "make_weights", "make_prompts",
    "make_prompt_lengths", "make_context_exit_depths", "c1_row_depths",
]


@dataclass(frozen=True)
class ModelDims:
    """Shape and fixed scalars of a looped LM.

    gate_bias is the calibrated scalar b of the exit gate
    z = w . RMSNorm(h) + b; gate_threshold is the logit threshold t (the gate
    fires when z > t; t = 0 is probability threshold 0.5).  gate_kind
    "convergence" replaces it by the training-free criterion: after loop
    d >= 2 the gate fires when |h_d - h_{d-1}| / |h_d| < conv_threshold.
    """
    name: str
    vocab: int
    hidden: int
    n_heads: int
    head_dim: int
    ffn: int
    n_prelude: int
    n_core: int
    n_coda: int
    r_max: int
    dtype: str                    # "fp32" or "bf16"
    inject: bool = False          # core input = h + e each loop (Huginn-like)
    rms_eps: float = 1e-6
    rope_theta: float = 10000.0
    gate_bias: float = 0.0
    gate_threshold: float = 0.0
    r_min: int = 2
    kv_layout: str = "depth"      # "depth" (r_max planes), "single" (1 plane), "first_shared" (2 planes);
                                  # the library also takes "depth_copy" (depth planes, copies made at exit)
    gate_kind: str = "linear"     # "linear" (w . RMSNorm(h) + b > t) or "convergence"
    conv_threshold: float = 0.0   # convergence gate: fires when the normalized step size is below this

    @property
    def qdim(self) -> int:
        return self.n_heads * self.head_dim

    def with_(self, **kw) -> "ModelDims":
        return dataclasses.replace(self, **kw)


@dataclass(frozen=True)
class Workload:
    """Request mix of a configuration (all synthetic, seeded)."""
    n_requests: int
    prompt_min: int
    prompt_max: int
    n_out: int
    prompt_dist: str = "uniform"      # "uniform", "fixed" or "lognormal"
    lognormal_median: float = 0.0
    lognormal_sigma: float = 0.0
    slots: tuple = (4,)               # max active sequences W
    mode: str = "refill"
    min_coda_batch: int = 1           # K
    max_batched_tokens: int = 8192    # M
    block_size: int = 16


# Gate biases were found by bisection with the oracle so that the mean exit
# depth of a short seeded calibration run lands near the configuration's
# target (oracle/calibrate_gate.py rewrites cdb_synth/gate_bias.json).
def _load_biases() -> Dict[str, float]:
    import json
    import os
    p = os.path.join(os.path.dirname(__file__), "gate_bias.json")
    if not os.path.exists(p):
        return {}
    with open(p) as f:
        d = json.load(f)
    return {k: float(np.float32(v["bias"])) for k, v in d.items()}


_BIAS = _load_biases()

CONFIGS: Dict[str, ModelDims] = {
    # tiny fp32 fully looped LM, 0-2-0, r_max 8, mean exit ~3
    "c0": ModelDims("c0", vocab=512, hidden=256, n_heads=4, head_dim=64, ffn=1024,
                    n_prelude=0, n_core=2, n_coda=0, r_max=8, dtype="fp32",
                    gate_bias=_BIAS.get("c0", 0.0)),
    # Ouro-like, 0-24-0, r_max 4, mean exit ~2.6, bf16
    "c1": ModelDims("c1", vocab=49152, hidden=2048, n_heads=16, head_dim=128, ffn=5632,
                    n_prelude=0, n_core=24, n_coda=0, r_max=4, dtype="bf16",
                    gate_bias=_BIAS.get("c1", 0.0)),
    # Huginn-like 2-4-2 with additive prelude injection, r_max 32, mean exit ~12
    "c3": ModelDims("c3", vocab=65536, hidden=5280, n_heads=55, head_dim=96, ffn=17920,
                    n_prelude=2, n_core=4, n_coda=2, r_max=32, dtype="bf16", inject=True,
                    gate_bias=_BIAS.get("c3", 0.0)),
}
CONFIGS["c2"] = CONFIGS["c1"].with_(name="c2")
CONFIGS["c4"] = CONFIGS["c1"].with_(name="c4")

# Mean exit-depth targets used when the biases were calibrated.
GATE_TARGETS = {"c0": 3.0, "c1": 2.6, "c3": 12.0}

WORKLOADS: Dict[str, Workload] = {
    "c0": Workload(n_requests=8, prompt_min=16, prompt_max=16, n_out=16,
                   prompt_dist="fixed", slots=(4,), mode="refill", min_coda_batch=1),
    "c2": Workload(n_requests=256, prompt_min=128, prompt_max=2048, n_out=256,
                   slots=(64, 128, 256), mode="refill", min_coda_batch=1),
    "c3": Workload(n_requests=128, prompt_min=256, prompt_max=1024, n_out=512,
                   slots=(64,), mode="refill", min_coda_batch=16),
    # log-normal with the ArXiv mean/median ratio (6989/6436) of the pages'
    # App. C.1 length statistics: sigma = sqrt(2 ln(6989/6436)) ~= 0.41
    "c4": Workload(n_requests=64, prompt_min=4096, prompt_max=16384, n_out=128,
                   prompt_dist="lognormal", lognormal_median=8192.0,
                   lognormal_sigma=math.sqrt(2.0 * math.log(6989.0 / 6436.0)),
                   slots=(8,), mode="refill", min_coda_batch=1),
}


# ---------------------------------------------------------------- bfloat16

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return the
    16-bit patterns as uint16.  NaN stays NaN (quiet)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    nan = np.isnan(x)
    r = ((u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16))
    r = r.astype(np.uint16)
    if nan.any():
        r = np.where(nan, np.uint16(0x7FC0), r)
    return r


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 values rounded to the nearest bfloat16, returned as float32."""
    return bits_to_f32(bf16_bits(x))


# ----------------------------------------------------------------- weights

def _layer_names(prefix: str) -> List[str]:
    return [f"{prefix}.wq", f"{prefix}.wk", f"{prefix}.wv", f"{prefix}.wo",
            f"{prefix}.wg", f"{prefix}.wu", f"{prefix}.wd"]


def tensor_order(d: ModelDims) -> List[tuple]:
    """(name, shape) of every drawn matrix, in the order the generator draws
    them.  Norm gains are not drawn (see make_weights)."""
    H, Q, F = d.hidden, d.qdim, d.ffn
    shapes = {"wq": (Q, H), "wk": (Q, H), "wv": (Q, H), "wo": (H, Q),
              "wg": (F, H), "wu": (F, H), "wd": (H, F)}
    out = [("embed", (d.vocab, H))]
    for stage, n in (("prelude", d.n_prelude), ("core", d.n_core), ("coda", d.n_coda)):
        for i in range(n):
            for nm in _layer_names(f"{stage}.{i}"):
                out.append((nm, shapes[nm.rsplit(".", 1)[1]]))
    out.append(("lm_head", (d.vocab, H)))
    out.append(("gate_w", (H,)))
    return out


def norm_names(d: ModelDims) -> List[str]:
    out = []
    for stage, n in (("prelude", d.n_prelude), ("core", d.n_core), ("coda", d.n_coda)):
        for i in range(n):
            out += [f"{stage}.{i}.attn_norm", f"{stage}.{i}.mlp_norm"]
    out.append("final_norm")
    return out


def make_weights(d: ModelDims, seed: int = 0, std: float = 0.02,
                 norm: str = "ones") -> Dict[str, np.ndarray]:
    """Seeded random-init weights.

    Matrices, embedding, LM head and gate vector: N(0, std) drawn in
    ``tensor_order`` from ``np.random.default_rng(seed)``.  Norm gains: all
    ones (``norm="ones"``) or 1 + 0.1 N(0,1) from a second stream seeded
    ``seed + 1000`` (``norm="random"``, used by tests so a dropped gain is
    visible).  bf16 configurations get every tensor rounded to bf16.
    Returns float32 arrays.
    """
    rng = np.random.default_rng(seed)
    w: Dict[str, np.ndarray] = {}
    for name, shape in tensor_order(d):
        a = rng.standard_normal(shape, dtype=np.float32)
        a *= np.float32(std)
        w[name] = a
    rng2 = np.random.default_rng(seed + 1000)
    for name in norm_names(d):
        if norm == "ones":
            w[name] = np.ones(d.hidden, dtype=np.float32)
        else:
            w[name] = (1.0 + 0.1 * rng2.standard_normal(d.hidden)).astype(np.float32)
    if d.dtype == "bf16":
        for k in list(w):
            w[k] = bf16_round(w[k])
    return w


# ---------------------------------------------------------------- workloads

def make_prompt_lengths(wl: Workload, seed: int = 1) -> np.ndarray:
    rng = np.random.default_rng(seed)
    n = wl.n_requests
    if wl.prompt_dist == "fixed":
        return np.full(n, wl.prompt_min, dtype=np.int64)
    if wl.prompt_dist == "uniform":
        return rng.integers(wl.prompt_min, wl.prompt_max + 1, size=n).astype(np.int64)
    if wl.prompt_dist == "lognormal":
        x = rng.lognormal(math.log(wl.lognormal_median), wl.lognormal_sigma, size=n)
        return np.clip(np.round(x), wl.prompt_min, wl.prompt_max).astype(np.int64)
    raise ValueError(wl.prompt_dist)


def make_prompts(vocab: int, lengths, seed: int = 1) -> List[np.ndarray]:
    """Uniform-random token ids in [0, vocab) for each prompt length."""
    rng = np.random.default_rng(seed + 7)
    return [rng.integers(0, vocab, size=int(L)).astype(np.int32) for L in lengths]


def make_context_exit_depths(n_pos: int, r_max: int, seed: int = 2) -> np.ndarray:
    """Per-position exit depths e_j ~ U{1..r_max} for synthetic cached
    context (the decode microbench).  Cached positions may carry any depth in
    [1, r_max]; only rows decoded under the lookahead gate are >= 2."""
    rng = np.random.default_rng(seed)
    return rng.integers(1, r_max + 1, size=n_pos).astype(np.uint8)


def c1_row_depths(n_rows: int, r_max: int = 4, seed: int = 2) -> np.ndarray:
    """Depth d_b of each row of a microbench core batch: drawn with weights
    proportional to in-flight survival for a mean exit of about 2.6
    (P(d = 1, 2, 3, 4) proportional to 1, 1, 0.45, 0.15)."""
    rng = np.random.default_rng(seed + 11)
    p = np.array([1.0, 1.0, 0.45, 0.15][:r_max])
    p = p / p.sum()
    return (rng.choice(np.arange(1, r_max + 1), size=n_rows, p=p)).astype(np.int32)
