"""Writes the oracle's outputs for small subsets of the end-to-end workloads
at their full model shapes (tests/golden/oracle_subsets/*.npz).

Calls only the oracle (oracle/) and the seeded input generators (cdb_synth);
nothing here comes from the HIP path.  The GPU test that reads these files
(tests/test_gpu_full_shape_subsets.py) runs the same requests through the
library and compares decision by decision.

    python -m tests.golden.make_oracle_subsets c2 c3 c4

Sequences never share state, so a subset of a workload decodes exactly as
it does inside the whole run ("Depth-adaptive Inference of Looped Language
Models via Continuous Depth Batching", §3: the batching changes neither the
predictions nor the exit decisions).  Subsets, from the workload's own
seeded prompt mix (the prompts of the end-to-end benchmark, seed 1):

* c2 (Ouro-like, 24 core layers, r_max 4): the shortest, the median and the
  longest prompt of the 256-request U{128..2048} mix; 6 output tokens.
* c3 (Huginn-like 2-4-2, r_max 32, prelude injection): the shortest and the
  longest prompt of the 128-request U{256..1024} mix; 3 output tokens.
* c4 (Ouro-like, log-normal prompts clipped to 4096..16384): the two
  shortest prompts of the 64-request mix; 4 output tokens.

Stored per request: the workload index, tokens, exits, per decision the
oracle's margins (top-2 logit gap of every token; every gate margin of
every decode pass), the exit state of every decode pass (fp32) and, for
the model with coda layers (c3), the logits of every decode pass as fp16
(at most 2^-11 relative rounding; the others recompute logits from the
stored exit state with the oracle's LM head).
"""
from __future__ import annotations

import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import cdb_synth as S  # noqa: E402
from oracle.model import OracleLM  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_subsets")

SUBSETS = {
    "c2": dict(dims="c2", n_out=6),
    "c3": dict(dims="c3", n_out=3),
    "c4": dict(dims="c4", n_out=4),
}


def pick(name, lengths):
    order = np.argsort(lengths, kind="stable")
    if name == "c2":
        return [int(order[0]), int(order[len(order) // 2]), int(order[-1])]
    if name == "c3":
        return [int(order[0]), int(order[-1])]
    return [int(order[0]), int(order[1])]


def make(name):
    spec = SUBSETS[name]
    d = S.CONFIGS[spec["dims"]]
    wl = S.WORKLOADS[name]
    lengths = S.make_prompt_lengths(wl, seed=1)
    prompts = S.make_prompts(d.vocab, lengths, seed=1)
    idx = pick(name, lengths)
    t0 = time.time()
    w = S.make_weights(d, seed=0)
    m = OracleLM(d, w, dtype=np.float32, keep_logits=True)
    print(f"{name}: weights in {time.time() - t0:.0f} s; requests {idx} lengths {[int(lengths[i]) for i in idx]}",
          flush=True)
    n_out = spec["n_out"]
    out = dict(requests=np.array(idx, np.int32), n_out=np.int32(n_out))
    for k, i in enumerate(idx):
        t1 = time.time()
        toks, exits, recs = m.decode_sequential(prompts[i], n_out, keep_state=True)
        margins = np.full((n_out - 1, d.r_max), np.nan, np.float32)
        for g in range(1, n_out):
            gm = recs[g].gate_margins
            margins[g - 1, :len(gm)] = gm
        out[f"r{k}_tokens"] = np.array(toks, np.int32)
        out[f"r{k}_exits"] = np.array(exits, np.int32)
        out[f"r{k}_logit_gap"] = np.array([r.logit_gap for r in recs], np.float32)
        out[f"r{k}_gate_margins"] = margins
        out[f"r{k}_exit_states"] = np.stack([recs[g].exit_state for g in range(1, n_out)]).astype(np.float32)
        if d.n_coda > 0:
            out[f"r{k}_logits_f16"] = np.stack([recs[g].logits for g in range(1, n_out)]).astype(np.float16)
        print(f"  request {i} (prompt {len(prompts[i])}): tokens {toks} exits {exits} in {time.time() - t1:.0f} s",
              flush=True)
    os.makedirs(OUT, exist_ok=True)
    np.savez(os.path.join(OUT, f"{name}.npz"), **out)


if __name__ == "__main__":
    for nm in sys.argv[1:] or list(SUBSETS):
        make(nm)
