"""Calibrate the exit-gate bias b of a configuration with the oracle.

Test infrastructure only; run as ``python -m oracle.calibrate_gate c0 c1``.
It rewrites ``cdb_synth/gate_bias.json`` (an input constant of the model,
not an expected value).

The pages replay recorded exit decisions of trained gates and sweep the
gate threshold to move the exit distribution ("Depth-adaptive Inference of
Looped Language Models via Continuous Depth Batching", §6.1 and App. C.2);
a random-init model has no trained gate, so the configuration fixes a mean
exit depth and b is chosen to reach it.  Method: decode a short seeded
calibration set at fixed depth, record each token's pre-bias gate value
s_d = w . RMSNorm(h_d) after every loop d < r_max, and bisect b so that the
mean of min(r_max, 1 + first d with s_d + b > t) hits the target.  (Under the
adaptive policy the trajectories shift slightly because earlier tokens'
exits change the cache; the realised mean is recomputed with the adaptive
oracle and stored next to b.)
"""
from __future__ import annotations

import json
import os
import sys
import time

import numpy as np

import cdb_synth as S
from .model import OracleLM, SeqCache

_JSON = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "cdb_synth", "gate_bias.json")


def record_gate_values(m: OracleLM, prompts, n_out):
    d = m.d
    traj = []
    for p in prompts:
        cache = SeqCache(d, len(p) + n_out, m.dt)
        tok, _, _ = m.prefill(p, cache)
        for i in range(n_out - 1):
            row = m.row_prelude(tok, len(p) + i, cache)
            s = []
            for depth in range(1, d.r_max + 1):
                m.row_core(row)
                if depth < d.r_max:
                    s.append(m.gate_logit(row.h[0]) - float(np.float32(d.gate_bias)))
            tok = m.row_coda(row)
            traj.append(s)
    return np.array(traj)


def mean_exit(traj, b, R, t=0.0):
    fire = (traj + b) > t
    out = []
    for row in fire:
        idx = np.flatnonzero(row)
        out.append(min(R, idx[0] + 2) if len(idx) else R)
    return float(np.mean(out))


def solve_bias(traj, R, target, t=0.0):
    lo, hi = -50.0, 50.0           # mean_exit decreases as b grows
    for _ in range(100):
        mid = 0.5 * (lo + hi)
        if mean_exit(traj, mid, R, t) > target:
            lo = mid
        else:
            hi = mid
    return float(np.float32(0.5 * (lo + hi)))


SETS = {  # (n_seq, prompt length or the workload whose length mix is drawn, n_out)
    "c0": (8, 16, 16),
    "c1": (6, "c2", 12),      # prompt lengths U{128..2048} as in the end-to-end workload
    "c3": (2, "c3", 8),       # prompt lengths U{256..1024} as in the Huginn-like workload
}


def calibrate(name: str, verify: bool = True):
    d = S.CONFIGS[name].with_(gate_bias=0.0)
    n_seq, plen, n_out = SETS[name]
    w = S.make_weights(d, seed=0)
    m = OracleLM(d, w)
    if isinstance(plen, str):
        lengths = [int(x) for x in S.make_prompt_lengths(S.WORKLOADS[plen], seed=101)[:n_seq]]
    else:
        lengths = [plen] * n_seq
    prompts = S.make_prompts(d.vocab, lengths, seed=101)
    t0 = time.time()
    traj = record_gate_values(m, prompts, n_out)
    target = S.GATE_TARGETS[name]
    b = solve_bias(traj, d.r_max, target)
    rec = {"bias": b, "target_mean_exit": target, "fixed_path_mean_exit": mean_exit(traj, b, d.r_max),
           "calibration_set": {"n_seq": n_seq, "prompt_len": plen, "prompt_lengths": lengths, "n_out": n_out,
                               "prompt_seed": 101}}
    if verify:
        # refine with the adaptive oracle itself (cheap for small models):
        # bisection around the fixed-path estimate
        def adaptive_mean(bb):
            m2 = OracleLM(d.with_(gate_bias=bb), w)
            ex = []
            for p in prompts:
                ex += m2.decode_sequential(p, n_out)[1]
            return float(np.mean(ex))
        lo, hi = b - 3.0, b + 3.0
        best = (abs(adaptive_mean(b) - target), b)
        for _ in range(24):
            mid = float(np.float32(0.5 * (lo + hi)))
            me = adaptive_mean(mid)
            best = min(best, (abs(me - target), mid))
            if me > target:
                lo = mid
            else:
                hi = mid
            if abs(me - target) <= 0.05:
                break
        b = best[1]
        rec["bias"] = b
        rec["adaptive_mean_exit"] = adaptive_mean(b)
    rec["seconds"] = round(time.time() - t0, 1)
    return rec


def main(argv):
    out = {}
    if os.path.exists(_JSON):
        with open(_JSON) as f:
            out = json.load(f)
    for name in argv or ["c0"]:
        out[name] = calibrate(name, verify=(name == "c0"))
        print(name, out[name], flush=True)
    with open(_JSON, "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main(sys.argv[1:])
