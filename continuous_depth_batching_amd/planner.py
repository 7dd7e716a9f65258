"""Latency-model planner for the CDB schedule (host side, no GPU work).

"Depth-adaptive Inference of Looped Language Models via Continuous Depth
Batching" models a recurrent step as t = delta + gamma N_b + alpha N_c
(Section 5), which at a fixed context L is linear in the batch (App. B,
Eq. 4), and a whole decode pass as tau(r) = tau_0 + tau_r r with tau_0 the
prelude + coda overhead (App. B, Eq. 3).  Section 5 draws the consequence:
refill pays in the memory-bound regime (a smaller batch costs almost as much
as a full one) and matters less once steps are compute bound.  Section 6.4
sweeps the minimum coda batch K: batching the coda saves boundary cost but
leaves exited rows waiting outside the core, shrinking the recurrent batch.

This module fits the two stage costs on measured stages and predicts the
decode rate (generated tokens per second, prefill excluded) of the three
schedules, so K and refill vs no-refill can be chosen from the model, in two
ways: closed-form steady-state rates (below) and a simulation of the
scheduler's queue rules with exits drawn from the measured distribution
(``simulate``), which keeps the burstiness of the exits:

* core step at B rows:        t(B)  = delta + slope * B (or the measured
                                 mean of B's power-of-two row bucket)
* boundary stage at E rows:   c(E)  = b0 + b1 * E     (coda + prelude)
* fixed depth: a cohort of W rows runs r_max steps and one boundary stage;
* no-refill (Alg. 1): a cohort of W rows shrinks as its tokens leave; step j
  runs while any row remains, with the surviving rows' expected count;
* refill (Alg. 2, minimum coda batch K): W rows in steady state, lambda =
  B / d_mean exits per step; the coda runs on E = max(K, lambda) rows every
  E / lambda steps and the rows waiting for it, (E - lambda) / 2 on average,
  are missing from the core batch B = W - (E - lambda) / 2.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Dict, Iterable, Optional, Sequence, Tuple

import numpy as np


def pow2(n: float) -> int:
    p = 1
    while p < n:
        p *= 2
    return p


@dataclass(frozen=True)
class StageModel:
    delta: float          # core step, seconds at B -> 0
    slope: float          # core step, seconds per row (gamma + alpha L at the workload's context)
    b0: float             # boundary stage, seconds at E -> 0
    b1: float             # boundary stage, seconds per row
    # measured mean core-step seconds per row bucket (a core step of B rows
    # runs the kernels of the power-of-two bucket holding B); when present
    # it replaces the line for the buckets it covers
    core_by_bucket: Optional[Tuple[Tuple[int, float], ...]] = None

    def core(self, B: float) -> float:
        if self.core_by_bucket:
            tab = dict(self.core_by_bucket)
            b = pow2(B)
            if b in tab:
                return tab[b]
        return self.delta + self.slope * B

    def boundary(self, E: float) -> float:
        return self.b0 + self.b1 * E


def _line_fit(xs: Sequence[float], ys: Sequence[float]) -> Tuple[float, float]:
    x = np.asarray(xs, dtype=np.float64)
    y = np.asarray(ys, dtype=np.float64)
    if len(x) == 0:
        raise ValueError("no samples")
    if np.ptp(x) == 0:                       # one batch size only: a flat cost
        return float(y.mean()), 0.0
    A = np.stack([np.ones_like(x), x], axis=1)
    (c0, c1), *_ = np.linalg.lstsq(A, y, rcond=None)
    return float(c0), float(c1)


def fit_stage_model(core: Iterable[Tuple[int, float]], boundary: Iterable[Tuple[int, float]],
                    buckets: bool = False) -> StageModel:
    """Least-squares lines through measured (rows, seconds) stage samples;
    with ``buckets`` also the mean core-step cost of each power-of-two row
    bucket that has samples."""
    core = list(core)
    boundary = list(boundary)
    d, s = _line_fit([b for b, _ in core], [t for _, t in core])
    b0, b1 = _line_fit([e for e, _ in boundary], [t for _, t in boundary])
    tab = None
    if buckets:
        acc: Dict[int, list] = {}
        for b, t in core:
            acc.setdefault(pow2(b), []).append(t)
        tab = tuple(sorted((k, float(np.mean(v))) for k, v in acc.items()))
    return StageModel(delta=d, slope=s, b0=b0, b1=b1, core_by_bucket=tab)


def exit_pmf(exits: Iterable[int], r_max: int) -> np.ndarray:
    """Empirical P(e = d) for d = 1..r_max (index d - 1)."""
    e = np.asarray(list(exits), dtype=np.int64)
    if e.size == 0 or e.min() < 1 or e.max() > r_max:
        raise ValueError("exit depths must lie in 1..r_max")
    return np.bincount(e - 1, minlength=r_max).astype(np.float64) / e.size


def rate_fixed(m: StageModel, W: int, r_max: int) -> float:
    return W / (r_max * m.core(W) + m.boundary(W))


def rate_norefill(m: StageModel, W: int, pmf: np.ndarray) -> float:
    """A cohort of W rows: step j runs while any row survives (probability
    1 - (1 - S_j)^W, S_j = P(e >= j)) on the survivors' expected count given
    that some survive; one boundary stage per cohort."""
    surv = np.cumsum(pmf[::-1])[::-1]        # S_j for j = 1..r_max
    t = 0.0
    for S in surv:
        p_any = 1.0 - (1.0 - S) ** W
        if p_any <= 0.0:
            continue
        t += p_any * m.core(W * S / p_any)
    return W / (t + m.boundary(W))


def rate_refill(m: StageModel, W: int, K: int, pmf: np.ndarray, iters: int = 200) -> float:
    """Steady state of Alg. 2 with minimum coda batch K (fixed point in B)."""
    d_mean = float(np.dot(np.arange(1, len(pmf) + 1), pmf))
    B = float(W)
    for _ in range(iters):
        lam = B / d_mean
        E = max(float(K), lam)
        B_new = max(1.0, W - (E - lam) / 2.0)
        if abs(B_new - B) < 1e-9:
            break
        B = 0.5 * (B + B_new)
    lam = B / d_mean
    E = max(float(K), lam)
    return lam / (m.core(B) + m.boundary(E) * lam / E)


def simulate(m: StageModel, mode: str, W: int, K: int, pmf: np.ndarray, n_req: int, n_out: int,
             S: int = 0, seed: int = 0, exits: Optional[Sequence[Sequence[int]]] = None) -> float:
    """Decode rate of a whole workload under the stage policy of Alg. 1 / 2
    (the scheduler's rules), with exit depths drawn from ``pmf`` and the
    stage costs of ``m``; prefill is taken as instantaneous, so the rate is
    generated tokens per second of core + boundary stages.

    refill: the coda runs when K tokens wait (or nothing else can run),
    otherwise a request is admitted when S slots are free, otherwise a core
    step runs; the coda's successors join the core batch.  no-refill:
    admit while possible, loop the cohort until every token has left, one
    coda.  fixed: no-refill with every exit at r_max.  Unlike the mean-field
    rates above, this keeps the burstiness of the exits (a bimodal exit
    distribution leaves many steps without exits).  With ``exits`` (per
    request, per decode token, in admission order) the recorded exit depths
    are replayed instead of drawn, as the pages replay recorded exits
    (App. C.2): a request whose tokens keep leaving early or late keeps doing
    so."""
    rng = np.random.default_rng(seed)
    R = len(pmf)
    cdf = np.cumsum(pmf)
    S = S or max(1, W // 8)
    done: Dict[int, int] = {}         # request -> decode tokens drawn so far

    def draw(r: int) -> int:
        i = done.get(r, 0)
        done[r] = i + 1
        if mode == "fixed":
            return R
        if exits is not None and i < len(exits[r]):
            return int(exits[r][i])
        return int(np.searchsorted(cdf, rng.random(), side="right")) + 1

    waiting = n_req
    left: Dict[int, int] = {}         # request -> decode tokens still to generate
    core = []                         # [request, depth, exit depth]
    qc = []                           # requests whose token waits for the coda
    t = 0.0
    tokens = 0
    nxt = 0

    def admit():
        nonlocal waiting, nxt
        waiting -= 1
        left[nxt] = n_out - 1
        if n_out > 1:
            core.append([nxt, 0, draw(nxt)])
        nxt += 1

    def core_step():
        nonlocal t
        t += m.core(len(core))
        keep = []
        for row in core:
            row[1] += 1
            (qc if row[1] == row[2] else keep).append(row if row[1] != row[2] else row[0])
        core[:] = keep

    def coda():
        nonlocal t, tokens
        t += m.boundary(len(qc))
        for r in qc:
            tokens += 1
            left[r] -= 1
            if left[r] > 0:
                core.append([r, 0, draw(r)])
            else:
                del left[r]
        qc.clear()

    while waiting or core or qc:
        active = len(left)
        if mode == "refill":
            if qc and (len(qc) >= K or (not core and not (waiting and W - active >= S))):
                coda()
            elif waiting and W - active >= S:
                while waiting and len(left) < W:
                    admit()
            elif core:
                core_step()
            else:
                break
        else:
            if waiting and W - len(left) >= S:      # a prefill stage packs requests up to W
                while waiting and len(left) < W:
                    admit()
            while core:
                core_step()
            if qc:
                coda()
            elif not core and not waiting:
                break
    return tokens / t if t > 0 else 0.0


def predict(m: StageModel, W: int, r_max: int, pmf: np.ndarray, Ks: Sequence[int]) -> Dict[str, float]:
    """Predicted decode rates: 'fixed', 'norefill' and 'refill_K<k>' per K."""
    out = {"fixed": rate_fixed(m, W, r_max), "norefill": rate_norefill(m, W, pmf)}
    for k in Ks:
        out[f"refill_K{k}"] = rate_refill(m, W, k, pmf)
    return out


def simulate_all(m: StageModel, W: int, r_max: int, pmf: np.ndarray, Ks: Sequence[int], n_req: int, n_out: int,
                 seed: int = 0, exits: Optional[Sequence[Sequence[int]]] = None) -> Dict[str, float]:
    """Simulated decode rates: 'fixed', 'norefill' and 'refill_K<k>' per K."""
    kw = dict(seed=seed, exits=exits)
    out = {"fixed": simulate(m, "fixed", W, 1, pmf, n_req, n_out, **kw),
           "norefill": simulate(m, "norefill", W, 1, pmf, n_req, n_out, **kw)}
    for k in Ks:
        out[f"refill_K{k}"] = simulate(m, "refill", W, k, pmf, n_req, n_out, **kw)
    return out


def recommend(rates: Dict[str, float]) -> str:
    """The depth-adaptive schedule with the highest predicted decode rate."""
    return max((k for k in rates if k != "fixed"), key=lambda k: rates[k])
