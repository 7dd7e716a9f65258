"""The looped LM decoded one sequence at a time — the definition CDB must
reproduce.  Test infrastructure only (see the package docstring).

Source: "Depth-adaptive Inference of Looped Language Models via Continuous
Depth Batching" (arXiv 2608.09444).

* §2 Problem Setup: prelude P, shared core R looped r_t <= r_max times,
  coda C; each token leaves the core at its own depth, decided at the end of
  a loop step.  A 0-N-0 model's prelude is the embedding and its coda the LM
  head.
* §3 (last sentence of "Depth-adaptive looped transformers") and §8: CDB
  does not change the model's predictions or exit decisions.  Hence the
  oracle is the plain per-sequence decode; every batched schedule must match
  it.
* §4.2 Depth-aware KV Cache, Fig. 2 right: the depth-indexed cache keeps
  r_max slots per (core layer, token); a token that exits at r_t < r_max has
  its final KV copied into the skipped slots (the last-exited cache).  The
  shared cache keeps one slot per (core layer, token) and every loop step
  overwrites it, so readers always see the most recent state.  App. E.1 adds
  first-then-shared (s = 2 slots): the first loop keeps a private slot and
  every later loop overwrites a second, shared one.  This oracle implements
  all three literally: each loop writes its slot and reads that slot of
  every position; the depth-indexed cache copies on exit; it never uses an
  index rule.
* §4.3 Asynchronous Scheduling and §7 "Designing exit gates": the lookahead
  gate's signal after step r decides whether the token runs step r+2, so the
  earliest exit is after step 2 (r_min = 2) and a token at r_max always
  leaves.  §7 (Setup and Results of the gating experiments): the
  training-free convergence criterion fires once the normalized L2 distance
  between consecutive loop states falls below a threshold; it needs two
  states, so with the lookahead its earliest exit is after step 3.
* App. A.1 (Preemption paragraph): prefill always runs at full depth, so
  every prompt position has exit depth r_max.
* App. A.5 (Attention and output projection): logits only for the final
  prompt token.

Readings where the pages are silent (each listed in the design notes):
gate z = w . RMSNorm(h) + b on the raw core output with a unit-gain norm,
firing when z > t (strict); the loop state passes between loops without an
extra norm; the Huginn-like model starts the core from h = 0 and adds the
prelude output e to the core input at every loop; greedy decoding takes the
lowest index among equal maxima; a single-slot cache under chunked prefill
reads same-chunk positions at the current loop and earlier-chunk positions
at their final state.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np

from .layers import attend, rmsnorm, rope, swiglu_mlp


def kv_slots(d) -> int:
    """KV slots per (core layer, token), s in App. E.1: r_max for the
    depth-indexed cache, 1 for single-slot sharing, 2 for first-then-shared."""
    return {"depth": d.r_max, "single": 1, "first_shared": 2}[d.kv_layout]


def kv_slot(d, depth: int) -> int:
    """Slot (0-based) that loop ``depth`` writes and reads: its own slot in
    the depth-indexed cache; the one slot under single-slot sharing; under
    first-then-shared the private slot for the first loop and the shared
    slot for every later loop (App. E.1)."""
    if d.kv_layout == "depth":
        return depth - 1
    if d.kv_layout == "single":
        return 0
    if d.kv_layout == "first_shared":
        return 0 if depth == 1 else 1
    raise ValueError(d.kv_layout)


class SeqCache:
    """All KV state of one sequence.

    core_k/core_v: [n_core, planes, cap, n_heads, head_dim] with planes =
    kv_slots (r_max depth-indexed, 1 single-slot, 2 first-then-shared);
    unwritten entries are NaN, so a read of a gap poisons the result.  bnd_k/bnd_v: one array per prelude or
    coda layer, [cap, n_heads, head_dim].  exit_depth[j] is e_j."""

    def __init__(self, d, cap: int, dtype):
        planes = kv_slots(d)
        shp = (d.n_core, planes, cap, d.n_heads, d.head_dim)
        self.core_k = np.full(shp, np.nan, dtype=dtype)
        self.core_v = np.full(shp, np.nan, dtype=dtype)
        self.bnd_k: Dict[str, np.ndarray] = {}
        self.bnd_v: Dict[str, np.ndarray] = {}
        for stage, n in (("prelude", d.n_prelude), ("coda", d.n_coda)):
            for i in range(n):
                self.bnd_k[f"{stage}.{i}"] = np.full((cap, d.n_heads, d.head_dim), np.nan, dtype=dtype)
                self.bnd_v[f"{stage}.{i}"] = np.full((cap, d.n_heads, d.head_dim), np.nan, dtype=dtype)
        self.exit_depth = np.zeros(cap, dtype=np.int32)
        self.cap = cap


@dataclass
class TokenRecord:
    """What one generated token looked like inside the oracle."""
    token: int                 # the token this step produced (own argmax)
    exit_depth: int            # the depth at which the step's input left the core
    logit_gap: float           # top-1 minus top-2 logit
    gate_margins: List[float] = field(default_factory=list)  # |sigmoid(z) - q| per gate evaluation
    gate_logits: List[float] = field(default_factory=list)
    exit_state: Optional[np.ndarray] = None   # h at the exit depth (before coda)
    logits: Optional[np.ndarray] = None
    own_exit: Optional[int] = None             # forced replay: the oracle's own exit decision
    own_token: Optional[int] = None            # forced replay: the oracle's own argmax


@dataclass
class Row:
    """A token in flight through the core: its position, loop state h (and
    injection vector), completed depth and scheduled exit depth."""
    pos: int
    h: np.ndarray
    inj: Optional[np.ndarray]
    cache: "SeqCache"
    exit_at: int
    depth: int = 0
    h_prev: Optional[np.ndarray] = None   # state before the last core step


def _sigmoid(z: float) -> float:
    import math
    return 1.0 / (1.0 + math.exp(-z))


class OracleLM:
    """Per-sequence looped LM.  ``dtype`` is the arithmetic type (float32 by
    default; float64 for pins).  In bf16 configurations the weights are the
    bf16-rounded values widened to ``dtype``; activations are not rounded."""

    def __init__(self, dims, weights: Dict[str, np.ndarray], dtype=np.float32,
                 keep_logits: bool = False):
        self.d = dims
        self.dt = np.dtype(dtype)
        self.w = {k: np.ascontiguousarray(v, dtype=self.dt) for k, v in weights.items()}
        self.keep_logits = keep_logits
        self.q_prob = _sigmoid(float(dims.gate_threshold))

    # ------------------------------------------------------------ one block
    def _block(self, x, positions, prefix, put_kv, get_kv):
        """Pre-norm attention + SwiGLU block on rows x[T, H] at positions[T].

        put_kv(k, v) stores this block's K/V rows ([T, nh, hd]); get_kv(i)
        returns (K, V) over positions 0..positions[i] for query row i."""
        d, w, eps = self.d, self.w, self.d.rms_eps
        T = x.shape[0]
        xn = rmsnorm(x, w[prefix + ".attn_norm"], eps)
        q = rope(xn @ w[prefix + ".wq"].T, positions, d.head_dim, d.rope_theta)
        k = rope(xn @ w[prefix + ".wk"].T, positions, d.head_dim, d.rope_theta)
        v = xn @ w[prefix + ".wv"].T
        put_kv(k.reshape(T, d.n_heads, d.head_dim), v.reshape(T, d.n_heads, d.head_dim))
        o = np.empty((T, d.qdim), dtype=self.dt)
        qh = q.reshape(T, d.n_heads, d.head_dim)
        for i in range(T):
            K, V = get_kv(i)
            o[i] = attend(qh[i], K, V).reshape(-1)
        x = x + o @ w[prefix + ".wo"].T
        xn = rmsnorm(x, w[prefix + ".mlp_norm"], eps)
        return x + swiglu_mlp(xn, w[prefix + ".wg"], w[prefix + ".wu"], w[prefix + ".wd"])

    def _boundary_layers(self, stage, n, x, positions, cache: SeqCache):
        for i in range(n):
            name = f"{stage}.{i}"
            Kc, Vc = cache.bnd_k[name], cache.bnd_v[name]

            def put(k, v, Kc=Kc, Vc=Vc):
                Kc[positions] = k
                Vc[positions] = v

            def get(r, Kc=Kc, Vc=Vc):
                p = positions[r]
                return Kc[: p + 1], Vc[: p + 1]
            x = self._block(x, positions, name, put, get)
        return x

    def core(self, h, positions, depth: int, cache: SeqCache):
        """One application of the shared core at loop ``depth`` (1-based).

        Depth-indexed cache: every row writes plane ``depth`` and reads plane
        ``depth`` of all positions up to its own (earlier positions that
        exited shallower hold their last-exited copy there).  Single-slot
        cache: the one plane is written and read, so under chunked prefill
        positions of earlier chunks are seen at their final (r_max) state and
        positions of the current chunk at loop ``depth``.  First-then-shared:
        loop 1 uses the private slot, later loops the shared one, which holds
        each earlier position's most recent (final) state."""
        d = self.d
        plane = kv_slot(d, depth)
        positions = np.asarray(positions)
        x = h
        for l in range(d.n_core):
            Kc, Vc = cache.core_k[l, plane], cache.core_v[l, plane]

            def put(k, v, Kc=Kc, Vc=Vc):
                Kc[positions] = k
                Vc[positions] = v

            def get(r, Kc=Kc, Vc=Vc):
                p = positions[r]
                return Kc[: p + 1], Vc[: p + 1]
            x = self._block(x, positions, f"core.{l}", put, get)
        return x

    def gate_eval(self, h_row: np.ndarray, h_prev_row: np.ndarray, depth: int):
        """The exit gate after loop ``depth``: (value, fires, margin), or None
        where it is not evaluated.  Linear gate: z = w . RMSNorm(h) + b,
        fires when z > t, margin |sigmoid(z) - q|.  Convergence gate (loops
        >= 2): c = |h_d - h_{d-1}|_2 / |h_d|_2, fires when c < tau, margin
        |c - tau|."""
        d = self.d
        if d.gate_kind == "linear":
            z = self.gate_logit(h_row)
            return z, z > float(d.gate_threshold), abs(_sigmoid(z) - self.q_prob)
        if d.gate_kind == "convergence":
            if depth < 2:
                return None
            c = float(np.linalg.norm(h_row - h_prev_row) / np.linalg.norm(h_row))
            tau = float(np.float32(d.conv_threshold))
            return c, c < tau, abs(c - tau)
        raise ValueError(d.gate_kind)

    def gate_logit(self, h_row: np.ndarray) -> float:
        """z = w . RMSNorm(h) + b with a unit-gain norm (exit head on the core
        output, §3 and §7; the concrete form is the configuration's)."""
        hn = rmsnorm(h_row, np.ones_like(h_row), self.d.rms_eps)
        return float(np.dot(hn, self.w["gate_w"])) + float(np.float32(self.d.gate_bias))

    def lm_head(self, x):
        """Final RMSNorm and the LM head projection (the 0-N-0 coda)."""
        xn = rmsnorm(x, self.w["final_norm"], self.d.rms_eps)
        return xn @ self.w["lm_head"].T

    def coda_logits(self, h_rows, positions, cache: SeqCache):
        x = self._boundary_layers("coda", self.d.n_coda, h_rows, positions, cache)
        return self.lm_head(x)

    def _prelude(self, tokens, positions, cache):
        x = self.w["embed"][np.asarray(tokens)]
        x = self._boundary_layers("prelude", self.d.n_prelude, x, positions, cache)
        if self.d.inject:
            return np.zeros_like(x), x
        return x, None

    def _last_exited_fill(self, cache: SeqCache, pos: int, e: int) -> None:
        """§4.2 (last-exited cache): a token that leaves the core after loop
        e < r_max never writes depth slots e+1..r_max; they receive a copy of
        the KV it wrote in its last loop (slot e, index e-1), in every core
        layer.  Only the depth-indexed layout has such slots."""
        d = self.d
        if d.kv_layout == "depth" and e < d.r_max:
            for l in range(d.n_core):
                cache.core_k[l, e:, pos] = cache.core_k[l, e - 1, pos]
                cache.core_v[l, e:, pos] = cache.core_v[l, e - 1, pos]

    # ------------------------------------------------------------- prefill
    def prefill(self, prompt: Sequence[int], cache: SeqCache, chunks=None):
        """Full-depth prefill of a prompt in the given chunks (list of
        (start, end)); returns (first token, logits of the last position,
        its core state at depth r_max).  The gate is not consulted, every
        prompt position gets exit depth r_max, and every position passes the
        coda layers (their KV is needed later) but only the last one reaches
        the LM head."""
        d = self.d
        P = len(prompt)
        if chunks is None:
            chunks = [(0, P)]
        assert chunks[0][0] == 0 and chunks[-1][1] == P
        for (s, e) in chunks:
            pos = np.arange(s, e)
            h, inj = self._prelude(np.asarray(prompt[s:e]), pos, cache)
            for depth in range(1, d.r_max + 1):
                h = self.core(h + inj if inj is not None else h, pos, depth, cache)
            cache.exit_depth[pos] = d.r_max
            x = self._boundary_layers("coda", d.n_coda, h, pos, cache)
        logits = self.lm_head(x[-1:])[0]
        return int(np.argmax(logits)), logits, h[-1].copy()

    # -------------------------------------------------------------- decode
    def decode_step(self, token: int, pos: int, cache: SeqCache, policy: str = "adaptive",
                    forced_exit: Optional[int] = None, keep_state: bool = False) -> TokenRecord:
        """Run one generated token through prelude, core loop and coda.

        policy "adaptive": lookahead gate — if it fires after step r the
        token runs step r+1 and then leaves; at r_max it always leaves; the
        gate is not evaluated at the step the token leaves.  policy "fixed": every
        token runs r_max loops.  ``forced_exit`` follows a given exit depth
        and records the oracle's own decision along that path (own_exit is
        None when the oracle would have looped past the forced depth)."""
        d = self.d
        R = d.r_max
        positions = np.array([pos])
        h, inj = self._prelude([token], positions, cache)
        exit_at = R
        first_fire = None
        margins, zs = [], []
        depth = 0
        for depth in range(1, R + 1):
            h_prev = h
            h = self.core(h + inj if inj is not None else h, positions, depth, cache)
            limit = forced_exit if forced_exit is not None else exit_at
            if depth == limit:
                break
            if policy == "fixed":
                continue
            g = self.gate_eval(h[0], h_prev[0], depth)
            if g is None:
                continue
            z, fires, margin = g
            zs.append(z)
            margins.append(margin)
            if fires and first_fire is None:
                first_fire = depth
                exit_at = depth + 1
        e = depth
        if policy == "fixed":
            own_exit = R
        elif first_fire is not None:
            own_exit = first_fire + 1
        else:
            own_exit = R if e == R else None
        self._last_exited_fill(cache, pos, e)
        cache.exit_depth[pos] = e
        logits = self.coda_logits(h, positions, cache)[0]
        top = int(np.argmax(logits))
        srt = np.sort(logits)
        rec = TokenRecord(token=top, exit_depth=e, logit_gap=float(srt[-1] - srt[-2]),
                          gate_margins=margins, gate_logits=zs, own_exit=own_exit, own_token=top)
        if keep_state:
            rec.exit_state = h[0].copy()
        if self.keep_logits:
            rec.logits = logits.copy()
        return rec

    def decode_sequential(self, prompt: Sequence[int], n_out: int, policy: str = "adaptive",
                          chunks=None, keep_state: bool = False,
                          forced_tokens: Optional[Sequence[int]] = None,
                          forced_exits: Optional[Sequence[int]] = None):
        """Decode one request alone: full-depth prefill, then n_out - 1 decode
        passes (the first output token comes from prefill; no EOS).

        Returns (tokens[n_out], exits[n_out - 1], records).  exits[i] is the
        exit depth of the pass whose input is tokens[i].  With
        forced_tokens / forced_exits (forced replay) the inputs and exits
        follow the given sequence and each record holds the oracle's own
        choice and margins at that decision."""
        P = len(prompt)
        cache = SeqCache(self.d, P + n_out, self.dt)
        tok0, logits0, _ = self.prefill(prompt, cache, chunks)
        srt = np.sort(logits0)
        first = TokenRecord(token=tok0, exit_depth=self.d.r_max, logit_gap=float(srt[-1] - srt[-2]),
                            own_token=tok0)
        if self.keep_logits:
            first.logits = logits0.copy()
        tokens = [tok0]
        exits: List[int] = []
        records = [first]
        for i in range(n_out - 1):
            inp = tokens[i] if forced_tokens is None else int(forced_tokens[i])
            fe = None if forced_exits is None else int(forced_exits[i])
            rec = self.decode_step(inp, P + i, cache, policy=policy, forced_exit=fe,
                                   keep_state=keep_state)
            tokens.append(rec.token)
            exits.append(rec.exit_depth)
            records.append(rec)
        return tokens, exits, records

    # ------------------------------------------- per-row stage functions
    # The CDB simulator drives the same arithmetic one row at a time, so
    # any batched schedule is batch-invariant by construction.
    def row_prelude(self, token: int, pos: int, cache: SeqCache) -> "Row":
        h, inj = self._prelude([token], np.array([pos]), cache)
        return Row(pos=pos, h=h, inj=inj, cache=cache, exit_at=self.d.r_max)

    def row_core(self, row: "Row") -> None:
        row.depth += 1
        row.h_prev = row.h
        x = row.h + row.inj if row.inj is not None else row.h
        row.h = self.core(x, np.array([row.pos]), row.depth, row.cache)

    def row_gate(self, row: "Row", policy: str = "adaptive") -> bool:
        """After a core step: True when the row leaves the core now.  Else,
        under the adaptive policy, a gate firing schedules the exit after the
        next step (lookahead)."""
        if row.depth == row.exit_at:
            return True
        if policy == "adaptive":
            g = self.gate_eval(row.h[0], row.h_prev[0], row.depth)
            if g is not None and g[1]:
                row.exit_at = row.depth + 1
        return False

    def row_coda(self, row: "Row") -> int:
        """Last-exited fill of the skipped depth slots, record e, then coda
        and greedy argmax."""
        e, pos, cache = row.depth, row.pos, row.cache
        self._last_exited_fill(cache, pos, e)
        cache.exit_depth[pos] = e
        logits = self.coda_logits(row.h, np.array([pos]), cache)[0]
        return int(np.argmax(logits))

    # ------------------------------------------------ single-row core step
    def core_step_row(self, h_row: np.ndarray, pos: int, depth: int, cache: SeqCache):
        """One core step of a single decode row at ``pos`` and ``depth`` on a
        cache whose earlier positions are complete (last-exited copies in
        place).  Returns (output state, K rows written [n_core, nh, hd],
        V rows written)."""
        out = self.core(np.asarray(h_row, dtype=self.dt)[None], np.array([pos]), depth, cache)
        plane = kv_slot(self.d, depth)
        return out[0], cache.core_k[:, plane, pos].copy(), cache.core_v[:, plane, pos].copy()


def cache_from_planes(dims, core_k, core_v, exit_depth, dtype=np.float32) -> SeqCache:
    """Build a SeqCache from synthetic planes with gaps.

    core_k, core_v: [n_core, planes, n_pos, nh, hd] holding valid data in
    planes < e_j of each position j (deeper planes may hold anything); the
    last-exited fill (§4.2) then copies plane e_j into the deeper ones.  For a
    single-slot layout (planes = 1) the arrays are taken as they are.  For
    first-then-shared (planes = 2: the first loop's state, then the most
    recent one) a position that left after its first loop never wrote the
    shared slot; its most recent state is the first loop's, so the private
    slot is copied there (synthetic contexts only: decoded tokens leave at
    depth >= 2)."""
    n_pos = core_k.shape[2]
    c = SeqCache(dims, n_pos + 1, dtype)
    c.core_k[:, :, :n_pos] = core_k
    c.core_v[:, :, :n_pos] = core_v
    c.exit_depth[:n_pos] = exit_depth
    if dims.kv_layout == "depth":
        R = dims.r_max
        for j in range(n_pos):
            e = int(exit_depth[j])
            if e < R:
                c.core_k[:, e:, j] = c.core_k[:, e - 1 : e, j]
                c.core_v[:, e:, j] = c.core_v[:, e - 1 : e, j]
    elif dims.kv_layout == "first_shared":
        for j in range(n_pos):
            if int(exit_depth[j]) == 1:
                c.core_k[:, 1, j] = c.core_k[:, 0, j]
                c.core_v[:, 1, j] = c.core_v[:, 0, j]
    return c
