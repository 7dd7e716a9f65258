"""CPU simulator of the CDB stage scheduler.  Test infrastructure only.

"Depth-adaptive Inference of Looped Language Models via Continuous Depth
Batching" (arXiv 2608.09444):

* §4.1 Stage-wise Scheduling: four queues — requests waiting for prefill,
  decode tokens awaiting the prelude, recurrent items ready for their next
  loop step, exited tokens awaiting the coda.
* Alg. 1 (App. A.3), no-refill: admit and prefill while CanPrefill allows,
  then prelude the whole decode queue, loop the cohort (the batch only
  shrinks as tokens exit) and run the coda once for the cohort.
* Alg. 2 (App. A.3), refill: each iteration runs, in priority order, coda
  (+ prelude) when at least K exits wait, else prefill (+ prelude) when
  CanPrefill allows, else one core step over every ready recurrent item.
* §6.1: continuous batching (CB), the baseline, runs r_max loops for every
  token with the same admission policy — here Alg. 1 with the gate off.
* App. A.1 "Chunked prefill" and Fig. 8 left: prompts are packed into
  prefill batches of at most M tokens; a prompt that does not fit is split
  and continues in the next prefill batch.
* App. A.2: at most W active sequences; prefill starts only when at least S
  slots are free; KV headroom rho_KV stops admission.
* App. A.4, Tables 2-3: the traces this module reproduces (queue sizes are
  taken after each stage; a loop stage lists how many tokens run their i-th
  loop step and how many exit).

Readings (the pages leave these open): a partially prefilled prompt always
continues before new requests are admitted and does not wait for S free
slots; a request is active (counts toward W) from its first prefill chunk
until its last token; when the recurrent queue is empty and nothing can be
prefilled, the coda runs even below K exits; admission reserves a request's
whole KV lifetime (prompt + outputs) because output lengths are fixed and
preemption is disabled (Table 1).

Two executors drive the stages: ``ModelExecutor`` runs the oracle model on
each row (the stage arithmetic is per row, so a batched schedule must give
exactly the tokens and exits of ``OracleLM.decode_sequential``), and
``ScriptedExecutor`` replays given exit depths without a model (the pages'
own exit-decision replay, App. C.2).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np


@dataclass
class Request:
    rid: int
    prompt: np.ndarray
    n_out: int
    prefilled: int = 0
    admitted: bool = False
    finished: bool = False
    tokens: List[int] = field(default_factory=list)
    exits: List[int] = field(default_factory=list)
    blocks: int = 0

    @property
    def prompt_len(self) -> int:
        return len(self.prompt)


@dataclass
class Item:
    """A decode token in flight: request, decode-pass index, position, and
    whatever the executor keeps for the row."""
    req: Request
    pass_idx: int
    pos: int
    token: int
    row: object = None
    depth: int = 0
    exit_at: int = 0


@dataclass
class Stage:
    kind: str            # prefill | prelude | loop | coda
    B: int
    detail: str
    queues: tuple        # refill: (Q_R, Q_C, Q_P); no-refill/fixed: (Q_D, Q_P)


class ScriptedExecutor:
    """Replays exit depths: script[rid][pass] = exit depth (default r_max).
    Tokens are dummies (0)."""

    def __init__(self, r_max: int, script: Optional[Dict[int, Dict[int, int]]] = None):
        self.r_max = r_max
        self.script = script or {}

    def begin(self, req: Request):
        pass

    def prefill_chunk(self, req: Request, start: int, end: int) -> Optional[int]:
        return 0 if end == req.prompt_len else None

    def prelude(self, it: Item):
        it.row = None

    def core(self, it: Item):
        pass

    def decide(self, it: Item, policy: str) -> bool:
        """After the core step at it.depth: does the token leave now?"""
        if it.depth == it.exit_at:
            return True
        if policy == "adaptive":
            e = self.script.get(it.req.rid, {}).get(it.pass_idx, self.r_max)
            if it.depth == e - 1:
                it.exit_at = e
        return False

    def coda(self, it: Item) -> int:
        return 0

    def end(self, req: Request):
        pass


class ModelExecutor:
    """Runs the oracle model one row at a time."""

    def __init__(self, model, chunks_of=None):
        self.m = model
        self.caches = {}
        self._chunked: Dict[int, list] = {}

    def begin(self, req: Request):
        from .model import SeqCache
        self.caches[req.rid] = SeqCache(self.m.d, req.prompt_len + req.n_out, self.m.dt)
        self._chunked[req.rid] = []

    def prefill_chunk(self, req: Request, start: int, end: int) -> Optional[int]:
        # Prefill arithmetic of a chunk depends only on the chunk boundaries
        # (depth-indexed: not even on those); the oracle's prefill runs the
        # whole recorded chunk list when the prompt completes.
        self._chunked[req.rid].append((start, end))
        if end < req.prompt_len:
            return None
        tok, _, _ = self.m.prefill(req.prompt, self.caches[req.rid], self._chunked[req.rid])
        return tok

    def prelude(self, it: Item):
        it.row = self.m.row_prelude(it.token, it.pos, self.caches[it.req.rid])
        it.row.exit_at = it.exit_at

    def core(self, it: Item):
        self.m.row_core(it.row)

    def decide(self, it: Item, policy: str) -> bool:
        it.row.exit_at = it.exit_at
        leave = self.m.row_gate(it.row, policy)
        it.exit_at = it.row.exit_at
        return leave

    def coda(self, it: Item) -> int:
        return self.m.row_coda(it.row)

    def end(self, req: Request):
        self.caches.pop(req.rid, None)


class CDBSimulator:
    """mode: "refill" (Alg. 2), "norefill" (Alg. 1) or "fixed" (CB: Alg. 1
    with every token at r_max)."""

    def __init__(self, requests: Sequence[Request], executor, r_max: int, mode: str,
                 W: int, K: int = 1, M: int = 8192, S: Optional[int] = None,
                 rho_kv: float = 0.0, kv_blocks: Optional[int] = None, block_size: int = 16):
        self.reqs = list(requests)
        self.ex = executor
        self.R = r_max
        self.mode = mode
        self.policy = "fixed" if mode == "fixed" else "adaptive"
        self.W, self.K, self.M = W, K, M
        self.S = max(1, W // 8) if S is None else S
        self.rho = rho_kv
        self.kv_blocks = kv_blocks
        self.bs = block_size
        self.free_blocks = kv_blocks
        self.q_pre: List[Request] = list(self.reqs)      # never admitted
        self.partial: Optional[Request] = None            # admitted, prompt not complete
        self.q_r: List[Item] = []
        self.q_c: List[Item] = []
        self.q_dec: List[Item] = []                       # Alg. 1 decode queue
        self.active = 0
        self.trace: List[Stage] = []
        self.n_core_steps = 0
        self.core_token_steps = 0

    # ------------------------------------------------------------ helpers
    def _blocks_for(self, req: Request) -> int:
        return -(-(req.prompt_len + req.n_out) // self.bs)

    def _kv_ok(self, req: Request) -> bool:
        if self.kv_blocks is None:
            return True
        need = self._blocks_for(req)
        return self.free_blocks - need >= self.rho * self.kv_blocks and need <= self.free_blocks

    def can_prefill(self) -> bool:
        if self.partial is not None:
            return True
        if not self.q_pre:
            return False
        return (self.W - self.active) >= self.S and self._kv_ok(self.q_pre[0])

    def _queues(self):
        if self.mode == "refill":
            return (len(self.q_r), len(self.q_c), len(self.q_pre))
        return (len(self.q_dec), len(self.q_pre))

    def _log(self, kind, B, detail):
        self.trace.append(Stage(kind, B, detail, self._queues()))

    def _finish(self, req: Request):
        req.finished = True
        self.active -= 1
        if self.kv_blocks is not None:
            self.free_blocks += req.blocks
        self.ex.end(req)

    def _new_item(self, req: Request, token: int) -> Item:
        i = len(req.tokens) - 1          # decode pass index; input = tokens[i]
        return Item(req=req, pass_idx=i, pos=req.prompt_len + i, token=token, exit_at=self.R)

    # ------------------------------------------------------------ stages
    def _prefill(self) -> List[Item]:
        """Pack up to M prompt tokens; returns the new decode items of prompts
        that completed (for sequences that need more tokens)."""
        budget = self.M
        parts = []                        # (req, start, end)
        if self.partial is not None:
            r = self.partial
            n = min(budget, r.prompt_len - r.prefilled)
            parts.append((r, r.prefilled, r.prefilled + n))
            budget -= n
            self.partial = None if r.prefilled + n == r.prompt_len else r
        while budget > 0 and self.partial is None and self.q_pre and self.active < self.W \
                and self._kv_ok(self.q_pre[0]):
            r = self.q_pre.pop(0)
            r.admitted = True
            self.active += 1
            if self.kv_blocks is not None:
                r.blocks = self._blocks_for(r)
                self.free_blocks -= r.blocks
            self.ex.begin(r)
            n = min(budget, r.prompt_len)
            parts.append((r, 0, n))
            budget -= n
            if n < r.prompt_len:
                self.partial = r
        done = []
        for (r, s, e) in parts:
            r.prefilled = e
            tok = self.ex.prefill_chunk(r, s, e)
            if tok is not None:
                r.tokens.append(tok)
                if len(r.tokens) >= r.n_out:
                    self._finish(r)
                else:
                    done.append(self._new_item(r, tok))
        self._pending_prefill_log = (len(parts), self.M - budget)
        return done

    def _prelude(self, items: List[Item]):
        for it in items:
            self.ex.prelude(it)

    def _core_step(self, items: List[Item]):
        """One loop step for every item; returns (exited, continuing)."""
        hist: Dict[int, int] = {}
        for it in items:
            self.ex.core(it)
            it.depth += 1
            hist[it.depth] = hist.get(it.depth, 0) + 1
        exited, cont = [], []
        for it in items:
            (exited if self.ex.decide(it, self.policy) else cont).append(it)
        self.n_core_steps += 1
        self.core_token_steps += len(items)
        detail = " ".join(f"r{d}:{hist[d]}" for d in sorted(hist))
        if exited:
            detail += f"; {len(exited)} exit" + ("s" if len(exited) > 1 else "")
        return exited, cont, detail

    def _coda(self, items: List[Item]) -> List[Item]:
        nxt = []
        for it in items:
            tok = self.ex.coda(it)
            r = it.req
            r.exits.append(it.depth)
            r.tokens.append(tok)
            if len(r.tokens) >= r.n_out:
                self._finish(r)
            else:
                nxt.append(self._new_item(r, tok))
        return nxt

    # ------------------------------------------------------------ drivers
    def _all_done(self):
        return all(r.finished for r in self.reqs)

    def run(self, max_stages: Optional[int] = None):
        while not self._all_done():
            if max_stages is not None and len(self.trace) >= max_stages:
                break
            if self.mode == "refill":
                self._step_refill()
            else:
                self._step_norefill(max_stages)
        return self

    def _step_refill(self):
        if self.q_c and (len(self.q_c) >= self.K or (not self.q_r and not self.can_prefill())):
            E, self.q_c = self.q_c, []
            nxt = self._coda(E)
            self._log("coda", len(E), "")
            if nxt:
                self._prelude(nxt)
                self.q_r.extend(nxt)
                self._log("prelude", len(nxt), "after coda")
        elif self.can_prefill():
            new = self._prefill()
            nseq, ntok = self._pending_prefill_log
            self._log("prefill", nseq, f"{ntok} prompt tokens")
            if new:
                self._prelude(new)
                self.q_r.extend(new)
                self._log("prelude", len(new), "after prefill")
        elif self.q_r:
            H, self.q_r = self.q_r, []
            exited, cont, detail = self._core_step(H)
            self.q_c.extend(exited)
            self.q_r.extend(cont)
            self._log("loop", len(H), detail)
        else:
            raise RuntimeError("refill scheduler stalled")

    def _step_norefill(self, max_stages):
        while self.can_prefill():
            new = self._prefill()
            self.q_dec.extend(new)
            nseq, ntok = self._pending_prefill_log
            self._log("prefill", nseq, f"{ntok} prompt tokens")
            if max_stages is not None and len(self.trace) >= max_stages:
                return
        if not self.q_dec:
            if self._all_done():
                return
            raise RuntimeError("no-refill scheduler stalled")
        B, self.q_dec = self.q_dec, []
        self._prelude(B)
        self._log("prelude", len(B), "")
        H, E = B, []
        for _ in range(self.R):
            exited, H, detail = self._core_step(H)
            E.extend(exited)
            self._log("loop", len(exited) + len(H), detail)
            if not H:
                break
        nxt = self._coda(E)
        self.q_dec = nxt
        self._log("coda", len(E), "")


def simulate(requests, executor, r_max, mode, W, **kw) -> CDBSimulator:
    return CDBSimulator(requests, executor, r_max, mode, W, **kw).run()
