"""Device buffers, the libcdb context, and the CPU stage scheduler.

"Depth-adaptive Inference of Looped Language Models via Continuous Depth
Batching" (arXiv 2608.09444):
* §4.1 and Alg. 2 (refill): in priority order — coda (+ prelude of the
  successors) once at least K exits wait; else prefill (+ prelude) when
  CanPrefill allows; else one recurrent-core step over the whole recurrent
  queue.  Alg. 1 (no-refill): prefill while CanPrefill allows, then loop the
  cohort until every token has exited, then one coda for the cohort.  Fixed
  depth (the CB baseline of §6.1): Alg. 1 with the gate off.
* App. A.1 / A.2: chunked prefill of at most M tokens; at most W active
  sequences; prefill waits for S free slots; paged KV of 16-token blocks.
* §4.3 / A.5: batches padded to power-of-two buckets.

The recurrent queue, the coda queue and the successor tokens live on the
device (cdb_gate_compact and cdb_boundary update them in place); the CPU
reads back only the per-step counts and the sequences that left, which it
needs for admission and for choosing the next bucket.  PyTorch provides the
device memory and the stream; every stage runs in libcdb's kernels.

Readings where the pages leave the policy open are the same as the ones
the design notes list: a partially prefilled prompt continues first and
does not wait for S; a request holds its slot from its first prefill chunk
to its last token; with an empty recurrent queue and nothing to prefill the
coda runs below K; admission reserves the request's whole KV lifetime
(prompt + outputs) because output lengths are fixed and preemption is off.
"""
from __future__ import annotations

import ctypes as C
import time
from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence

import numpy as np
import torch

from . import _lib as L


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def pow2(n: int) -> int:
    p = 1
    while p < n:
        p *= 2
    return p


class DeviceModel:
    """Weights on the device in the library's layouts (see include/cdb.h)."""

    def __init__(self, dims, weights: Dict[str, np.ndarray], device="cuda"):
        self.dims = dims
        wdt = torch.bfloat16 if dims.dtype == "bf16" else torch.float32
        self.wdt = wdt
        t = lambda a, dt=wdt: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device=device, dtype=dt)
        c_dtype = L.CDB_BF16 if dims.dtype == "bf16" else L.CDB_FP32
        stream = torch.cuda.current_stream(device)

        def packed(a):
            """Row-major [out][in] on the device, rewritten by the library into
            its fragment-packed layout."""
            src = t(a)
            dst = torch.empty_like(src)
            L.check(L.lib.cdb_pack_weight(c_dtype, _ptr(src), _ptr(dst), src.shape[0], src.shape[1],
                                          C.c_void_p(stream.cuda_stream)))
            stream.synchronize()
            return dst

        self.keep = []

        def layer(prefix):
            lw = dict(
                attn_norm=t(weights[prefix + ".attn_norm"], torch.float32),
                wqkv=packed(np.concatenate([weights[prefix + ".wq"], weights[prefix + ".wk"],
                                            weights[prefix + ".wv"]])),
                wo=packed(weights[prefix + ".wo"]),
                mlp_norm=t(weights[prefix + ".mlp_norm"], torch.float32),
                wgu=packed(np.concatenate([weights[prefix + ".wg"], weights[prefix + ".wu"]])),
                wd=packed(weights[prefix + ".wd"]),
            )
            self.keep.append(lw)
            return L.cdb_layer(*[_ptr(lw[k]) for k in ("attn_norm", "wqkv", "wo", "mlp_norm", "wgu", "wd")])

        self.embed = t(weights["embed"])
        self.final_norm = t(weights["final_norm"], torch.float32)
        self.lm_head = packed(weights["lm_head"])
        self.gate_w = t(weights["gate_w"], torch.float32)
        mk = lambda stage, n: (L.cdb_layer * max(n, 1))(*[layer(f"{stage}.{i}") for i in range(n)])
        self.pre = mk("prelude", dims.n_prelude)
        self.core = mk("core", dims.n_core)
        self.coda = mk("coda", dims.n_coda)
        self.c_weights = L.cdb_weights(_ptr(self.embed), self.pre, self.core, self.coda,
                                       _ptr(self.final_norm), _ptr(self.lm_head), _ptr(self.gate_w))

    def c_dims(self, kv_layout=None):
        d = self.dims
        lay = {"depth": L.CDB_KV_DEPTH, "single": L.CDB_KV_SINGLE, "first_shared": L.CDB_KV_FIRST_SHARED,
               "depth_copy": L.CDB_KV_DEPTH_COPY}[kv_layout or d.kv_layout]
        kind = {"linear": L.CDB_GATE_LINEAR, "convergence": L.CDB_GATE_CONVERGENCE}[d.gate_kind]
        return L.cdb_dims(d.vocab, d.hidden, d.n_heads, d.head_dim, d.ffn, d.n_prelude, d.n_core, d.n_coda,
                          d.r_max, L.CDB_BF16 if d.dtype == "bf16" else L.CDB_FP32, lay, 1 if d.inject else 0,
                          kind, d.rms_eps, d.rope_theta, float(np.float32(d.gate_bias)), d.gate_threshold,
                          float(np.float32(d.conv_threshold)))


class Engine:
    """One libcdb context with every buffer it needs."""

    def __init__(self, model: DeviceModel, n_slots: int, max_rows: int, num_blocks: int, max_seqs: int,
                 max_blocks_per_seq: int, max_out: int, max_prefill_tokens: int = 8192,
                 kv_layout: Optional[str] = None, device="cuda", kv_fill: Optional[float] = None,
                 static_workspace: bool = False):
        d = model.dims
        self.m, self.d = model, d
        # One non-default stream (default priority) carries the library's
        # work and the caller's torch work on the engine's buffers, so they
        # stay ordered; a non-default stream can also be captured into graphs.
        self.prev_stream = torch.cuda.current_stream(device)
        self.stream = torch.cuda.Stream(device=device)
        self.stream.wait_stream(self.prev_stream)
        torch.cuda.set_stream(self.stream)
        self.kv_layout = kv_layout or d.kv_layout
        self.planes = {"depth": d.r_max, "single": 1, "first_shared": 2, "depth_copy": d.r_max}[self.kv_layout]
        self.max_rows, self.n_slots = max_rows, n_slots
        self.num_blocks, self.max_seqs, self.mbps, self.max_out = num_blocks, max_seqs, max_blocks_per_seq, max_out
        self.max_T = max_prefill_tokens
        dev = device
        kvdt = model.wdt
        i32 = dict(dtype=torch.int32, device=dev)
        per_plane = num_blocks * d.n_heads * 16 * d.head_dim
        fill = float("nan") if kv_fill is None else kv_fill
        self.core_k = torch.full((d.n_core * self.planes * per_plane,), fill, dtype=kvdt, device=dev)
        self.core_v = torch.full_like(self.core_k, fill)
        nb = d.n_prelude + d.n_coda
        self.bnd_k = torch.full((max(nb, 1) * per_plane,), fill, dtype=kvdt, device=dev) if nb else None
        self.bnd_v = torch.full_like(self.bnd_k, fill) if nb else None
        self.emap = torch.zeros(num_blocks * 16, dtype=torch.uint8, device=dev)
        self.btab = torch.zeros(max_seqs * max_blocks_per_seq, **i32)
        self.state = torch.zeros(n_slots, d.hidden, dtype=torch.float32, device=dev)
        self.inject = torch.zeros_like(self.state) if d.inject else None
        self.prev_state = torch.zeros_like(self.state) if d.gate_kind == "convergence" else None
        self.tokens_out = torch.full((max_seqs, max_out), -1, **i32)
        self.exits_out = torch.zeros((max_seqs, max_out), **i32)
        self.n_gen = torch.zeros(max_seqs, **i32)
        self.n_out = torch.zeros(max_seqs, **i32)
        # core batch (recurrent queue) and coda queue at fixed addresses
        cap = max_rows
        self.desc_t = torch.zeros(5 * cap + 1, **i32)
        self.desc = L.cdb_core_desc(*[_ptr(x) for x in (self.desc_t[0:1], self.desc_t[1:1 + cap],
                                                        self.desc_t[1 + cap:1 + 2 * cap],
                                                        self.desc_t[1 + 2 * cap:1 + 3 * cap],
                                                        self.desc_t[1 + 3 * cap:1 + 4 * cap],
                                                        self.desc_t[1 + 4 * cap:1 + 5 * cap])], cap)
        self.q_t = torch.zeros(4 * cap + 1, **i32)
        self.q_seq_view = self.q_t[1 + cap:1 + 2 * cap]
        self.exq = L.cdb_exit_queue(*[_ptr(x) for x in (self.q_t[0:1], self.q_t[1:1 + cap], self.q_t[1 + cap:1 + 2 * cap],
                                                        self.q_t[1 + 2 * cap:1 + 3 * cap], self.q_t[1 + 3 * cap:1 + 4 * cap])],
                                    cap)
        self.counts = torch.zeros(4, **i32)
        self.fired = torch.zeros(cap, **i32)
        # two pinned readback buffers, so a step's counts can be read while the next step runs
        self.h_counts = torch.zeros((2, 4), dtype=torch.int32, pin_memory=True)
        self.h_fired = torch.zeros((2, cap), dtype=torch.int32, pin_memory=True)
        self.cout = [L.cdb_compact_out(_ptr(self.counts), _ptr(self.fired), _ptr(self.h_counts[i]),
                                       _ptr(self.h_fired[i]), None) for i in range(2)]
        cdims = model.c_dims(self.kv_layout)
        self.cdims = cdims
        wsb = L.lib.cdb_workspace_bytes(C.byref(cdims), max_rows, max_prefill_tokens, max_blocks_per_seq * 16)
        if wsb == 0:
            raise L.CDBError(L.CDB_EINVAL, L.lib.cdb_last_error().decode())
        # static_workspace: the context uses the library's static device
        # scratch (cdb_init_static) and no workspace is allocated here
        self.workspace = None if static_workspace else torch.zeros(wsb, dtype=torch.uint8, device=dev)
        self.c_kv = L.cdb_kv(16, num_blocks, _ptr(self.core_k), _ptr(self.core_v), _ptr(self.bnd_k), _ptr(self.bnd_v),
                             _ptr(self.emap), _ptr(self.btab), max_seqs, max_blocks_per_seq)
        self.c_pools = L.cdb_pools(_ptr(self.state), _ptr(self.inject), _ptr(self.prev_state), n_slots,
                                   _ptr(self.workspace), 0 if static_workspace else wsb, max_rows,
                                   max_prefill_tokens, max_blocks_per_seq * 16)
        self.c_seqs = L.cdb_seqs(_ptr(self.tokens_out), _ptr(self.exits_out), _ptr(self.n_gen), _ptr(self.n_out), max_out)
        self.ctx = C.c_void_p()
        init = L.lib.cdb_init_static if static_workspace else L.lib.cdb_init
        L.check(init(C.byref(cdims), C.byref(model.c_weights), C.byref(self.c_kv), C.byref(self.c_pools),
                     C.byref(self.c_seqs), C.c_void_p(self.stream.cuda_stream), C.byref(self.ctx)))

    def close(self):
        if self.ctx:
            self.stream.synchronize()
            L.lib.cdb_destroy(self.ctx)
            self.ctx = C.c_void_p()
            if torch.cuda.current_stream(self.stream.device) == self.stream:
                torch.cuda.set_stream(self.prev_stream)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # ------------------------------------------------------------ stages
    def core_step(self, rows_pad: int):
        L.check(L.lib.cdb_core_step(self.ctx, C.byref(self.desc), rows_pad))

    def gate_compact(self, rows_pad: int, gate_enabled: bool = True, buf: int = 0):
        L.check(L.lib.cdb_gate_compact(self.ctx, C.byref(self.desc), rows_pad, 1 if gate_enabled else 0,
                                       C.byref(self.exq), C.byref(self.cout[buf])))

    def boundary(self, rows_pad: int, exit_states: Optional[torch.Tensor] = None,
                 logits: Optional[torch.Tensor] = None, tokens_rows: Optional[torch.Tensor] = None):
        bd = L.cdb_boundary_desc(rows_pad, _ptr(exit_states), _ptr(logits), _ptr(tokens_rows))
        L.check(L.lib.cdb_boundary(self.ctx, C.byref(self.exq), C.byref(self.desc), C.byref(bd)))

    def prefill(self, parts, logits: Optional[torch.Tensor] = None):
        """parts: list of (seq, slot, start_pos, token array, is_final).  The
        token and descriptor arrays go up through a ring of pinned buffers
        with an asynchronous copy, so a prefill does not wait for the work
        queued before it."""
        cu = np.zeros(len(parts) + 1, dtype=np.int32)
        for i, p in enumerate(parts):
            cu[i + 1] = cu[i] + len(p[3])
        toks = np.concatenate([np.asarray(p[3], dtype=np.int32) for p in parts])
        seq = np.array([p[0] for p in parts], dtype=np.int32)
        slot = np.array([p[1] for p in parts], dtype=np.int32)
        start = np.array([p[2] for p in parts], dtype=np.int32)
        fin = np.array([1 if p[4] else 0 for p in parts], dtype=np.int32)
        host = np.concatenate([toks, cu, seq, start, slot, fin])
        n, T = len(parts), len(toks)
        if not hasattr(self, "_pf_ring"):
            cap_i = self.max_T + 5 * (self.max_T + 1) + 8
            self._pf_ring = [(torch.empty(cap_i, dtype=torch.int32, pin_memory=True),
                              torch.empty(cap_i, dtype=torch.int32, device=self.state.device),
                              torch.cuda.Event()) for _ in range(4)]
            self._pf_next = 0
        hbuf, dbuf, ev = self._pf_ring[self._pf_next]
        self._pf_next = (self._pf_next + 1) % len(self._pf_ring)
        ev.synchronize()                      # the slot's previous upload and prefill have finished
        if len(host) > hbuf.numel():
            raise ValueError("prefill chunk larger than max_prefill_tokens")
        hbuf[: len(host)].copy_(torch.from_numpy(host))
        dbuf[: len(host)].copy_(hbuf[: len(host)], non_blocking=True)
        o = [0, T, T + n + 1, T + 2 * n + 1, T + 3 * n + 1, T + 4 * n + 1]
        self._pf_keep = (cu, start, fin)
        pd = L.cdb_prefill_desc(n, T, _ptr(dbuf[o[0]:]), _ptr(dbuf[o[1]:]), _ptr(dbuf[o[2]:]), _ptr(dbuf[o[3]:]),
                                _ptr(dbuf[o[4]:]), _ptr(dbuf[o[5]:]), cu.ctypes.data_as(C.c_void_p),
                                start.ctypes.data_as(C.c_void_p), fin.ctypes.data_as(C.c_void_p), _ptr(logits))
        L.check(L.lib.cdb_prefill(self.ctx, C.byref(pd), C.byref(self.desc)))
        ev.record(self.stream)

    def sync(self):
        L.check(L.lib.cdb_sync(self.ctx))

    # ------------------------------------------------------------ graphs
    def capture(self, fn):
        """Record the library calls made by fn() into a HIP graph (handle)."""
        self.stream.synchronize()
        L.check(L.lib.cdb_graph_begin(self.ctx))
        try:
            fn()
        finally:
            g = C.c_void_p()
            rc = L.lib.cdb_graph_end(self.ctx, C.byref(g))
        L.check(rc)
        return g

    def replay(self, g):
        L.check(L.lib.cdb_graph_launch(self.ctx, g))

    @staticmethod
    def drop(g):
        if g:
            L.lib.cdb_graph_destroy(g)

    def read_counts(self, buf: int = 0):
        self.sync()
        return [int(x) for x in self.h_counts[buf].tolist()]


# ------------------------------------------------------------ scheduler
@dataclass
class Req:
    rid: int
    prompt: np.ndarray
    n_out: int
    prefilled: int = 0
    slot: int = -1
    blocks: List[int] = field(default_factory=list)
    n_gen: int = 0
    finished: bool = False
    admitted: bool = False


@dataclass
class StageLog:
    kind: str
    B: int
    detail: str
    gpu_s: float = 0.0


class Scheduler:
    """CPU side of CDB: admission, prefill packing, stage order, buckets."""

    def __init__(self, eng: Engine, prompts: Sequence[np.ndarray], n_out, mode: str = "refill", W: int = 64,
                 K: int = 1, M: int = 8192, S: Optional[int] = None, rho_kv: float = 0.0, timing: bool = False,
                 capture_states: bool = False, capture_logits: bool = False, graphs: bool = False,
                 events: bool = False, gate: bool = True):
        if mode not in ("refill", "norefill", "fixed"):
            raise ValueError(mode)
        # gate=False keeps the mode's stage policy but never exits early:
        # CDB at full depth, the overhead comparison with fixed-depth CB (§6.2)
        self.gate_on = gate and mode != "fixed"
        self.e = eng
        outs = [n_out] * len(prompts) if np.isscalar(n_out) else list(n_out)
        self.reqs = [Req(i, np.asarray(p, dtype=np.int32), int(o)) for i, (p, o) in enumerate(zip(prompts, outs))]
        if len(self.reqs) > eng.max_seqs:
            raise ValueError("more requests than max_seqs")
        if W > eng.n_slots or W > eng.max_rows:
            raise ValueError("W exceeds the engine's slots or rows")
        if M > eng.max_T:
            raise ValueError("M exceeds max_prefill_tokens")
        self.mode, self.W, self.K, self.M = mode, W, K, M
        self.S = max(1, W // 8) if S is None else S
        self.rho = rho_kv
        self.waiting = list(self.reqs)
        self.partial: Optional[Req] = None
        self.active = 0
        self.free_slots = list(range(W))[::-1]
        self.free_blocks = list(range(eng.num_blocks))[::-1]
        self.qr = 0               # recurrent queue rows (device n_valid)
        self.qc = 0               # coda queue rows
        self.qc_seqs: List[int] = []
        self.log: List[StageLog] = []
        self.core_steps = 0
        self.core_token_steps = 0
        self.timing = timing
        self.capture = capture_states
        self.exit_states: Dict[tuple, np.ndarray] = {}     # (seq, token index) -> state at exit
        self._st_buf = torch.zeros(eng.max_rows, eng.d.hidden, dtype=torch.float32,
                                   device=eng.state.device) if capture_states else None
        self.capture_logits = capture_logits
        self.logits: Dict[tuple, np.ndarray] = {}          # (seq, token index) -> logits of that token
        self._lg_buf = torch.zeros(eng.max_rows, eng.d.vocab, dtype=torch.float32,
                                   device=eng.state.device) if capture_logits else None
        # core step + gate/compaction recorded once per row bucket and replayed
        # (the descriptor lives at fixed device addresses, so a graph stays valid)
        self.use_graphs = graphs
        self.graphs: Dict[int, object] = {}
        self.progress = None      # optional callable(finished requests, core steps), every ~20 s of host time
        self._t_prog = 0.0
        self.t_prefill = 0.0
        self.t_core = 0.0
        self.t_coda = 0.0
        self.t_total = 0.0
        # events around every stage's GPU work: (kind, start, end), for the
        # GPU idle fraction of the run
        self.events = events
        self._evs = []
        eng.n_gen.zero_()
        eng.n_out[: len(self.reqs)] = torch.tensor([r.n_out for r in self.reqs], dtype=torch.int32)
        eng.desc_t[0] = 0
        eng.q_t[0] = 0

    # -------------------------------------------------------- admission
    def _blocks_for(self, r: Req) -> int:
        return -(-(len(r.prompt) + r.n_out) // 16)

    def _kv_ok(self, r: Req) -> bool:
        need = self._blocks_for(r)
        return need <= len(self.free_blocks) and len(self.free_blocks) - need >= self.rho * self.e.num_blocks

    def can_prefill(self) -> bool:
        if self.partial is not None:
            return True
        return bool(self.waiting) and (self.W - self.active) >= self.S and self._kv_ok(self.waiting[0])

    def _admit(self, r: Req):
        r.admitted = True
        r.slot = self.free_slots.pop()
        nb = self._blocks_for(r)
        if nb > self.e.mbps:
            raise ValueError(f"request {r.rid} needs {nb} blocks > max_blocks_per_seq")
        r.blocks = [self.free_blocks.pop() for _ in range(nb)]
        row = torch.tensor(r.blocks, dtype=torch.int32)
        self.e.btab[r.rid * self.e.mbps: r.rid * self.e.mbps + nb] = row.to(self.e.btab.device)
        self.active += 1

    def _finish(self, r: Req):
        r.finished = True
        self.active -= 1
        self.free_slots.append(r.slot)
        self.free_blocks.extend(r.blocks)
        r.blocks = []

    def _pack(self):
        budget = self.M
        parts = []
        if self.partial is not None:
            r = self.partial
            n = min(budget, len(r.prompt) - r.prefilled)
            parts.append((r, r.prefilled, r.prefilled + n))
            budget -= n
            self.partial = None if r.prefilled + n == len(r.prompt) else r
        while budget > 0 and self.partial is None and self.waiting and self.active < self.W \
                and self._kv_ok(self.waiting[0]):
            r = self.waiting.pop(0)
            self._admit(r)
            n = min(budget, len(r.prompt))
            parts.append((r, 0, n))
            budget -= n
            if n < len(r.prompt):
                self.partial = r
        return parts, self.M - budget

    # ------------------------------------------------------------ stages
    def _t0(self):
        if self.timing:
            torch.cuda.synchronize()
        return time.perf_counter()

    def _do_prefill(self):
        parts, ntok = self._pack()
        t0 = self._t0()
        self._stage("prefill", lambda: self.e.prefill(
            [(r.rid, r.slot, s, r.prompt[s:e], e == len(r.prompt)) for (r, s, e) in parts]))
        for (r, s, e) in parts:
            r.prefilled = e
        done = 0
        for (r, s, e) in parts:
            if e == len(r.prompt):
                r.n_gen = 1
                if r.n_gen >= r.n_out:
                    self._finish(r)
                else:
                    done += 1
        self.qr += done
        dt = self._t1(t0)
        self.t_prefill += dt
        self.log.append(StageLog("prefill", len(parts), f"{ntok} prompt tokens", dt))
        if done:
            self.log.append(StageLog("prelude", done, "after prefill"))

    def _stage(self, kind, fn):
        """Launch one stage, bracketed by events when recording them."""
        if not self.events:
            fn()
            return
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(self.e.stream)
        fn()
        b.record(self.e.stream)
        self._evs.append((kind, a, b))

    def gpu_idle_fraction(self) -> Optional[float]:
        """Share of the GPU time span from the first stage's start to the
        last stage's end during which no stage ran (Fig. 3's idle time):
        1 - sum of stage durations / span.  Needs the stage events (the
        lookahead scheduler always records them)."""
        if not self._evs:
            return None
        torch.cuda.synchronize()
        busy = sum(a.elapsed_time(b) for _, a, b in self._evs)
        span = self._evs[0][1].elapsed_time(self._evs[-1][2])
        return max(0.0, 1.0 - busy / span) if span > 0 else 0.0

    def _t1(self, t0):
        if self.timing:
            torch.cuda.synchronize()
        return time.perf_counter() - t0

    def _do_core(self):
        B = self.qr
        rows = pow2(B)
        t0 = self._t0()
        if self.use_graphs:
            g = self.graphs.get(rows)
            if g is None:
                g = self.graphs[rows] = self.e.capture(lambda: self._core_calls(rows))
            self._stage("core", lambda: self.e.replay(g))
        else:
            self._stage("core", lambda: self._core_calls(rows))
        cont, n_exit, _, _ = self.e.read_counts()
        dt = self._t1(t0)
        self.t_core += dt
        if n_exit:
            self.qc_seqs += self.e.q_seq_view[self.qc:self.qc + n_exit].tolist()
        self.qr, self.qc = cont, self.qc + n_exit
        self.core_steps += 1
        self.core_token_steps += B
        self.log.append(StageLog("loop", B, f"{n_exit} exits", dt))

    def _core_calls(self, rows):
        self.e.core_step(rows)
        self.e.gate_compact(rows, gate_enabled=self.gate_on)

    def _do_coda(self):
        E = self.qc
        t0 = self._t0()
        self._stage("coda", lambda: self.e.boundary(pow2(E), exit_states=self._st_buf, logits=self._lg_buf))
        dt = self._t1(t0)
        self.t_coda += dt
        states = self._st_buf[:E].cpu().numpy() if self.capture else None
        lgs = self._lg_buf[:E].cpu().numpy() if self.capture_logits else None
        succ = 0
        for i, sid in enumerate(self.qc_seqs):
            r = self.reqs[sid]
            if states is not None:
                self.exit_states[(sid, r.n_gen)] = states[i]
            if lgs is not None:
                self.logits[(sid, r.n_gen)] = lgs[i]
            r.n_gen += 1
            if r.n_gen >= r.n_out:
                self._finish(r)
            else:
                succ += 1
        self.qc, self.qc_seqs = 0, []
        self.qr += succ
        self.log.append(StageLog("coda", E, "", dt))
        if succ:
            self.log.append(StageLog("prelude", succ, "after coda"))

    def _report(self):
        if self.progress is not None:
            now = time.perf_counter()
            if now - self._t_prog >= 20.0:
                self._t_prog = now
                self.progress(sum(r.finished for r in self.reqs), self.core_steps)

    def run(self):
        t_start = self._t_prog = time.perf_counter()
        while not all(r.finished for r in self.reqs):
            self._report()
            if self.mode == "refill":
                if self.qc and (self.qc >= self.K or (not self.qr and not self.can_prefill())):
                    self._do_coda()
                elif self.can_prefill():
                    self._do_prefill()
                elif self.qr:
                    self._do_core()
                else:
                    raise RuntimeError("scheduler stalled")
            else:
                while self.can_prefill():
                    self._do_prefill()
                if not self.qr and not self.qc:
                    if all(r.finished for r in self.reqs):
                        break
                    raise RuntimeError("scheduler stalled")
                while self.qr:
                    self._do_core()
                if self.qc:
                    self._do_coda()
        torch.cuda.synchronize()
        self.t_total = time.perf_counter() - t_start
        for g in self.graphs.values():
            self.e.drop(g)
        self.graphs = {}
        return self

    def results(self):
        toks = self.e.tokens_out[: len(self.reqs)].cpu().numpy()
        exits = self.e.exits_out[: len(self.reqs)].cpu().numpy()
        return [(toks[r.rid, : r.n_out].tolist(), exits[r.rid, 1: r.n_out].tolist()) for r in self.reqs]


class AsyncScheduler(Scheduler):
    """The same stage policy as Scheduler (refill Alg. 2, no-refill Alg. 1,
    fixed depth), run with the lookahead of §4.3 so that the host does not
    wait for the stage it has just launched.

    Each core step's gate reports the sequences that leave after the NEXT
    step (rows that fired, and rows that reach r_max).  A core step is
    launched knowing only the size of the core batch; its exits are the
    lookahead list of the core step before it, read back from the pinned
    buffer of that step (two buffers, used in turn) at the next decision,
    while the new step runs.  So the host's picture of both queues is exact
    at every decision and one stage is always queued on the GPU.  Rows enter
    the core at depth 1 with exit_at r_max, so with r_max >= 2 no row leaves
    at its first step.  Stage GPU times come from events (no
    synchronisation)."""

    def __init__(self, *args, arrivals: Optional[Sequence[float]] = None, **kw):
        kw.setdefault("graphs", True)
        super().__init__(*args, **kw)
        if self.e.d.r_max < 2:
            raise ValueError("the lookahead needs r_max >= 2")
        # online serving (§6.3): request i becomes admissible arrivals[i]
        # seconds after run() starts (non-decreasing); its finish time is the
        # GPU time of the stage that produced its last token
        self.arrivals = None if arrivals is None else [float(x) for x in arrivals]
        if self.arrivals is not None:
            if len(self.arrivals) != len(self.reqs) or any(b < a for a, b in zip(self.arrivals, self.arrivals[1:])):
                raise ValueError("arrivals: one non-decreasing time per request")
            self.pending = list(self.waiting)
            self.waiting = []
        self._fin_evs = []            # (request ids finished by the stage, event after it)
        self.finish_s: Dict[int, float] = {}
        if self.capture or self.capture_logits:
            raise ValueError("state/logit capture needs the synchronous Scheduler")
        self.qc_seqs = []
        self._rb = []                 # launched core steps not read back: (buf, event)
        self._next = []               # lookahead list of the core step before the last one
        self._unfolded = False        # the last core step's exits are not yet in qr / qc
        self._buf = 0
        self._evs = []                # (kind, start event, end event)
        self._phase = "prefill"       # Alg. 1 phases

    def _timed(self, kind, fn):
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(self.e.stream)
        fn()
        b.record(self.e.stream)
        self._evs.append((kind, a, b))

    def _fold(self):
        """Fold the exits of the last launched core step into the queues."""
        if not self._unfolded:
            return
        if len(self._rb) == 2:        # the step before the last one: its lookahead list
            buf, ev = self._rb.pop(0)
            ev.synchronize()
            n_next = int(self.e.h_counts[buf, 3])
            self._next = self.e.h_fired[buf, :n_next].tolist() if n_next else []
        exits, self._next = self._next, None
        self.qr -= len(exits)
        self.qc_seqs += exits
        self.qc = len(self.qc_seqs)
        self._unfolded = False
        self.log[-1].detail = f"{len(exits)} exits"

    def _core(self):
        B = self.qr
        rows = pow2(B)
        key = (rows, self._buf)
        g = self.graphs.get(key)
        if g is None:
            buf = self._buf
            g = self.graphs[key] = self.e.capture(
                lambda: (self.e.core_step(rows), self.e.gate_compact(rows, self.gate_on, buf)))
        self._timed("core", lambda: self.e.replay(g))
        ev = torch.cuda.Event()
        ev.record(self.e.stream)
        self._rb.append((self._buf, ev))
        self._buf ^= 1
        self._unfolded = True
        self.core_steps += 1
        self.core_token_steps += B
        self.log.append(StageLog("loop", B, ""))

    def _arrive(self):
        """Requests whose arrival time has passed join the waiting queue."""
        if self.arrivals is None:
            return
        now = time.perf_counter() - self._t_start
        while self.pending and self.arrivals[self.pending[0].rid] <= now:
            self.waiting.append(self.pending.pop(0))

    def _mark_finished(self, rids):
        if rids and self.arrivals is not None:
            ev = torch.cuda.Event(enable_timing=True)
            ev.record(self.e.stream)
            self._fin_evs.append((rids, ev))

    def _coda(self):
        E = len(self.qc_seqs)
        self._timed("coda", lambda: self.e.boundary(pow2(E)))
        succ = 0
        fin = []
        for sid in self.qc_seqs:
            r = self.reqs[sid]
            r.n_gen += 1
            if r.n_gen >= r.n_out:
                self._finish(r)
                fin.append(r.rid)
            else:
                succ += 1
        self._mark_finished(fin)
        self.qc_seqs = []
        self.qc = 0
        self.qr += succ
        self.log.append(StageLog("coda", E, ""))
        if succ:
            self.log.append(StageLog("prelude", succ, "after coda"))

    def _prefill(self):
        parts, ntok = self._pack()
        self._timed("prefill", lambda: self.e.prefill(
            [(r.rid, r.slot, s, r.prompt[s:e], e == len(r.prompt)) for (r, s, e) in parts]))
        done = 0
        fin = []
        for (r, s, e) in parts:
            r.prefilled = e
            if e == len(r.prompt):
                r.n_gen = 1
                if r.n_gen >= r.n_out:
                    self._finish(r)
                    fin.append(r.rid)
                else:
                    done += 1
        self._mark_finished(fin)
        self.qr += done
        self.log.append(StageLog("prefill", len(parts), f"{ntok} prompt tokens"))
        if done:
            self.log.append(StageLog("prelude", done, "after prefill"))

    def normalized_latency(self) -> Dict[int, float]:
        """Per request: (finish - arrival) / output tokens (online serving)."""
        return {rid: (t - self.arrivals[rid]) / self.reqs[rid].n_out for rid, t in self.finish_s.items()}

    def _decide(self):
        if self.mode == "refill":                     # Alg. 2 priority
            if self.qc and (self.qc >= self.K or (not self.qr and not self.can_prefill())):
                return "coda"
            if self.can_prefill():
                return "prefill"
            return "core" if self.qr else None
        # Alg. 1: prefill while possible, loop the cohort to the end, one coda
        for _ in range(3):
            if self._phase == "prefill":
                if self.can_prefill():
                    return "prefill"
                self._phase = "core"
            if self._phase == "core":
                if self.qr:
                    return "core"
                self._phase = "coda"
            if self._phase == "coda":
                self._phase = "prefill"
                if self.qc:
                    return "coda"
        return None

    def run(self):
        t_start = self._t_prog = self._t_start = time.perf_counter()
        ev0 = torch.cuda.Event(enable_timing=True)
        ev0.record(self.e.stream)
        while True:
            self._report()
            self._arrive()
            self._fold()
            st = self._decide()
            if st is None:
                if all(r.finished for r in self.reqs):
                    break
                if self.arrivals is not None and self.pending:
                    # idle until the next request arrives
                    wait = self.arrivals[self.pending[0].rid] - (time.perf_counter() - t_start)
                    if wait > 0:
                        time.sleep(wait)
                    continue
                raise RuntimeError("scheduler stalled")
            {"core": self._core, "coda": self._coda, "prefill": self._prefill}[st]()
        torch.cuda.synchronize()
        self.t_total = time.perf_counter() - t_start
        for rids, ev in self._fin_evs:
            t = ev0.elapsed_time(ev) / 1e3
            for rid in rids:
                self.finish_s[rid] = t
        tot = {"prefill": 0.0, "core": 0.0, "coda": 0.0}
        # per-stage GPU seconds with the stage's batch (the log lists the
        # timed stages in launch order, interleaved with untimed preludes)
        timed = [st for st in self.log if st.kind in ("loop", "coda", "prefill")]
        self.samples = []
        for (kind, a, b), st in zip(self._evs, timed):
            sec = a.elapsed_time(b) / 1e3
            tot[kind] += sec
            st.gpu_s = sec
            self.samples.append((kind, st.B, sec))
        self.t_prefill, self.t_core, self.t_coda = tot["prefill"], tot["core"], tot["coda"]
        for g in self.graphs.values():
            self.e.drop(g)
        self.graphs = {}
        return self
