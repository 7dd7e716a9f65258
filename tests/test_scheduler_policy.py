"""The product scheduler (continuous_depth_batching_amd.engine.Scheduler)
against the pages' printed stage traces, on the CPU.

"Depth-adaptive Inference of Looped Language Models via Continuous Depth
Batching", App. A.4, Tables 2-3: the first 20 stages of refill (K = 1 and
K = 16) and no-refill CDB on a ShareGPT-like mix at W = 64.  The same exit
script and prompt lengths that make the oracle's simulator reproduce those
tables (tests/test_oracle_sched.py) drive the product scheduler through a
test double of the device: a plain Python model of the library's queues
(core batch in row order, exit queue, successors appended at depth 1) with
the scripted lookahead exits.  The scheduler's stage sequence must be the
printed one: the kind and batch of every stage, and the queue sizes after
every loop and prelude stage (refill: Q_R, Q_C, Q_P; no-refill: Q_P).
"""
import os
import subprocess
import sys

import numpy as np
import pytest

from tests.conftest import read_tsv
from tests.test_oracle_sched import huginn_exit_script, huginn_prompt_lengths, ouro_exit_script, ouro_prompt_lengths

pytestmark = pytest.mark.cpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def eng_mod():
    if not os.path.exists(os.path.join(ROOT, "continuous_depth_batching_amd", "libcdb.so")):
        subprocess.check_call([sys.executable, "-m", "continuous_depth_batching_amd.build"], cwd=ROOT)
    from continuous_depth_batching_amd import engine
    return engine


class _Enough(Exception):
    pass


class _Log(list):
    """The scheduler's stage log; records the queue sizes after each stage
    and stops the run after n stages."""

    def __init__(self, sch, n):
        super().__init__()
        self.sch, self.n, self.queues = sch, n, []

    def append(self, st):
        super().append(st)
        s = self.sch
        self.queues.append((s.qr, s.qc, len(s.waiting)))
        if len(self) >= self.n:
            raise _Enough()


class FakeDevice:
    """Test double of the library's device queues: the core batch (rows in
    order), the exit queue, and the successor refill, with scripted exits
    (script[rid][pass] = exit depth, r_max by default) taken through the
    lookahead gate: a row whose scripted exit is e is marked after loop
    e - 1 and leaves after loop e."""

    def __init__(self, torch, r_max, script, n_req, W):
        self.R, self.script = r_max, script
        self.n_slots = self.max_rows = W
        self.max_seqs, self.mbps, self.max_T = n_req, 64, 8192
        self.num_blocks = n_req * 64
        self.btab = torch.zeros(n_req * 64, dtype=torch.int32)
        self.n_gen = torch.zeros(n_req, dtype=torch.int32)
        self.n_out = torch.zeros(n_req, dtype=torch.int32)
        self.desc_t = torch.zeros(1, dtype=torch.int32)
        self.q_t = torch.zeros(1, dtype=torch.int32)
        self.torch = torch
        self.rows, self.exitq, self.counts = [], [], [0, 0, 0, 0]
        self.q_seq_view = torch.zeros(0, dtype=torch.int32)

    def _row(self, seq, p):
        return {"seq": seq, "pass": p, "depth": 0, "exit_at": self.R}

    def prefill(self, parts, logits=None):
        for (rid, slot, start, toks, final) in parts:
            if final:
                self.n_gen[rid] = 1
                if int(self.n_out[rid]) > 1:
                    self.rows.append(self._row(rid, 0))

    def core_step(self, rows):
        assert len(self.rows) <= rows
        for r in self.rows:
            r["depth"] += 1

    def gate_compact(self, rows, gate_enabled=True, buf=0):
        cont, ex, fired, nxt = [], [], 0, []
        for r in self.rows:
            if r["depth"] == r["exit_at"]:
                ex.append(r)
                continue
            if gate_enabled and r["depth"] == self.script.get(r["seq"], {}).get(r["pass"], self.R) - 1:
                r["exit_at"] = r["depth"] + 1
                fired += 1
            cont.append(r)
            if r["exit_at"] == r["depth"] + 1:
                nxt.append(r["seq"])
        self.rows = cont
        self.exitq += ex
        self.counts = [len(cont), len(ex), fired, len(nxt)]
        self.q_seq_view = self.torch.tensor([r["seq"] for r in self.exitq], dtype=self.torch.int32)

    def boundary(self, rows, exit_states=None, logits=None, tokens_rows=None):
        for r in self.exitq:
            self.n_gen[r["seq"]] += 1
            if int(self.n_gen[r["seq"]]) < int(self.n_out[r["seq"]]):
                self.rows.append(self._row(r["seq"], r["pass"] + 1))
        self.exitq = []

    def read_counts(self, buf=0):
        return list(self.counts)


def _run(eng_mod, lengths, r_max, script, mode, K, n=20):
    import torch
    prompts = [np.zeros(L, dtype=np.int32) for L in lengths]
    dev = FakeDevice(torch, r_max, script, len(prompts), 64)
    sch = eng_mod.Scheduler(dev, prompts, 100, mode=mode, W=64, K=K, M=8192)
    sch.log = _Log(sch, n)
    with pytest.raises(_Enough):
        sch.run()
    return sch


def _check(sch, gold, refill):
    for i, (st, row) in enumerate(zip(sch.log, gold)):
        kind, B = row[1], int(row[2])
        if not refill and kind == "prelude":
            continue
        assert (st.kind, st.B) == (kind, B), (row[0], st.kind, st.B)
        q = sch.log.queues[i]
        if refill and kind in ("loop", "prelude"):
            assert q == tuple(int(x) for x in row[4:7]), (row[0], q, row[4:7])
        if not refill:
            assert q[2] == int(row[5]), (row[0], q, row)


def _gold(name, refill):
    rows = read_tsv(name)
    if refill:
        return rows
    return [r for r in rows if r[1] != "prelude"]


@pytest.mark.parametrize("name,lengths,r_max,script,K", [
    ("table2_ouro_refill_k1.tsv", ouro_prompt_lengths(), 4, ouro_exit_script(), 1),
    ("table2_huginn_refill_k1.tsv", huginn_prompt_lengths(), 16, huginn_exit_script(), 1),
    ("table3_ouro_refill_k16.tsv", ouro_prompt_lengths(), 4, ouro_exit_script(), 16),
])
def test_product_scheduler_reproduces_refill_traces(eng_mod, name, lengths, r_max, script, K):
    sch = _run(eng_mod, lengths, r_max, script, "refill", K)
    _check(sch, _gold(name, True), True)


def test_product_scheduler_reproduces_norefill_trace(eng_mod):
    gold = _gold("table3_ouro_norefill.tsv", False)
    sch = _run(eng_mod, ouro_prompt_lengths(), 4, ouro_exit_script(), "norefill", 1, n=40)
    stages = [st for st in sch.log if st.kind != "prelude"]
    queues = [q for st, q in zip(sch.log, sch.log.queues) if st.kind != "prelude"]
    for st, q, row in zip(stages, queues, gold):
        assert (st.kind, st.B) == (row[1], int(row[2])), (row[0], st.kind, st.B)
        assert q[2] == int(row[5]), (row[0], q)
