"""GPU parity of the lookahead gate + stream compaction and of the refill
that follows it, at batch sizes that span several wavefronts and several
256-row chunks (needs an MI355X).

"Depth-adaptive Inference of Looped Language Models via Continuous Depth
Batching": Alg. 2 (Gate: tokens that reached their exit go to the coda queue,
the rest stay in the recurrent queue; Coda and Prelude: each finished token's
successor re-enters the recurrent queue at depth 1), §4.3 (the lookahead gate
fired after step d makes the token leave after step d + 1, and the host is
told one step ahead which tokens leave next).

One decode step -- core step, gate + compaction, boundary (coda and the
successors' prelude) -- is captured as a HIP graph and replayed once, as the
benchmark runs it.  The expected queues come from a plain host partition in
row order of the same rows, with the gate decisions taken from the exit head
evaluated in fp64 on the GPU's own post-step states (every case asserts that
no gate value lies within 1e-3 of the threshold, so fp32 rounding cannot flip
a decision).  Everything is compared element by element, bit-exact: the
continue list (slot, seq, pos, depth + 1, exit_at), the exit queue in row
order (slot, seq, pos, depth), counts[0..3], the lookahead list fired_seq,
the successors appended behind the continue list (slot, seq, pos + 1,
depth 1, exit_at r_max), and their tokens against the oracle's LM head.
"""
import sys

import numpy as np
import pytest

import cdb_synth as S

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def eng_mod():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from continuous_depth_batching_amd import engine
    return engine


DIMS = S.ModelDims("t", vocab=512, hidden=256, n_heads=4, head_dim=64, ffn=1024, n_prelude=0, n_core=2,
                   n_coda=0, r_max=6, dtype="fp32", gate_bias=0.0)


def _setup(eng_mod, B, seed, L=40, n_out=None):
    d = DIMS
    R = d.r_max
    w = S.make_weights(d, seed=seed, std=0.05)
    dm = eng_mod.DeviceModel(d, w)
    mbps = (L + 32) // 16 + 1
    rows = eng_mod.pow2(B)
    e = eng_mod.Engine(dm, n_slots=B, max_rows=rows, num_blocks=B * mbps, max_seqs=B, max_blocks_per_seq=mbps,
                       max_out=8, max_prefill_tokens=16, kv_fill=0.0)
    gen = torch.Generator(device="cuda").manual_seed(seed)
    e.core_k.copy_(torch.randn(e.core_k.numel(), generator=gen, device="cuda"))
    e.core_v.copy_(torch.randn(e.core_v.numel(), generator=gen, device="cuda"))
    rng = np.random.default_rng(seed)
    e.btab.copy_(torch.from_numpy(rng.permutation(B * mbps).astype(np.int32)))
    emap = S.make_context_exit_depths(B * mbps * 16, R, seed=seed + 1)
    e.emap.copy_(torch.from_numpy(emap))
    e.state.copy_(torch.randn((B, d.hidden), generator=gen, device="cuda"))
    cap = e.max_rows
    # rows in a shuffled slot order; depth U{1..R}; exit_at >= depth, equal
    # to depth for about a third of the rows (they leave this step)
    slot = rng.permutation(B).astype(np.int32)
    seq = rng.permutation(B).astype(np.int32)
    pos = (L - rng.integers(0, 8, size=B)).astype(np.int32)
    depth = rng.integers(1, R + 1, size=B).astype(np.int32)
    leave = rng.random(B) < 0.35
    exit_at = np.where(leave, depth, rng.integers(depth, R + 1)).astype(np.int32)
    exit_at = np.where(depth == R, R, exit_at).astype(np.int32)
    desc = np.zeros(5 * cap + 1, dtype=np.int32)
    desc[0] = B
    for k, a in enumerate((slot, seq, pos, depth, exit_at)):
        desc[1 + k * cap:1 + k * cap + B] = a
    e.desc_t.copy_(torch.from_numpy(desc))
    e.q_t.zero_()
    # every sequence has produced one token; some have produced their last
    n_out_arr = np.full(B, 8, dtype=np.int32)
    if n_out is not None:
        n_out_arr = n_out(rng, B)
    e.n_gen.fill_(1)
    e.n_out[:B] = torch.from_numpy(n_out_arr).cuda()
    return d, w, e, dict(slot=slot, seq=seq, pos=pos, depth=depth, exit_at=exit_at, n_out=n_out_arr)


def _host_partition(d, w, rows, state1, q_n0=0):
    """Plain partition of the valid rows in row order (Alg. 2 Gate with the
    lookahead of §4.3), given the post-step states."""
    R = d.r_max
    B = len(rows["slot"])
    g = np.asarray(w["gate_w"], np.float64)
    cont, ex, fired, nxt = [], [], 0, []
    zmin = np.inf
    for b in range(B):
        dep, ea = int(rows["depth"][b]), int(rows["exit_at"][b])
        if dep == ea:
            ex.append(b)
            continue
        h = state1[rows["slot"][b]].astype(np.float64)
        z = float(np.dot(h / np.sqrt(np.mean(h * h) + d.rms_eps), g)) + float(np.float32(d.gate_bias))
        zmin = min(zmin, abs(z))
        fire = z > d.gate_threshold
        fired += int(fire)
        new_ea = dep + 1 if fire else ea
        cont.append((b, new_ea))
        if new_ea == dep + 1:
            nxt.append(int(rows["seq"][b]))
    return cont, ex, fired, nxt, zmin


def _check_step(eng_mod, B, seed, n_out=None):
    d, w, e, rows = _setup(eng_mod, B, seed, n_out=n_out)
    R = d.r_max
    cap = e.max_rows
    rp = eng_mod.pow2(B)
    _say(f"[case] gate + compaction + refill, captured step: B={B} rows_pad={rp} seed={seed}")
    state0 = e.state.clone()
    e.core_step(rp)                              # the post-step states the gate will see
    torch.cuda.synchronize()
    state1 = e.state.cpu().numpy().astype(np.float64)
    e.state.copy_(state0)
    cont, ex, fired, nxt, zmin = _host_partition(d, w, rows, state1)
    _say(f"  host: {len(cont)} continue, {len(ex)} leave, {fired} fired, {len(nxt)} leave next; min |z| {zmin:.2e}")
    assert zmin > 1e-3, "a gate value within 1e-3 of the threshold: choose another seed"
    waves = {b // 64 for b in ex}
    assert waves == set(range((B + 63) // 64)), f"exits must fall in every wave, got waves {sorted(waves)}"
    g = e.capture(lambda: (e.core_step(rp), e.gate_compact(rp, True), e.boundary(rp)))
    e.replay(g)
    torch.cuda.synchronize()
    e.drop(g)
    np.testing.assert_array_equal(e.state.cpu().numpy()[[rows["slot"][b] for b, _ in cont]],
                                  state1[[rows["slot"][b] for b, _ in cont]].astype(np.float32))
    counts = e.counts.cpu().numpy().tolist()
    assert counts == [len(cont), len(ex), fired, len(nxt)], (counts, [len(cont), len(ex), fired, len(nxt)])
    assert e.fired.cpu().numpy()[:len(nxt)].tolist() == nxt
    desc = e.desc_t.cpu().numpy()
    get = lambda k, n0, n1: desc[1 + k * cap + n0:1 + k * cap + n1]
    nc = len(cont)
    want = np.array([[rows["slot"][b], rows["seq"][b], rows["pos"][b], rows["depth"][b] + 1, ea] for b, ea in cont],
                    dtype=np.int32).reshape(-1, 5)
    got = np.stack([get(k, 0, nc) for k in range(5)], axis=1)
    np.testing.assert_array_equal(got, want)
    # the exit queue (row order); the boundary consumed it (n = 0), its arrays stay
    q = e.q_t.cpu().numpy()
    assert int(q[0]) == 0
    qg = np.stack([q[1 + k * cap:1 + k * cap + len(ex)] for k in range(4)], axis=1)
    qw = np.array([[rows["slot"][b], rows["seq"][b], rows["pos"][b], rows["depth"][b]] for b in ex],
                  dtype=np.int32).reshape(-1, 4)
    np.testing.assert_array_equal(qg, qw)
    # successors: the exits whose sequence still generates, in exit-queue order
    succ = [b for b in ex if rows["n_out"][rows["seq"][b]] > 2]
    n_succ = len(succ)
    assert int(desc[0]) == nc + n_succ
    sg = np.stack([get(k, nc, nc + n_succ) for k in range(5)], axis=1)
    sw = np.array([[rows["slot"][b], rows["seq"][b], rows["pos"][b] + 1, 1, R] for b in succ],
                  dtype=np.int32).reshape(-1, 5)
    np.testing.assert_array_equal(sg, sw)
    # tokens of the leaving rows (greedy argmax of the LM head on their state)
    from oracle.model import OracleLM
    m = OracleLM(d, w, dtype=np.float64)
    toks = e.tokens_out.cpu().numpy()
    exits_out = e.exits_out.cpu().numpy()
    n_gen = e.n_gen.cpu().numpy()
    low = 0
    for b in ex:
        sq = rows["seq"][b]
        lg = m.lm_head(state1[rows["slot"][b]][None])[0]
        top = int(np.argmax(lg))
        srt = np.sort(lg)
        assert n_gen[sq] == 2
        assert exits_out[sq, 1] == rows["depth"][b]
        if toks[sq, 1] != top:
            assert srt[-1] - srt[-2] < 1e-5, f"row {b}: token {toks[sq, 1]} vs oracle {top}"
            low += 1
        # the freed slot of a successor holds the embedding of the new token
        if b in succ:
            np.testing.assert_array_equal(e.state.cpu().numpy()[rows["slot"][b]],
                                          w["embed"][toks[sq, 1]].astype(np.float32))
    _say(f"  device queues, counts, lookahead list and successors match; tokens of {len(ex)} exits "
         f"({low} within 1e-5 of a tie)")
    e.close()


@pytest.mark.parametrize("B,seed", [(200, 21), (256, 22), (512, 23), (300, 24)])
def test_gate_compaction_refill_multi_wave(eng_mod, B, seed):
    """200 rows (four waves, the last partial), 256 (four full waves), 512
    (two 256-row chunks) and 300 (a partial second chunk)."""
    _check_step(eng_mod, B, seed)


def test_gate_compaction_some_sequences_finish(eng_mod):
    """Sequences that have produced their last token get no successor: the
    refill appends only the others, still in exit-queue order."""
    _check_step(eng_mod, 256, 25, n_out=lambda rng, B: rng.choice([2, 8], size=B).astype(np.int32))


def test_gate_compaction_appends_to_a_waiting_exit_queue(eng_mod):
    """With K > 1 exits wait in the coda queue across core steps: a gate
    step appends its exits behind the ones already queued (Alg. 2: the coda
    waits for K exits).  Two gate steps without a boundary in between."""
    B = 256
    d, w, e, rows = _setup(eng_mod, B, 26)
    cap = e.max_rows
    _say(f"[case] gate + compaction twice into one exit queue: B={B}")
    state = e.state.cpu().numpy().astype(np.float64)
    cont, ex, fired, nxt, zmin = _host_partition(d, w, rows, state)
    assert zmin > 1e-3
    e.gate_compact(B, True)
    torch.cuda.synchronize()
    n1 = len(ex)
    assert int(e.q_t[0].item()) == n1
    # second step: the compacted batch, depth + 1, no core step in between
    desc = e.desc_t.cpu().numpy()
    nc = int(desc[0])
    rows2 = {k: desc[1 + i * cap:1 + i * cap + nc].copy() for i, k in enumerate(("slot", "seq", "pos", "depth",
                                                                                    "exit_at"))}
    cont2, ex2, fired2, nxt2, zmin2 = _host_partition(d, w, rows2, state)
    assert zmin2 > 1e-3
    e.gate_compact(eng_mod.pow2(nc), True)
    torch.cuda.synchronize()
    q = e.q_t.cpu().numpy()
    assert int(q[0]) == n1 + len(ex2)
    qs = q[1 + cap:1 + cap + n1 + len(ex2)].tolist()
    assert qs == [int(rows["seq"][b]) for b in ex] + [int(rows2["seq"][b]) for b in ex2]
    assert e.counts.cpu().numpy().tolist() == [len(cont2), len(ex2), fired2, len(nxt2)]
    _say(f"  exit queue {n1} + {len(ex2)} in order")
    e.close()
