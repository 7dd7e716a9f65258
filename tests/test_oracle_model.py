"""Pins of the oracle's looped LM (CPU only).

* Gate off, the looped model equals an independently written unrolled
  transformer (fp64) — the §2 layer count p + c*r + q with tied core weights
  and one KV per unrolled layer.
* §4.2 / Fig. 2 (right): the cells each cache design holds for tokens that
  exit at (2, 1, 3).
* The shared single-slot cache reads the latest state of every position;
  first-then-shared (App. E.1) reads the first-loop state in loop 1 and the
  latest state in later loops, and equals the depth-indexed cache at r_max 2.
* §4.3 / §7: lookahead exit depth = min(r_max, 1 + first firing step),
  never below 2, by enumeration of every firing pattern.
"""
import itertools

import numpy as np
import pytest

import cdb_synth as S
from oracle.model import OracleLM, SeqCache, cache_from_planes
from oracle.unrolled import unrolled_forward, unrolled_forward_exits
from tests.conftest import read_tsv

pytestmark = pytest.mark.cpu


def tiny(**kw):
    base = dict(name="t", vocab=97, hidden=32, n_heads=2, head_dim=16, ffn=48,
                n_prelude=0, n_core=2, n_coda=0, r_max=3, dtype="fp32")
    base.update(kw)
    return S.ModelDims(**base)


def _check_unrolled(d, prompt_len=5, n_out=4, seed=0):
    w = S.make_weights(d, seed=seed, norm="random", std=0.2)
    m = OracleLM(d, w, dtype=np.float64, keep_logits=True)
    prompt = S.make_prompts(d.vocab, [prompt_len], seed=seed)[0]
    toks, exits, recs = m.decode_sequential(prompt, n_out, policy="fixed", keep_state=True)
    assert exits == [d.r_max] * (n_out - 1)
    seq = np.concatenate([prompt, np.array(toks[:-1], dtype=np.int32)])
    core_out, logits = unrolled_forward(d, w, seq, loops=d.r_max)
    # prefill logits of the last prompt position
    np.testing.assert_allclose(recs[0].logits, logits[prompt_len - 1], rtol=1e-10, atol=1e-11)
    for i in range(1, n_out):
        p = prompt_len + i - 1
        np.testing.assert_allclose(recs[i].exit_state, core_out[p], rtol=1e-10, atol=1e-11)
        np.testing.assert_allclose(recs[i].logits, logits[p], rtol=1e-10, atol=1e-11)
        assert recs[i].token == int(np.argmax(logits[p]))


def test_fixed_depth_equals_unrolled_transformer():
    _check_unrolled(tiny())


def test_one_loop_is_plain_transformer():
    _check_unrolled(tiny(r_max=1, n_core=3), prompt_len=4, n_out=3)


def test_prelude_coda_and_injection_equal_unrolled():
    _check_unrolled(tiny(n_prelude=1, n_coda=1, inject=True, r_max=4), prompt_len=4, n_out=4)


def test_chunked_prefill_depth_indexed_is_chunk_independent():
    d = tiny(r_max=2)
    w = S.make_weights(d, seed=3, norm="random", std=0.2)
    m = OracleLM(d, w, dtype=np.float64)
    prompt = S.make_prompts(d.vocab, [9], seed=3)[0]
    a = m.decode_sequential(prompt, 4)[0:2]
    b = m.decode_sequential(prompt, 4, chunks=[(0, 2), (2, 7), (7, 9)])[0:2]
    assert a == b


def _labelled_planes(R, exits, nh=1, hd=1):
    """K planes whose value is the loop step that wrote them; deeper slots
    than a token's exit stay empty (NaN)."""
    n = len(exits)
    K = np.full((1, R, n, nh, hd), np.nan)
    for j, e in enumerate(exits):
        for s in range(e):
            K[0, s, j] = s + 1
    return K


def test_fig2_last_exited_and_shared_cells():
    gold = read_tsv("fig2_kv_designs.tsv")
    exits = [2, 1, 3]
    d = tiny(r_max=3, n_core=1, n_heads=1, head_dim=1, hidden=1)
    K = _labelled_planes(3, exits)
    c = cache_from_planes(d, K, K.copy(), np.array(exits))
    for layout, slot, *cells in gold:
        if layout == "last_exited":
            got = [int(c.core_k[0, int(slot) - 1, j, 0, 0]) for j in range(3)]
            assert got == [int(x) for x in cells]
    # shared: the fixture's single row says the slot ends at each token's
    # last step; the single-slot oracle must leave exactly the KV of the exit
    # step in its one plane (checked below on a real model)
    shared = [r for r in gold if r[0] == "shared"][0]
    assert [int(x) for x in shared[2:]] == exits


def test_single_slot_holds_exit_step_kv():
    import copy
    ds = tiny(r_max=4, kv_layout="single")
    w = S.make_weights(ds, seed=2, norm="random", std=0.2)
    prompt = S.make_prompts(ds.vocab, [4], seed=2)[0]
    m = OracleLM(ds, w, dtype=np.float64)
    base = SeqCache(ds, 6, np.float64)
    m.prefill(prompt, base)
    for e in range(1, 5):
        c = copy.deepcopy(base)
        m.decode_step(7, 4, c, forced_exit=e)
        # manual loop: steps 1..e, reading the slot after step e
        c2 = copy.deepcopy(base)
        h, _ = m._prelude([7], np.array([4]), c2)
        for depth in range(1, e + 1):
            h = m.core(h, np.array([4]), depth, c2)
        np.testing.assert_array_equal(c.core_k[:, 0, 4], c2.core_k[:, 0, 4])
        if e > 1:     # and it differs from what step e-1 left there
            c3 = copy.deepcopy(base)
            h, _ = m._prelude([7], np.array([4]), c3)
            for depth in range(1, e):
                h = m.core(h, np.array([4]), depth, c3)
            assert np.abs(c3.core_k[:, 0, 4] - c.core_k[:, 0, 4]).max() > 1e-9


def test_last_exited_equals_min_rule_on_random_maps():
    rng = np.random.default_rng(7)
    R, n = 6, 40
    d = tiny(r_max=R, n_core=2)
    exits = rng.integers(1, R + 1, size=n)
    K = rng.standard_normal((2, R, n, 2, 16))
    V = rng.standard_normal((2, R, n, 2, 16))
    for j, e in enumerate(exits):          # poison the gaps
        K[:, e:, j] = np.nan
        V[:, e:, j] = np.nan
    c = cache_from_planes(d, K, V, exits, dtype=np.float64)
    for depth in range(1, R + 1):
        for j, e in enumerate(exits):
            src = min(depth, int(e)) - 1
            np.testing.assert_array_equal(c.core_k[:, depth - 1, j], K[:, src, j])
            np.testing.assert_array_equal(c.core_v[:, depth - 1, j], V[:, src, j])


def test_single_slot_reads_latest_state():
    """Single slot, gate off: a decode token at loop d sees every prompt
    position at its final (r_max) state.  Equivalent construction: the
    depth-indexed cache with each prompt position's final plane copied into
    all planes."""
    dd = tiny(r_max=3)
    ds = dd.with_(kv_layout="single")
    w = S.make_weights(dd, seed=5, norm="random", std=0.2)
    prompt = S.make_prompts(dd.vocab, [6], seed=5)[0]
    ms, md = OracleLM(ds, w, dtype=np.float64), OracleLM(dd, w, dtype=np.float64)
    cs, cd = SeqCache(ds, 8, np.float64), SeqCache(dd, 8, np.float64)
    ts, _, _ = ms.prefill(prompt, cs)
    td, _, _ = md.prefill(prompt, cd)
    # one-chunk prefill: at loop d every prompt position reads the others at
    # loop d in both layouts, so the results agree and the single slot ends
    # holding the final plane
    assert ts == td
    np.testing.assert_array_equal(cs.core_k[:, 0, :6], cd.core_k[:, 2, :6])
    np.testing.assert_array_equal(cs.core_v[:, 0, :6], cd.core_v[:, 2, :6])
    # single-slot decode reads the prompt at its final state at every loop:
    # make the depth-indexed cache hold the final plane in every plane
    cd.core_k[:, :, :6] = cd.core_k[:, 2:3, :6]
    cd.core_v[:, :, :6] = cd.core_v[:, 2:3, :6]
    rs = ms.decode_step(11, 6, cs, policy="fixed", keep_state=True)
    rd = md.decode_step(11, 6, cd, policy="fixed", keep_state=True)
    np.testing.assert_allclose(rs.exit_state, rd.exit_state, rtol=1e-12)
    assert rs.token == rd.token


def test_single_slot_chunked_prefill_sees_earlier_chunks_at_final_state():
    """With one slot, a prompt prefilled in two chunks differs from one chunk
    (the second chunk sees the first at its final state at every loop), and
    equals the depth-indexed computation where the first chunk's planes all
    hold the final plane."""
    dd = tiny(r_max=3)
    ds = dd.with_(kv_layout="single")
    w = S.make_weights(dd, seed=6, norm="random", std=0.3)
    prompt = S.make_prompts(dd.vocab, [8], seed=6)[0]
    ms, md = OracleLM(ds, w, dtype=np.float64), OracleLM(dd, w, dtype=np.float64)
    cs = SeqCache(ds, 8, np.float64)
    _, lg_s, _ = ms.prefill(prompt, cs, chunks=[(0, 3), (3, 8)])
    cd = SeqCache(dd, 8, np.float64)
    md.prefill(prompt[:3], cd)
    cd.core_k[:, :, :3] = cd.core_k[:, 2:3, :3]
    cd.core_v[:, :, :3] = cd.core_v[:, 2:3, :3]
    pos = np.arange(3, 8)
    h, _ = md._prelude(prompt[3:8], pos, cd)
    for depth in range(1, 4):
        h = md.core(h, pos, depth, cd)
    lg_d = md.lm_head(h[-1:])[0]
    np.testing.assert_allclose(lg_s, lg_d, rtol=1e-12)
    cs1 = SeqCache(ds, 8, np.float64)
    _, lg_1, _ = ms.prefill(prompt, cs1)
    assert np.abs(lg_1 - lg_s).max() > 1e-6


def test_first_shared_with_two_loops_is_depth_indexed():
    """With r_max = 2 the first-then-shared cache has one slot per loop (the
    shared slot only ever holds loop 2), so it must equal the depth-indexed
    cache bit for bit: prefill, adaptive decode, exits and states."""
    dd = tiny(r_max=2, gate_bias=0.05)
    df = dd.with_(kv_layout="first_shared")
    w = S.make_weights(dd, seed=8, norm="random", std=0.2)
    prompt = S.make_prompts(dd.vocab, [7], seed=8)[0]
    md, mf = OracleLM(dd, w, dtype=np.float64), OracleLM(df, w, dtype=np.float64)
    td, ed, rd = md.decode_sequential(prompt, 6, keep_state=True)
    tf, ef, rf = mf.decode_sequential(prompt, 6, keep_state=True)
    assert (td, ed) == (tf, ef)
    for a, b in zip(rd[1:], rf[1:]):
        np.testing.assert_array_equal(a.exit_state, b.exit_state)


def test_first_shared_reads_first_loop_then_latest_state():
    """First-then-shared, gate off, r_max 3.  One-chunk prefill reads the
    loop's own states in every layout, so it agrees with the depth-indexed
    cache and leaves the first loop in the private slot and the last loop in
    the shared one.  A decode token then sees the prompt at its first-loop
    state in loop 1 and at its final state in loops 2 and 3: equivalently,
    the depth-indexed cache with planes 2 and 3 of the prompt replaced by
    the final plane."""
    dd = tiny(r_max=3)
    df = dd.with_(kv_layout="first_shared")
    w = S.make_weights(dd, seed=9, norm="random", std=0.2)
    prompt = S.make_prompts(dd.vocab, [6], seed=9)[0]
    mf, md = OracleLM(df, w, dtype=np.float64), OracleLM(dd, w, dtype=np.float64)
    cf, cd = SeqCache(df, 8, np.float64), SeqCache(dd, 8, np.float64)
    tf, _, _ = mf.prefill(prompt, cf)
    td, _, _ = md.prefill(prompt, cd)
    assert tf == td
    assert cf.core_k.shape[1] == 2
    np.testing.assert_array_equal(cf.core_k[:, 0, :6], cd.core_k[:, 0, :6])
    np.testing.assert_array_equal(cf.core_k[:, 1, :6], cd.core_k[:, 2, :6])
    np.testing.assert_array_equal(cf.core_v[:, 1, :6], cd.core_v[:, 2, :6])
    cd.core_k[:, 1:, :6] = cd.core_k[:, 2:3, :6]
    cd.core_v[:, 1:, :6] = cd.core_v[:, 2:3, :6]
    rf = mf.decode_step(11, 6, cf, policy="fixed", keep_state=True)
    rd = md.decode_step(11, 6, cd, policy="fixed", keep_state=True)
    np.testing.assert_allclose(rf.exit_state, rd.exit_state, rtol=1e-12)
    assert rf.token == rd.token
    # and it is neither the depth-indexed nor the single-slot computation
    cd2 = SeqCache(dd, 8, np.float64)
    md.prefill(prompt, cd2)
    r_plain = md.decode_step(11, 6, cd2, policy="fixed", keep_state=True)
    ds = dd.with_(kv_layout="single")
    ms = OracleLM(ds, w, dtype=np.float64)
    cs = SeqCache(ds, 8, np.float64)
    ms.prefill(prompt, cs)
    r_single = ms.decode_step(11, 6, cs, policy="fixed", keep_state=True)
    assert np.abs(rf.exit_state - r_plain.exit_state).max() > 1e-9
    assert np.abs(rf.exit_state - r_single.exit_state).max() > 1e-9


def test_first_shared_slots_hold_first_and_exit_step_kv():
    """After a decode token leaves at depth e, the private slot holds the KV
    of its first loop and the shared slot the KV of loop e (e >= 2)."""
    import copy
    df = tiny(r_max=4, kv_layout="first_shared")
    w = S.make_weights(df, seed=4, norm="random", std=0.2)
    prompt = S.make_prompts(df.vocab, [4], seed=4)[0]
    m = OracleLM(df, w, dtype=np.float64)
    base = SeqCache(df, 6, np.float64)
    m.prefill(prompt, base)
    for e in range(2, 5):
        c = copy.deepcopy(base)
        m.decode_step(7, 4, c, forced_exit=e)
        dd = df.with_(kv_layout="depth")
        md = OracleLM(dd, w, dtype=np.float64)
        # reference: the same token through the depth-indexed cache whose
        # prompt planes 2..4 hold the final plane (what the shared slot shows)
        cd = SeqCache(dd, 6, np.float64)
        md.prefill(prompt, cd)
        cd.core_k[:, 1:, :4] = cd.core_k[:, 3:4, :4]
        cd.core_v[:, 1:, :4] = cd.core_v[:, 3:4, :4]
        md.decode_step(7, 4, cd, forced_exit=e)
        np.testing.assert_allclose(c.core_k[:, 0, 4], cd.core_k[:, 0, 4], rtol=1e-12)
        np.testing.assert_allclose(c.core_k[:, 1, 4], cd.core_k[:, e - 1, 4], rtol=1e-12)
        np.testing.assert_allclose(c.core_v[:, 1, 4], cd.core_v[:, e - 1, 4], rtol=1e-12)


def _identity_core_weights(d, seed):
    """Weights whose core layers contribute nothing (every core projection
    zero), so each core layer, and the core, is the identity map."""
    w = S.make_weights(d, seed=seed, norm="random", std=0.2)
    for k in w:
        if k.startswith("core.") and not k.endswith("norm"):
            w[k] = np.zeros_like(w[k])
    return w


@pytest.mark.parametrize("tau,expect", [(0.6, 3), (0.5, 4), (0.3, 5), (0.26, 5), (0.24, 6), (0.1, 8)])
def test_convergence_gate_closed_form_injection(tau, expect):
    """Identity core with the prelude output e added at every loop: h_d =
    d e, so the normalized step |h_d - h_{d-1}| / |h_d| is exactly 1 / d.
    The gate first fires at the smallest d >= 2 with 1/d < tau (strict) and
    the token leaves one step later (lookahead), at r_max at the latest:
    tau 0.6 -> 3 (the earliest exit), 0.5 -> 4 (1/2 is not below 0.5),
    0.3 -> 5, 0.26 -> 5, 0.24 -> 6, 0.1 -> r_max = 8.  Normalizing by the
    older state instead (1/(d-1)) or firing in the same step would move
    every one of these."""
    d = tiny(r_max=8, inject=True, gate_kind="convergence", conv_threshold=tau)
    w = _identity_core_weights(d, seed=3)
    m = OracleLM(d, w, dtype=np.float64)
    prompt = S.make_prompts(d.vocab, [5], seed=3)[0]
    toks, exits, recs = m.decode_sequential(prompt, 4, keep_state=True)
    assert exits == [expect] * 3
    for r in recs[1:]:
        ks = np.arange(2, len(r.gate_logits) + 2)
        np.testing.assert_allclose(r.gate_logits, 1.0 / ks, rtol=1e-12)


def test_convergence_gate_identity_core_without_injection():
    """Identity core, no injection: consecutive states are equal, the step
    size is 0, so any tau > 0 fires at loop 2 (exit 3) and tau = 0 never
    fires (strict), leaving at r_max."""
    for tau, expect in ((0.01, 3), (0.0, 6)):
        d = tiny(r_max=6, gate_kind="convergence", conv_threshold=tau)
        w = _identity_core_weights(d, seed=4)
        m = OracleLM(d, w, dtype=np.float64)
        prompt = S.make_prompts(d.vocab, [4], seed=4)[0]
        _, exits, _ = m.decode_sequential(prompt, 3)
        assert exits == [expect] * 2


class _ScriptedConvergence(OracleLM):
    """Oracle whose convergence values follow a script from loop 2 on."""
    def __init__(self, *a, cs=None, **k):
        super().__init__(*a, **k)
        self.cs = list(cs)

    def gate_eval(self, h_row, h_prev_row, depth):
        if depth < 2:
            return None
        c = self.cs.pop(0)
        tau = float(self.d.conv_threshold)
        return c, c < tau, abs(c - tau)


def test_convergence_exit_rule_by_enumeration():
    """Every firing pattern of loops 2..r_max-1: e = min(r_max, 1 + first
    firing loop), so e >= 3 always."""
    R = 6
    d = tiny(r_max=R, hidden=8, n_heads=1, head_dim=8, ffn=8, n_core=1, vocab=11, gate_kind="convergence",
             conv_threshold=0.5)
    w = S.make_weights(d, seed=1)
    prompt = S.make_prompts(d.vocab, [3], seed=1)[0]
    seen = set()
    for pattern in itertools.product([0, 1], repeat=R - 2):
        cs = [0.1 if f else 0.9 for f in pattern] + [0.9] * 4
        m = _ScriptedConvergence(d, w, dtype=np.float64, cs=cs)
        cache = SeqCache(d, 5, np.float64)
        m.prefill(prompt, cache)
        rec = m.decode_step(5, 3, cache)
        fires = [i + 2 for i, f in enumerate(pattern) if f]
        want = min(R, fires[0] + 1) if fires else R
        assert rec.exit_depth == want
        assert rec.exit_depth >= 3
        seen.add(rec.exit_depth)
    assert seen == set(range(3, R + 1))


class _ScriptedGate(OracleLM):
    """Oracle whose gate logits follow a script (the loop itself is real)."""
    def __init__(self, *a, zs=None, **k):
        super().__init__(*a, **k)
        self.zs = list(zs)

    def gate_logit(self, h_row):
        return self.zs.pop(0)


def test_lookahead_exit_rule_by_enumeration():
    R = 5
    d = tiny(r_max=R, hidden=8, n_heads=1, head_dim=8, ffn=8, n_core=1, vocab=11)
    w = S.make_weights(d, seed=0)
    for pattern in itertools.product([False, True], repeat=R - 1):
        zs = [1.0 if f else -1.0 for f in pattern]
        m = _ScriptedGate(d, w, dtype=np.float64, zs=zs)
        c = SeqCache(d, 4, np.float64)
        m.prefill([1, 2], c)
        rec = m.decode_step(3, 2, c)
        fired = [i + 1 for i, f in enumerate(pattern) if f]
        want = min(R, fired[0] + 1) if fired else R
        assert rec.exit_depth == want
        assert 2 <= rec.exit_depth <= R
        # the gate is evaluated after every step except the one the token leaves at
        assert len(rec.gate_logits) == rec.exit_depth - 1
        # the exit depth recorded for the position
        assert c.exit_depth[2] == want


def test_gate_threshold_is_strict():
    d = tiny(r_max=3, hidden=8, n_heads=1, head_dim=8, ffn=8, n_core=1, vocab=11)
    w = S.make_weights(d, seed=0)
    m = _ScriptedGate(d, w, dtype=np.float64, zs=[0.0, 0.0])
    c = SeqCache(d, 4, np.float64)
    m.prefill([1, 2], c)
    assert m.decode_step(3, 2, c).exit_depth == 3


def test_forced_replay_records_own_decisions():
    R = 4
    d = tiny(r_max=R, hidden=8, n_heads=1, head_dim=8, ffn=8, n_core=1, vocab=11)
    w = S.make_weights(d, seed=0)
    # own gate fires after step 1 (own exit 2); replay forces exit 3
    m = _ScriptedGate(d, w, dtype=np.float64, zs=[1.0, -1.0])
    c = SeqCache(d, 4, np.float64)
    m.prefill([1, 2], c)
    rec = m.decode_step(3, 2, c, forced_exit=3)
    assert rec.exit_depth == 3 and rec.own_exit == 2
    # own gate never fires; forced exit 2 -> own decision unknown beyond 2 (None)
    m = _ScriptedGate(d, w, dtype=np.float64, zs=[-1.0])
    c = SeqCache(d, 4, np.float64)
    m.prefill([1, 2], c)
    rec = m.decode_step(3, 2, c, forced_exit=2)
    assert rec.exit_depth == 2 and rec.own_exit is None


def test_decode_token_nan_gaps_never_read():
    """Depth-indexed decode on a cache whose unused planes are NaN gives finite
    results (the last-exited fill covers every gap that is read)."""
    d = tiny(r_max=4)
    w = S.make_weights(d, seed=9, std=0.2)
    d = d.with_(gate_bias=0.0)
    m = OracleLM(d, w, dtype=np.float64)
    prompt = S.make_prompts(d.vocab, [5], seed=9)[0]
    toks, exits, recs = m.decode_sequential(prompt, 10, keep_state=True)
    assert all(np.isfinite(r.exit_state).all() for r in recs[1:])
    assert all(2 <= e <= 4 for e in exits)


# ------------------------------------------------------------------ gate value
class _GateGain(OracleLM):
    """Planted mistake: the exit head's norm applies the final norm's gain."""
    def gate_logit(self, h_row):
        from oracle.layers import rmsnorm
        hn = rmsnorm(h_row, self.w["final_norm"], self.d.rms_eps)
        return float(np.dot(hn, self.w["gate_w"])) + float(np.float32(self.d.gate_bias))


class _GateNoEps(OracleLM):
    """Planted mistake: epsilon dropped from the norm."""
    def gate_logit(self, h_row):
        hn = h_row / np.sqrt(np.mean(h_row * h_row))
        return float(np.dot(hn, self.w["gate_w"])) + float(np.float32(self.d.gate_bias))


class _GateEpsOutside(OracleLM):
    """Planted mistake: epsilon added outside the square root."""
    def gate_logit(self, h_row):
        hn = h_row / (np.sqrt(np.mean(h_row * h_row)) + self.d.rms_eps)
        return float(np.dot(hn, self.w["gate_w"])) + float(np.float32(self.d.gate_bias))


class _GateBiasTwice(OracleLM):
    """Planted mistake: the bias added twice."""
    def gate_logit(self, h_row):
        return OracleLM.gate_logit(self, h_row) + float(np.float32(self.d.gate_bias))


def _gate_case(cls=OracleLM):
    """Hidden size 8, h = 2 * (+1, -1, ...): mean(h^2) = 4 exactly.  With
    eps = 5 under the root the norm divides by sqrt(4 + 5) = 3, so with
    w = (1, 0, ..., 0, 0.5) and b = 0.25 the exit head gives
    z = (2 - 0.5 * 2) / 3 + 0.25 = 1/3 + 1/4 = 7/12, by hand.  The norm gains
    of the model are random (not 1), and the exit head must not use them."""
    d = tiny(hidden=8, n_heads=1, head_dim=8, ffn=8, vocab=11, rms_eps=5.0, gate_bias=0.25)
    w = S.make_weights(d, seed=3, norm="random")
    w["gate_w"] = np.array([1, 0, 0, 0, 0, 0, 0, 0.5], dtype=np.float32)
    h = 2.0 * np.array([1, -1, 1, -1, 1, -1, 1, -1], dtype=np.float64)
    return cls(d, w, dtype=np.float64), h


def test_gate_logit_hand_value():
    """Exit head z = w . RMSNorm(h) + b (§3: a small exit head on the core
    output; §7 gating): the hand value 7/12 of _gate_case."""
    m, h = _gate_case()
    assert abs(m.gate_logit(h) - 7.0 / 12.0) < 1e-15
    # a second hand value: h = 3 e_1 (mean(h^2) = 9/8), eps 5 -> sqrt(49/8)
    h2 = np.zeros(8)
    h2[0] = 3.0
    assert abs(m.gate_logit(h2) - (3.0 / np.sqrt(49.0 / 8.0) + 0.25)) < 1e-15


def test_gate_logit_ignores_every_norm_gain():
    m, h = _gate_case()
    z = m.gate_logit(h)
    for k in list(m.w):
        if k.endswith("norm"):
            m.w[k] = m.w[k] * 3.0 + 1.0
    assert m.gate_logit(h) == z


@pytest.mark.parametrize("cls", [_GateGain, _GateNoEps, _GateEpsOutside, _GateBiasTwice])
def test_gate_logit_pin_catches_planted_mistakes(cls):
    m, h = _gate_case(cls)
    assert abs(m.gate_logit(h) - 7.0 / 12.0) > 1e-3


def test_gate_logit_decides_the_exit():
    """The value drives the decision: with the hand case's model, a token
    whose gate value is 7/12 > 0 after loop 1 leaves after loop 2, and with
    a bias of -1 (z = 1/3 - 1 < 0 for the same state) it does not fire."""
    m, h = _gate_case()
    z, fires, margin = m.gate_eval(h, h, 1)
    assert fires and abs(margin - abs(1.0 / (1.0 + np.exp(-7.0 / 12.0)) - 0.5)) < 1e-15
    m.d = m.d.with_(gate_bias=-1.0)
    assert not m.gate_eval(h, h, 1)[1]


# ------------------------------------------------- last-exited fill at decode
class _FillFromFirstPlane(OracleLM):
    """Planted mistake: skipped slots get the first loop's KV instead of the
    last loop's."""
    def _last_exited_fill(self, cache, pos, e):
        if self.d.kv_layout == "depth" and e < self.d.r_max:
            for l in range(self.d.n_core):
                cache.core_k[l, e:, pos] = cache.core_k[l, 0, pos]
                cache.core_v[l, e:, pos] = cache.core_v[l, 0, pos]


class _FillOffByOne(OracleLM):
    """Planted mistake: skipped slots start one too late (slot e+1 is left
    as the gap, i.e. never filled)."""
    def _last_exited_fill(self, cache, pos, e):
        if self.d.kv_layout == "depth" and e < self.d.r_max:
            for l in range(self.d.n_core):
                cache.core_k[l, e + 1:, pos] = cache.core_k[l, e - 1, pos]
                cache.core_v[l, e + 1:, pos] = cache.core_v[l, e - 1, pos]


FORCED = [2, 3, 1, 4, 2, 3]


def _fill_case(cls=OracleLM, inject=False, n_coda=0):
    d = tiny(r_max=4, inject=inject, n_prelude=1 if inject else 0, n_coda=n_coda)
    w = S.make_weights(d, seed=12, norm="random", std=0.25)
    prompt = S.make_prompts(d.vocab, [5], seed=12)[0]
    m = cls(d, w, dtype=np.float64, keep_logits=True)
    toks, exits, recs = m.decode_sequential(prompt, len(FORCED) + 1, keep_state=True, forced_exits=FORCED)
    seq = np.concatenate([prompt, np.array(toks[:-1], dtype=np.int32)])
    ex = [d.r_max] * len(prompt) + FORCED
    states, logits = unrolled_forward_exits(d, w, seq, ex)
    return d, prompt, recs, states, logits


@pytest.mark.parametrize("inject,n_coda", [(False, 0), (True, 1)])
def test_decode_last_exited_fill_equals_unrolled_with_exits(inject, n_coda):
    """§4.2, decode side: after a token leaves at depth e < r_max its skipped
    slots hold the KV of loop e, so every later token that runs loop d > e
    reads it there.  Pinned against the independently written unrolled
    transformer with per-position exit depths (tokens leave at 2, 3, 1, 4,
    2, 3; later tokens read them at deeper loops): exit states and logits of
    every decoded token agree to fp64 rounding."""
    d, prompt, recs, states, logits = _fill_case(inject=inject, n_coda=n_coda)
    P = len(prompt)
    for i in range(1, len(FORCED) + 1):
        np.testing.assert_allclose(recs[i].exit_state, states[P + i - 1], rtol=1e-10, atol=1e-12)
        np.testing.assert_allclose(recs[i].logits, logits[P + i - 1], rtol=1e-10, atol=1e-11)


@pytest.mark.parametrize("cls", [_FillFromFirstPlane, _FillOffByOne])
def test_decode_fill_pin_catches_planted_mistakes(cls):
    """The same comparison fails for a fill from the wrong slot (no NaN
    reaches the result, so a finiteness check alone would pass) and for a
    fill that leaves a gap (NaN reaches the result)."""
    d, prompt, recs, states, logits = _fill_case(cls)
    P = len(prompt)
    errs = []
    for i in range(1, len(FORCED) + 1):
        a = recs[i].exit_state
        errs.append(np.inf if not np.isfinite(a).all() else float(np.abs(a - states[P + i - 1]).max()))
    assert max(errs) > 1e-6


def test_decode_fill_matches_min_rule_cache():
    """The slots a decoded token's fill writes equal what cache_from_planes
    builds from the same planes and exit depths (the min rule of §4.2: slot
    d of position j reads loop min(d, e_j))."""
    import copy
    d = tiny(r_max=4)
    w = S.make_weights(d, seed=13, norm="random", std=0.25)
    prompt = S.make_prompts(d.vocab, [4], seed=13)[0]
    m = OracleLM(d, w, dtype=np.float64)
    c = SeqCache(d, 4 + len(FORCED), np.float64)
    m.prefill(prompt, c)
    tok = int(prompt[-1])
    for i, e in enumerate(FORCED):
        rec = m.decode_step(tok, 4 + i, c, forced_exit=e)
        tok = rec.token
    n = 4 + len(FORCED)
    gapped_k = c.core_k[:, :, :n].copy()
    gapped_v = c.core_v[:, :, :n].copy()
    for j in range(n):
        gapped_k[:, c.exit_depth[j]:, j] = np.nan
        gapped_v[:, c.exit_depth[j]:, j] = np.nan
    c2 = cache_from_planes(d, gapped_k, gapped_v, c.exit_depth[:n], dtype=np.float64)
    np.testing.assert_array_equal(c2.core_k[:, :, :n], c.core_k[:, :, :n])
    np.testing.assert_array_equal(c2.core_v[:, :, :n], c.core_v[:, :, :n])
