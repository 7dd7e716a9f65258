"""The latency-model planner (host side): fits and closed forms."""
import numpy as np
import pytest

from continuous_depth_batching_amd import planner as P

pytestmark = pytest.mark.cpu


def test_fit_recovers_lines():
    m = P.fit_stage_model([(b, 1e-3 + 2e-5 * b) for b in (1, 7, 30, 64)],
                          [(e, 4e-4 + 1e-6 * e) for e in (1, 5, 16)])
    assert m.delta == pytest.approx(1e-3) and m.slope == pytest.approx(2e-5)
    assert m.b0 == pytest.approx(4e-4) and m.b1 == pytest.approx(1e-6)
    flat = P.fit_stage_model([(64, 2e-3), (64, 2e-3)], [(8, 1e-3)])
    assert flat.delta == pytest.approx(2e-3) and flat.slope == 0.0


def test_bucketed_core_cost():
    """A core step of B rows costs what its power-of-two bucket costs."""
    m = P.fit_stage_model([(33, 2.0), (64, 2.2), (17, 1.5), (20, 1.7)], [(4, 1.0)], buckets=True)
    assert m.core(40) == pytest.approx(2.1)       # bucket 64: mean of 2.0 and 2.2
    assert m.core(32) == pytest.approx(1.6)       # bucket 32: mean of 1.5 and 1.7
    assert m.core(3) == pytest.approx(m.delta + 3 * m.slope)     # no sample in bucket 4: the line


def test_exit_pmf():
    pmf = P.exit_pmf([2, 2, 3, 4], 4)
    assert pmf.tolist() == [0.0, 0.5, 0.25, 0.25]
    with pytest.raises(ValueError):
        P.exit_pmf([0, 2], 4)
    with pytest.raises(ValueError):
        P.exit_pmf([5], 4)


def test_memory_bound_closed_forms():
    """Constant step cost delta and a free boundary: a step costs the same
    at any batch, so fixed depth makes W tokens per r_max steps, refill at
    K = 1 W tokens per d_mean steps, and no-refill with every token leaving
    at depth d W tokens per d steps."""
    m = P.StageModel(delta=1e-3, slope=0.0, b0=0.0, b1=0.0)
    W, R = 64, 4
    pmf = P.exit_pmf([2] * 5 + [3] * 3 + [4] * 2, R)
    d_mean = float(np.dot(np.arange(1, R + 1), pmf))
    assert P.rate_fixed(m, W, R) == pytest.approx(W / (R * 1e-3))
    assert P.rate_refill(m, W, 1, pmf) == pytest.approx(W / (d_mean * 1e-3))
    assert P.rate_norefill(m, W, P.exit_pmf([3], R)) == pytest.approx(W / (3 * 1e-3))
    assert P.rate_norefill(m, W, P.exit_pmf([R], R)) == pytest.approx(P.rate_fixed(m, W, R))


def test_compute_bound_closed_forms():
    """Step cost proportional to the batch (delta = 0): every schedule pays
    per token-step, so refill and (for a large cohort) no-refill both reach
    1 / (slope d_mean), fixed depth 1 / (slope r_max)."""
    s = 2e-5
    m = P.StageModel(delta=0.0, slope=s, b0=0.0, b1=0.0)
    R = 4
    pmf = P.exit_pmf([2] * 5 + [3] * 3 + [4] * 2, R)
    d_mean = float(np.dot(np.arange(1, R + 1), pmf))
    assert P.rate_fixed(m, 64, R) == pytest.approx(1 / (s * R))
    assert P.rate_refill(m, 64, 1, pmf) == pytest.approx(1 / (s * d_mean))
    assert P.rate_norefill(m, 10**6, pmf) == pytest.approx(1 / (s * d_mean), rel=1e-6)


def test_refill_batch_fixed_point():
    """With K above the exits per step the core batch settles at
    B = (W - K/2) / (1 - 1/(2 d_mean)) and the coda runs on K rows."""
    m = P.StageModel(delta=1e-3, slope=1e-5, b0=5e-4, b1=2e-6)
    W, K, R = 64, 16, 32
    pmf = P.exit_pmf([12] * 10, R)
    d = 12.0
    B = (W - K / 2) / (1 - 1 / (2 * d))
    lam = B / d
    want = lam / (m.core(B) + m.boundary(K) * lam / K)
    assert P.rate_refill(m, W, K, pmf) == pytest.approx(want, rel=1e-9)


def test_simulation_closed_forms():
    """Every token leaves at depth d: W requests start together and stay in
    step, so each round is d core steps on W rows and one coda on W rows
    whatever the schedule (refill at K = 1 or K = W, no-refill); fixed depth
    is the same with d = r_max."""
    m = P.StageModel(delta=1e-3, slope=2e-5, b0=2e-3, b1=1e-5)
    W, d, R, n_out = 16, 3, 6, 9
    pmf = P.exit_pmf([d], R)
    want = W / (d * m.core(W) + m.boundary(W))
    for mode, K in (("refill", 1), ("refill", W), ("norefill", 1)):
        assert P.simulate(m, mode, W, K, pmf, W, n_out) == pytest.approx(want), (mode, K)
    assert P.simulate(m, "fixed", W, 1, pmf, W, n_out) == pytest.approx(W / (R * m.core(W) + m.boundary(W)))


def test_simulation_refill_memory_bound_limit():
    """Constant step cost, free boundary, many requests: refill at K = 1
    keeps the core batch full, so the rate tends to W / (d_mean delta);
    no-refill pays every cohort's longest token."""
    m = P.StageModel(delta=1e-3, slope=0.0, b0=0.0, b1=0.0)
    W, R = 32, 4
    pmf = P.exit_pmf([2] * 6 + [3] * 3 + [4], R)
    d_mean = float(np.dot(np.arange(1, R + 1), pmf))
    got = P.simulate(m, "refill", W, 1, pmf, 64, 200, seed=1)
    assert got == pytest.approx(W / (d_mean * 1e-3), rel=0.03)
    assert P.simulate(m, "norefill", W, 1, pmf, 64, 200, seed=1) < 0.8 * got


def test_simulation_replays_recorded_exits():
    """Two requests, two decode tokens each, recorded exits [2, 2] and
    [4, 4], refill at K = 1, unit-cost steps and free codas: request 0's
    tokens leave after steps 2 and 4, request 1's after steps 4 and 8, so
    4 tokens take 8 steps."""
    m = P.StageModel(delta=1.0, slope=0.0, b0=0.0, b1=0.0)
    pmf = P.exit_pmf([2, 4], 4)
    got = P.simulate(m, "refill", 2, 1, pmf, 2, 3, S=1, exits=[[2, 2], [4, 4]])
    assert got == pytest.approx(4 / 8)
    # no-refill: cohort of both, each token pass lasts 4 steps -> 4 tokens in 8 steps as well,
    # fixed depth (r_max 4 for every token) the same here
    assert P.simulate(m, "norefill", 2, 1, pmf, 2, 3, S=1, exits=[[2, 2], [4, 4]]) == pytest.approx(4 / 8)


def test_recommendation_follows_boundary_cost():
    """Cheap boundary (Ouro-like): immediate coda (K = 1) is best; a costly
    boundary (Huginn-like prelude/coda layers) moves the best K up."""
    pmf = P.exit_pmf([2] * 6 + [3] * 3 + [4], 4)
    cheap = P.StageModel(delta=1.4e-3, slope=3.8e-5, b0=1e-4, b1=1e-7)
    rates = P.predict(cheap, 64, 4, pmf, [1, 4, 8, 16])
    best = P.recommend(rates)
    assert best == "refill_K1"
    assert rates["refill_K1"] > rates["fixed"]
    costly = P.StageModel(delta=1.0e-3, slope=1.0e-5, b0=2.5e-3, b1=1e-6)
    pmf_h = P.exit_pmf(list(range(3, 23)), 32)
    rates_h = P.predict(costly, 64, 32, pmf_h, [1, 4, 8, 16])
    best_h = P.recommend(rates_h)
    assert best_h in ("refill_K8", "refill_K16", "norefill")
    assert rates_h["refill_K16"] > rates_h["refill_K1"]
