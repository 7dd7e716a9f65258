"""GPU parity of the HIP path against the CPU oracle (needs an MI355X).

Every case prints its name, shapes and seed before touching the GPU.
Bars (fp32 mode): token ids and exit depths bit-exact, hidden states at exit
within 1e-4 relative (norm-wise).  bf16 mode: hidden states within 2e-2
relative, logits within 5e-2 absolute, token/exit differences only where
the oracle's own margin is below 1e-2 (counted and printed).
"""
import ctypes as C
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


def _rel(a, b):
    return float(np.linalg.norm(np.asarray(a, np.float64) - np.asarray(b, np.float64)) /
                 max(np.linalg.norm(np.asarray(b, np.float64)), 1e-30))


def _c0_run(eng_mod, mode, W=4, K=1, kv_layout="depth", n_req=8, plen=16, n_out=16, M=8192, prompt_lens=None,
            **dims_kw):
    from oracle.model import OracleLM
    d = S.CONFIGS["c0"].with_(kv_layout=kv_layout, **dims_kw)
    # the explicit last-exited copies compute what the oracle's depth-indexed cache holds
    d_or = d.with_(kv_layout="depth") if kv_layout == "depth_copy" else d
    _say(f"[case] c0 end-to-end mode={mode} W={W} K={K} kv={kv_layout} n_req={n_req} plen={plen} n_out={n_out} "
         f"{dims_kw}")
    w = S.make_weights(d, seed=0)
    lens = prompt_lens or [plen] * n_req
    prompts = S.make_prompts(d.vocab, lens, seed=1)
    dm = eng_mod.DeviceModel(d, w)
    max_len = max(lens) + n_out
    e = eng_mod.Engine(dm, n_slots=W, max_rows=max(W, 4), num_blocks=len(lens) * (max_len // 16 + 2),
                       max_seqs=len(lens), max_blocks_per_seq=max_len // 16 + 2, max_out=n_out,
                       max_prefill_tokens=max(M, max(lens)))
    sch = eng_mod.Scheduler(e, prompts, n_out, mode=mode, W=W, K=K, M=M, capture_states=True).run()
    got = sch.results()
    m = OracleLM(d_or, w, dtype=np.float32)
    policy = "fixed" if mode == "fixed" else "adaptive"
    worst = 0.0
    for i, p in enumerate(prompts):
        chunks = None
        toks, exits, recs = m.decode_sequential(p, n_out, policy=policy, keep_state=True, chunks=chunks)
        gt, ge = got[i]
        assert gt == toks, f"request {i}: tokens differ\n gpu    {gt}\n oracle {toks}"
        assert ge == exits, f"request {i}: exits differ\n gpu    {ge}\n oracle {exits}"
        for g in range(1, n_out):
            st = sch.exit_states[(i, g)]
            worst = max(worst, _rel(st, recs[g].exit_state))
    _say(f"  max relative exit-state error {worst:.3e}")
    assert worst < 1e-4
    # the product scheduler's stage policy against the oracle's CDB simulator
    # (Alg. 1 / Alg. 2, pinned on the pages' Tables 2-3) driving the oracle
    # model on the same prompts, W, K, M and KV blocks: fp32 exits are
    # bit-exact, so every prefill, loop and coda stage must have the same
    # kind and batch size, in the same order (preludes run inside the
    # library's prefill and boundary calls and are not separate stages)
    from oracle.cdb_sim import CDBSimulator, ModelExecutor, Request
    reqs = [Request(i, np.asarray(p, np.int32), n_out) for i, p in enumerate(prompts)]
    sim = CDBSimulator(reqs, ModelExecutor(m), r_max=d_or.r_max, mode=mode, W=W, K=K, M=M,
                       kv_blocks=e.num_blocks).run()
    gpu_stages = [(st.kind, st.B) for st in sch.log if st.kind != "prelude"]
    sim_stages = [(st.kind, st.B) for st in sim.trace if st.kind != "prelude"]
    assert gpu_stages == sim_stages, f"stage sequences differ:\n gpu {gpu_stages}\n sim {sim_stages}"
    assert [(r.tokens, r.exits) for r in reqs] == got
    _say(f"  stage sequence equals the oracle simulator's ({len(gpu_stages)} stages)")
    # the lookahead scheduler: same tokens and exits, and the same stages with
    # the same batch sizes (its host picture of the queues is exact)
    if e.d.r_max >= 2:
        asch = eng_mod.AsyncScheduler(e, prompts, n_out, mode=mode, W=W, K=K, M=M).run()
        assert asch.results() == got, "lookahead scheduler: tokens / exits differ"
        stages = lambda sc: [(st.kind, st.B) for st in sc.log]
        assert stages(asch) == stages(sch), "lookahead scheduler: stage sequence differs"
        _say(f"  lookahead scheduler: identical results and {len(asch.log)} identical stages")
    e.close()
    return sch


def test_c0_refill_k1_bit_exact(eng_mod):
    sch = _c0_run(eng_mod, "refill")
    assert sch.core_steps > 0


def test_c0_norefill_bit_exact(eng_mod):
    _c0_run(eng_mod, "norefill")


def test_c0_fixed_depth_bit_exact(eng_mod):
    _c0_run(eng_mod, "fixed")


def test_c0_refill_k2_chunked_ragged(eng_mod):
    # ragged prompts and a small M force chunked prefill across batches
    _c0_run(eng_mod, "refill", W=3, K=2, M=24, prompt_lens=[5, 17, 9, 30, 12, 3], n_out=10)


@pytest.mark.parametrize("mode", ["refill", "norefill"])
def test_c0_online_arrivals_bit_exact(eng_mod, mode):
    """Online serving (Poisson-like staggered arrivals, some while others
    decode): the lookahead scheduler admits requests only after they
    arrive, and every request still decodes to the oracle's tokens and
    exits; normalized latencies are positive and finite."""
    from oracle.model import OracleLM
    d = S.CONFIGS["c0"]
    _say(f"[case] c0 online arrivals mode={mode}")
    w = S.make_weights(d, seed=0)
    lens = [16, 9, 23, 12, 16, 30]
    prompts = S.make_prompts(d.vocab, lens, seed=1)
    n_out = 8
    arrivals = [0.0, 0.0, 0.03, 0.05, 0.2, 0.21]
    dm = eng_mod.DeviceModel(d, w)
    e = eng_mod.Engine(dm, n_slots=4, max_rows=4, num_blocks=len(lens) * 4, max_seqs=len(lens),
                       max_blocks_per_seq=4, max_out=n_out, max_prefill_tokens=256)
    sch = eng_mod.AsyncScheduler(e, prompts, n_out, mode=mode, W=4, K=1, M=256, arrivals=arrivals).run()
    got = sch.results()
    nl = sch.normalized_latency()
    e.close()
    m = OracleLM(d, w, dtype=np.float32)
    for i, p in enumerate(prompts):
        toks, exits, _ = m.decode_sequential(p, n_out)
        assert got[i] == (toks, exits), f"request {i}"
    assert sorted(nl) == list(range(len(lens)))
    assert all(0.0 < v < 10.0 for v in nl.values()), nl
    # the last two arrive after 0.2 s: they cannot finish before they arrive
    assert sch.finish_s[4] > 0.2 and sch.finish_s[5] > 0.21
    _say(f"  normalized latency ms/token: {[round(1e3 * nl[i], 2) for i in range(len(lens))]}")


@pytest.mark.parametrize("mode", ["refill", "norefill"])
def test_c0_convergence_gate_bit_exact(eng_mod, mode):
    """The training-free convergence gate (loops >= 2, normalized step below
    0.36, lookahead exit): tokens and exits bit-exact, exits >= 3."""
    sch = _c0_run(eng_mod, mode, n_req=6, n_out=10, gate_kind="convergence", conv_threshold=0.36)
    exits = [e for _, ex in sch.results() for e in ex]
    assert min(exits) >= 3 and len(set(exits)) > 1


@pytest.mark.parametrize("kv_layout", ["single", "first_shared"])
def test_c0_shared_slot_caches(eng_mod, kv_layout):
    _c0_run(eng_mod, "refill", kv_layout=kv_layout, n_req=4, n_out=10)


def test_c0_explicit_last_exited_copies(eng_mod):
    """CDB_KV_DEPTH_COPY: at exit the boundary copies a token's last-loop
    K/V into the planes above its exit depth in every core layer (§4.2's
    last-exited cache made explicit) and attention reads every earlier
    position at its own plane, without the depth map.  Tokens, exits and
    the stage sequence bit-exact against the oracle (r_max 8, so most exits
    leave planes to fill); every exit state bit-identical to the run with
    the index rule min(d, e_j), since the same values are read."""
    a = _c0_run(eng_mod, "refill", kv_layout="depth_copy", n_req=6, n_out=12)
    b = _c0_run(eng_mod, "refill", kv_layout="depth", n_req=6, n_out=12)
    assert a.results() == b.results()
    assert a.exit_states.keys() == b.exit_states.keys()
    for k, v in a.exit_states.items():
        assert np.array_equal(v, b.exit_states[k]), f"exit state {k} differs between the two caches"


def _synthetic_core_case(eng_mod, d, B, L, seed=3, kv_layout="depth", rows_pad=None, n_check=None, coda=False):
    """One core step of B rows at context L over synthetic KV (exit depths
    U{1..r_max}, NaN gaps above them) against the oracle's single-row step.
    With coda=True every row is scheduled to leave after this step
    (exit_at = depth), and gate/compaction plus the boundary follow: the
    checked rows' exit states (2e-2), logits (5e-2 absolute) and tokens are
    compared with the oracle's LM head on its own core-step output."""
    from oracle.model import OracleLM, cache_from_planes
    d = d.with_(kv_layout=kv_layout)
    d_or = d.with_(kv_layout="depth") if kv_layout == "depth_copy" else d   # same values, copies made at exit
    _say(f"[case] synthetic core step H={d.hidden} heads={d.n_heads}x{d.head_dim} layers={d.n_core} "
         f"R={d.r_max} dtype={d.dtype} kv={kv_layout} B={B} L={L} seed={seed}")
    w = S.make_weights(d, seed=seed)
    dm = eng_mod.DeviceModel(d, w)
    R = d.r_max
    planes = {"depth": R, "single": 1, "first_shared": 2, "depth_copy": R}[kv_layout]
    mbps = (L + 1) // 16 + 1
    nblk = B * mbps
    e = eng_mod.Engine(dm, n_slots=B, max_rows=eng_mod.pow2(B), num_blocks=nblk, max_seqs=B,
                       max_blocks_per_seq=mbps, max_out=2, max_prefill_tokens=16)
    rng = np.random.default_rng(seed)
    perm = rng.permutation(nblk).astype(np.int32)            # non-contiguous physical blocks
    e.btab.copy_(torch.from_numpy(perm))
    nh, hd = d.n_heads, d.head_dim
    exit_d = rng.integers(1, R + 1, size=(B, L)).astype(np.uint8)
    depth = rng.integers(1, R + 1, size=B).astype(np.int32)
    kvdt = dm.wdt
    gen = torch.Generator(device="cuda").manual_seed(seed)
    # pool layout [n_core][num_blocks][n_heads][planes][16][head_dim]
    K = torch.randn((d.n_core, nblk, nh, planes, 16, hd), generator=gen, device="cuda").to(kvdt)
    V = torch.randn((d.n_core, nblk, nh, planes, 16, hd), generator=gen, device="cuda").to(kvdt)
    emap = torch.zeros(nblk * 16, dtype=torch.uint8)
    bt = perm.reshape(B, mbps)
    for b in range(B):
        for j in range(L):
            emap[bt[b, j // 16] * 16 + j % 16] = int(exit_d[b, j])
    # explicit copies: every gap (planes >= e_j) holds plane e_j - 1, as the
    # boundary leaves it, and the depth map is poisoned (all 1: a reader
    # that still applied min(d, e_j) would read plane 0 everywhere)
    if kv_layout == "depth_copy":
        ed = torch.zeros((nblk, 16), dtype=torch.long)
        for b in range(B):
            for j in range(L):
                ed[bt[b, j // 16], j % 16] = int(exit_d[b, j])
        ed = ed.cuda()
        pl = torch.arange(planes, device="cuda")[None, :, None]          # [1, planes, 1]
        src = torch.minimum(pl, (ed[:, None, :] - 1).clamp(min=0))       # [nblk, planes, 16]
        idx = src[None, :, None, :, :, None].expand_as(K)
        K = torch.gather(K, 3, idx)
        V = torch.gather(V, 3, idx)
        emap.fill_(1)
    # poison every gap (planes >= e_j of cached positions) with NaN
    elif planes > 1:
        gap = torch.zeros((nblk, planes, 16), dtype=torch.bool)
        for b in range(B):
            for j in range(L):
                gap[bt[b, j // 16], int(exit_d[b, j]):, j % 16] = True
        gap = gap.cuda()[None, :, None, :, :, None].expand_as(K)
        K = torch.where(gap, torch.full_like(K, float("nan")), K)
        V = torch.where(gap, torch.full_like(V, float("nan")), V)
    e.core_k.copy_(K.reshape(-1))
    e.core_v.copy_(V.reshape(-1))
    e.emap.copy_(emap)
    state0 = torch.randn((B, d.hidden), generator=gen, device="cuda")
    e.state.copy_(state0)
    inj0 = None
    if d.inject:                                 # prelude output e, added to the core input every loop
        inj0 = torch.randn((B, d.hidden), generator=gen, device="cuda")
        e.inject.copy_(inj0)
        inj0 = inj0.cpu().numpy()
    rows = rows_pad or eng_mod.pow2(B)
    desc = np.zeros(5 * e.max_rows + 1, dtype=np.int32)
    cap = e.max_rows
    desc[0] = B
    desc[1:1 + B] = np.arange(B)                 # slot
    desc[1 + cap:1 + cap + B] = np.arange(B)     # seq
    desc[1 + 2 * cap:1 + 2 * cap + B] = L        # pos
    desc[1 + 3 * cap:1 + 3 * cap + B] = depth
    desc[1 + 4 * cap:1 + 4 * cap + B] = depth if coda else R
    e.desc_t.copy_(torch.from_numpy(desc))
    e.core_step(rows)
    torch.cuda.synchronize()
    out = e.state.cpu().numpy()
    if coda:
        e.q_t.zero_()
        e.n_gen.fill_(1)
        e.n_out.fill_(2)
        lg_buf = torch.zeros((rows, d.vocab), dtype=torch.float32, device="cuda")
        st_buf = torch.zeros((rows, d.hidden), dtype=torch.float32, device="cuda")
        e.gate_compact(rows, True)
        e.boundary(rows, exit_states=st_buf, logits=lg_buf)
        e.sync()
        assert e.read_counts()[:2] == [0, B]
        lg_gpu = lg_buf.cpu().numpy()
        st_gpu = st_buf.cpu().numpy()
        toks_gpu = e.tokens_out.cpu().numpy()[:, 1]
    Kh = K.float().cpu().numpy()
    Vh = V.float().cpu().numpy()
    s0 = state0.cpu().numpy()
    m = OracleLM(d_or, w, dtype=np.float32)
    worst = worst_logit = 0.0
    check = range(B) if n_check is None else sorted(set(np.linspace(0, B - 1, n_check).astype(int).tolist()))
    for b in check:
        # gather this row's planes in logical order for the oracle
        kb = np.stack([Kh[:, bt[b, j // 16], :, :, j % 16, :].transpose(0, 2, 1, 3) for j in range(L)], axis=2)
        vb = np.stack([Vh[:, bt[b, j // 16], :, :, j % 16, :].transpose(0, 2, 1, 3) for j in range(L)], axis=2)
        cache = cache_from_planes(d_or, kb, vb, exit_d[b], dtype=np.float32)
        x_in = s0[b] + inj0[b] if inj0 is not None else s0[b]
        ref, kref, vref = m.core_step_row(x_in, L, int(depth[b]), cache)
        assert np.isfinite(out[b]).all(), f"row {b}: non-finite output (a gap was read?)"
        err = _rel(out[b], ref)
        worst = max(worst, err)
        # K/V written for this row at plane depth (or the single plane)
        pl = min(int(depth[b]), planes) - 1
        kg = e.core_k.view(d.n_core, nblk, nh, planes, 16, hd)[:, bt[b, L // 16], :, pl, L % 16, :].float().cpu().numpy()
        tol_kv = 1e-5 if d.dtype == "fp32" else 1e-2
        assert _rel(kg, kref) < tol_kv, f"row {b}: written K differs ({_rel(kg, kref):.2e})"
        if coda:                                 # exit queue = rows in row order (all leave)
            assert np.array_equal(st_gpu[b], out[b])
            lg = m.lm_head(ref[None])[0]
            lerr = float(np.abs(lg_gpu[b] - lg).max())
            worst_logit = max(worst_logit, lerr)
            top = int(np.argmax(lg))
            srt = np.sort(lg)
            assert toks_gpu[b] == top or srt[-1] - srt[-2] < 1e-2, f"row {b}: token {toks_gpu[b]} vs {top}"
    if coda:
        _say(f"  max logit abs error {worst_logit:.3e} (bar 5e-2)")
        assert worst_logit < 5e-2
    _say(f"  max relative state error {worst:.3e} over rows {list(check)}")
    e.close()
    return worst


@pytest.mark.parametrize("ffn,B", [(256, 5), (272, 5), (256, 70)])
def test_plane_rule_fp32_tiny_many_tiles(eng_mod, ffn, B):
    """ffn 256 takes the fused gate/up + SwiGLU decode kernel; 272 (not a
    multiple of 32, allowed for fp32's 16-wide k-steps) the split gate/up
    projection and the separate SwiGLU kernel; B = 70 runs the decode GEMMs
    on two 64-row blocks."""
    d = S.ModelDims("t", vocab=64, hidden=128, n_heads=2, head_dim=64, ffn=ffn, n_prelude=0, n_core=2,
                    n_coda=0, r_max=4, dtype="fp32")
    assert _synthetic_core_case(eng_mod, d, B=B, L=77) < 1e-4


@pytest.mark.parametrize("B", [5, 40, 70])
def test_fp32_tiny_fused_residual_projections(eng_mod, monkeypatch, B):
    """The fused residual projections (unsplit O and down with the deferred
    RMSNorm scale) in fp32 (16-wide k-steps) with one, four and two blocks of
    four 16-row tiles, both fusions forced on at every batch size
    (CDB_FUSE_*_ROWS=256); two core layers, so the deferred scale crosses a
    layer boundary."""
    monkeypatch.setenv("CDB_FUSE_O_ROWS", "256")
    monkeypatch.setenv("CDB_FUSE_DOWN_ROWS", "256")
    d = S.ModelDims("t", vocab=64, hidden=64, n_heads=2, head_dim=32, ffn=256, n_prelude=0, n_core=2,
                    n_coda=0, r_max=3, dtype="fp32")
    assert _synthetic_core_case(eng_mod, d, B=B, L=77) < 1e-4


@pytest.mark.parametrize("B", [3, 20, 40, 100])
def test_plane_rule_bf16_head128_ragged(eng_mod, B):
    """B = 3, 20 and 40 run the decode GEMMs (split and fused gate/up) with
    one, two and four 16-row tiles; B = 100 with two 64-row blocks."""
    d = S.ModelDims("t", vocab=64, hidden=256, n_heads=2, head_dim=128, ffn=512, n_prelude=0, n_core=2,
                    n_coda=0, r_max=4, dtype="bf16")
    assert _synthetic_core_case(eng_mod, d, B=B, L=150) < 2e-2


@pytest.mark.parametrize("kv_layout", ["single", "first_shared", "depth_copy"])
def test_shared_slot_core_step_bf16(eng_mod, kv_layout):
    d = S.ModelDims("t", vocab=64, hidden=256, n_heads=2, head_dim=128, ffn=512, n_prelude=0, n_core=2,
                    n_coda=0, r_max=4, dtype="bf16")
    assert _synthetic_core_case(eng_mod, d, B=4, L=64, kv_layout=kv_layout) < 2e-2


def test_huginn_dims_core_step_injection_sampled_rows(eng_mod):
    """Huginn-like core shapes (hidden 5280, 55 x 96 heads, SwiGLU 17920,
    4 core layers, r_max 32, bf16) with the prelude injection, at context
    200; the vocabulary and the prelude/coda layers play no part in a core
    step and are left out."""
    d = S.CONFIGS["c3"].with_(vocab=512, n_prelude=0, n_coda=0)
    assert _synthetic_core_case(eng_mod, d, B=4, L=200, n_check=4) < 2e-2


def test_ouro_dims_core_step_sampled_rows(eng_mod):
    """Full Ouro-like shapes (24 layers, 2048 hidden, 16x128 heads, SwiGLU
    5632, r_max 4, bf16) at context 200, every row checked."""
    assert _synthetic_core_case(eng_mod, S.CONFIGS["c1"], B=4, L=200, n_check=4) < 2e-2


def test_bench_shape_graph_step_sampled_rows(eng_mod):
    """The benchmark's own configuration: Ouro-like bf16 model, 64 rows at
    context 1024 on non-contiguous blocks with cached exit depths U{1..4},
    one decode step (core step + gate/compaction + coda/prelude) captured as
    a HIP graph and replayed, as bench.py times it (here the boundary also
    writes exit states and logits).  Four continuing rows must hold the
    oracle's core-step output (2e-2 relative) and have written its K; every
    row that leaves must have the oracle's exit state (2e-2), logits within
    5e-2 absolute over the whole vocabulary (all 24 layers behind them), the
    oracle's token (unless its top-2 logit gap is below 1e-2), and its slot
    must hold the successor's embedding."""
    import bench
    from oracle.model import OracleLM, cache_from_planes
    d = S.CONFIGS["c1"]
    B, L = 64, 1024
    _say(f"[case] bench shape: Ouro-like bf16 B={B} L={L}, captured decode step, sampled rows")
    w = S.make_weights(d, seed=0)
    dm = eng_mod.DeviceModel(d, w)
    db = bench.DecodeBench(eng_mod, dm, d, B, L, steps_total=8, seed=3)
    e = db.e
    cap = e.max_rows
    state0 = e.state.cpu().numpy().copy()
    desc0 = e.desc_t.cpu().numpy().copy()
    depth0 = desc0[1 + 3 * cap:1 + 3 * cap + B].copy()
    emap = e.emap.cpu().numpy()
    bt = e.btab.cpu().numpy().reshape(B, db.mbps)
    rows_pad = db.rows
    lg_buf = torch.zeros((rows_pad, d.vocab), dtype=torch.float32, device="cuda")
    st_buf = torch.zeros((rows_pad, d.hidden), dtype=torch.float32, device="cuda")
    # the benchmark's step (core step, gate/compaction, boundary), with the
    # boundary also writing the exit states and logits of the rows that leave
    g = e.capture(lambda: (e.core_step(rows_pad), e.gate_compact(rows_pad, True),
                           e.boundary(rows_pad, exit_states=st_buf, logits=lg_buf)))
    e.replay(g)
    torch.cuda.synchronize()
    e.drop(g)
    state1 = e.state.cpu().numpy()
    toks = e.tokens_out.cpu().numpy()
    lg_gpu = lg_buf.cpu().numpy()
    st_gpu = st_buf.cpu().numpy()
    m = OracleLM(d, w, dtype=np.float32)
    R, nh, hd = d.r_max, d.n_heads, d.head_dim
    K5 = e.core_k.view(d.n_core, -1, nh, R, 16, hd)
    V5 = e.core_v.view(d.n_core, -1, nh, R, 16, hd)
    cont = [b for b in range(B) if depth0[b] < R]
    leave = [b for b in range(B) if depth0[b] == R]
    rows = cont[:4] + leave
    _say(f"  rows checked {rows} (depths {[int(depth0[b]) for b in rows]})")
    nb = L // 16
    worst = worst_logit = 0.0
    for b in rows:
        blocks = torch.from_numpy(bt[b, :nb].astype(np.int64)).cuda()
        kb = K5.index_select(1, blocks).float().cpu().numpy()      # [n_core, nb, nh, R, 16, hd]
        vb = V5.index_select(1, blocks).float().cpu().numpy()
        kb = kb.transpose(0, 3, 1, 4, 2, 5).reshape(d.n_core, R, L, nh, hd)
        vb = vb.transpose(0, 3, 1, 4, 2, 5).reshape(d.n_core, R, L, nh, hd)
        ex = np.array([emap[bt[b, j // 16] * 16 + j % 16] for j in range(L)], dtype=np.uint8)
        cache = cache_from_planes(d, kb, vb, ex, dtype=np.float32)
        del kb, vb
        ref, kref, _ = m.core_step_row(state0[b], L, int(depth0[b]), cache)
        kg = K5[:, int(bt[b, L // 16]), :, int(depth0[b]) - 1, L % 16, :].float().cpu().numpy()
        assert _rel(kg, kref) < 1e-2, f"row {b}: written K differs ({_rel(kg, kref):.2e})"
        if depth0[b] < R:
            err = _rel(state1[b], ref)
            worst = max(worst, err)
            assert err < 2e-2, f"row {b}: state rel err {err:.3e}"
        else:
            # leaving rows reach the exit queue in row order
            qi = leave.index(b)
            err = _rel(st_gpu[qi], ref)
            worst = max(worst, err)
            assert err < 2e-2, f"row {b}: exit state rel err {err:.3e}"
            lg = m.lm_head(ref[None])[0]
            lerr = float(np.abs(lg_gpu[qi] - lg).max())
            worst_logit = max(worst_logit, lerr)
            assert lerr < 5e-2, f"row {b}: logit abs err {lerr:.3e}"
            top = int(np.argmax(lg))
            gap = float(np.sort(lg)[-1] - np.sort(lg)[-2])
            got = int(toks[b, 1])
            assert got == top or gap < 1e-2, f"row {b}: token {got} vs oracle {top} (gap {gap:.3e})"
            emb = w["embed"][got]
            assert np.array_equal(state1[b], emb.astype(np.float32)), f"row {b}: slot does not hold the successor"
            _say(f"  leaving row {b}: token {got} (oracle {top}, top-2 gap {gap:.3f}), logit err {lerr:.3e}")
    _say(f"  max relative state error {worst:.3e}, max logit abs error {worst_logit:.3e}")
    e.close()


def test_empty_core_batch_is_a_no_op(eng_mod):
    """A core step, gate/compaction and boundary over a batch with no valid
    row leave the loop state, the queues and the tokens untouched."""
    d = S.CONFIGS["c0"]
    _say("[case] empty core batch (n_valid = 0), c0 dims")
    w = S.make_weights(d, seed=0)
    dm = eng_mod.DeviceModel(d, w)
    e = eng_mod.Engine(dm, n_slots=4, max_rows=4, num_blocks=8, max_seqs=4, max_blocks_per_seq=2, max_out=4,
                       max_prefill_tokens=16, kv_fill=0.0)
    e.state.copy_(torch.randn((4, d.hidden), device="cuda"))
    e.desc_t.zero_()
    e.q_t.zero_()
    s0 = e.state.clone()
    tok0 = e.tokens_out.clone()
    for rows in (1, 4):
        e.core_step(rows)
        e.gate_compact(rows, True)
        e.boundary(rows)
    counts = e.read_counts()
    assert counts == [0, 0, 0, 0], counts
    assert torch.equal(e.state, s0)
    assert torch.equal(e.tokens_out, tok0)
    assert int(e.desc_t[0].item()) == 0 and int(e.q_t[0].item()) == 0
    e.close()


def test_c0_refill_with_the_gate_off_is_full_depth(eng_mod):
    """Refill (Alg. 2) with the gate switched off never exits early: every
    token leaves at r_max, and the tokens equal the oracle's fixed-depth
    decode bit for bit (fp32), through CDB's staged schedule -- the
    configuration the pages compare with fixed-depth CB to measure CDB's own
    overhead (§6.2)."""
    from oracle.model import OracleLM
    d = S.CONFIGS["c0"]
    _say("[case] c0 refill with the gate off, W=4")
    w = S.make_weights(d, seed=0)
    n_out, lens = 12, [16, 40, 9, 23, 31, 12]
    prompts = S.make_prompts(d.vocab, lens, seed=1)
    dm = eng_mod.DeviceModel(d, w)
    max_len = max(lens) + n_out
    e = eng_mod.Engine(dm, n_slots=4, max_rows=4, num_blocks=len(lens) * (max_len // 16 + 2), max_seqs=len(lens),
                       max_blocks_per_seq=max_len // 16 + 2, max_out=n_out, max_prefill_tokens=8192)
    sch = eng_mod.AsyncScheduler(e, prompts, n_out, mode="refill", W=4, K=1, M=8192, gate=False).run()
    got = sch.results()
    m = OracleLM(d, w, dtype=np.float32)
    for i, p in enumerate(prompts):
        toks, exits, _ = m.decode_sequential(p, n_out, policy="fixed")
        assert list(got[i][0]) == list(toks), f"request {i}: tokens differ"
        assert list(got[i][1]) == list(exits) and all(x == d.r_max for x in exits), f"request {i}: {got[i][1]}"
    assert sch.core_token_steps == sum((n_out - 1) * d.r_max for _ in prompts)
    e.close()


def test_c0_single_loop_model_bit_exact(eng_mod):
    """Degenerate depth: r_max = 1, so every token leaves after its first
    loop and the gate is never evaluated; bit-exact tokens against the
    oracle (synchronous scheduler: the lookahead needs two loops)."""
    _c0_run(eng_mod, "refill", n_req=4, n_out=8, r_max=1)


def test_bf16_decode_batch_above_64_rows(eng_mod):
    """200 rows (bucket 256): the weight-streaming decode projections in four
    64-row blocks; attention without context splits."""
    d = S.ModelDims("t", vocab=64, hidden=256, n_heads=2, head_dim=128, ffn=512, n_prelude=0, n_core=2,
                    n_coda=0, r_max=4, dtype="bf16")
    assert _synthetic_core_case(eng_mod, d, B=200, L=40, n_check=6) < 2e-2


@pytest.mark.parametrize("B", [300, 512])
def test_bf16_ouro_width_decode_above_256_rows_with_coda(eng_mod, B):
    """Ouro-like widths (H 2048, 16 x 128 heads, SwiGLU 5632, vocabulary
    49152) with 2 core layers and more than 256 rows (bucket 512): the
    projections leave the weight-streaming decode kernels for the LDS-tiled
    MFMA GEMM split over K (partials reduced by the norm and by attention)
    and its SwiGLU epilogue; the LM head streams its weights in 64-row
    blocks with the argmax epilogue.  Every row leaves, so the boundary runs
    at 512 rows.  Sampled rows against the oracle: states 2e-2, logits 5e-2."""
    d = S.CONFIGS["c1"].with_(n_core=2)
    assert _synthetic_core_case(eng_mod, d, B=B, L=48, n_check=8, coda=True) < 2e-2


@pytest.mark.parametrize("B,fuse", [(1, "both"), (16, "both"), (32, "both"), (64, "both"), (100, "both"),
                                    (16, "o"), (16, "down"), (16, "none"), (48, "none"), (48, "plain"),
                                    (100, "none")])
def test_bf16_ouro_width_fused_residual_projections(eng_mod, monkeypatch, B, fuse):
    """Decode layers whose O and down projections complete the residual
    stream themselves (no K split) and hand the next norm's input g * x
    unscaled, with per-8-column sums of x^2 from which attention and the
    gate/up kernel apply the row's 1 / rms; or (fuse "none") split
    projections whose partials a separate kernel adds with the norm deferred
    the same way (sums per 256 columns); or ("plain") split projections and
    norm kernels.  Ouro-like widths with 3 core layers, so the deferred scale
    crosses layer boundaries, and every row leaves (coda boundary and LM
    head).  One, two and four 16-row tiles and two 64-row blocks with both
    projections fused; at 16 rows each one alone and neither
    (CDB_FUSE_O_ROWS / CDB_FUSE_DOWN_ROWS / CDB_DEFER_NORM_ROWS).  Sampled
    rows against the oracle: states 2e-2, logits 5e-2."""
    monkeypatch.setenv("CDB_FUSE_O_ROWS", "0" if fuse in ("none", "down", "plain") else "256")
    monkeypatch.setenv("CDB_FUSE_DOWN_ROWS", "0" if fuse in ("none", "o", "plain") else "256")
    monkeypatch.setenv("CDB_DEFER_NORM_ROWS", "0" if fuse == "plain" else "256")
    d = S.CONFIGS["c1"].with_(n_core=3)
    assert _synthetic_core_case(eng_mod, d, B=B, L=200, n_check=min(B, 6), coda=True) < 2e-2


@pytest.mark.parametrize("dtype,B", [("bf16", 3), ("fp32", 4)])
def test_o_projection_merging_attention_splits_matches_merge_kernel(eng_mod, monkeypatch, dtype, B):
    """At one piece per lane (here 4 heads of 128, bucket 4, 16 context
    splits) the fused O projection merges the attention's split partials
    itself instead of the merge kernel.  The same core step with that fold
    switched off (CDB_FOLD_MERGE=0) gives bitwise the same states: the merge
    is the same arithmetic in the same order."""
    hd = 128 if dtype == "bf16" else 64
    d = S.ModelDims("t", vocab=64, hidden=512, n_heads=4, head_dim=hd, ffn=1024, n_prelude=0, n_core=2,
                    n_coda=0, r_max=4, dtype=dtype)
    _say(f"[case] merge fold vs merge kernel, {dtype} H=512 4x{hd} B={B}")
    L = 300

    def run(fold):
        monkeypatch.setenv("CDB_FOLD_MERGE", fold)
        w = S.make_weights(d, seed=5)
        dm = eng_mod.DeviceModel(d, w)
        mbps = (L + 1) // 16 + 1
        e = eng_mod.Engine(dm, n_slots=B, max_rows=eng_mod.pow2(B), num_blocks=B * mbps, max_seqs=B,
                           max_blocks_per_seq=mbps, max_out=2, max_prefill_tokens=16)
        gen = torch.Generator(device="cuda").manual_seed(11)
        e.btab.copy_(torch.arange(B * mbps, dtype=torch.int32, device="cuda"))
        e.core_k.copy_(torch.randn(e.core_k.numel(), generator=gen, device="cuda").to(e.core_k.dtype))
        e.core_v.copy_(torch.randn(e.core_v.numel(), generator=gen, device="cuda").to(e.core_v.dtype))
        e.emap.copy_(torch.from_numpy(S.make_context_exit_depths(B * mbps * 16, d.r_max, seed=2)))
        e.state.copy_(torch.randn((B, d.hidden), generator=gen, device="cuda"))
        cap = e.max_rows
        desc = np.zeros(5 * cap + 1, dtype=np.int32)
        desc[0] = B
        desc[1:1 + B] = np.arange(B)
        desc[1 + cap:1 + cap + B] = np.arange(B)
        desc[1 + 2 * cap:1 + 2 * cap + B] = L - np.arange(B) * 37
        desc[1 + 3 * cap:1 + 3 * cap + B] = np.arange(B) % d.r_max + 1
        desc[1 + 4 * cap:1 + 4 * cap + B] = d.r_max
        e.desc_t.copy_(torch.from_numpy(desc))
        for _ in range(3):
            e.core_step(eng_mod.pow2(B))
        torch.cuda.synchronize()
        return e.state.cpu().numpy(), e.core_k.cpu().float().numpy()

    s1, k1 = run("1")
    s0, k0 = run("0")
    assert np.isfinite(s1).all()
    assert np.array_equal(s1, s0)
    assert np.array_equal(k1, k0)


def test_graph_replays_match_eager_steps(eng_mod):
    """A captured decode step (core step + gate/compaction + coda/prelude),
    replayed several times with eager work and synchronisations between the
    replays, gives bitwise the states of the same steps run eagerly."""
    d = S.ModelDims("t", vocab=256, hidden=256, n_heads=2, head_dim=128, ffn=512, n_prelude=0, n_core=2,
                    n_coda=0, r_max=4, dtype="bf16", gate_bias=0.0)
    _say(f"[case] graph replay vs eager, bf16 H=256 2x128 layers=2 R=4 B=8 L=40")

    def make():
        w = S.make_weights(d, seed=4)
        dm = eng_mod.DeviceModel(d, w)
        B, L = 8, 40
        mbps = (L + 64) // 16 + 1
        e = eng_mod.Engine(dm, n_slots=B, max_rows=B, num_blocks=B * mbps, max_seqs=B, max_blocks_per_seq=mbps,
                           max_out=64, max_prefill_tokens=16, kv_fill=0.0)
        gen = torch.Generator(device="cuda").manual_seed(9)
        e.core_k.copy_(torch.randn(e.core_k.numel(), generator=gen, device="cuda").to(e.core_k.dtype))
        e.core_v.copy_(torch.randn(e.core_v.numel(), generator=gen, device="cuda").to(e.core_v.dtype))
        e.btab.copy_(torch.arange(B * mbps, dtype=torch.int32, device="cuda"))
        emap = torch.full((B * mbps * 16,), d.r_max, dtype=torch.uint8)
        emap[: B * mbps * 16] = torch.from_numpy(S.make_context_exit_depths(B * mbps * 16, d.r_max, seed=3))
        e.emap.copy_(emap)
        e.state.copy_(torch.randn((B, d.hidden), generator=gen, device="cuda"))
        cap = e.max_rows
        desc = np.zeros(5 * cap + 1, dtype=np.int32)
        desc[0] = B
        desc[1:1 + B] = np.arange(B)
        desc[1 + cap:1 + cap + B] = np.arange(B)
        desc[1 + 2 * cap:1 + 2 * cap + B] = L
        desc[1 + 3 * cap:1 + 3 * cap + B] = S.c1_row_depths(B, 4, seed=1)
        desc[1 + 4 * cap:1 + 4 * cap + B] = d.r_max
        e.desc_t.copy_(torch.from_numpy(desc))
        e.n_gen.fill_(1)
        e.n_out.fill_(60)
        return e

    def step(e):
        e.core_step(8)
        e.gate_compact(8, True)
        e.boundary(8)

    ea, eb = make(), make()
    g = eb.capture(lambda: step(eb))
    for i in range(6):
        step(ea)
        eb.replay(g)
        torch.cuda.synchronize()
        junk = torch.randn(1000, device="cuda").sum().item()      # eager work between replays
        assert torch.equal(ea.state, eb.state), f"replay {i}: state differs"
        assert torch.equal(ea.desc_t, eb.desc_t), f"replay {i}: core batch differs"
        assert torch.equal(ea.tokens_out, eb.tokens_out), f"replay {i}: tokens differ"
        assert torch.equal(ea.emap, eb.emap)
    eb.drop(g)
    assert int(ea.n_gen.sum().item()) > 8          # some rows exited and were refilled
    ea.close(); eb.close()


class LogitBarExceeded(AssertionError):
    """The bf16 logits missed the 5e-2 absolute bar (every other check of
    the case passed before this one was made)."""


def _bf16_replay_check(eng_mod, d, prompt_lens, n_out, W, M, mode="refill", seed=0):
    """bf16 bar: follow the GPU's tokens and exits in the oracle (forced
    replay); exit states within 2e-2 relative, logits within 5e-2 absolute;
    a token or exit the oracle would have chosen differently is allowed only
    where its own margin there is below 1e-2 (such cases are counted).  The
    logit bar is checked last and raises LogitBarExceeded."""
    from oracle.model import OracleLM
    _say(f"[case] bf16 end-to-end H={d.hidden} {d.n_heads}x{d.head_dim} layers={d.n_core} R={d.r_max} "
         f"prompts={prompt_lens} n_out={n_out} W={W} M={M} mode={mode}")
    w = S.make_weights(d, seed=seed)
    prompts = S.make_prompts(d.vocab, prompt_lens, seed=seed + 1)
    dm = eng_mod.DeviceModel(d, w)
    mbps = max(prompt_lens) // 16 + n_out // 16 + 3
    e = eng_mod.Engine(dm, n_slots=W, max_rows=eng_mod.pow2(max(W, 2)), num_blocks=len(prompts) * mbps,
                       max_seqs=len(prompts), max_blocks_per_seq=mbps, max_out=n_out, max_prefill_tokens=M)
    sch = eng_mod.Scheduler(e, prompts, n_out, mode=mode, W=W, K=1, M=M, capture_states=True,
                            capture_logits=True).run()
    got = sch.results()
    e.close()
    m = OracleLM(d, w, dtype=np.float32, keep_logits=True)
    worst_state = worst_logit = 0.0
    logit_std = 0.0
    allowed = 0
    for i, p in enumerate(prompts):
        gt, ge = got[i]
        toks, exits, recs = m.decode_sequential(p, n_out, keep_state=True, forced_tokens=gt[:-1], forced_exits=ge)
        logit_std = max(logit_std, max(float(np.std(r.logits)) for r in recs[1:]))
        if toks[0] != gt[0]:
            assert recs[0].logit_gap < 1e-2, f"request {i}: first token differs with gap {recs[0].logit_gap}"
            allowed += 1
        for g in range(1, n_out):
            rec = recs[g]
            worst_state = max(worst_state, _rel(sch.exit_states[(i, g)], rec.exit_state))
            worst_logit = max(worst_logit, float(np.abs(sch.logits[(i, g)] - rec.logits).max()))
            if rec.own_token != gt[g]:
                assert rec.logit_gap < 1e-2, f"request {i} token {g}: differs with logit gap {rec.logit_gap}"
                allowed += 1
            if rec.own_exit != ge[g - 1]:
                # the decision that differs is the gate evaluation closest to the GPU's exit
                m_near = min(rec.gate_margins) if rec.gate_margins else 1.0
                assert m_near < 1e-2, f"request {i} token {g}: exit differs with gate margin {m_near}"
                allowed += 1
    _say(f"  max exit-state rel err {worst_state:.3e}, max logit abs err {worst_logit:.3e} "
         f"(bar 5e-2, logit std {logit_std:.3f}), allowed low-margin disagreements {allowed}")
    assert worst_state < 2e-2
    if not worst_logit < 5e-2:
        raise LogitBarExceeded(f"max logit abs err {worst_logit:.3e} >= 5e-2 (logit std {logit_std:.3f})")
    return sch


def test_bf16_head128_long_prompts_chunked_prefill(eng_mod):
    d = S.ModelDims("t", vocab=512, hidden=256, n_heads=2, head_dim=128, ffn=512, n_prelude=0, n_core=2,
                    n_coda=0, r_max=4, dtype="bf16", gate_bias=0.1)
    _bf16_replay_check(eng_mod, d, [150, 37, 300, 91], n_out=12, W=3, M=128)


def test_bf16_huginn_like_tiny_injection(eng_mod):
    d = S.ModelDims("t", vocab=512, hidden=192, n_heads=2, head_dim=96, ffn=384, n_prelude=2, n_core=2,
                    n_coda=2, r_max=8, dtype="bf16", inject=True, gate_bias=0.1)
    _bf16_replay_check(eng_mod, d, [40, 75, 20], n_out=8, W=2, M=64)


def test_bf16_huginn_like_tiny_convergence_gate(eng_mod):
    d = S.ModelDims("t", vocab=512, hidden=192, n_heads=2, head_dim=96, ffn=384, n_prelude=2, n_core=2,
                    n_coda=2, r_max=8, dtype="bf16", inject=True, gate_kind="convergence", conv_threshold=0.21)
    _bf16_replay_check(eng_mod, d, [40, 75, 20], n_out=8, W=2, M=64)


@pytest.mark.parametrize("ffn", [5632, 3040])
def test_bf16_wide_prefill_chunk_tiled_projections(eng_mod, ffn):
    """Ouro-width layers (H 2048, 16 x 128 heads) with one core layer and
    r_max 3, so that a single 2100-token prefill chunk reaches the LDS-tiled
    MFMA GEMM for all four projections (QKV, O with the residual add,
    gate/up with SwiGLU, down with the residual add), with a ragged last row
    tile.  F = 3040 (95 k-steps of 32) gives the down projection a final
    half k-tile."""
    d = S.ModelDims("t", vocab=512, hidden=2048, n_heads=16, head_dim=128, ffn=ffn, n_prelude=0, n_core=1,
                    n_coda=0, r_max=3, dtype="bf16", gate_bias=0.0)
    _bf16_replay_check(eng_mod, d, [2100, 40], n_out=4, W=2, M=8192)


def test_bf16_ouro_width_prefill_wide_tiles_match_tiled(eng_mod, monkeypatch):
    """Ouro-like widths with one core layer: a 4,200-token prompt (one
    4,240-row chunk) puts all four projections on the 256 x 128 GEMM --
    QKV (fp32 store) and gate/up with SwiGLU in its two-barrier form, O and
    down with the residual add in its prefetching form -- with a ragged last
    row tile.  The same run with that kernel off (CDB_TILE_WIDE=0: the
    128 x 128 kernel, which the test above checks against the oracle) must
    give the same tokens, exits, logits and exit states bit for bit."""
    d = S.ModelDims("t", vocab=512, hidden=2048, n_heads=16, head_dim=128, ffn=5632, n_prelude=0, n_core=1,
                    n_coda=1, r_max=3, dtype="bf16", gate_bias=0.0)
    prompt_lens, n_out, W, M = [4200, 40], 4, 2, 8192
    w = S.make_weights(d, seed=0)
    prompts = S.make_prompts(d.vocab, prompt_lens, seed=1)
    mbps = max(prompt_lens) // 16 + n_out // 16 + 3

    def run(wide):
        monkeypatch.setenv("CDB_TILE_WIDE", "1" if wide else "0")
        _say(f"[case] Ouro-width prefill {prompt_lens}, 256 x 128 GEMM {'on' if wide else 'off'}")
        dm = eng_mod.DeviceModel(d, w)
        e = eng_mod.Engine(dm, n_slots=W, max_rows=eng_mod.pow2(W), num_blocks=len(prompts) * mbps,
                           max_seqs=len(prompts), max_blocks_per_seq=mbps, max_out=n_out, max_prefill_tokens=M)
        sch = eng_mod.Scheduler(e, prompts, n_out, mode="refill", W=W, K=1, M=M, capture_states=True,
                                capture_logits=True).run()
        res = sch.results()
        e.close()
        return res, sch

    ra, sa = run(True)
    rb, sb = run(False)
    for i in range(len(prompts)):
        assert list(ra[i][0]) == list(rb[i][0]) and list(ra[i][1]) == list(rb[i][1])
    assert sorted(sa.logits) == sorted(sb.logits) and len(sa.logits) > 0
    for key in sa.logits:
        assert np.array_equal(np.asarray(sa.logits[key]), np.asarray(sb.logits[key])), key
    for key in sa.exit_states:
        assert np.array_equal(np.asarray(sa.exit_states[key]), np.asarray(sb.exit_states[key])), key


HUGINN_LOGIT_REASON = (
    "bf16 storage floor at hidden 5280: measured 6.87e-2 max logit error on the GPU (states 1.22e-2, within "
    "2e-2); the oracle itself, rounding only K/V and the GEMM inputs to bf16, moves the logits by 6.6e-2 "
    "(K/V alone 4.3e-2, QKV input alone 5.3e-2, LM-head input alone 1.1e-2), so no bf16-KV path meets 5e-2 "
    "at this width")


@pytest.mark.xfail(strict=True, raises=LogitBarExceeded, reason=HUGINN_LOGIT_REASON)
def test_bf16_huginn_width_prefill_injection(eng_mod):
    """Huginn-like widths (H 5280, 55 x 96 heads, F 17920) with one prelude,
    one core and one coda layer, r_max 3 and the prelude injection: a
    300-token prompt reaches the LDS-tiled GEMM (K = 5280 ends in a half
    k-tile) and the head-dim-96 MFMA prefill attention at full width.
    States, tokens and exits meet their bars; the logits miss 5e-2 (see the
    xfail reason), which this test records as an expected failure."""
    d = S.ModelDims("t", vocab=4096, hidden=5280, n_heads=55, head_dim=96, ffn=17920, n_prelude=1, n_core=1,
                    n_coda=1, r_max=3, dtype="bf16", inject=True, gate_bias=0.0)
    _bf16_replay_check(eng_mod, d, [300, 41], n_out=4, W=2, M=8192)


@pytest.mark.xfail(strict=True, raises=LogitBarExceeded, reason=(
    "bf16 storage floor at hidden 5280: measured 7.86e-2 max logit error on the GPU with states at 1.38e-2 "
    "(within 2e-2), tokens and exits equal to the oracle's; see HUGINN_LOGIT_REASON"))
def test_bf16_huginn_width_prefill_big_tiles_oracle(eng_mod):
    """Huginn-like widths (H 5280, 55 x 96 heads, F 17920), one core layer,
    r_max 2: a 2,400-token prompt (one 2,441-row prefill chunk with the
    41-token one) gives the QKV projection 10 x 62 and the gate/up
    projection 10 x 140 tiles of 256 x 256 with K = 5280, so both run on the
    256 x 256 GEMM with 32x32x16 MFMAs (the O and down projections have
    too few tiles and take the 128 x 128 kernel); against the oracle."""
    d = S.ModelDims("t", vocab=4096, hidden=5280, n_heads=55, head_dim=96, ffn=17920, n_prelude=0, n_core=1,
                    n_coda=0, r_max=2, dtype="bf16", gate_bias=0.0)
    _bf16_replay_check(eng_mod, d, [2400, 41], n_out=3, W=2, M=8192)


def test_bf16_huginn_width_prefill_big_tiles_match_tiled(eng_mod, monkeypatch):
    """Huginn-like widths with a 6,200-token prompt: the prefill chunk has
    enough rows for the 256 x 256 GEMM with 32x32x16 MFMAs (K >= 4096 and
    at least two workgroups per CU) in all four projections -- QKV (fp32
    store), O and down (residual add), gate/up (SwiGLU) -- with a ragged
    last row tile, and K = 5280 runs an odd number (165) of 32-wide k-tiles.
    The same run with that kernel switched off (CDB_TILE256=0: the 128 x 128
    kernel, parity-tested against the oracle above at this width) must give
    the same tokens, exits, logits and exit states bit for bit (the oracle's
    per-row attention loop is too slow for a prompt of this length)."""
    d = S.ModelDims("t", vocab=4096, hidden=5280, n_heads=55, head_dim=96, ffn=17920, n_prelude=1, n_core=1,
                    n_coda=1, r_max=3, dtype="bf16", inject=True, gate_bias=0.0)
    prompt_lens, n_out, W, M = [6200, 41], 3, 2, 8192
    w = S.make_weights(d, seed=0)
    prompts = S.make_prompts(d.vocab, prompt_lens, seed=1)
    mbps = max(prompt_lens) // 16 + n_out // 16 + 3

    def run(big):
        monkeypatch.setenv("CDB_TILE256", "1" if big else "0")
        _say(f"[case] Huginn-width prefill {prompt_lens}, 256 x 256 GEMM {'on' if big else 'off'}")
        dm = eng_mod.DeviceModel(d, w)
        e = eng_mod.Engine(dm, n_slots=W, max_rows=eng_mod.pow2(W), num_blocks=len(prompts) * mbps,
                           max_seqs=len(prompts), max_blocks_per_seq=mbps, max_out=n_out, max_prefill_tokens=M)
        sch = eng_mod.Scheduler(e, prompts, n_out, mode="refill", W=W, K=1, M=M, capture_states=True,
                                capture_logits=True).run()
        res = sch.results()
        e.close()
        return res, sch

    ra, sa = run(True)
    rb, sb = run(False)
    for i in range(len(prompts)):
        assert list(ra[i][0]) == list(rb[i][0]) and list(ra[i][1]) == list(rb[i][1])
    assert sorted(sa.logits) == sorted(sb.logits) and len(sa.logits) > 0
    for key in sa.logits:
        assert np.array_equal(np.asarray(sa.logits[key]), np.asarray(sb.logits[key])), key
    for key in sa.exit_states:
        assert np.array_equal(np.asarray(sa.exit_states[key]), np.asarray(sb.exit_states[key])), key


@pytest.mark.parametrize("hd", [128, 96])
def test_bf16_prefill_attention_128_row_tiles_oracle(eng_mod, monkeypatch, hd):
    """Prefill attention on 128-row query tiles (two groups of 16 queries per
    wave; CDB_PF_TILE_ROWS=128 forces them) in chunks that start past
    position 0 and end in ragged tiles, against the oracle."""
    monkeypatch.setenv("CDB_PF_TILE_ROWS", "128")
    d = S.ModelDims("t", vocab=512, hidden=256, n_heads=2, head_dim=hd, ffn=512, n_prelude=0, n_core=2,
                    n_coda=0, r_max=4, dtype="bf16", gate_bias=0.1)
    _bf16_replay_check(eng_mod, d, [150, 37, 300, 91], n_out=12, W=3, M=192)


@pytest.mark.parametrize("hd", [128, 96])
def test_bf16_prefill_attention_tile_rows_same_bits(eng_mod, monkeypatch, hd):
    """The same prompts prefilled on 64-row and on 128-row query tiles give
    bit for bit the same tokens, exits, logits and exit states: the tile size
    changes which queries share a workgroup, not the arithmetic per query."""
    d = S.ModelDims("t", vocab=512, hidden=384, n_heads=4, head_dim=hd, ffn=768, n_prelude=0, n_core=2,
                    n_coda=1, r_max=3, dtype="bf16", gate_bias=0.0)
    prompt_lens, n_out, W, M = [2300, 900, 41], 4, 3, 2048
    w = S.make_weights(d, seed=2)
    prompts = S.make_prompts(d.vocab, prompt_lens, seed=3)
    mbps = max(prompt_lens) // 16 + n_out // 16 + 3

    def run(rows):
        monkeypatch.setenv("CDB_PF_TILE_ROWS", rows)
        _say(f"[case] prefill tiles of {rows} rows, head_dim {hd}, prompts {prompt_lens}, M={M}")
        dm = eng_mod.DeviceModel(d, w)
        e = eng_mod.Engine(dm, n_slots=W, max_rows=eng_mod.pow2(W), num_blocks=len(prompts) * mbps,
                           max_seqs=len(prompts), max_blocks_per_seq=mbps, max_out=n_out, max_prefill_tokens=M)
        sch = eng_mod.Scheduler(e, prompts, n_out, mode="refill", W=W, K=1, M=M, capture_states=True,
                                capture_logits=True).run()
        res = sch.results()
        e.close()
        return res, sch

    ra, sa = run("128")
    rb, sb = run("64")
    for i in range(len(prompts)):
        assert list(ra[i][0]) == list(rb[i][0]) and list(ra[i][1]) == list(rb[i][1])
    assert sorted(sa.logits) == sorted(sb.logits) and len(sa.logits) > 0
    for key in sa.logits:
        assert np.array_equal(np.asarray(sa.logits[key]), np.asarray(sb.logits[key])), key
    for key in sa.exit_states:
        assert np.array_equal(np.asarray(sa.exit_states[key]), np.asarray(sb.exit_states[key])), key


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_pack_weight_layout(eng_mod, dtype):
    """cdb_pack_weight writes the documented fragment-packed layout: tiles of
    16 rows x KS columns in (row tile, column tile) order, piece l of a tile
    = row l % 16, columns (l // 16) * VEC .. + VEC."""
    import torch
    from continuous_depth_batching_amd import _lib as L
    _say(f"[case] pack_weight layout dtype={dtype}")
    ks, vec = (32, 8) if dtype == "bf16" else (16, 4)
    rows, cols = 48, 5 * ks
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    rng = np.random.default_rng(11)
    src_h = torch.from_numpy(rng.standard_normal((rows, cols)).astype(np.float32)).to(tdt)
    src = src_h.cuda()
    dst = torch.full_like(src, float("nan"))
    L.check(L.lib.cdb_pack_weight(L.CDB_BF16 if dtype == "bf16" else L.CDB_FP32, C.c_void_p(src.data_ptr()),
                                  C.c_void_p(dst.data_ptr()), rows, cols, None))
    torch.cuda.synchronize()
    got = dst.cpu().float().numpy().reshape(-1)
    want = (src_h.float().numpy().reshape(rows // 16, 16, cols // ks, ks // vec, vec)
            .transpose(0, 2, 3, 1, 4).reshape(-1))
    assert np.array_equal(got, want)
