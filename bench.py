"""Benchmark of the CDB decode hot path on one MI355X.

Workload: the Ouro-like fully looped model (vocab 49152, hidden 2048, 16
heads x 128, SwiGLU 5632, 24-layer core, r_max 4, bf16, seeded random
init), decode-only, every sequence at context 1024 with seeded per-position
exit depths 1-4 and non-contiguous KV blocks.  One step = one pass of the
whole decode hot path over a batch of B rows at mixed depths: slot gather,
the 24 core layers (RMSNorm, QKV / O / SwiGLU GEMMs, RoPE, depth-indexed
attention with K/V write), the lookahead gate with stream compaction, and
the boundary for the rows that left (depth-map write, final norm, LM head,
greedy argmax, successor prelude refilling the freed slots).  Sequences
never finish, so every step runs B rows.  Inputs are resident in HBM when
the timed region starts; the region holds no host synchronisation.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--batch B] [--context L]
                    [--sweep 1,2,4,...] [--no-cpu]

Prints one JSON line (metric, value, ..., roofline, cpu_baseline).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

# The oracle's CPU baseline runs on the host cores this process may use: its
# BLAS threads are pinned to that count before numpy is first imported.
HOST_CORES = len(os.sched_getaffinity(0))
for _v in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS"):
    os.environ[_v] = str(HOST_CORES)

import numpy as np  # noqa: E402

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_traffic_ouro_b64_ctx1024.txt")
ATTN_SRC = [os.path.join(ROOT, "continuous_depth_batching_amd", "csrc", f)
            for f in ("k_attn.hip", "attn_common.h", "common.h")]
CALIB_BYTES = 1 << 30          # plain copy of known size, profiled beside the kernels


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--batch", type=int, default=64)
    ap.add_argument("--context", type=int, default=1024)
    ap.add_argument("--sweep", type=str, default="")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-e2e", action="store_true",
                    help="skip the short end-to-end C2 segment (fixed depth vs refill, S_dec, S_e2e)")
    ap.add_argument("--points", type=str, default="1,16,256",
                    help="further batch sizes timed at --context beside the headline batch (graph step time and "
                         "fraction of the step bound each; empty to skip)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--sweep-contexts", type=str, default="",
                    help="contexts for the batch sweep (default: --context only); two or more fit Eq. 4")
    ap.add_argument("--e2e", action="store_true",
                    help="end-to-end run with prefill (default workload: 256 requests, prompts U{128..2048}, "
                         "256 outputs)")
    ap.add_argument("--workload", type=str, default="c2", choices=["c2", "c3", "c4"],
                    help="c2: Ouro-like, prompts U{128..2048}; c3: Huginn-like 2-4-2 (r_max 32, injection), "
                         "prompts U{256..1024}, 512 outputs, K = 16; c4: Ouro-like, log-normal prompts "
                         "(median 8192, 4096..16384)")
    ap.add_argument("--K", type=int, default=0, help="minimum coda batch (default: the workload's)")
    ap.add_argument("--gate", type=str, default="linear", choices=["linear", "convergence"],
                    help="exit gate of the end-to-end runs: the configuration's calibrated linear lookahead gate, "
                         "or the training-free convergence criterion with --conv-threshold")
    ap.add_argument("--conv-threshold", type=float, default=0.0)
    ap.add_argument("--k-sweep", type=str, default="",
                    help="end to end: fit the latency model (Eq. 3/4 stage costs) on the fixed-depth and no-refill "
                         "runs, predict refill at each of these K, then run them (first W of --slots)")
    ap.add_argument("--serve", action="store_true",
                    help="online serving (Section 6.3): Poisson arrivals at each --rates for --duration seconds, "
                         "normalized latency (end-to-end time / output tokens) per schedule")
    ap.add_argument("--rates", type=str, default="4,8,12,16")
    ap.add_argument("--duration", type=float, default=40.0)
    ap.add_argument("--samples-out", type=str, default="",
                    help="--k-sweep: write the stage samples and recorded exits the model was fitted on (JSON)")
    ap.add_argument("--slots", type=str, default="")
    ap.add_argument("--modes", type=str, default="fixed,norefill,refill")
    ap.add_argument("--layouts", type=str, default="depth")
    ap.add_argument("--kv-layout", type=str, default="depth", choices=["depth", "depth_copy", "single", "first_shared"],
                    help="KV layout of the decode step measurements (depth_copy: explicit last-exited copies)")
    ap.add_argument("--requests", type=int, default=0)
    ap.add_argument("--n-out", type=int, default=0)
    ap.add_argument("--max-blocks", type=int, default=20480)
    ap.add_argument("--sync-scheduler", action="store_true",
                    help="read back every core step before the next stage (no lookahead pipelining)")
    return ap.parse_args()


class DecodeBench:
    """Engine set up with synthetic cached context for B rows at context L."""

    def __init__(self, eng_mod, dm, dims, B, L, steps_total, seed=3, kv_layout=None):
        import torch
        self.torch = torch
        self.B, self.L = B, L
        R = dims.r_max
        mbps = (L + steps_total + 32) // 16 + 1
        self.mbps = mbps
        # When the depth-indexed cache of B rows does not fit in HBM (512 rows
        # at context 1024 need 413 GB), rows b and b + distinct share their KV
        # blocks: the traffic is the same, the contents are synthetic anyway.
        planes = {"single": 1, "first_shared": 2}.get(kv_layout or "depth", R)
        block_bytes = 2 * dims.n_core * planes * 16 * dims.qdim * 2
        free, _ = torch.cuda.mem_get_info()
        distinct = max(1, min(B, int((free - 24e9) // (mbps * block_bytes))))
        self.distinct = distinct
        nblk = distinct * mbps
        self.e = e = eng_mod.Engine(dm, n_slots=B, max_rows=eng_mod.pow2(B), num_blocks=nblk, max_seqs=B,
                                    max_blocks_per_seq=mbps, max_out=steps_total + 8, max_prefill_tokens=16,
                                    kv_fill=0.0, kv_layout=kv_layout)
        rng = np.random.default_rng(seed)
        perm = rng.permutation(nblk).astype(np.int32)
        e.btab.copy_(torch.from_numpy(np.concatenate([perm] * (-(-B // distinct)))[: B * mbps]))
        gen = torch.Generator(device="cuda").manual_seed(seed)
        # K/V everywhere bf16 N(0,1): one seeded 512 MiB random chunk, tiled
        step = 1 << 28
        chunk = torch.randn(step, generator=gen, device="cuda", dtype=torch.float32).to(e.core_k.dtype)
        for pool in (e.core_k, e.core_v):
            n = pool.numel()
            for s in range(0, n, step):
                m = min(step, n - s)
                pool[s:s + m].copy_(chunk[:m])
        del chunk
        import cdb_synth as S
        ex = S.make_context_exit_depths(nblk * 16, R, seed=seed + 1)
        emap = ex.reshape(nblk, 16).copy()
        bt = perm.reshape(distinct, mbps)
        for b in range(distinct):            # positions >= L: in flight / future
            for j in range(L, mbps * 16):
                emap[bt[b, j // 16], j % 16] = R
        e.emap.copy_(torch.from_numpy(emap.reshape(-1)))
        e.state.copy_(torch.randn((B, dims.hidden), generator=gen, device="cuda"))
        cap = e.max_rows
        desc = np.zeros(5 * cap + 1, dtype=np.int32)
        desc[0] = B
        desc[1:1 + B] = np.arange(B)
        desc[1 + cap:1 + cap + B] = np.arange(B)
        desc[1 + 2 * cap:1 + 2 * cap + B] = L
        desc[1 + 3 * cap:1 + 3 * cap + B] = S.c1_row_depths(B, R, seed=seed)
        desc[1 + 4 * cap:1 + 4 * cap + B] = R
        e.desc_t.copy_(torch.from_numpy(desc))
        e.q_t[0] = 0
        e.n_gen.fill_(1)
        e.n_out.fill_(steps_total + 8)
        self.rows = eng_mod.pow2(B)

    def step(self):
        e = self.e
        e.core_step(self.rows)
        e.gate_compact(self.rows, True)
        e.boundary(self.rows)

    def positions(self):
        cap = self.e.max_rows
        n = int(self.e.desc_t[0].item())
        return self.e.desc_t[1 + 2 * cap:1 + 2 * cap + n].cpu().numpy()

    def generated(self):
        return int(self.e.n_gen.sum().item())


def run_point(eng_mod, dm, dims, B, L, steps, warmup, profile=True, kv_layout=None):
    import torch
    from continuous_depth_batching_amd import _lib as LL
    import ctypes as C
    bench = DecodeBench(eng_mod, dm, dims, B, L, steps * 3 + warmup + 4, kv_layout=kv_layout)
    for _ in range(warmup):
        bench.step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    # eager launches (reference)
    t0.record()
    for _ in range(steps):
        bench.step()
    t1.record()
    torch.cuda.synchronize()
    ms_eager = t0.elapsed_time(t1)
    # one step captured as a HIP graph (fixed buffers, device-resident counts)
    graph = bench.e.capture(bench.step)
    bench.e.replay(graph)
    torch.cuda.synchronize()
    g0 = bench.generated()
    t0.record()
    for _ in range(steps):
        bench.e.replay(graph)
    t1.record()
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1)
    g1 = bench.generated()
    bench.e.drop(graph)
    res = dict(B=B, L=L, kv_rows_distinct=bench.distinct, ms_per_step=ms / steps, ms_per_step_eager=ms_eager / steps,
               core_token_steps_per_s=B * steps / (ms / 1e3),
               decoded_tokens_per_s=(g1 - g0) / (ms / 1e3))
    if profile:
        pos_a = bench.positions()
        LL.check(LL.lib.cdb_profile(bench.e.ctx, 1))
        for _ in range(steps):
            bench.step()
        LL.check(LL.lib.cdb_profile(bench.e.ctx, 0))
        pos_b = bench.positions()
        prof = {}
        for cls in ("attn", "gemm_qkv", "gemm_o", "gemm_gu", "gemm_down", "lm_head", "norm", "gate", "boundary"):
            tot, cnt = C.c_double(), C.c_int64()
            LL.check(LL.lib.cdb_profile_read(bench.e.ctx, cls.encode(), C.byref(tot), C.byref(cnt)))
            prof[cls] = dict(total_ms=tot.value, launches=cnt.value,
                             avg_us=(1e3 * tot.value / cnt.value) if cnt.value else None)
        res["profile"] = prof
        res["mean_context"] = float((pos_a.mean() + pos_b.mean()) / 2.0)
    bench.e.close()
    del bench
    torch.cuda.empty_cache()
    return res


def source_sha(paths):
    import hashlib
    h = hashlib.sha256()
    for path in paths:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary, or None when it is absent or was taken on other kernel source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    with open(TRAFFIC_FILE) as f:
        for line in f:
            if "=" in line and not line.lstrip().startswith("#"):
                k, v = line.split("=", 1)
                kv[k.strip()] = v.strip()
    if kv.get("k_attn_source_sha256_16") != source_sha(ATTN_SRC):
        return None
    try:
        return int(float(kv["hbm_bytes_per_launch"]))
    except (KeyError, ValueError):
        return None


def calibration_copy():
    """Plain device copies of CALIB_BYTES (read + write): the first lets a
    counter run scale FETCH_SIZE / WRITE_SIZE against known bytes; the next
    ones, timed with events, give the HBM rate this device reaches on a
    copy, reported beside the datasheet peak.  Returns GB/s (bytes read +
    written per second, best of the timed copies)."""
    import torch
    a = torch.ones(CALIB_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(5):
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0.record()
        b.copy_(a)
        t1.record()
        torch.cuda.synchronize()
        best = max(best, 2.0 * CALIB_BYTES / (t0.elapsed_time(t1) * 1e-3) / 1e9)
    del a, b
    torch.cuda.empty_cache()
    return best


def device_peaks():
    """Compute units and peak engine clock from the HIP runtime, and the dense
    bf16 matrix peak they imply (CDNA4: 2048 bf16 multiply-adds, 4096 flops,
    per compute unit per clock -- the datasheet's 2.5 PFLOP/s at 256 CUs and
    2.4 GHz)."""
    import ctypes as C
    try:
        hip = C.CDLL("libamdhip64.so")
        dev = C.c_int()
        hip.hipGetDevice(C.byref(dev))
        cu, clk = C.c_int(), C.c_int()
        hip.hipDeviceGetAttribute(C.byref(cu), 63, dev)      # hipDeviceAttributeMultiprocessorCount
        hip.hipDeviceGetAttribute(C.byref(clk), 5, dev)      # hipDeviceAttributeClockRate (kHz)
        return dict(compute_units=cu.value, clock_mhz=clk.value / 1e3,
                    bf16_dense_tflops=round(cu.value * clk.value * 1e3 * 4096 / 1e12, 1))
    except Exception as ex:                                  # reported, not fatal
        return dict(error=str(ex))


def latency_fit(points):
    """Least-squares fit of the pages' step-latency model at context L,
    t(B) = delta + (gamma + alpha_kv L) B (Eq. 4), on the measured graph
    step times, and the saturation batch B* = delta / (gamma + alpha_kv L)
    at each swept context.  With a single context only delta and the slope
    gamma + alpha_kv L are identifiable."""
    B = np.array([p["B"] for p in points], dtype=np.float64)
    L = np.array([p["L"] for p in points], dtype=np.float64)
    t = np.array([p["ms_per_step"] * 1e3 for p in points], dtype=np.float64)   # us
    ctxs = sorted(set(L.tolist()))
    if len(ctxs) >= 2:
        A = np.stack([np.ones_like(B), B, B * L], axis=1)
        (delta, gamma, alpha), *_ = np.linalg.lstsq(A, t, rcond=None)
        slopes = {int(c): gamma + alpha * c for c in ctxs}
        out = {"delta_us": round(float(delta), 2), "gamma_us_per_row": round(float(gamma), 4),
               "alpha_kv_us_per_row_per_position": float(alpha)}
    else:
        A = np.stack([np.ones_like(B), B], axis=1)
        (delta, slope), *_ = np.linalg.lstsq(A, t, rcond=None)
        slopes = {int(ctxs[0]): slope}
        out = {"delta_us": round(float(delta), 2)}
    pred = A @ np.linalg.lstsq(A, t, rcond=None)[0]
    out["r2"] = round(float(1.0 - ((t - pred) ** 2).sum() / ((t - t.mean()) ** 2).sum()), 5)
    out["slope_us_per_row"] = {str(c): round(float(v), 3) for c, v in slopes.items()}
    out["saturation_batch"] = {str(c): round(float(delta / v), 2) for c, v in slopes.items()}
    return out


def step_bound_us(dims, B, L):
    """Roofline step time: core weights once + per-row KV traffic at HBM peak,
    GEMM flops at the bf16 MFMA peak (the larger of the two per GEMM)."""
    H, Q, F, n = dims.hidden, dims.qdim, dims.ffn, dims.n_core
    wbytes = 2 * n * (3 * Q * H + H * Q + 2 * F * H + H * F)
    kv = B * n * (2 * Q * 2) * (L + 1)
    flops = 2 * B * wbytes / 2
    return max(wbytes / (HBM_PEAK_GBS * 1e3), flops / (BF16_PEAK_TFLOPS * 1e6)) + kv / (HBM_PEAK_GBS * 1e3)


def cpu_baseline(dims, w, L, budget_s=15.0, max_rows=2048, seed=5):
    """The oracle's single-row core step at the bench's context, timed on the
    host cores on a bounded sample: rows at depths 1..r_max over one synthetic
    cached context, run until about budget_s seconds of oracle time.  BLAS
    runs with one thread per core of this process's affinity mask (set
    before numpy was imported)."""
    from oracle.model import OracleLM, cache_from_planes
    blas_threads = None
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        pass
    import cdb_synth as S
    m = OracleLM(dims, w, dtype=np.float32)
    rng = np.random.default_rng(seed)
    R = dims.r_max
    kb = rng.standard_normal((dims.n_core, R, L, dims.n_heads, dims.head_dim), dtype=np.float32)
    vb = rng.standard_normal((dims.n_core, R, L, dims.n_heads, dims.head_dim), dtype=np.float32)
    ex = S.make_context_exit_depths(L, R, seed=seed)
    cache = cache_from_planes(dims, kb, vb, ex, dtype=np.float32)
    del kb, vb
    total, rows = 0.0, 0
    while total < budget_s and rows < max_rows:
        h = rng.standard_normal(dims.hidden).astype(np.float32)
        t0 = time.perf_counter()
        m.core_step_row(h, L, 1 + rows % R, cache)
        total += time.perf_counter() - t0
        rows += 1
    return dict(value=rows / total, unit="core token-steps/s", cores=HOST_CORES, blas_threads=blas_threads,
                kind="oracle",
                sample=f"{rows} single-row core steps (24 layers, fp32 numpy) at context {L}, depths 1..{R}; "
                       f"{total:.1f} s of oracle time")


def e2e_bounds(dims, lengths, exits, log, R):
    """FLOP bound of Eq. 1 summed per decode token, and the sum-of-stages
    roofline time of a run.

    Eq. 1 (per token t): F0 = 2 H V (coda LM head; the prelude of a fully
    looped model is an embedding gather), F_r(t) = 2 * core parameters +
    4 * n_L * nh * hd * (L_t + 1) (attention over the L_t earlier positions
    and itself).  Stage roofline: each core step max(weight bytes / BW, GEMM
    flops / P) plus its KV bytes / BW; each coda max(LM head bytes / BW,
    flops / P); each prefill chunk r_max * its GEMM and attention flops / P."""
    H, Q, F, V, n = dims.hidden, dims.qdim, dims.ffn, dims.vocab, dims.n_core
    lp = 3 * Q * H + H * Q + 2 * F * H + H * F   # parameters of one transformer layer
    nb = dims.n_prelude + dims.n_coda            # boundary (prelude + coda) layers
    params = n * lp
    attn_row = 4.0 * n * Q                       # flops per attended position per loop
    kv_row = 2.0 * n * 2 * Q                     # K+V bytes per position per loop (bf16)
    fix = ada = 0.0
    kv_bytes = 0.0
    for P, ex in zip(lengths, exits):
        for g, d in enumerate(ex):               # pass g+1 has P + g earlier positions
            Lt = P + g
            F0 = 2.0 * H * V + 2.0 * nb * lp + 4.0 * nb * Q * (Lt + 1)
            Fr = 2.0 * params + attn_row * (Lt + 1)
            fix += F0 + R * Fr
            ada += F0 + d * Fr
            kv_bytes += d * kv_row * (Lt + 1) + nb * 2 * 2 * Q * (Lt + 1)
    bw, pk = HBM_PEAK_GBS * 1e9, BF16_PEAK_TFLOPS * 1e12
    t = kv_bytes / bw
    bnd_w = 2.0 * (H * V + nb * lp)               # LM head + boundary layers, bf16
    for st in log:
        if st.kind == "loop":
            t += max(2.0 * params / bw, 2.0 * params * st.B / pk)
        elif st.kind == "coda":
            t += max(bnd_w / bw, bnd_w * st.B / pk)
    pf = 0.0
    for P in lengths:
        pf += (R * n + nb) * (2.0 * lp * P + 4.0 * Q * P * (P + 1) / 2.0) + 2.0 * H * V
    t += pf / pk
    return fix / ada, t


def prefill_profile(eng, eng_mod, dims, prompts, max_tokens=16384):
    """Kernel-class times of prefill alone (chunks of <= 8192 tokens at full
    depth, first token from the coda), with the prefill GEMMs' achieved
    TFLOP/s against the bf16 MFMA peak."""
    from continuous_depth_batching_amd import _lib as LL
    import ctypes as C
    import torch
    sel, tot = [], 0
    for p in prompts:
        if tot + len(p) > max_tokens:
            break
        sel.append(p)
        tot += len(p)
    LL.check(LL.lib.cdb_profile(eng.ctx, 1))
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    eng_mod.Scheduler(eng, sel, 1, mode="fixed", W=min(len(sel), eng.n_slots), M=8192).run()
    wall = time.perf_counter() - t0
    LL.check(LL.lib.cdb_profile(eng.ctx, 0))
    out = {"tokens": tot, "requests": len(sel), "wall_s": round(wall, 4)}
    for cls in ("prefill_gemm", "prefill_attn", "norm", "lm_head", "boundary", "other"):
        ms, cnt = C.c_double(), C.c_int64()
        LL.check(LL.lib.cdb_profile_read(eng.ctx, cls.encode(), C.byref(ms), C.byref(cnt)))
        out[cls + "_ms"] = round(ms.value, 3)
    H, Q, F = dims.hidden, dims.qdim, dims.ffn
    lp = 3 * Q * H + H * Q + 2 * F * H + H * F
    gemm_flops = 2.0 * lp * tot * (dims.n_core * dims.r_max + dims.n_prelude + dims.n_coda)
    if out["prefill_gemm_ms"] > 0:
        tf = gemm_flops / (out["prefill_gemm_ms"] * 1e-3) / 1e12
        out["prefill_gemm_tflops"] = round(tf, 1)
        out["prefill_gemm_mfma_frac"] = round(tf / BF16_PEAK_TFLOPS, 4)
    out["prefill_tokens_per_s"] = round(tot / wall, 1)
    return out


def e2e_engine(eng_mod, dm, dims, layout, lengths, n_out, Wmax, max_blocks, n_req):
    import torch
    planes = {"depth": dims.r_max, "single": 1, "first_shared": 2, "depth_copy": dims.r_max}[layout]
    mbps = -(-(int(lengths.max()) + n_out) // 16)
    block_bytes = 2 * (dims.n_core * planes + dims.n_prelude + dims.n_coda) * 16 * dims.qdim * 2
    free, _ = torch.cuda.mem_get_info()
    fit = int((free - 16e9) // block_bytes)
    nblk = max(min(max_blocks, fit), mbps)
    log(f"e2e engine: layout {layout}, KV blocks {nblk} ({nblk * block_bytes / 1e9:.1f} GB), W <= {Wmax}")
    eng = eng_mod.Engine(dm, n_slots=Wmax, max_rows=eng_mod.pow2(Wmax), num_blocks=nblk, max_seqs=n_req,
                         max_blocks_per_seq=mbps, max_out=n_out, max_prefill_tokens=8192, kv_fill=0.0,
                         kv_layout=layout)
    return eng, nblk


def run_e2e(a, eng_mod, dm, dims):
    import torch
    import cdb_synth as S
    R = dims.r_max
    base = S.WORKLOADS[a.workload]
    slots = tuple(int(x) for x in a.slots.split(",")) if a.slots else base.slots
    wl = S.Workload(**{**base.__dict__, "n_requests": a.requests or base.n_requests,
                       "n_out": a.n_out or base.n_out, "slots": slots})
    a.K = a.K or wl.min_coda_batch
    lengths = S.make_prompt_lengths(wl, seed=1)
    prompts = S.make_prompts(dims.vocab, lengths, seed=1)
    n_out = wl.n_out
    log(f"e2e {a.workload}: {len(prompts)} requests, prompts {int(lengths.min())}..{int(lengths.max())} "
        f"(mean {lengths.mean():.0f}), n_out {n_out}, slots {slots}")
    runs, pf_prof = [], None
    for layout in a.layouts.split(","):
        eng, nblk = e2e_engine(eng_mod, dm, dims, layout, lengths, n_out, max(slots), a.max_blocks, len(prompts))
        # warm-up: load every kernel once
        wp = [p[:64] for p in prompts[:8]]
        for mode in ("fixed", "refill"):
            eng_mod.Scheduler(eng, wp, 6, mode=mode, W=8, M=8192, graphs=True).run()
        if pf_prof is None:
            pf_prof = prefill_profile(eng, eng_mod, dims, prompts)
            log(json.dumps({"prefill_profile": pf_prof}))
        runs += e2e_layout_runs(a, eng, eng_mod, dims, lengths, prompts, n_out, slots, layout, nblk)
        eng.close()
        del eng
        torch.cuda.empty_cache()
    return runs, dict(workload=a.workload, K=a.K, requests=len(prompts), prompt_min=int(lengths.min()),
                      prompt_max=int(lengths.max()), prompt_mean=float(lengths.mean()), n_out=n_out), pf_prof


def e2e_layout_runs(a, eng, eng_mod, dims, lengths, prompts, n_out, slots, layout, nblk):
    R = dims.r_max
    runs = []
    for W in slots:
        per_mode = {}
        for mode in a.modes.split(","):
            # "<mode>_gateoff": the mode's stage policy with the gate off (full depth)
            base, gate = (mode[:-len("_gateoff")], False) if mode.endswith("_gateoff") else (mode, True)
            if a.sync_scheduler:
                sch = eng_mod.Scheduler(eng, prompts, n_out, mode=base, W=W, K=a.K, M=8192, timing=True, graphs=True,
                                        gate=gate)
            else:
                sch = eng_mod.AsyncScheduler(eng, prompts, n_out, mode=base, W=W, K=a.K, M=8192, gate=gate)
            sch.progress = lambda done, steps: log(f"  {mode} W={W}: {done}/{len(prompts)} requests finished, "
                                                   f"{steps} core steps")
            sch.run()
            res = sch.results()
            exits = [ex for _, ex in res]
            n_dec = sum(len(t) for t, _ in res)
            dbar = float(np.mean(np.concatenate([np.asarray(e, dtype=np.float64) for e in exits])))
            sdec, t_bound = e2e_bounds(dims, lengths, exits, sch.log, R)
            r = dict(mode=mode, W=W, layout=layout, kv_blocks=nblk, scheduler="sync" if a.sync_scheduler else "lookahead",
                     wall_s=round(sch.t_total, 3), decoded_tokens=n_dec,
                     decoded_tokens_per_s=round(n_dec / sch.t_total, 1),
                     core_token_steps=sch.core_token_steps, core_steps=sch.core_steps,
                     core_token_steps_per_s=round(sch.core_token_steps / sch.t_core, 1) if sch.t_core else None,
                     mean_core_batch=round(sch.core_token_steps / max(sch.core_steps, 1), 2),
                     prefill_s=round(sch.t_prefill, 3), core_s=round(sch.t_core, 3), coda_s=round(sch.t_coda, 3),
                     prefill_share=round(sch.t_prefill / sch.t_total, 4), mean_exit=round(dbar, 4),
                     s_dec_flops=round(sdec, 4), stage_bound_s=round(t_bound, 3),
                     frac_of_stage_bound=round(t_bound / sch.t_total, 4))
            per_mode[mode] = (r, res)
            runs.append(r)
            log(json.dumps(r))
        if "fixed" in per_mode:
            fx = per_mode["fixed"][0]
            alpha = fx["prefill_share"]
            for mode in ("refill", "norefill"):
                if mode not in per_mode:
                    continue
                r, res = per_mode[mode]
                sdec = r["s_dec_flops"]
                se2e = 1.0 / (alpha + (1.0 - alpha) / sdec)
                r["speedup_vs_fixed"] = round(fx["wall_s"] / r["wall_s"], 4)
                r["s_e2e_bound"] = round(se2e, 4)
                r["frac_of_s_e2e"] = round(r["speedup_vs_fixed"] / se2e, 4)
                r["alpha_pf_fixed"] = alpha
            # CDB at full depth against fixed-depth CB (§6.2: 95-99% of CB's throughput)
            for mode in ("refill_gateoff", "norefill_gateoff"):
                if mode in per_mode:
                    per_mode[mode][0]["throughput_vs_fixed"] = round(fx["wall_s"] / per_mode[mode][0]["wall_s"], 4)
        if "refill" in per_mode and "norefill" in per_mode:
            a_res, b_res = per_mode["refill"][1], per_mode["norefill"][1]
            same = sum(1 for x, y in zip(a_res, b_res) if x == y)
            per_mode["refill"][0]["identical_requests_vs_norefill"] = f"{same}/{len(a_res)}"
        log(json.dumps({"W": W, "layout": layout,
                        "summary": {m: {k: v for k, v in per_mode[m][0].items()
                                        if k in ("wall_s", "speedup_vs_fixed", "s_e2e_bound", "frac_of_s_e2e")}
                                    for m in per_mode}}))
    return runs


def cdb_e2e_segment(eng_mod, dm, dims, n_requests=128, n_out=64, W=64, max_blocks=9000):
    """A short end-to-end run of the Ouro-like model on the C2 prompt mix
    (prompt lengths U{128..2048}, the first n_requests of the workload's
    seeded requests, n_out tokens each, W slots, K = 1, chunks of <= 8192
    tokens): fixed-depth continuous batching against CDB refill (Alg. 2)
    with the lookahead scheduler, refill once more with the synchronous
    scheduler (every core step read back before the next stage), and refill
    with the gate off (full depth: CDB's own overhead against fixed-depth
    CB, §6.2).  Reports the realised speedup, the FLOP bound of Eq. 1 summed
    per token (S_dec), the prefill-corrected bound of Eq. 2 (S_e2e, alpha =
    the fixed-depth run's prefill share of GPU time) and realised / S_e2e,
    the full-depth throughput relative to fixed depth, and the GPU idle
    fraction of each schedule (share of the stage span with no stage on the
    GPU)."""
    import torch
    import cdb_synth as S
    R = dims.r_max
    lengths = S.make_prompt_lengths(S.WORKLOADS["c2"], seed=1)[:n_requests]
    prompts = S.make_prompts(dims.vocab, S.make_prompt_lengths(S.WORKLOADS["c2"], seed=1), seed=1)[:n_requests]
    eng, nblk = e2e_engine(eng_mod, dm, dims, "depth", lengths, n_out, W, max_blocks, len(prompts))
    wp = [p[:64] for p in prompts[:8]]
    for mode in ("fixed", "refill"):
        eng_mod.Scheduler(eng, wp, 6, mode=mode, W=8, M=8192, graphs=True).run()
    out = dict(workload=f"ouro-like c2 prompt mix, first {len(prompts)} requests, prompts "
                        f"{int(lengths.min())}..{int(lengths.max())}, {n_out} outputs, W={W}, K=1",
               requests=len(prompts), n_out=n_out, W=W, kv_blocks=nblk)
    runs = {}
    for name, mode, sync, gate in (("fixed", "fixed", False, True), ("refill", "refill", False, True),
                                   ("refill_sync", "refill", True, True), ("refill_gateoff", "refill", False, False)):
        if sync:
            sch = eng_mod.Scheduler(eng, prompts, n_out, mode=mode, W=W, K=1, M=8192, graphs=True, events=True,
                                    gate=gate)
        else:
            sch = eng_mod.AsyncScheduler(eng, prompts, n_out, mode=mode, W=W, K=1, M=8192, gate=gate)
        sch.run()
        res = sch.results()
        exits = [ex for _, ex in res]
        n_dec = sum(len(t) for t, _ in res)
        sdec, t_bound = e2e_bounds(dims, lengths, exits, sch.log, R)
        busy = sum(a_.elapsed_time(b_) for _, a_, b_ in sch._evs) / 1e3
        pf = sum(a_.elapsed_time(b_) for k_, a_, b_ in sch._evs if k_ == "prefill") / 1e3
        runs[name] = dict(wall_s=round(sch.t_total, 4), decoded_tokens_per_s=round(n_dec / sch.t_total, 1),
                          core_token_steps=sch.core_token_steps, mean_exit=round(float(np.mean(np.concatenate(
                              [np.asarray(e_, np.float64) for e_ in exits]))), 4),
                          prefill_share=round(pf / busy, 4) if busy else None, s_dec=round(sdec, 4),
                          gpu_idle_fraction=round(sch.gpu_idle_fraction(), 4))
        log(json.dumps({"cdb_e2e": name, **runs[name]}))
    fx, rf = runs["fixed"], runs["refill"]
    alpha = fx["prefill_share"]
    sdec = rf["s_dec"]
    se2e = 1.0 / (alpha + (1.0 - alpha) / sdec)
    speed = fx["wall_s"] / rf["wall_s"]
    out.update(runs=runs, speedup_refill_vs_fixed=round(speed, 4), s_dec=sdec, alpha_pf_fixed=alpha,
               s_e2e=round(se2e, 4), frac_of_s_e2e=round(speed / se2e, 4),
               speedup_refill_sync_vs_fixed=round(fx["wall_s"] / runs["refill_sync"]["wall_s"], 4),
               full_depth_refill_vs_fixed=round(fx["wall_s"] / runs["refill_gateoff"]["wall_s"], 4))
    eng.close()
    del eng
    torch.cuda.empty_cache()
    return out


def run_k_sweep(a, eng_mod, dm, dims):
    """Latency-model-driven choice of K and of refill vs no-refill: fit the
    core-step and boundary-stage costs on the fixed-depth and no-refill
    runs, predict the decode rate of refill at every K, then measure them."""
    import torch
    import cdb_synth as S
    from continuous_depth_batching_amd import planner as PL
    R = dims.r_max
    base = S.WORKLOADS[a.workload]
    slots = tuple(int(x) for x in a.slots.split(",")) if a.slots else base.slots
    W = slots[0]
    wl = S.Workload(**{**base.__dict__, "n_requests": a.requests or base.n_requests,
                       "n_out": a.n_out or base.n_out, "slots": (W,)})
    lengths = S.make_prompt_lengths(wl, seed=1)
    prompts = S.make_prompts(dims.vocab, lengths, seed=1)
    n_out = wl.n_out
    Ks = [int(x) for x in a.k_sweep.split(",") if x]
    layout = a.layouts.split(",")[0]
    eng, nblk = e2e_engine(eng_mod, dm, dims, layout, lengths, n_out, W, a.max_blocks, len(prompts))
    wp = [p[:64] for p in prompts[:8]]
    for mode in ("fixed", "refill"):
        eng_mod.Scheduler(eng, wp, 6, mode=mode, W=8, M=8192, graphs=True).run()
    n_dec = len(prompts) * (n_out - 1)
    stage_seqs = {}

    def measure(mode, K):
        sch = eng_mod.AsyncScheduler(eng, prompts, n_out, mode=mode, W=W, K=K, M=8192)
        sch.progress = lambda done, steps: log(f"  {mode} K={K}: {done}/{len(prompts)} requests finished, "
                                               f"{steps} core steps")
        sch.run()
        per_req = [ex for _, ex in sch.results()]
        stage_seqs[f"{mode}_K{K}"] = [[st.kind, st.B] for st in sch.log]
        exits = [e for ex in per_req for e in ex]
        r = dict(mode=mode, K=K, wall_s=round(sch.t_total, 3), core_s=round(sch.t_core, 3),
                 coda_s=round(sch.t_coda, 3), prefill_s=round(sch.t_prefill, 3),
                 decode_rate=round(n_dec / (sch.t_core + sch.t_coda), 1),
                 decoded_tokens_per_s=round(len(prompts) * n_out / sch.t_total, 1),
                 mean_core_batch=round(sch.core_token_steps / max(sch.core_steps, 1), 2),
                 mean_exit=round(float(np.mean(exits)), 3))
        log(json.dumps(r))
        return r, sch, per_req

    fixed, s_fix, _ = measure("fixed", 1)
    noref, s_nor, ex_nor = measure("norefill", 1)
    # fixed depth and no-refill run every coda on a whole cohort; a short
    # refill calibration (the first W requests, 32 outputs, K = 1) adds
    # boundary stages of every size
    cal = eng_mod.AsyncScheduler(eng, prompts[:W], min(n_out, 32), mode="refill", W=W, K=1, M=8192).run()
    core = [(B, t) for s in (s_fix, s_nor, cal) for kind, B, t in s.samples if kind == "core"]
    bnd = [(B, t) for s in (s_fix, s_nor, cal) for kind, B, t in s.samples if kind == "coda"]
    m = PL.fit_stage_model(core, bnd, buckets=True)
    pmf = PL.exit_pmf([e for ex in ex_nor for e in ex], R)
    pred_mf = PL.predict(m, W, R, pmf, Ks)
    # the no-refill run's exits, replayed per request (the pages' recorded-exit replay, App. C.2)
    pred = PL.simulate_all(m, W, R, pmf, Ks, len(prompts), n_out, exits=ex_nor)
    best_pred = PL.recommend(pred)
    log(json.dumps({"stage_model": m.__dict__, "simulated_decode_rate": pred, "mean_field_decode_rate": pred_mf,
                    "recommended": best_pred}))
    if a.samples_out:
        with open(a.samples_out, "w") as f:
            json.dump({"core": core, "boundary": bnd, "exits": ex_nor, "W": W, "r_max": R, "Ks": Ks,
                       "n_req": len(prompts), "n_out": n_out}, f)
    runs = {"fixed": fixed, "norefill": noref}
    for K in Ks:
        runs[f"refill_K{K}"] = measure("refill", K)[0]
    if a.samples_out:
        with open(a.samples_out.replace(".json", "_stages.json"), "w") as f:
            json.dump(stage_seqs, f)
    eng.close()
    del eng
    torch.cuda.empty_cache()
    best_meas = max((k for k in runs if k != "fixed"), key=lambda k: runs[k]["decode_rate"])
    best_wall = max((k for k in runs if k != "fixed"), key=lambda k: runs[k]["decoded_tokens_per_s"])
    rows = [dict(schedule=k, predicted_decode_rate=round(pred[k], 1), mean_field_rate=round(pred_mf[k], 1),
                 **runs[k]) for k in runs]
    family = "Huginn-like" if dims.inject else "Ouro-like"
    print(json.dumps({
        "metric": f"decode rate by schedule ({family} bf16, workload {a.workload}, W = {W}): latency-model "
                  f"prediction vs measurement",
        "unit": "generated tokens/s over core + boundary stages", "n_gpus": 1, "data": "synthetic",
        "config": dict(workload=a.workload, W=W, layout=layout, requests=len(prompts), n_out=n_out,
                       gate=a.gate, Ks=Ks),
        "stage_model": {k: (float(v) if not isinstance(v, tuple) else v) for k, v in m.__dict__.items()},
        "exit_pmf": [round(float(x), 4) for x in pmf],
        "recommended": best_pred, "best_measured_decode_rate": best_meas, "best_measured_wall": best_wall,
        "runs": rows}), flush=True)


def run_serve(a, eng_mod, dm, dims):
    """Online serving: requests arrive by a Poisson process at rate lambda
    for a fixed window (§6.3); each schedule serves the same arrivals and
    reports normalized latency, end-to-end time / output tokens per request."""
    import torch
    import cdb_synth as S
    base = S.WORKLOADS[a.workload]
    W = int(a.slots.split(",")[0]) if a.slots else 64
    n_out = a.n_out or base.n_out
    rates = [float(x) for x in a.rates.split(",") if x]
    modes = a.modes.split(",")
    rng = np.random.default_rng(11)
    traces = {}
    for lam in rates:
        t, arr = 0.0, []
        while True:
            t += rng.exponential(1.0 / lam)
            if t > a.duration:
                break
            arr.append(t)
        wl = S.Workload(**{**base.__dict__, "n_requests": len(arr), "n_out": n_out})
        lengths = S.make_prompt_lengths(wl, seed=int(lam * 1000) + 1)
        traces[lam] = (np.array(arr), lengths, S.make_prompts(dims.vocab, lengths, seed=int(lam * 1000) + 1))
    n_max = max(len(v[0]) for v in traces.values())
    all_len = np.concatenate([v[1] for v in traces.values()])
    eng, nblk = e2e_engine(eng_mod, dm, dims, a.layouts.split(",")[0], all_len, n_out, W, a.max_blocks, n_max)
    wp = [p[:64] for p in traces[rates[0]][2][:8]]
    for mode in ("fixed", "refill"):
        eng_mod.Scheduler(eng, wp, 6, mode=mode, W=8, M=8192, graphs=True).run()
    runs = []
    for lam in rates:
        arr, lengths, prompts = traces[lam]
        for mode in modes:
            sch = eng_mod.AsyncScheduler(eng, prompts, n_out, mode=mode, W=W, K=a.K or base.min_coda_batch, M=8192,
                                         arrivals=arr)
            sch.progress = lambda done, steps: log(f"  rate {lam} {mode}: {done}/{len(prompts)} finished")
            sch.run()
            nl = np.array(list(sch.normalized_latency().values()))
            r = dict(rate=lam, mode=mode, requests=len(prompts), wall_s=round(sch.t_total, 3),
                     norm_latency_mean_ms=round(1e3 * float(nl.mean()), 2),
                     norm_latency_p50_ms=round(1e3 * float(np.median(nl)), 2),
                     norm_latency_p90_ms=round(1e3 * float(np.percentile(nl, 90)), 2),
                     decoded_tokens_per_s=round(len(prompts) * n_out / sch.t_total, 1))
            log(json.dumps(r))
            runs.append(r)
    eng.close()
    del eng
    torch.cuda.empty_cache()
    family = "Huginn-like" if dims.inject else "Ouro-like"
    print(json.dumps({
        "metric": f"normalized latency under Poisson arrivals ({family} bf16, workload {a.workload}, W = {W})",
        "unit": "ms per output token (end-to-end time / output tokens)", "higher_is_better": False,
        "n_gpus": 1, "data": "synthetic",
        "config": dict(workload=a.workload, W=W, n_out=n_out, duration_s=a.duration, rates_per_s=rates,
                       K=a.K or base.min_coda_batch),
        "runs": runs}), flush=True)


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1 (no multi-GPU path)"}))
        sys.exit(2)
    import torch
    import cdb_synth as S
    from continuous_depth_batching_amd import engine as eng_mod
    dims = S.CONFIGS["c3" if ((a.e2e or a.serve) and a.workload == "c3") else "c1"]
    if (a.e2e or a.serve) and a.gate == "convergence":
        dims = dims.with_(gate_kind="convergence", conv_threshold=a.conv_threshold)
    t0 = time.time()
    w = S.make_weights(dims, seed=a.seed)
    log(f"weights generated in {time.time() - t0:.1f} s")
    dm = eng_mod.DeviceModel(dims, w)
    torch.cuda.synchronize()
    log(f"weights on device after {time.time() - t0:.1f} s")
    if a.serve:
        run_serve(a, eng_mod, dm, dims)
        return
    if a.e2e and a.k_sweep:
        run_k_sweep(a, eng_mod, dm, dims)
        return
    if a.e2e:
        runs, wl, pf_prof = run_e2e(a, eng_mod, dm, dims)
        best = max((r for r in runs if r["mode"] in ("refill", "norefill")), key=lambda r: r["decoded_tokens_per_s"],
                   default=runs[-1])
        family = "Huginn-like" if dims.inject else "Ouro-like"
        shape = (f"{family.lower()} {dims.n_prelude}-{dims.n_core}-{dims.n_coda} r_max {dims.r_max}"
                 + (" with prelude injection" if dims.inject else ""))
        print(json.dumps({
            "metric": f"decoded tokens/s ({family} bf16, end to end with prefill, workload {a.workload})",
            "value": best["decoded_tokens_per_s"], "unit": "decoded tokens/s", "n_gpus": 1,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic",
            "config": {**wl, "workload_id": wl["workload"], "gate": a.gate,
                       "conv_threshold": a.conv_threshold if a.gate == "convergence" else None,
                       "workload": f"{shape}, end to end: prefill chunks of <= 8192 tokens, "
                                   f"decode until every request has its outputs (K = {a.K})"},
            "best": {k: best[k] for k in ("mode", "W")}, "prefill_profile": pf_prof, "runs": runs}), flush=True)
        return
    copy_gbs = calibration_copy()
    peaks = device_peaks()
    log(json.dumps({"copy_gbs": round(copy_gbs, 1), "device": peaks, "host_cores": HOST_CORES}))
    main_pt = run_point(eng_mod, dm, dims, a.batch, a.context, a.steps, a.warmup, profile=True, kv_layout=a.kv_layout)
    log(json.dumps(main_pt))
    sweep = []
    fit = None
    if a.sweep:
        ctxs = [int(x) for x in a.sweep_contexts.split(",") if x] or [a.context]
        for L in ctxs:
            for B in [int(x) for x in a.sweep.split(",") if x]:
                pt = run_point(eng_mod, dm, dims, B, L, a.steps, a.warmup, profile=True, kv_layout=a.kv_layout)
                pt["bound_us"] = step_bound_us(dims, B, L)
                pt["frac_of_step_bound"] = pt["bound_us"] / (pt["ms_per_step"] * 1e3)
                log(json.dumps({k: v for k, v in pt.items() if k != "profile"}))
                sweep.append(pt)
        fit = latency_fit(sweep)
        log(json.dumps({"latency_fit": fit}))
    # dominant kernel: depth-indexed attention (KV streaming) at B >= ~12, else the weight GEMMs
    B, L = a.batch, main_pt["mean_context"]
    prof = main_pt["profile"]
    Q = dims.qdim
    attn_bytes = B * (2 * Q * 2 * (L + 1) + L)            # K+V read at one plane per position, K/V write, depth map
    attn_avg_s = prof["attn"]["avg_us"] * 1e-6
    gemm_bytes = {"gemm_qkv": 2 * 3 * Q * dims.hidden, "gemm_o": 2 * dims.hidden * Q,
                  "gemm_gu": 2 * 2 * dims.ffn * dims.hidden, "gemm_down": 2 * dims.hidden * dims.ffn}
    kernels = {"attn": dict(bytes=attn_bytes, avg_us=prof["attn"]["avg_us"])}
    for k, by in gemm_bytes.items():
        kernels[k] = dict(bytes=by, avg_us=prof[k]["avg_us"],
                          gbs=by / (prof[k]["avg_us"] * 1e-6) / 1e9 if prof[k]["avg_us"] else None)
    step_time_kernels = {k: prof[k]["total_ms"] for k in prof}
    dom = max(step_time_kernels, key=lambda k: step_time_kernels[k])
    achieved = attn_bytes / attn_avg_s / 1e9
    roof = {"bound": "hbm", "kernel": "attn (depth-indexed decode attention)", "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
            "peak_measured_copy": round(copy_gbs, 1), "frac_of_measured_copy": round(achieved / copy_gbs, 4),
            "traffic": measured_traffic() if (B == 64 and a.context == 1024) else None,
            "bytes_per_launch": int(attn_bytes), "avg_launch_us": round(prof["attn"]["avg_us"], 2),
            "dominant_by_time": dom}
    points = []
    if a.points and not a.sweep:
        for Bp in [int(x) for x in a.points.split(",") if x]:
            pt = run_point(eng_mod, dm, dims, Bp, a.context, a.steps, a.warmup, profile=False, kv_layout=a.kv_layout)
            bnd = step_bound_us(dims, Bp, a.context)
            points.append(dict(batch=Bp, ms_per_step=round(pt["ms_per_step"], 4),
                               core_token_steps_per_s=round(pt["core_token_steps_per_s"], 1),
                               decoded_tokens_per_s=round(pt["decoded_tokens_per_s"], 1),
                               step_bound_us=round(bnd, 1),
                               frac_of_step_bound=round(bnd / (pt["ms_per_step"] * 1e3), 4)))
            log(json.dumps({"point": points[-1]}))
    e2e = None
    if not a.no_e2e:
        t1 = time.time()
        e2e = cdb_e2e_segment(eng_mod, dm, dims)
        log(f"cdb e2e segment in {time.time() - t1:.1f} s")
    cpu = None
    if not a.no_cpu:
        t1 = time.time()
        cpu = cpu_baseline(dims, w, a.context)
        log(f"cpu baseline {cpu} in {time.time() - t1:.1f} s")
    bound = step_bound_us(dims, B, a.context)
    out = {
        "metric": "core token-steps/s (Ouro-like bf16 decode hot path, context 1024)",
        "value": round(main_pt["core_token_steps_per_s"], 1),
        "unit": "core token-steps/s",
        "n_gpus": 1, "steps": a.steps, "warmup": a.warmup,
        "ms_per_step": round(main_pt["ms_per_step"], 4),
        "ms_per_step_eager": round(main_pt["ms_per_step_eager"], 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "ouro-like 0-24-0 r_max 4 decode core step + gate/compaction + coda/prelude refill, "
                               "synthetic cached context with exit depths U{1..4}",
                   "batch": B, "context": a.context, "vocab": dims.vocab, "hidden": dims.hidden,
                   "heads": f"{dims.n_heads}x{dims.head_dim}", "ffn": dims.ffn, "core_layers": dims.n_core,
                   "r_max": dims.r_max, "kv_layout": a.kv_layout},
        "decoded_tokens_per_s": round(main_pt["decoded_tokens_per_s"], 1),
        "step_bound_us": round(bound, 1),
        "frac_of_step_bound": round(bound / (main_pt["ms_per_step"] * 1e3), 4),
        "roofline": roof,
        "kernels": kernels,
        "device_peaks": {**peaks, "hbm_copy_gbs": round(copy_gbs, 1), "hbm_datasheet_gbs": HBM_PEAK_GBS,
                         "bf16_datasheet_tflops": BF16_PEAK_TFLOPS},
        "batch_points": points,
        "cdb_e2e": e2e,
        "cpu_baseline": cpu,
    }
    if sweep:
        out["sweep"] = [{k: v for k, v in p.items() if k != "profile"} for p in sweep]
        out["latency_fit"] = fit
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
