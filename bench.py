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

import numpy as np

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_traffic_ouro_b64_ctx1024.txt")
ATTN_SRC = os.path.join(ROOT, "continuous_depth_batching_amd", "csrc", "k_attn.hip")
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
    ap.add_argument("--seed", type=int, default=0)
    return ap.parse_args()


class DecodeBench:
    """Engine set up with synthetic cached context for B rows at context L."""

    def __init__(self, eng_mod, dm, dims, B, L, steps_total, seed=3):
        import torch
        self.torch = torch
        self.B, self.L = B, L
        R = dims.r_max
        mbps = (L + steps_total + 32) // 16 + 1
        self.mbps = mbps
        nblk = B * mbps
        self.e = e = eng_mod.Engine(dm, n_slots=B, max_rows=eng_mod.pow2(B), num_blocks=nblk, max_seqs=B,
                                    max_blocks_per_seq=mbps, max_out=steps_total + 8, max_prefill_tokens=16,
                                    kv_fill=0.0)
        rng = np.random.default_rng(seed)
        perm = rng.permutation(nblk).astype(np.int32)
        e.btab.copy_(torch.from_numpy(perm))
        gen = torch.Generator(device="cuda").manual_seed(seed)
        # random K/V everywhere (bf16 N(0,1)), in chunks to bound temporaries
        for pool in (e.core_k, e.core_v):
            n = pool.numel()
            step = 1 << 28
            for s in range(0, n, step):
                m = min(step, n - s)
                pool[s:s + m].copy_(torch.randn(m, generator=gen, device="cuda", dtype=torch.float32).to(pool.dtype))
        import cdb_synth as S
        ex = S.make_context_exit_depths(nblk * 16, R, seed=seed + 1)
        emap = ex.reshape(nblk, 16).copy()
        bt = perm.reshape(B, mbps)
        for b in range(B):                   # positions >= L: in flight / future
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


def run_point(eng_mod, dm, dims, B, L, steps, warmup, profile=True):
    import torch
    from continuous_depth_batching_amd import _lib as LL
    import ctypes as C
    bench = DecodeBench(eng_mod, dm, dims, B, L, steps * 3 + warmup + 4)
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
    res = dict(B=B, L=L, ms_per_step=ms / steps, ms_per_step_eager=ms_eager / steps,
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


def source_sha(path):
    import hashlib
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


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
    """One plain device copy of CALIB_BYTES (read + write), so a counter run
    can scale FETCH_SIZE / WRITE_SIZE against known bytes."""
    import torch
    a = torch.ones(CALIB_BYTES // 2, dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    del a, b
    torch.cuda.empty_cache()


def step_bound_us(dims, B, L):
    """Roofline step time: core weights once + per-row KV traffic at HBM peak,
    GEMM flops at the bf16 MFMA peak (the larger of the two per GEMM)."""
    H, Q, F, n = dims.hidden, dims.qdim, dims.ffn, dims.n_core
    wbytes = 2 * n * (3 * Q * H + H * Q + 2 * F * H + H * F)
    kv = B * n * (2 * Q * 2) * (L + 1)
    flops = 2 * B * wbytes / 2
    return max(wbytes / (HBM_PEAK_GBS * 1e3), flops / (BF16_PEAK_TFLOPS * 1e6)) + kv / (HBM_PEAK_GBS * 1e3)


def cpu_baseline(dims, w, L, budget_s=10.0, max_rows=256, seed=5):
    """The oracle's single-row core step at the bench's context, timed on the
    host cores on a bounded sample: rows at depths 1..r_max over one synthetic
    cached context, run until about budget_s seconds of oracle time."""
    from oracle.model import OracleLM, cache_from_planes
    try:
        from threadpoolctl import threadpool_info
        threads = max([d.get("num_threads", 1) for d in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
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
    return dict(value=rows / total, unit="core token-steps/s", cores=int(threads), kind="oracle",
                sample=f"{rows} single-row core steps (24 layers, fp32 numpy) at context {L}, depths 1..{R}; "
                       f"{total:.1f} s of oracle time")


def main():
    a = parse()
    if a.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU; --gpus must be 1 (no multi-GPU path)"}))
        sys.exit(2)
    import torch
    import cdb_synth as S
    from continuous_depth_batching_amd import engine as eng_mod
    dims = S.CONFIGS["c1"]
    t0 = time.time()
    w = S.make_weights(dims, seed=a.seed)
    log(f"weights generated in {time.time() - t0:.1f} s")
    dm = eng_mod.DeviceModel(dims, w)
    torch.cuda.synchronize()
    log(f"weights on device after {time.time() - t0:.1f} s")
    calibration_copy()
    main_pt = run_point(eng_mod, dm, dims, a.batch, a.context, a.steps, a.warmup, profile=True)
    log(json.dumps(main_pt))
    sweep = []
    if a.sweep:
        for B in [int(x) for x in a.sweep.split(",") if x]:
            pt = run_point(eng_mod, dm, dims, B, a.context, a.steps, a.warmup, profile=True)
            pt["bound_us"] = step_bound_us(dims, B, a.context)
            pt["frac_of_step_bound"] = pt["bound_us"] / (pt["ms_per_step"] * 1e3)
            log(json.dumps({k: v for k, v in pt.items() if k != "profile"}))
            sweep.append(pt)
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
            "traffic": measured_traffic() if (B == 64 and a.context == 1024) else None,
            "bytes_per_launch": int(attn_bytes), "avg_launch_us": round(prof["attn"]["avg_us"], 2),
            "dominant_by_time": dom}
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
                   "r_max": dims.r_max},
        "decoded_tokens_per_s": round(main_pt["decoded_tokens_per_s"], 1),
        "step_bound_us": round(bound, 1),
        "frac_of_step_bound": round(bound / (main_pt["ms_per_step"] * 1e3), 4),
        "roofline": roof,
        "kernels": kernels,
        "cpu_baseline": cpu,
    }
    if sweep:
        out["sweep"] = [{k: v for k, v in p.items() if k != "profile"} for p in sweep]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
