#!/usr/bin/env python3
"""Benchmark of the routed attention hot path on one MI355X.

One step = mono_build_index + mono_route + mono_selected_attention over one
batch of synthetic q, k, v already resident in HBM (the scaling-sweep
workload at T = 32768: batch 1, 16 heads, d 64, block 64, 1024 addresses,
capacity 64, 4 probes, R = 2 remote + 2 local blocks, bf16).  Prints one JSON
line: tokens/s, the dominant kernel's roofline, and the CPU oracle timed on a
bounded sample on the host cores.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-sweep] [--no-cpu-baseline]
"""
import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
FP32_VECTOR_TFLOPS = 157.3       # MI355X fp32 vector peak
BF16_MFMA_TFLOPS = 2500.0        # MI355X dense bf16 MFMA peak


def workload_bytes_flops(cfg, sel_np=None):
    """Algorithmic bytes and flops of each stage for one step (what the method
    must move or compute), per the per-unit figures in the design doc."""
    es = 2 if cfg.dtype == "bf16" else 4
    B, T, Hq, Hkv, d, R = cfg.B, cfg.T, cfg.Hq, cfg.Hkv, cfg.d, cfg.R
    NB = cfg.NB
    build_bytes = B * T * Hkv * d * es + B * Hkv * NB * (4 * d + 4 + 4) + \
        B * Hkv * (2 * cfg.A + 2) * 4
    t = np.arange(T)
    qb = t // cfg.beta
    E = np.maximum(0, qb - cfg.L + 1)
    searched = (E > R).sum()
    route_bytes = B * Hq * searched * d * es + B * Hq * T * R * 4
    route_flops = B * Hq * searched * (2 * cfg.K * d + 2 * R * d)
    # attended keys per query: selected remote tokens + local tokens <= t
    lo = np.maximum(0, qb - cfg.L + 1) * cfg.beta
    local = t - lo + 1
    if sel_np is not None:
        nrem = (sel_np >= 0).sum(-1).astype(np.float64) * cfg.beta        # [B,Hq,T]
        keys = (nrem + local[None, None, :]).sum()
    else:
        keys = B * Hq * (np.minimum(E, R) * cfg.beta + local).sum()
    attn_flops = 4.0 * d * keys
    attn_bytes = (B * T * Hq * d * es) * 2 + 2 * B * T * Hkv * d * es + B * Hq * T * R * 4
    return dict(build_bytes=build_bytes, route_bytes=route_bytes, route_flops=route_flops,
                attn_bytes=attn_bytes, attn_flops=attn_flops)


def run_gpu(cfg, steps, warmup, per_stage=True):
    import torch
    from learned_sparse_causal_amd import binding, synth
    d = synth.qkv_device(cfg)
    cos, sin = binding.device_rope(cfg)
    cb = torch.from_numpy(d["codebooks"]).cuda()
    idx = binding.empty_index(cfg)
    sel = torch.empty((cfg.B, cfg.Hq, cfg.T, cfg.R), dtype=torch.int32, device="cuda")
    out = torch.empty((cfg.B, cfg.T, cfg.Hq, cfg.d), dtype=d["q"].dtype, device="cuda")
    ws = torch.empty(max(1, binding.workspace_bytes(cfg, binding.WS_ATTENTION)), dtype=torch.uint8,
                     device="cuda")

    def step(ev=None):
        if ev: ev[0].record()
        binding.build_index(cfg, d["k"], cos, sin, cb, idx)
        if ev: ev[1].record()
        binding.route(cfg, d["q"], cos, sin, cb, idx, sel)
        if ev: ev[2].record()
        binding.selected_attention(cfg, d["q"], d["k"], d["v"], cos, sin, sel, out, ws)
        if ev: ev[3].record()

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # whole-step timing: exactly `steps` steps between two synchronizations
    t0 = time.perf_counter()
    for _ in range(steps):
        step()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    stage = None
    if per_stage:
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
        for e in evs:
            step(e)
        torch.cuda.synchronize()
        stage = {k: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in evs])) * 1e3
                 for i, k in enumerate(("build", "route", "attend"))}
    stats = dict(overflow=int(idx["overflow"].sum().item()), max_load=int(idx["load"].max().item()))
    return wall_ms, stage, stats, sel


def cpu_baseline(cfg, budget_s=15.0):
    """The oracle (as it stands) on the host: the whole index build, then route
    + attention for a random sample of routes sized to the time budget; the
    full-step time is extrapolated from the per-route rate."""
    import oracle
    from learned_sparse_causal_amd import synth
    oracle.build_oracle(force=False)
    threads = min(16, os.cpu_count() or 1)
    inp = synth.qkv(cfg)
    c, s = oracle.rope_table(cfg.T, cfg.d)
    sh = oracle.Shape.of(**cfg.shape_kw())
    t0 = time.perf_counter()
    idx = oracle.build_index(sh, inp["k"], c, s, inp["codebooks"], threads)
    t_build = time.perf_counter() - t0
    rng = np.random.default_rng(0)
    n = 2000
    spent, done = 0.0, 0
    while True:
        ids = rng.choice(cfg.routes, size=n, replace=False).astype(np.int64)
        t0 = time.perf_counter()
        sel, _ = oracle.route(sh, inp["q"], c, s, inp["codebooks"], idx, ids, threads)
        oracle.attention(sh, inp["q"], inp["k"], inp["v"], c, s, sel, ids, threads)
        dt = time.perf_counter() - t0
        spent += dt
        done += n
        if spent + t_build > budget_s * 0.5 or done >= cfg.routes:
            break
        n = min(cfg.routes, int(n * max(2.0, (budget_s * 0.5 - t_build) / max(dt, 1e-3))))
    per_route = spent / done
    t_step = t_build + per_route * cfg.routes
    return dict(value=cfg.B * cfg.T / t_step, unit="tokens/s", cores=threads, kind="oracle",
                sample="full index build (%.2f s) + route and attention of %d random routes of "
                       "%d (%.2f s), full step extrapolated from the per-route rate: %.1f s"
                       % (t_build, done, cfg.routes, spent, t_step))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the routed attention path is built and timed on a "
              "single MI355X (--gpus 1); multi-GPU runs are not part of this build.",
              file=sys.stderr)
        sys.exit(2)
    from learned_sparse_causal_amd import configs

    cfg = configs.SWEEP_32K
    wall_ms, stage, stats, sel = run_gpu(cfg, args.steps, args.warmup)
    w = workload_bytes_flops(cfg, sel.cpu().numpy())
    tokens = cfg.B * cfg.T
    # per-stage roofline floors and the dominant stage
    floors = {
        "build": w["build_bytes"] / (HBM_PEAK_GBS * 1e9),
        "route": max(w["route_bytes"] / (HBM_PEAK_GBS * 1e9),
                     w["route_flops"] / (FP32_VECTOR_TFLOPS * 1e12)),
        "attend": max(w["attn_bytes"] / (HBM_PEAK_GBS * 1e9),
                      w["attn_flops"] / (BF16_MFMA_TFLOPS * 1e12)),
    }
    dom = max(stage, key=stage.get)
    t_dom = stage[dom] * 1e-6
    if dom == "route":
        roof = dict(bound="alu", achieved=w["route_flops"] / t_dom / 1e12,
                    peak=FP32_VECTOR_TFLOPS, unit="TFLOP/s")
    elif dom == "build":
        roof = dict(bound="hbm", achieved=w["build_bytes"] / t_dom / 1e9, peak=HBM_PEAK_GBS,
                    unit="GB/s")
    else:
        roof = dict(bound="hbm", achieved=w["attn_bytes"] / t_dom / 1e9, peak=HBM_PEAK_GBS,
                    unit="GB/s")
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    roof["kernel"] = {"route": "k_route", "build": "k_block_address+k_posting_lists",
                      "attend": "mono_selected_attention (6 kernels)"}[dom]
    line = dict(
        metric="routed-attn tokens/s (build+route+attend) at T=32K; % HBM/MFMA roofline",
        value=tokens / (wall_ms * 1e-3), unit="tokens/s", n_gpus=1, steps=args.steps,
        warmup=args.warmup, ms_per_step=wall_ms, higher_is_better=True, scaling="weak",
        vs_baseline=None, dtype="bf16", data="synthetic",
        config=dict(workload=cfg.name, B=cfg.B, T=cfg.T, Hq=cfg.Hq, Hkv=cfg.Hkv, d=cfg.d,
                    block=cfg.beta, P=cfg.P, K=cfg.K, capacity=cfg.cap, n_probes=cfg.n_probes,
                    R=cfg.R, L=cfg.L),
        roofline=roof,
        stage_us=stage,
        path_roofline_frac=sum(floors.values()) / (wall_ms * 1e-3),
        floors_us={k: v * 1e6 for k, v in floors.items()},
        index=stats,
    )
    if not args.no_sweep:
        pts = []
        for T in configs.SWEEP_T:
            c = configs.sweep(T)
            times = []
            for _ in range(3):
                ms, _, _, _ = run_gpu(c, 1, 1, per_stage=False)
                times.append(ms)
            pts.append((T, float(np.median(times))))
        x = np.log([p[0] for p in pts])
        y = np.log([p[1] for p in pts])
        line["sweep"] = dict(points_ms={str(T): ms for T, ms in pts},
                             exponent=float(np.polyfit(x, y, 1)[0]))
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
