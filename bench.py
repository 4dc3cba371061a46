#!/usr/bin/env python3
"""Benchmark of the routed attention hot path on one MI355X.

One step = index build + route + selected-set attention (mono_routed_attention,
which equals mono_build_index + mono_route + mono_selected_attention bit for
bit) over one batch of synthetic q, k, v already resident in HBM (the scaling-sweep
workload at T = 32768: batch 1, 16 heads, d 64, block 64, 1024 addresses,
capacity 64, 4 probes, R = 2 remote + 2 local blocks, bf16).  Prints one JSON
line: tokens/s, the dominant kernel's roofline (its duration taken from HIP
events recorded around its launches inside the timed steps), the per-stage
floors, the 4K-32K sweep exponent, the routed step against the dense causal
attention kernel (mono_dense_attention) at 4K-64K tokens, one decode step
(mono_decode_step) and index update (mono_decode_index) on the batch-8
64K-token cache, spherical codebook calibration (mono_calibrate_codebooks) on
the 8192-token capacity workload with held-out overflow before and after,
the whole step on the batch-8 64K-token workload (d 128, R 8) with its overflow
and maximum list load, peaks measured on the GPU (a 1 GiB device copy, a
library bf16 GEMM) with the path's roofline fraction against them, and the CPU
oracle timed on the host cores (plus its index build and route alone on 4
threads over the sweep, with their exponent).

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-sweep] [--no-dense]
                    [--dense-sizes 4096,...] [--no-decode] [--no-calibration]
                    [--no-onbox-peaks] [--no-large] [--no-cpu-baseline]
                    [--copy-calibration]

--copy-calibration runs a plain 256 MiB device copy before the steps; hardware
counter runs use it to scale FETCH_SIZE / WRITE_SIZE to bytes.
"""
import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, GB/s
FP32_VECTOR_TFLOPS = 157.3       # MI355X fp32 vector peak
BF16_MFMA_TFLOPS = 2500.0        # MI355X dense bf16 MFMA peak
COPY_BYTES = 256 << 20

# Hardware-counter traffic of a kernel, kept as a short text summary with the
# sha256 of the source it was measured on (a changed source voids it).
TRAFFIC_FILES = {"k_route": ("profiles/k_route_sweep_T32768_traffic.md",
                             "learned_sparse_causal_amd/csrc/route.hip")}


def workload_bytes_flops(cfg, sel_np=None):
    """Algorithmic bytes and flops of each stage for one step (what the method
    must move or compute)."""
    es = 2 if cfg.dtype == "bf16" else 4
    B, T, Hq, Hkv, d, R = cfg.B, cfg.T, cfg.Hq, cfg.Hkv, cfg.d, cfg.R
    NB = cfg.NB
    # build: read k once; write the summaries, addresses and the lists
    build_bytes = B * T * Hkv * d * es + B * Hkv * NB * (4 * d + 4 + 4) + \
        B * Hkv * (2 * cfg.A + 2) * 4
    t = np.arange(T)
    qb = t // cfg.beta
    E = np.maximum(0, qb - cfg.L + 1)
    searched = int((E > R).sum()) * B * Hq
    # route: read q of every searched query once, write R ids per route;
    # per searched route K*d MACs (codebook scores), A adds (address sums),
    # R*d MACs (rerank of at least R candidates)
    route_bytes = searched * d * es + B * Hq * T * R * 4
    route_flops = searched * (2 * cfg.K * d + cfg.A + 2 * R * d)
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
                attn_bytes=attn_bytes, attn_flops=attn_flops, searched_routes=searched)


def copy_calibration():
    """A plain device copy of COPY_BYTES (read COPY_BYTES, write COPY_BYTES),
    three launches: the reference for the hardware byte counters."""
    import torch
    src = torch.ones(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()


ROUTE_EVENT_EVERY = 4


def run_gpu(cfg, steps, warmup, route_events=True):
    """Times `steps` steps (mono_routed_attention) between two
    synchronizations; HIP events the library records on the launch stream
    between the stages of every timed step give the per-stage (and, for
    route, per-kernel: the route stage launches k_route only) durations."""
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

    # mono_routed_attention: index build, route and attention in one call;
    # arguments are checked and marshalled once, and the library records the
    # four stage events on the launch stream
    launch = binding.routed_attention_launcher(cfg, d["q"], d["k"], d["v"], cos, sin, cb, idx,
                                               sel, out, ws)

    def step(ev=None):
        launch(ev)

    for _ in range(warmup):
        step()
    # timed region: one event pair around it and, if asked, the route stage of
    # every fourth step (the first included) bracketed by events; each timed
    # event stalls the queue for a few microseconds, so fewer of them perturb
    # the measured throughput less
    evs = [[None, torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True), None]
           if route_events and i % ROUTE_EVENT_EVERY == 0 else None for i in range(steps)]
    r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    r0.record()
    for e in evs:
        step(e)
    r1.record()
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    region_us = r0.elapsed_time(r1) * 1e3 / steps
    route_us = (float(np.mean([e[1].elapsed_time(e[2]) for e in evs if e is not None])) * 1e3
                if route_events else None)
    # stage breakdown and per-step spread: further steps with all four events
    n_bd = max(3, min(steps, 10))
    full = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_bd)]
    for e in full:
        step(e)
    torch.cuda.synchronize()
    step_us = [e[0].elapsed_time(e[3]) * 1e3 for e in full]
    stage = {k: float(np.mean([e[i].elapsed_time(e[i + 1]) for e in full])) * 1e3
             for i, k in enumerate(("build", "route", "attend"))}
    stage["route_in_timed_steps"] = route_us
    stage["step_gpu_us"] = region_us
    stats = dict(overflow=int(idx["overflow"].sum().item()), max_load=int(idx["load"].max().item()),
                 mean_load=float(cfg.NB / cfg.A))
    return wall_ms, stage, step_us, stats, sel


def time_step_median(cfg, reps=3, warmup=1):
    """The scaling study's protocol (technical report page, section
    "Finite-range scaling": one warm-up, then three timed runs, the median):
    `warmup` untimed steps, then `reps` steps each timed by its own HIP event
    pair on the launch stream; returns (median ms, every timed ms)."""
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
    launch = binding.routed_attention_launcher(cfg, d["q"], d["k"], d["v"], cos, sin, cb, idx,
                                               sel, out, ws)
    for _ in range(warmup):
        launch(None)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    torch.cuda.synchronize()
    for e in ev:
        e[0].record()
        launch(None)
        e[1].record()
        torch.cuda.synchronize()
    ms = [e[0].elapsed_time(e[1]) for e in ev]
    return float(np.median(ms)), ms


def time_dense(cfg, reps=3, warmup=1):
    """mono_dense_attention on the same inputs as the routed step: median of
    `reps` calls timed with HIP events on the launch stream (ms)."""
    import torch
    from learned_sparse_causal_amd import binding, synth
    d = synth.qkv_device(cfg)
    cos, sin = binding.device_rope(cfg)
    out = torch.empty((cfg.B, cfg.T, cfg.Hq, cfg.d), dtype=d["q"].dtype, device="cuda")
    ws = torch.empty(binding.workspace_bytes(cfg, binding.WS_DENSE), dtype=torch.uint8,
                     device="cuda")
    for _ in range(warmup):
        binding.dense_attention(cfg, d["q"], d["k"], d["v"], cos, sin, out, ws)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
    for e in ev:
        e[0].record()
        binding.dense_attention(cfg, d["q"], d["k"], d["v"], cos, sin, out, ws)
        e[1].record()
    torch.cuda.synchronize()
    return float(np.median([e[0].elapsed_time(e[1]) for e in ev]))


def run_decode(cfg, steps=20, warmup=3):
    """Decode on a full cache of cfg.T tokens, the index holding its rotated-key
    copy: mono_decode_step for the last position (route + attend of B x Hq
    new-token queries) and mono_decode_index re-indexing the last block (its
    summary, address and rotated keys, then the list rebuild), each timed with
    HIP events on the launch stream; medians in us.
    Algorithmic bytes of a step: per (batch, kv-head) the key and value rows
    of the union of its heads' selected and local tokens, plus q, out and sel."""
    import torch
    from learned_sparse_causal_amd import binding, synth
    d = synth.qkv_device(cfg)
    cos, sin = binding.device_rope(cfg)
    cb = torch.from_numpy(d["codebooks"]).cuda()
    idx = binding.build_index(cfg, d["k"], cos, sin, cb, rotated_keys=True)
    pos = cfg.T - 1
    q = d["q"][:, pos].contiguous()
    sel = torch.empty((cfg.B, cfg.Hq, cfg.R), dtype=torch.int32, device="cuda")
    out = torch.empty((cfg.B, cfg.Hq, cfg.d), dtype=q.dtype, device="cuda")

    def timed(fn):
        for _ in range(warmup):
            fn()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(steps)]
        for e in ev:
            e[0].record()
            fn()
            e[1].record()
        torch.cuda.synchronize()
        return float(np.median([e[0].elapsed_time(e[1]) for e in ev])) * 1e3

    step_us = timed(lambda: binding.decode_step(cfg, q, d["k"], d["v"], cos, sin, cb, idx, pos,
                                                sel, out))
    index_us = timed(lambda: binding.decode_index(cfg, d["k"], cos, sin, cb, idx, cfg.NB - 1,
                                                  cfg.T))
    es = 2 if cfg.dtype == "bf16" else 4
    s_np = sel.cpu().numpy()
    qb = pos // cfg.beta
    local = set(range(max(0, qb - cfg.L + 1), qb + 1))
    tokens = 0
    for b in range(cfg.B):
        for g in range(cfg.Hkv):
            blocks = set(local)
            for h in range(g * cfg.G, (g + 1) * cfg.G):
                blocks.update(int(x) for x in s_np[b, h] if x >= 0)
            tokens += sum(min(cfg.beta, pos + 1 - n * cfg.beta) for n in blocks)
    step_bytes = tokens * 2 * cfg.d * es + cfg.B * cfg.Hq * (2 * cfg.d * es + 4 * cfg.R)
    return dict(workload=cfg.name, B=cfg.B, cache_tokens=cfg.T, position=pos,
                step_us=step_us, tokens_per_s=cfg.B / (step_us * 1e-6),
                index_update_us=index_us,
                roofline=dict(bound="hbm", achieved=step_bytes / (step_us * 1e-6) / 1e9,
                              peak=HBM_PEAK_GBS, unit="GB/s",
                              frac=step_bytes / (step_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                              bytes=step_bytes),
                dense_kv_floor_us=cfg.B * cfg.Hkv * cfg.T * 2 * cfg.d * es / (HBM_PEAK_GBS * 1e9)
                * 1e6)


def run_calibration(cfg, train_sequences=8, rounds=10, reps=5):
    """Spherical codebook calibration on the capacity workload: codebooks
    calibrated on `train_sequences` synthetic concentrated-key sequences
    (mono_build_index, then mono_calibrate_codebooks timed with HIP events,
    median of `reps`), and a held-out sequence indexed with the codebooks
    before and after.  Algorithmic flops per round: 2 K d/P per (point,
    component) for the assignment plus d/P per point for the sums."""
    import torch
    from learned_sparse_causal_amd import binding, synth
    tcfg = cfg.with_(B=train_sequences)
    k_train, cb0 = synth.concentrated_keys(tcfg, seed=53)
    k_test, _ = synth.concentrated_keys(cfg, seed=54)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    cos, sin = binding.device_rope(cfg)
    cb0_d = torch.from_numpy(cb0).cuda()
    tidx = binding.build_index(tcfg, torch.from_numpy(k_train).cuda().to(dt), cos, sin, cb0_d)
    ws = torch.empty(binding.workspace_bytes(tcfg, binding.WS_CALIBRATE), dtype=torch.uint8,
                     device="cuda")
    cb = cb0_d.clone()
    times = []
    for _ in range(reps + 1):
        cb.copy_(cb0_d)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        binding.calibrate_codebooks(tcfg, tidx["kbar"], cb, rounds, ws)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3)
    cal_us = float(np.median(times[1:]))
    kt = torch.from_numpy(k_test).cuda().to(dt)
    before = binding.build_index(cfg, kt, cos, sin, cb0_d)
    after = binding.build_index(cfg, kt, cos, sin, cb)
    torch.cuda.synchronize()
    n_points = tcfg.B * tcfg.NB
    flops = rounds * tcfg.Hkv * tcfg.P * n_points * (2 * tcfg.K + 1) * (tcfg.d // tcfg.P)
    achieved = flops / (cal_us * 1e-6) / 1e12
    return dict(workload=cfg.name + "_concentrated_keys", train_sequences=train_sequences,
                rounds=rounds, calibrate_us=cal_us,
                held_out=dict(overflow_before=int(before["overflow"].sum().item()),
                              overflow_after=int(after["overflow"].sum().item()),
                              max_load_before=int(before["load"].max().item()),
                              max_load_after=int(after["load"].max().item()),
                              capacity=cfg.cap),
                roofline=dict(bound="alu", achieved=achieved, peak=FP32_VECTOR_TFLOPS,
                              unit="TFLOP/s", frac=achieved / FP32_VECTOR_TFLOPS, flops=flops))


def dense_flops(cfg):
    """Causal dense attention: 2 d flops for q.k and 2 d for p.v per (query, key <= query)."""
    return 4.0 * cfg.d * cfg.B * cfg.Hq * cfg.T * (cfg.T + 1) / 2


def measured_traffic(kernel):
    """Bytes per launch from the committed counter summary, or None if there is
    none or the kernel's source changed since it was taken."""
    if kernel not in TRAFFIC_FILES:
        return None
    summary, src = (os.path.join(ROOT, p) for p in TRAFFIC_FILES[kernel])
    if not os.path.exists(summary):
        return None
    text = open(summary).read()
    m_sha = re.search(r"source sha256: ([0-9a-f]{64})", text)
    m_val = re.search(r"traffic bytes per launch: ([0-9.eE+]+)", text)
    if not (m_sha and m_val):
        return None
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    return float(m_val.group(1)) if sha == m_sha.group(1) else None


def cpu_baseline(cfg, reps=3):
    """The oracle (as it stands) on the host cores: the whole step (index
    build, route and attention of every query) run `reps` times, median."""
    import oracle
    from learned_sparse_causal_amd import synth
    oracle.build_oracle(force=False)
    threads = min(16, oracle.max_threads())
    inp = synth.qkv(cfg)
    c, s = oracle.rope_table(cfg.T, cfg.d)
    sh = oracle.Shape.of(**cfg.shape_kw())
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        idx = oracle.build_index(sh, inp["k"], c, s, inp["codebooks"], threads)
        sel, _ = oracle.route(sh, inp["q"], c, s, inp["codebooks"], idx, None, threads)
        oracle.attention(sh, inp["q"], inp["k"], inp["v"], c, s, sel, None, threads)
        times.append(time.perf_counter() - t0)
    t_step = float(np.median(times))
    # the index build and the route alone on 4 threads over the 4K-32K sweep
    # (the configuration the pages time their build and search on), with the
    # least-squares exponent of ln t on ln T
    from learned_sparse_causal_amd import configs
    pts = {}
    for T in configs.SWEEP_T:
        c4 = configs.sweep(T)
        inp4 = synth.qkv(c4)
        cc, ss = oracle.rope_table(c4.T, c4.d)
        sh4 = oracle.Shape.of(**c4.shape_kw())
        t0 = time.perf_counter()
        idx = oracle.build_index(sh4, inp4["k"], cc, ss, inp4["codebooks"], 4)
        oracle.route(sh4, inp4["q"], cc, ss, inp4["codebooks"], idx, None, 4)
        pts[T] = time.perf_counter() - t0
    ts = sorted(pts)
    expo = float(np.polyfit(np.log(ts), np.log([pts[T] for T in ts]), 1)[0])
    model = ""
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                model = ln.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    return dict(value=cfg.B * cfg.T / t_step, unit="tokens/s", cores=threads, kind="oracle",
                sample="the whole step (index build, route and fp64 attention of all %d queries, "
                       "numpy-drawn inputs of the same distribution), %d runs, median %.2f s"
                       % (cfg.routes, reps, t_step),
                cpu_model=model, host_cpus=os.cpu_count(),
                build_route_4_threads=dict(seconds={str(T): pts[T] for T in ts}, exponent=expo))


def onbox_peaks():
    """Peaks measured on this GPU: a device-to-device copy of 1 GiB (read +
    write bytes / time) and a library bf16 GEMM (8192^3, torch.matmul)."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    a = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)
    b = torch.randn(8192, 8192, device="cuda").to(torch.bfloat16)

    def timed(fn, reps):
        fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / reps

    t_copy = timed(lambda: dst.copy_(src), 10)
    t_gemm = timed(lambda: torch.matmul(a, b), 5)
    out = dict(hbm_copy_GBs=2 * n / t_copy / 1e9, bf16_gemm_TFLOPs=2 * 8192 ** 3 / t_gemm / 1e12)
    del src, dst, a, b
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-calibration", action="store_true")
    ap.add_argument("--no-onbox-peaks", action="store_true")
    ap.add_argument("--no-large", action="store_true")
    ap.add_argument("--dense-sizes", default="4096,8192,16384,32768,65536",
                    help="token counts of the routed-vs-dense comparison")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the routed attention path is built and timed on a "
              "single MI355X (--gpus 1); runs on several GPUs are not supported.",
              file=sys.stderr)
        sys.exit(2)
    from learned_sparse_causal_amd import configs

    if args.copy_calibration:
        copy_calibration()
    cfg = configs.SWEEP_32K
    wall_ms, stage, step_us, stats, sel = run_gpu(cfg, args.steps, args.warmup)
    w = workload_bytes_flops(cfg, sel.cpu().numpy())
    tokens = cfg.B * cfg.T
    floors = {
        "build": w["build_bytes"] / (HBM_PEAK_GBS * 1e9),
        "route": max(w["route_bytes"] / (HBM_PEAK_GBS * 1e9),
                     w["route_flops"] / (FP32_VECTOR_TFLOPS * 1e12)),
        "attend": max(w["attn_bytes"] / (HBM_PEAK_GBS * 1e9),
                      w["attn_flops"] / (BF16_MFMA_TFLOPS * 1e12)),
    }
    # the dominant single kernel is the router (the route stage launches
    # k_route only), timed by events inside the timed steps
    t_route = stage["route_in_timed_steps"] * 1e-6
    roof = dict(bound="alu", achieved=w["route_flops"] / t_route / 1e12,
                peak=FP32_VECTOR_TFLOPS, unit="TFLOP/s")
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = measured_traffic("k_route")
    roof["kernel"] = "k_route"
    roof["kernel_us"] = stage["route_in_timed_steps"]
    roof["hbm_GBs"] = w["route_bytes"] / t_route / 1e9
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
        step_us_spread=dict(min=min(step_us), median=float(np.median(step_us)), max=max(step_us)),
        path_roofline_frac=sum(floors.values()) / (wall_ms * 1e-3),
        floors_us={k: v * 1e6 for k, v in floors.items()},
        index=stats,
    )
    routed_ms = {}
    if not args.no_sweep:
        # 1 warm-up + 3 separately timed steps per length, median (the
        # protocol of the report page's scaling study), and the least-squares
        # exponent of ln t on ln T
        pts, runs = [], {}
        for T in configs.SWEEP_T:
            med, ms = time_step_median(configs.sweep(T))
            pts.append((T, med))
            runs[str(T)] = ms
        routed_ms.update(pts)
        x = np.log([p[0] for p in pts])
        y = np.log([p[1] for p in pts])
        line["sweep"] = dict(points_ms={str(T): ms for T, ms in pts}, timed_runs_ms=runs,
                             protocol="1 warm-up + 3 timed steps, median",
                             exponent=float(np.polyfit(x, y, 1)[0]))
    if not args.no_dense:
        # routed step (index build + route + attention) against dense causal
        # attention on the same q, k, v, 4K to 64K tokens
        cmp_t = [int(x) for x in args.dense_sizes.split(",") if x]
        pts = {}
        for T in cmp_t:
            c = configs.sweep(T)
            if T not in routed_ms:
                routed_ms[T] = time_step_median(c)[0]
            dms = time_dense(c)
            pts[str(T)] = dict(routed_ms=routed_ms[T], dense_ms=dms,
                               dense_over_routed=dms / routed_ms[T],
                               dense_mfma_frac=dense_flops(c) / (dms * 1e-3) / 1e12 /
                               BF16_MFMA_TFLOPS)
        line["dense_vs_routed"] = pts
    if not args.no_large:
        # the whole step on the largest workload (batch 8, 64K tokens, d 128,
        # R 8), 1 warm-up + 3 timed steps, with its index statistics
        c5 = configs.LARGE
        _, st5, _, stats5, sel5 = run_gpu(c5, 3, 1, route_events=False)
        w5 = workload_bytes_flops(c5, sel5.cpu().numpy())
        del sel5
        f5 = {
            "build": w5["build_bytes"] / (HBM_PEAK_GBS * 1e9),
            "route": max(w5["route_bytes"] / (HBM_PEAK_GBS * 1e9),
                         w5["route_flops"] / (FP32_VECTOR_TFLOPS * 1e12)),
            "attend": max(w5["attn_bytes"] / (HBM_PEAK_GBS * 1e9),
                          w5["attn_flops"] / (BF16_MFMA_TFLOPS * 1e12)),
        }
        t5 = st5["step_gpu_us"] * 1e-6
        line["large"] = dict(
            workload=c5.name, step_ms=t5 * 1e3, tokens_per_s=c5.B * c5.T / t5,
            stage_us={k: st5[k] for k in ("build", "route", "attend")},
            floors_us={k: v * 1e6 for k, v in f5.items()},
            path_roofline_frac=sum(f5.values()) / t5,
            attend_mfma_frac=w5["attn_flops"] / (st5["attend"] * 1e-6) / 1e12 / BF16_MFMA_TFLOPS,
            index=stats5)
    if not args.no_decode:
        line["decode"] = run_decode(configs.LARGE)
    if not args.no_calibration:
        line["calibration"] = run_calibration(configs.ALL_ELIGIBLE)
    if not args.no_onbox_peaks:
        peaks = onbox_peaks()
        f_box = {
            "build": w["build_bytes"] / (peaks["hbm_copy_GBs"] * 1e9),
            "route": max(w["route_bytes"] / (peaks["hbm_copy_GBs"] * 1e9),
                         w["route_flops"] / (FP32_VECTOR_TFLOPS * 1e12)),
            "attend": max(w["attn_bytes"] / (peaks["hbm_copy_GBs"] * 1e9),
                          w["attn_flops"] / (peaks["bf16_gemm_TFLOPs"] * 1e12)),
        }
        peaks["path_roofline_frac"] = sum(f_box.values()) / (wall_ms * 1e-3)
        line["onbox_peaks"] = peaks
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
