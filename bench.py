#!/usr/bin/env python3
"""Throughput of the DLA layer forward pass on one MI355X.

Headline (the JSON line's value): prefill tokens/s of the Gated-DeltaNet-1.3B
shaped layer at T = 32768 (B=2, H=16, d_k=128, d_v=256, C=32, tau=0.3, bf16),
one step = one dla_prefill call over the whole batch (score, boundaries,
greedy capacity merges, chunked MFMA read/update).  Inputs are synthetic
(seeded piecewise-regime keys) and resident in HBM before timing starts.

Also reported on the same line:
  roofline      the algorithmic flops of the prefill (sum over token-heads of
                2 (m_t + 1) d_k d_v, m_t from the run's own schedule) over the
                whole prefill's HIP-event time (every kernel of the call, from
                the score to the sweep), against the dense bf16 MFMA peak;
                kernel_* fields give the same for the chunk kernel (the
                sweep) alone, and mfma_ops_ratio / mfma_busy_frac its MFMA
                counters (issued MFMA flops over the algorithmic flops, share
                of SIMD cycles the matrix cores were busy), from the counter
                summary committed under profiles/;
  decode        batched decode (B=256, H=16, d=128, C=32 full fp32 caches):
                steps/s over a loop of dla_decode_step calls and the decode
                kernel's algorithmic HBM bytes per launch over its duration,
                against the HBM peak; inputs from the tested recipe
                (workloads.decode_inputs), distinct caches tiled over the
                streams;
  cpu_baseline  the CPU oracle on a bounded sample of the prefill workload, on
                the CPU threads the process is granted;
  prefill_density_merge_rule
                the same prefill with the capacity merges choosing the pair
                of lowest information density instead of smallest summed
                information (--no-density skips it);
  prefill_streamed_kernel
                the same prefill on the streamed chunk kernel (the kernel of
                fp32 io and C > 32; --no-streamed skips it);
  prefill_workloads
                the other prefill workloads in their full launch
                configurations: Mamba-2-780M-shaped, long context (T=131072),
                Mamba-2-shaped with C=64, tiny fp32, and the state information
                score on the Mamba-2-shaped layer with values that follow the
                key segments (--no-other skips them); the long-context one
                also timed with its sweep unsplit (`unsplit`: its grid of 128
                blocks is split along the sequence), and the Mamba-2-shaped
                one over batch sizes 1, 2, 4 with the library's sweep and
                unsplit (`batch_sweep`: the pages measure prefill over batch
                sizes);
  decode_bf16_states
                the same decode on caches storing closed states as bf16 (the
                most recent one stays fp32), with its algorithmic bytes
                (--no-bf16-states skips it);
  prefill_fenwick_schedule
                the same prefill under the Log-Linear fixed schedule (Fenwick
                buckets, lam = the first 16 columns, one weight per level),
                the comparison the pages draw between the two methods; its
                algorithmic flops count 2 (popcount(t) + 2) d_k d_v per
                token-head, the buckets read plus the update (--no-fenwick
                skips it);
  prefill_literal_reading
                the same prefill on the literal reading of the key noise
                (0.2 N(0, I) per coordinate: every token opens a state, so
                every chunk merges), 5 timed steps (--no-literal skips it);
  prefill_context_sweep
                DLA and the fixed schedule on the first T' tokens of the same
                streams, T' = 4096 .. 32768 (the pages compare the two
                methods' prefill over context lengths); --no-sweep or
                --no-fenwick skips it;
  decode_fenwick_schedule
                batched decode (B=256, H=16, d=128, C=32) under the same
                schedule, from position 2^20 (the cache preloaded with the one
                bucket of the first 2^20 tokens), with its algorithmic bytes:
                the popcount(t) buckets read, the token's bucket written
                (--no-fenwick skips it).

roofline.traffic is the kernel's HBM bytes per launch from the hardware
counters FETCH_SIZE and WRITE_SIZE (two rocprofv3 --pmc passes over this
script with --copy-probe-mib, each scaled by what the counter reads for a plain
device copy of known size), read from the counter summary committed under
profiles/.  It is null when that summary is missing or was taken on kernel
sources other than the ones built now (sha256 over the files it names).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "DLA prefill tokens/s at T=32K; decode steps/s at B=256; % MFMA / HBM peak"
PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def measured_traffic(summary: str, kernel: str):
    """HBM bytes per launch of `kernel` from a committed counter summary
    (key: value lines), or None when it is absent, names another kernel, or
    its kernel sources no longer hash to what it recorded."""
    path = os.path.join(ROOT, "profiles", summary)
    try:
        kv = {}
        for line in open(path):
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                kv[key.strip()] = val.strip()
        if kv.get("kernel") != kernel:
            return None
        h = hashlib.sha256()
        for f in kv["sources"].split():
            h.update(open(os.path.join(ROOT, f), "rb").read())
        if h.hexdigest() != kv["sources_sha256"]:
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def measured_mfma(summary: str, kernel: str):
    """MFMA counters of `kernel` from a committed counter summary: the MFMA
    flops it issues per launch and the share of SIMD cycles its matrix cores
    were busy; None when the summary is absent, names another kernel, or was
    taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", summary)
    try:
        kv = {}
        for line in open(path):
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                kv[key.strip()] = val.strip()
        if kv.get("kernel") != kernel:
            return None
        h = hashlib.sha256()
        for f in kv["sources"].split():
            h.update(open(os.path.join(ROOT, f), "rb").read())
        if h.hexdigest() != kv["sources_sha256"]:
            return None
        return dict(mfma_flop_per_launch=float(kv["mfma_flop_per_launch"]),
                    mfma_busy_frac=float(kv["mfma_busy_frac"]))
    except (OSError, KeyError, ValueError):
        return None


def copy_probe(torch, mib):
    """A plain device-to-device copy of mib MiB, three times: the counter
    passes scale FETCH_SIZE and WRITE_SIZE by what they read for it."""
    if mib <= 0:
        return
    n = mib * (1 << 20)
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"copy probe: 3 x {n} bytes")
    del src, dst
    torch.cuda.empty_cache()


def upload(torch, d, cfg, dev, T=None):
    """q, k, v, lam of a workload draw as device tensors [B, H, T, d] in the io dtype."""
    T = cfg.T if T is None else T
    dt = torch.bfloat16 if cfg.io == "bf16" else torch.float32

    def up(a, dd):
        return torch.from_numpy(a).to(dev).to(dt).view(cfg.B, cfg.H, T, dd)

    return up(d["q"], cfg.dk), up(d["k"], cfg.dk), up(d["v"], cfg.dv), up(d["lam"], cfg.C)


def prefill_leg(args, torch, dla, cfg, x, steps=None, rule="sum", score_rule="cosine", tau=None, path=None):
    """One prefill workload timed: an untimed call exporting the schedule (its
    m_t gives the algorithmic flops), the warmup, then `steps` timed calls.
    Each timed step resets the cache (a prefill continues what the cache
    holds) and runs dla_prefill; HIP events on the call's stream bracket the
    whole prefill (every kernel from the score to the sweep, not the reset),
    and the library's hook brackets the chunk kernel (the sweep)."""
    steps = args.steps if steps is None else steps
    tau = cfg.tau if tau is None else tau
    B, H, T, dk, dv, C = cfg.B, cfg.H, x[0].shape[2], cfg.dk, cfg.dv, cfg.C
    BH = B * H
    dev = x[0].device
    q, k, v, lam = x
    if path is not None:
        dla.dla_set_prefill_path(path, 0)
    try:
        cache = dla.Cache(B, H, C, dk, dv, device=dev, merge_rule=rule, score_rule=score_rule)
        ws = dla.prefill_workspace(B, H, T, C, dk, dv, dev)
        o = torch.empty(B, H, T, dv, dtype=q.dtype, device=dev)
        m_t = torch.empty(BH, T, dtype=torch.int32, device=dev)
        bnd = torch.empty(BH, T, dtype=torch.uint8, device=dev)
        n_ev = torch.empty(BH, dtype=torch.int32, device=dev)
        dla.prefill(q, k, v, lam, tau, cache, o=o, workspace=ws, sched=dict(m_t=m_t, boundary=bnd, n_ev=n_ev))
        torch.cuda.synchronize()
        m_sum = int(m_t.sum(dtype=torch.int64).item())
        flops = 2.0 * (m_sum + BH * T) * dk * dv
        stats = dict(mean_live_states=m_sum / (BH * T),
                     boundaries_per_stream=float(bnd.sum(dtype=torch.int64).item()) / BH,
                     merges_per_stream=float(n_ev.sum(dtype=torch.int64).item()) / BH)
        del m_t, bnd, n_ev
        for _ in range(args.warmup):
            cache.reset()
            dla.prefill(q, k, v, lam, tau, cache, o=o, workspace=ws)
        ev = lambda: torch.cuda.Event(enable_timing=True)
        whole = [(ev(), ev()) for _ in range(steps)]
        sweep = [(ev(), ev()) for _ in range(steps)]
        for pair in whole + sweep:          # materialise the event handles
            pair[0].record()
            pair[1].record()
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        for (a, b), (c, e) in zip(whole, sweep):
            cache.reset()
            dla.dla_set_prefill_events(c.cuda_event, e.cuda_event)
            a.record()
            dla.prefill(q, k, v, lam, tau, cache, o=o, workspace=ws)
            b.record()
        torch.cuda.synchronize()
        wall = time.perf_counter() - w0
        dla.dla_set_prefill_events(None, None)
        kernel = dla.dla_prefill_kernel(dla.DLA_BF16 if q.dtype == torch.bfloat16 else dla.DLA_F32, B, H, C, dk, dv)
    finally:
        if path is not None:
            dla.dla_set_prefill_path(dla.DLA_PATH_AUTO, 0)
    whole_ms = sum(a.elapsed_time(b) for a, b in whole) / steps
    sweep_ms = sum(a.elapsed_time(b) for a, b in sweep) / steps
    ach = flops / (whole_ms * 1e-3) / 1e12
    sweep_ach = flops / (sweep_ms * 1e-3) / 1e12
    del cache, ws, o
    return dict(value=B * T * steps / wall, unit="tokens/s", steps=steps, ms_per_step=wall * 1e3 / steps,
                prefill_ms=whole_ms, achieved=ach, unit_achieved="TFLOP/s", frac=ach / PEAK_BF16_TFLOPS,
                kernel=kernel, kernel_ms=sweep_ms, kernel_achieved=sweep_ach,
                kernel_frac=sweep_ach / PEAK_BF16_TFLOPS, algorithmic_flop_per_launch=flops, schedule=stats)


def _leg_log(name, r):
    log(f"{name}: {r['ms_per_step']:.3f} ms/step, prefill {r['prefill_ms']:.3f} ms "
        f"({100 * r['frac']:.1f}% of bf16 peak), chunk kernel {r['kernel']} {r['kernel_ms']:.3f} ms "
        f"({100 * r['kernel_frac']:.1f}%), mean live states {r['schedule']['mean_live_states']:.2f}, "
        f"boundaries/stream {r['schedule']['boundaries_per_stream']:.1f}, merges/stream "
        f"{r['schedule']['merges_per_stream']:.1f}")


def prefill_bench(args, torch, dla, workloads):
    cfg = workloads.CONFIGS[args.workload]
    B, H, T, dk, dv, C = cfg.B, cfg.H, cfg.T, cfg.dk, cfg.dv, cfg.C
    BH = B * H
    dev = torch.device("cuda:0")
    t0 = time.time()
    d = workloads.prefill_inputs(cfg, reading=args.reading)
    log(f"prefill inputs {args.workload} ({args.reading}) generated in {time.time() - t0:.1f}s")
    q, k, v, lam = upload(torch, d, cfg, dev)
    sample = None
    if not args.no_cpu:
        S = min(BH, args.cpu_streams)
        sample = {x: d[x][:S].copy() for x in ("q", "k", "v", "lam")}
    del d
    head = prefill_leg(args, torch, dla, cfg, (q, k, v, lam))
    _leg_log("prefill", head)
    tokens = B * T
    density = None
    if not args.no_density:
        density = prefill_leg(args, torch, dla, cfg, (q, k, v, lam), rule="density")
        density["merge_rule"] = "density"
        _leg_log("prefill, density merge rule", density)
    literal = None
    if args.reading == "relative" and not args.no_literal:
        # the literal reading of the key noise: every token opens a state
        dl = workloads.prefill_inputs(cfg, reading="literal")
        xl = upload(torch, dl, cfg, dev)
        del dl
        literal = prefill_leg(args, torch, dla, cfg, xl, steps=5)
        literal["reading"] = "literal"
        del xl
        _leg_log("prefill, literal noise reading", literal)
    streamed = None
    if not args.no_streamed:
        # the streamed chunk kernel (states read from the cache every chunk) on
        # the same workload: the kernel fp32 io and C > 32 take
        streamed = prefill_leg(args, torch, dla, cfg, (q, k, v, lam), steps=5, path=dla.DLA_PATH_STREAMED)
        streamed["path"] = "streamed"
        _leg_log("prefill, streamed kernel", streamed)
    fenwick = sweep = None
    if not args.no_fenwick:
        o = torch.empty(B, H, T, dv, dtype=q.dtype, device=dev)
        ws = dla.prefill_workspace(B, H, T, C, dk, dv, dev)
        fenwick = fenwick_leg(args, torch, dla, cfg, q, k, v, lam, o, ws, head["ms_per_step"])
        del o, ws
        if not args.no_sweep:
            sweep = context_sweep(torch, dla, cfg, q, k, v, lam)
    kernel = head["kernel"]
    traffic = measured_traffic(f"{_kernel_file(kernel)}_{args.workload}_hbm_traffic.txt", kernel)
    mfma = measured_mfma(f"{_kernel_file(kernel)}_{args.workload}_mfma.txt", kernel)
    roof = dict(bound="mfma", achieved=head["achieved"], peak=PEAK_BF16_TFLOPS, unit="TFLOP/s", frac=head["frac"],
                traffic=traffic, scope="whole prefill (score, compaction, greedy scan, pre-pass, sweep)",
                prefill_ms=head["prefill_ms"], kernel=kernel, kernel_ms=head["kernel_ms"],
                kernel_achieved=head["kernel_achieved"], kernel_frac=head["kernel_frac"],
                algorithmic_flop_per_launch=head["algorithmic_flop_per_launch"])
    if mfma is not None:
        # counters of the sweep kernel: MFMA flops issued over the algorithmic
        # flops, and the share of SIMD cycles the matrix cores were busy
        roof["mfma_ops_ratio"] = mfma["mfma_flop_per_launch"] / head["algorithmic_flop_per_launch"]
        roof["mfma_busy_frac"] = mfma["mfma_busy_frac"]
    else:
        roof["mfma_ops_ratio"] = roof["mfma_busy_frac"] = None
    res = dict(
        value=tokens / (head["ms_per_step"] * 1e-3), ms_per_step=head["ms_per_step"],
        config=dict(workload=f"{args.workload} prefill", B=B, H=H, T=T, d_k=dk, d_v=dv, C=C,
                    tau=cfg.tau, io=cfg.io, keys=f"piecewise-regime, {args.reading} noise",
                    segment_means=list(cfg.seg_means)),
        roofline=roof, schedule=head["schedule"],
        token_heads_per_s=BH * T / (head["ms_per_step"] * 1e-3),
        density_rule=density, fenwick=fenwick, context_sweep=sweep, literal=literal, streamed=streamed,
    )
    del q, k, v, lam
    torch.cuda.empty_cache()
    return res, sample, cfg


def other_prefill_legs(args, torch, dla, workloads):
    """The other prefill workloads, each in its own full launch configuration:
    the Mamba-2-780M-shaped layer (B=4, H=24, T=8192, d_k=128, d_v=64, C=16),
    the long-context one (B=1, H=16, T=131072, d=128, C=32), the same
    Mamba-2-shaped tokens with C=64 (the streamed kernel), the tiny fp32 layer
    (the streamed kernel in fp32), and the state information score on the
    Mamba-2-shaped layer with values that follow the key segments."""
    dev = torch.device("cuda:0")
    out = {}
    import dataclasses
    legs = [("mamba2_780m_bf16", "mamba2_780m_bf16", {}, {}),
            ("long_t131k_bf16", "long_t131k_bf16", {}, {}),
            ("mamba2_780m_bf16_c64", "mamba2_780m_bf16", dict(C=64), {}),
            ("tiny_fp32", "tiny_fp32", {}, {}),
            ("mamba2_780m_bf16_state_score", "mamba2_780m_bf16", {}, dict(score_rule="state", tau=0.6))]
    for name, base, repl, kw in legs:
        cfg = dataclasses.replace(workloads.CONFIGS[base], **repl)
        t0 = time.time()
        d = workloads.prefill_inputs(cfg, values="regime" if kw.get("score_rule") == "state" else "random")
        x = upload(torch, d, cfg, dev)
        del d
        log(f"{name}: inputs generated in {time.time() - t0:.1f}s")
        r = prefill_leg(args, torch, dla, cfg, x, steps=10 if cfg.T >= 4096 else 50, **kw)
        if name == "long_t131k_bf16":
            # its sweep grid (128 blocks) is split along the sequence; the same
            # call with the split turned off, for comparison
            u = prefill_leg(args, torch, dla, cfg, x, steps=5, path=dla.DLA_PATH_UNSPLIT, **kw)
            r["unsplit"] = {kk: u[kk] for kk in ("ms_per_step", "prefill_ms", "kernel_ms", "frac", "kernel_frac")}
            log(f"{name} unsplit: {u['ms_per_step']:.3f} ms/step, sweep {u['kernel_ms']:.3f} ms")
        if name == "mamba2_780m_bf16":
            r["batch_sweep"] = batch_sweep(torch, dla, cfg, x)
        r["config"] = dict(workload=name, B=cfg.B, H=cfg.H, T=cfg.T, d_k=cfg.dk, d_v=cfg.dv, C=cfg.C,
                           tau=kw.get("tau", cfg.tau), io=cfg.io, score_rule=kw.get("score_rule", "cosine"),
                           values="regime" if kw.get("score_rule") == "state" else "random",
                           segment_means=list(cfg.seg_means))
        kernel = r["kernel"]
        r["traffic"] = measured_traffic(f"{_kernel_file(kernel)}_{name}_hbm_traffic.txt", kernel)
        _leg_log(name, r)
        out[name] = r
        del x
        torch.cuda.empty_cache()
    return out


def fenwick_leg(args, torch, dla, cfg, q, k, v, lam, o, ws, dla_ms):
    """The same tokens under the Log-Linear fixed schedule: L = bit_length(T-1)+1
    level weights (the first L columns of the workload's lam), a cache of C = L
    slots, reset before every call (a prefill continues the cache)."""
    B, H, T, dk, dv = cfg.B, cfg.H, cfg.T, cfg.dk, cfg.dv
    L = (T - 1).bit_length() + 1
    lamL = lam[..., :L].contiguous()
    cache = dla.Cache(B, H, L, dk, dv, device=q.device, merge_rule="fenwick")
    for _ in range(max(args.warmup, 1)):
        cache.reset()
        dla.prefill(q, k, v, lamL, 0.0, cache, o=o, workspace=ws)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    for a, b in evs:
        a.record()
        b.record()
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for a, b in evs:
        cache.reset()
        dla.dla_set_prefill_events(a.cuda_event, b.cuda_event)
        dla.prefill(q, k, v, lamL, 0.0, cache, o=o, workspace=ws)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - w0) * 1e3 / args.steps
    dla.dla_set_prefill_events(None, None)
    kern = sum(a.elapsed_time(b) for a, b in evs) / len(evs)
    read = sum(bin(t).count("1") + 1 for t in range(T))        # buckets read per stream
    flops = 2.0 * B * H * (read + T) * dk * dv
    ach = flops / (kern * 1e-3) / 1e12
    kernel = dla.dla_prefill_kernel(dla.DLA_BF16, B, H, L, dk, dv)
    log(f"prefill, Log-Linear fixed schedule (C = L = {L}): {ms:.3f} ms/step, chunk kernel {kern:.3f} ms, "
        f"{100 * ach / PEAK_BF16_TFLOPS:.1f}% of bf16 peak, buckets read per token {read / T:.2f}, "
        f"DLA/Log-Linear time {dla_ms / ms:.2f}")
    del cache
    return dict(schedule="Log-Linear fixed (Fenwick)", value=B * T / (ms * 1e-3), unit="tokens/s",
                ms_per_step=ms, kernel=kernel, kernel_ms=kern, C=L, achieved=ach, unit_achieved="TFLOP/s",
                frac=ach / PEAK_BF16_TFLOPS, algorithmic_flop_per_launch=flops,
                buckets_read_per_token=read / T, dla_over_fenwick_time=dla_ms / ms)


def batch_sweep(torch, dla, cfg, x, batches=(1, 2, 4), steps=10):
    """Prefill tokens/s of the workload's layer at batch sizes B' <= B (the
    first B' sequences of its batch): the library's choice of sweep, which
    splits a small grid along the sequence, and the same calls with the split
    turned off.  Wall time over `steps` calls after one warmup call."""
    q, k, v, lam = x
    H, T, dk, dv, C = cfg.H, q.shape[2], cfg.dk, cfg.dv, cfg.C
    out = []
    for Bn in batches:
        if Bn > cfg.B:
            continue
        xs = [t[:Bn].contiguous() for t in (q, k, v, lam)]
        on = torch.empty(Bn, H, T, dv, dtype=q.dtype, device=q.device)
        cache = dla.Cache(Bn, H, C, dk, dv, device=q.device)
        wsn = dla.prefill_workspace(Bn, H, T, C, dk, dv, q.device)
        res = dict(B=Bn, T=T)
        for name, path in (("split", dla.DLA_PATH_AUTO), ("unsplit", dla.DLA_PATH_UNSPLIT)):
            dla.dla_set_prefill_path(path, 0)
            try:
                def call():
                    cache.reset()
                    dla.prefill(*xs, cfg.tau, cache, o=on, workspace=wsn)

                call()
                torch.cuda.synchronize()
                w0 = time.perf_counter()
                for _ in range(steps):
                    call()
                torch.cuda.synchronize()
                ms = (time.perf_counter() - w0) * 1e3 / steps
            finally:
                dla.dla_set_prefill_path(dla.DLA_PATH_AUTO, 0)
            res[f"{name}_ms_per_step"] = ms
            res[f"{name}_tokens_per_s"] = Bn * T / (ms * 1e-3)
        del cache, wsn, on, xs
        out.append(res)
        log(f"batch sweep B={Bn}: {res['split_ms_per_step']:.3f} ms (library's sweep), "
            f"{res['unsplit_ms_per_step']:.3f} ms unsplit")
    return out


def context_sweep(torch, dla, cfg, q, k, v, lam, lengths=(4096, 8192, 16384, 32768), steps=5):
    """Prefill tokens/s of DLA (summed-information merges, C = cfg.C) and of the
    Log-Linear fixed schedule (C = L(T')) on the first T' tokens of the
    workload's streams: wall time over `steps` calls after one warmup call."""
    B, H, dk, dv = cfg.B, cfg.H, cfg.dk, cfg.dv
    out = []
    for Tn in lengths:
        if Tn > cfg.T:
            continue
        L = (Tn - 1).bit_length() + 1
        qn, kn, vn = (x[:, :, :Tn].contiguous() for x in (q, k, v))
        lam_d = lam[:, :, :Tn].contiguous()
        lam_f = lam[:, :, :Tn, :L].contiguous()
        on = torch.empty(B, H, Tn, dv, dtype=q.dtype, device=q.device)
        res = dict(T=Tn)
        for name, rule, C, ln in (("dla", "sum", cfg.C, lam_d), ("fenwick", "fenwick", L, lam_f)):
            cache = dla.Cache(B, H, C, dk, dv, device=q.device, merge_rule=rule)
            wsn = dla.prefill_workspace(B, H, Tn, C, dk, dv, q.device)

            def call():
                cache.reset()
                dla.prefill(qn, kn, vn, ln, cfg.tau, cache, o=on, workspace=wsn)

            call()
            torch.cuda.synchronize()
            w0 = time.perf_counter()
            for _ in range(steps):
                call()
            torch.cuda.synchronize()
            ms = (time.perf_counter() - w0) * 1e3 / steps
            res[f"{name}_ms_per_step"] = ms
            res[f"{name}_tokens_per_s"] = B * Tn / (ms * 1e-3)
            del cache, wsn
        res["dla_over_fenwick_time"] = res["dla_ms_per_step"] / res["fenwick_ms_per_step"]
        out.append(res)
        log(f"context sweep T={Tn}: DLA {res['dla_ms_per_step']:.3f} ms, Log-Linear fixed schedule "
            f"{res['fenwick_ms_per_step']:.3f} ms, ratio {res['dla_over_fenwick_time']:.2f}")
    return out


def decode_inputs_tiled(torch, workloads, cfg, steps, dev, distinct):
    """The batched-decode workload from workloads.decode_inputs (the recipe the
    parity tests check): `distinct` caches and their step inputs drawn on the
    host, tiled over the B*H streams on the device (stream i gets draw
    i mod distinct); step inputs as [steps, B*H, d] bf16."""
    BH = cfg.B * cfg.H
    d = workloads.decode_inputs(cfg, caches=range(distinct), steps=steps)
    ti = torch.arange(BH, device=dev) % distinct

    def tile(a):          # [distinct, steps, n] -> [steps, B*H, n] bf16
        return torch.from_numpy(np.ascontiguousarray(np.swapaxes(a, 0, 1))).to(dev).to(torch.bfloat16)[:, ti]

    out = dict(states=torch.from_numpy(d["states"]).to(dev)[ti], info=torch.from_numpy(d["info"]).to(dev)[ti],
               count=torch.from_numpy(d["count"]).to(dev)[ti], start=torch.from_numpy(d["start"]).to(dev)[ti],
               t_seen=d["t_seen"])
    for x in ("q", "k", "v", "lam"):
        out[x] = tile(d[x])
    return out


def decode_bench(args, torch, dla, workloads, state_dtype="f32"):
    """Batched decode on preloaded full caches: every state fp32 ("f32"), or
    closed states bf16 and the most recent fp32 ("bf16")."""
    cfg = workloads.CONFIGS[args.decode_workload]
    B, H, C, dk, dv = cfg.B, cfg.H, cfg.C, cfg.dk, cfg.dv
    BH = B * H
    dev = torch.device("cuda:0")
    S, W = args.decode_steps, args.decode_warmup
    t0 = time.time()
    d = decode_inputs_tiled(torch, workloads, cfg, S + W, dev, args.decode_distinct)
    cache = dla.Cache(B, H, C, dk, dv, device=dev, state_dtype=state_dtype,
                      preload=dict(m0=C, states=d["states"], info=d["info"], count=d["count"],
                                   start=d["start"], t_seen=d["t_seen"]))
    del d["states"]
    torch.cuda.synchronize()
    log(f"decode inputs generated in {time.time() - t0:.1f}s")
    o = torch.empty(B, H, dv, dtype=torch.bfloat16, device=dev)
    bnd = torch.empty(S + W, BH, dtype=torch.uint8, device=dev)
    evi = torch.empty(S + W, BH, dtype=torch.int32, device=dev)
    mt = torch.empty(S + W, BH, dtype=torch.int32, device=dev)

    def step(j):
        dla.decode_step(d["q"][j].view(B, H, dk), d["k"][j].view(B, H, dk), d["v"][j].view(B, H, dv),
                        d["lam"][j].view(B, H, C), cfg.tau, cache, o=o,
                        sched=dict(boundary=bnd[j], ev_i=evi[j], m_t=mt[j]))

    for j in range(W):
        step(j)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(S)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for i, (a, b) in enumerate(evs):
        a.record()
        step(W + i)
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    kern = [a.elapsed_time(b) for a, b in evs]
    kern_avg = sum(kern) / S
    # algorithmic bytes: every live state read once, the states a step changes
    # written once; q, k, v, lam in, o out (bf16); the stream's metadata read
    # and written
    b_ = bnd[W:].to(torch.int64)
    e_ = evi[W:].to(torch.int64)
    m_prev = torch.cat([mt[W - 1:W] if W > 0 else torch.full((1, BH), C, dtype=torch.int32, device=dev),
                        mt[W:-1]], 0).to(torch.int64)
    D2 = dk * dv
    if state_dtype == "f32":
        # fp32 states: one written, or two for a merge away from the newest pair
        writes = torch.where((b_ == 1) & (e_ >= 0) & (e_ < m_prev - 1), 2, 1)
        st_bytes = (m_prev * 4 + writes * 4) * D2
    else:
        # m - 1 closed bf16 states and the fp32 active one read; written: the
        # active one (4 B) always, plus the closing active state (2 B) when a
        # new state opens without absorbing the token, plus a merged pair's
        # result (2 B) when the merge is not into the active state
        closes = (b_ == 1) & ((e_ < 0) | (e_ < m_prev - 2))
        merged = (b_ == 1) & (e_ >= 0) & (e_ < m_prev - 1)
        st_bytes = ((m_prev - 1) * 2 + 4 + 4 + 2 * closes.to(torch.int64) + 2 * merged.to(torch.int64)) * D2
    meta_rw = 2 * (32 + 64 + 20 * m_prev + 4 * dk)
    io_bytes = 2 * (2 * dk + dv + C + dv)
    total = (st_bytes + meta_rw + io_bytes).sum().item()
    bytes_per_step = total / S
    achieved = bytes_per_step / (kern_avg * 1e-3) / 1e9
    res = dict(
        workload=f"{args.decode_workload}", B=B, H=H, d_k=dk, d_v=dv, C=C, steps=S, warmup=W,
        state_dtype=state_dtype,
        steps_per_s=S / wall, ms_per_step=wall * 1e3 / S, tokens_per_s=BH * S / wall,
        boundaries_per_stream=float(b_.sum().item()) / BH,
        merges_per_stream=float((e_ >= 0).sum().item()) / BH,
        roofline=dict(bound="hbm", achieved=achieved, peak=PEAK_HBM_GBS, unit="GB/s",
                      frac=achieved / PEAK_HBM_GBS,
                      traffic=measured_traffic(f"k_decode_{args.decode_workload}_hbm_traffic.txt", "k_decode")
                      if state_dtype == "f32" else
                      measured_traffic(f"k_decode_bf16_states_{args.decode_workload}_hbm_traffic.txt",
                                       "k_decode(bf16 states)"),
                      kernel="k_decode",
                      kernel_ms=kern_avg, algorithmic_bytes_per_launch=bytes_per_step),
        inputs=f"workloads.decode_inputs: {args.decode_distinct} distinct caches and step inputs tiled over the "
               f"{BH} streams",
    )
    log(f"decode ({state_dtype} states): {res['steps_per_s']:.1f} steps/s, kernel {kern_avg:.3f} ms, "
        f"{achieved:.0f} GB/s algorithmic ({100 * achieved / PEAK_HBM_GBS:.1f}% of HBM peak)")
    return res


def fenwick_decode_bench(args, torch, dla, workloads):
    """Batched decode under the Log-Linear fixed schedule: the decode workload's
    shapes and token draws (lam = the level weights), caches preloaded with the
    one bucket of positions [0, 2^20), then S + W steps from there."""
    cfg = workloads.CONFIGS[args.decode_workload]
    B, H, C, dk, dv = cfg.B, cfg.H, cfg.C, cfg.dk, cfg.dv
    BH = B * H
    dev = torch.device("cuda:0")
    S, W = args.decode_steps, args.decode_warmup
    t0 = 1 << 20
    d = decode_inputs_tiled(torch, workloads, cfg, S + W, dev, args.decode_distinct)
    first = d.pop("states")[:, :1].contiguous()
    cache = dla.Cache(B, H, C, dk, dv, device=dev, merge_rule="fenwick",
                      preload=dict(m0=1, states=first, info=torch.zeros(BH, 1, dtype=torch.int64, device=dev),
                                   count=torch.full((BH, 1), t0, dtype=torch.int32, device=dev),
                                   start=torch.zeros(BH, 1, dtype=torch.int64, device=dev), t_seen=t0))
    del first
    torch.cuda.synchronize()
    o = torch.empty(B, H, dv, dtype=torch.bfloat16, device=dev)

    def step(j):
        dla.decode_step(d["q"][j].view(B, H, dk), d["k"][j].view(B, H, dk), d["v"][j].view(B, H, dv),
                        d["lam"][j].view(B, H, C), 0.0, cache, o=o)

    for j in range(W):
        step(j)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(S)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    for i, (a, b) in enumerate(evs):
        a.record()
        step(W + i)
        b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    kern_avg = sum(a.elapsed_time(b) for a, b in evs) / S
    # algorithmic bytes per stream-step at position t: the popcount(t) buckets
    # read and the token's bucket written (fp32), the metadata read and
    # written, q, k, v, lam in and o out (bf16)
    m_sum = sum(bin(t0 + W + i).count("1") for i in range(S))
    D2 = dk * dv
    per_stream = 4 * D2 * (m_sum + S) + 2 * (96 * S + 20 * m_sum) + 2 * (2 * dk + dv + C + dv) * S
    bytes_per_step = BH * per_stream / S
    achieved = bytes_per_step / (kern_avg * 1e-3) / 1e9
    res = dict(workload=f"{args.decode_workload}, Log-Linear fixed schedule from position 2^20",
               B=B, H=H, d_k=dk, d_v=dv, C=C, steps=S, warmup=W, steps_per_s=S / wall,
               ms_per_step=wall * 1e3 / S, tokens_per_s=BH * S / wall, mean_live_states=m_sum / S,
               roofline=dict(bound="hbm", achieved=achieved, peak=PEAK_HBM_GBS, unit="GB/s",
                             frac=achieved / PEAK_HBM_GBS, kernel="k_decode_fenwick", kernel_ms=kern_avg,
                             algorithmic_bytes_per_launch=bytes_per_step))
    log(f"decode, Log-Linear fixed schedule: {res['steps_per_s']:.1f} steps/s, kernel {kern_avg:.3f} ms, "
        f"{achieved:.0f} GB/s algorithmic ({100 * achieved / PEAK_HBM_GBS:.1f}% of HBM peak), "
        f"mean buckets read {m_sum / S:.2f}")
    del d, cache
    return res


def _kernel_file(kernel: str) -> str:
    """k_prefill_rs<128,16,8> -> k_prefill_rs_128_16_8 (a file-name form)."""
    return kernel.replace("<", "_").replace(">", "").replace(",", "_")


def cpu_baseline(args, sample, cfg):
    """The oracle as it stands on S streams x the first Ts tokens, one stream
    per thread on every CPU thread the process is granted (OMP_NUM_THREADS
    where it is set, else all host threads); Ts doubles from 512 until one run
    takes a third of the time budget, and that run is reported."""
    import oracle
    S = sample["k"].shape[0]
    granted = int(os.environ.get("OMP_NUM_THREADS") or 0) or (os.cpu_count() or 1)
    cores = min(S, granted)
    Ts = 512
    while True:
        t0 = time.perf_counter()
        oracle.run(*(sample[x][:, :Ts] for x in ("q", "k", "v", "lam")), cfg.C, cfg.tau,
                   final_states=False, nthreads=cores)
        dt = time.perf_counter() - t0
        if dt >= args.cpu_seconds / 3 or Ts >= cfg.T:
            break
        Ts = min(cfg.T, 2 * Ts)
    # a token of the layer is d_k x d_v work in each of the H heads
    val = S * Ts / dt / cfg.H
    log(f"cpu oracle: {S} streams x {Ts} tokens in {dt:.1f}s on {cores} threads "
        f"(host threads {os.cpu_count()}, granted {granted})")
    return dict(value=val, unit="tokens/s", cores=cores, kind="oracle",
                sample=f"{S} of {cfg.B * cfg.H} streams x first {Ts} of {cfg.T} tokens of the "
                       f"prefill workload (schedule, states and every output, float64), "
                       f"{dt:.1f} s; value = stream-tokens/s / H",
                host_threads=os.cpu_count(), granted_threads=granted, host_cpu=_cpu_model())


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="gdn_1p3b_t32k_bf16")
    ap.add_argument("--reading", default="relative", choices=["relative", "literal"])
    ap.add_argument("--decode-workload", default="decode_b256_bf16")
    ap.add_argument("--decode-steps", type=int, default=4096)
    ap.add_argument("--decode-warmup", type=int, default=8)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-bf16-states", action="store_true",
                    help="skip the second decode measurement on a cache with bf16 closed states")
    ap.add_argument("--no-density", action="store_true",
                    help="skip the second prefill measurement under the information-density merge rule")
    ap.add_argument("--no-literal", action="store_true",
                    help="skip the prefill measurement on the literal reading of the key noise")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the DLA vs Log-Linear context sweep")
    ap.add_argument("--no-fenwick", action="store_true",
                    help="skip the prefill measurement under the Log-Linear fixed schedule")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--cpu-streams", type=int, default=32)
    ap.add_argument("--decode-distinct", type=int, default=128,
                    help="distinct decode caches drawn on the host and tiled over the B*H streams")
    ap.add_argument("--no-streamed", action="store_true",
                    help="skip the prefill measurement on the streamed chunk kernel")
    ap.add_argument("--no-other", action="store_true",
                    help="skip the other prefill workloads (Mamba-2-shaped, long context, C=64, fp32, state score)")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="after the prefill, copy this many MiB three times (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures the layer on one GPU only (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE {world}): streams shard over GPUs with no communication, so a "
              f"multi-GPU figure is N independent copies of this one.", file=sys.stderr)
        sys.exit(2)

    import torch

    import dynamic_state_memory_amd as dla
    import workloads
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dla.load()
    pre, sample, cfg = prefill_bench(args, torch, dla, workloads)
    other = None if args.no_other else other_prefill_legs(args, torch, dla, workloads)
    copy_probe(torch, args.copy_probe_mib)
    dec = None if args.no_decode else decode_bench(args, torch, dla, workloads)
    torch.cuda.empty_cache()
    dec_bf = None if (args.no_decode or args.no_bf16_states) else \
        decode_bench(args, torch, dla, workloads, state_dtype="bf16")
    torch.cuda.empty_cache()
    dec_fen = None if (args.no_decode or args.no_fenwick) else fenwick_decode_bench(args, torch, dla, workloads)
    cpu = None if args.no_cpu else cpu_baseline(args, sample, cfg)
    out = {
        "metric": METRIC, "value": pre["value"], "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": pre["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic", "config": pre["config"], "roofline": pre["roofline"],
        "cpu_baseline": cpu, "decode": dec, "schedule": pre["schedule"],
        "token_heads_per_s": pre["token_heads_per_s"],
        "prefill_density_merge_rule": pre["density_rule"],
        "decode_bf16_states": dec_bf,
        "prefill_literal_reading": pre["literal"],
        "prefill_fenwick_schedule": pre["fenwick"],
        "prefill_context_sweep": pre["context_sweep"],
        "prefill_streamed_kernel": pre["streamed"],
        "prefill_workloads": other,
        "decode_fenwick_schedule": dec_fen,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
