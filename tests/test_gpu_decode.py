"""GPU parity of dla_decode_step: stream equivalence with prefill and the
oracle, and the batched-decode workload in its full launch configuration."""
import dataclasses

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_common import (STATE_TOL_BF16_STORAGE, TOL, compare_outputs, gpu_prefill, oracle_threads, say,
                              torch_mod)
from tests.helpers import mat_rel_err

pytestmark = pytest.mark.gpu


def _decode_steps_dev(cache, tq, tk, tv, tl, tau, B, H):
    """Run tq.shape[0] decode steps on device inputs [steps, B*H, d].  Returns
    the outputs [steps, B*H, d_v] and the per-step schedule, on the device."""
    torch = torch_mod()
    import dynamic_state_memory_amd as dla
    dev = tq.device
    n, BH = tq.shape[:2]
    sched = dict(s=torch.empty(n, BH, dtype=torch.float32, device=dev),
                 boundary=torch.empty(n, BH, dtype=torch.uint8, device=dev),
                 m_t=torch.empty(n, BH, dtype=torch.int32, device=dev),
                 ev_i=torch.empty(n, BH, dtype=torch.int32, device=dev))
    o = torch.empty(n, BH, tv.shape[2], dtype=tq.dtype, device=dev)
    for j in range(n):
        dla.decode_step(tq[j].view(B, H, -1), tk[j].view(B, H, -1), tv[j].view(B, H, -1),
                        tl[j].view(B, H, -1), tau, cache, o=o[j].view(B, H, -1),
                        sched={kk: vv[j] for kk, vv in sched.items()})
    torch.cuda.synchronize()
    return o, sched


def _decode_steps(cache, q, k, v, lam, tau, io, B, H):
    """Run q.shape[1] decode steps; inputs [S, steps, d] numpy.  Returns o and per-step schedule."""
    torch = torch_mod()
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if io == "bf16" else torch.float32

    def up(a):
        return torch.from_numpy(np.ascontiguousarray(np.swapaxes(a, 0, 1))).to(dev).to(dt)

    o, sched = _decode_steps_dev(cache, up(q), up(k), up(v), up(lam), tau, B, H)
    out = o.float().cpu().numpy().swapaxes(0, 1)
    return out, {kk: vv.cpu().numpy().swapaxes(0, 1) for kk, vv in sched.items()}


def _merge_log(r, S, n):
    """Oracle merges as a per-step array (-1 = none)."""
    ev = np.full((S, n), -1, np.int32)
    for i in range(S):
        for t, e in r["events"][i]:
            ev[i, t] = e
    return ev


def _config(name):
    """A workload, or a variant of one with other key and value widths."""
    extra = {"dk256_dv128_bf16": ("long_t131k_bf16", dict(dk=256, dv=128, C=24)),
             "dk64_dv256_bf16": ("gdn_1p3b_t32k_bf16", dict(dk=64, dv=256, C=16)),
             "dk128_f32": ("tiny_fp32", dict(dk=128, dv=64, C=12))}
    if name in extra:
        base, kw = extra[name]
        return dataclasses.replace(workloads.CONFIGS[base], **kw)
    return workloads.CONFIGS[name]


@pytest.mark.parametrize("name,io,T,j,means,rule,sdt", [
    ("tiny_fp32", "f32", 512, 100, None, "sum", "f32"),
    ("mamba2_780m_bf16", "bf16", 1300, 200, (20,), "sum", "f32"),
    ("mamba2_780m_bf16", "bf16", 1300, 200, (20,), "density", "bf16"),
    ("gdn_1p3b_t32k_bf16", "bf16", 1100, 150, (16, 60), "sum", "f32"),
    ("gdn_1p3b_t32k_bf16", "bf16", 1100, 150, (16, 60), "sum", "bf16"),
    ("dk256_dv128_bf16", "bf16", 900, 120, (20,), "sum", "f32"),
    ("dk64_dv256_bf16", "bf16", 900, 120, (20,), "density", "f32"),
    ("dk128_f32", "f32", 700, 100, (20,), "sum", "f32"),
    ("long_t131k_bf16", "bf16", 1500, 300, (20,), "sum", "f32"),
    ("long_t131k_bf16", "bf16", 1500, 300, (20,), "density", "f32"),
    ("tiny_fp32", "f32", 512, 100, None, "density", "f32"),
    ("long_t131k_bf16", "bf16", 1500, 300, (20,), "sum", "bf16"),
    ("long_t131k_bf16", "bf16", 1500, 300, (20,), "density", "bf16"),
])
def test_prefill_then_decode_equals_one_prefill(name, io, T, j, means, rule, sdt):
    """Prefill T - j tokens, then j decode steps on the same cache: the
    outputs, the schedule of the decode steps and the final cache are those of
    one oracle pass over the T tokens (the cache carries the stream, whatever
    d_k and d_v)."""
    torch = torch_mod()
    import dynamic_state_memory_amd as dla
    cfg = _config(name)
    if means is not None:
        cfg = dataclasses.replace(cfg, seg_means=means)
    streams = [0] if cfg.B * cfg.H == 1 else [0, 1, 2]
    d = workloads.prefill_inputs(cfg, streams=streams, T=T)
    S = len(streams)
    say(f"decode equivalence {name} ({rule} rule, {sdt} states): prefill {T - j} + {j} steps")
    r = oracle.run(d["q"], d["k"], d["v"], d["lam"], cfg.C, cfg.tau, nthreads=oracle_threads(), merge_rule=rule)
    # prefill of the first T - j tokens
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    cache = dla.Cache(1, S, cfg.C, cfg.dk, cfg.dv, device=dev, merge_rule=rule, state_dtype=sdt)

    def up(a, d_):
        return torch.from_numpy(np.ascontiguousarray(a[:, :T - j])).to(dev).to(dt).reshape(1, S, T - j, d_)

    o1 = dla.prefill(up(d["q"], cfg.dk), up(d["k"], cfg.dk), up(d["v"], cfg.dv), up(d["lam"], cfg.C),
                     cfg.tau, cache)
    torch.cuda.synchronize()
    o1 = o1.float().cpu().numpy().reshape(S, T - j, cfg.dv)
    o2, sc = _decode_steps(cache, d["q"][:, T - j:], d["k"][:, T - j:], d["v"][:, T - j:],
                           d["lam"][:, T - j:], cfg.tau, io, 1, S)
    compare_outputs(o1, r["o"][:, :T - j], TOL[io], "prefill part")
    compare_outputs(o2, r["o"][:, T - j:], TOL[io], "decode part")
    assert np.array_equal(sc["s"].view(np.uint32), r["s"][:, T - j:].view(np.uint32))
    assert np.array_equal(sc["boundary"], r["b"][:, T - j:])
    assert np.array_equal(sc["m_t"], r["m_t"][:, T - j:])
    assert np.array_equal(sc["ev_i"], _merge_log(r, S, T)[:, T - j:])
    fin = cache.read()
    assert np.array_equal(fin["m"], r["fin_m"])
    for i in range(S):
        m = int(r["fin_m"][i])
        assert np.array_equal(fin["start"][i, :m], r["fin_start"][i, :m])
        assert np.array_equal(fin["info"][i, :m], r["fin_I"][i, :m])
        tol = STATE_TOL_BF16_STORAGE if sdt == "bf16" else 1e-4
        assert mat_rel_err(fin["S"][i, :m], r["fin_S"][i, :m]) <= tol
        # the most recent state is fp32 either way
        assert mat_rel_err(fin["S"][i, m - 1:m], r["fin_S"][i, m - 1:m]) <= 1e-4
    say(f"decode equivalence {name}: ok")


@pytest.mark.parametrize("sdt", ["f32", "bf16"])
@pytest.mark.parametrize("rule", ["sum", "density"])
def test_prefill_decode_prefill_is_one_stream(rule, sdt):
    """Prefill, decode steps, then another prefill on the same cache: the
    outputs and final cache equal one pass over all the tokens (oracle)."""
    torch = torch_mod()
    import dynamic_state_memory_amd as dla
    cfg = dataclasses.replace(workloads.CONFIGS["long_t131k_bf16"], C=16, seg_means=(7,))
    T1, T2, T3 = 330, 57, 401
    T = T1 + T2 + T3
    d = workloads.prefill_inputs(cfg, streams=[0, 1, 2], T=T)
    S = 3
    say(f"prefill {T1} + decode {T2} + prefill {T3} ({rule} rule, {sdt} states)")
    r = oracle.run(d["q"], d["k"], d["v"], d["lam"], cfg.C, cfg.tau, nthreads=oracle_threads(), merge_rule=rule)
    dev = torch.device("cuda:0")
    cache = dla.Cache(1, S, cfg.C, cfg.dk, cfg.dv, device=dev, merge_rule=rule, state_dtype=sdt)

    def up(a, lo, hi, d_):
        return torch.from_numpy(np.ascontiguousarray(a[:, lo:hi])).to(dev).to(torch.bfloat16).reshape(1, S, hi - lo, d_)

    def pre(lo, hi):
        o = dla.prefill(up(d["q"], lo, hi, cfg.dk), up(d["k"], lo, hi, cfg.dk), up(d["v"], lo, hi, cfg.dv),
                        up(d["lam"], lo, hi, cfg.C), cfg.tau, cache)
        torch.cuda.synchronize()
        return o.float().cpu().numpy().reshape(S, hi - lo, cfg.dv)

    o1 = pre(0, T1)
    o2, _ = _decode_steps(cache, d["q"][:, T1:T1 + T2], d["k"][:, T1:T1 + T2], d["v"][:, T1:T1 + T2],
                          d["lam"][:, T1:T1 + T2], cfg.tau, "bf16", 1, S)
    o3 = pre(T1 + T2, T)
    compare_outputs(np.concatenate([o1, o2, o3], 1), r["o"], TOL["bf16"], "prefill-decode-prefill")
    fin = cache.read()
    assert np.array_equal(fin["m"], r["fin_m"]) and np.array_equal(fin["t_seen"], r["fin_t_seen"])
    tol = STATE_TOL_BF16_STORAGE if sdt == "bf16" else 1e-4
    for i in range(S):
        m = int(r["fin_m"][i])
        assert fin["start"][i, :m].tolist() == r["fin_start"][i, :m].tolist()
        assert fin["info"][i, :m].tolist() == r["fin_I"][i, :m].tolist()
        assert fin["count"][i, :m].tolist() == r["fin_n"][i, :m].tolist()
        assert mat_rel_err(fin["S"][i, :m], r["fin_S"][i, :m]) <= tol
    assert r["n_ev"].min() > 0
    say("prefill-decode-prefill: ok")


@pytest.mark.parametrize("B,H,n_unique,steps,rule,sdt", [
    (1, 32, 32, 4096, "sum", "f32"), (256, 16, 32, 400, "sum", "f32"), (1, 32, 32, 1000, "density", "f32"),
    (1, 32, 32, 4096, "sum", "bf16"), (256, 16, 32, 400, "sum", "bf16"), (1, 32, 32, 1000, "density", "bf16")])
def test_batched_decode_workload(B, H, n_unique, steps, rule, sdt):
    """Full caches preloaded, then steps of fresh tokens: 32 distinct caches
    over all 4096 steps of the workload (B=1, H=32), and the full launch
    configuration (B=256, H=16) with the 32 caches tiled over its 4096
    streams.  The first 32 streams are checked against the oracle (outputs,
    every step's schedule, the whole final cache); every other stream must
    equal its tile's first copy bit for bit, outputs, schedule and final
    cache."""
    torch = torch_mod()
    import dynamic_state_memory_amd as dla
    d = workloads.decode_inputs(caches=range(n_unique), steps=steps)
    cfg = d["cfg"]
    C, dk, dv = cfg.C, cfg.dk, cfg.dv
    S, BH = n_unique, B * H
    say(f"batched decode B={B} H={H} unique={S} steps={steps} ({rule} rule, {sdt} states): oracle")
    init = dict(m=np.full(S, C, np.int32), S=d["states"], I=d["info"], n=d["count"], start=d["start"],
                has_prev=np.zeros(S, np.int32), s_prev=np.ones(S, np.float32),
                k_prev=np.zeros((S, dk), np.float32), t_seen=np.full(S, d["t_seen"], np.int64))
    r = oracle.run(d["q"], d["k"], d["v"], d["lam"], C, cfg.tau, init=init, nthreads=oracle_threads(),
                   merge_rule=rule)
    if rule == "density":
        r_sum = oracle.run(d["q"], d["k"], d["v"], d["lam"], C, cfg.tau, init=init, outputs=False,
                           final_states=False, nthreads=oracle_threads())
        assert any(a != b for a, b in zip(r["events"], r_sum["events"])), "the two rules agree on this input"
    dev = torch.device("cuda:0")
    say(f"batched decode B={B} H={H}: GPU")
    ti = torch.arange(BH, device=dev) % S          # stream -> its distinct cache
    pre = dict(m0=C, states=torch.from_numpy(d["states"]).to(dev)[ti],
               info=torch.from_numpy(d["info"]).to(dev)[ti],
               count=torch.from_numpy(d["count"]).to(dev)[ti],
               start=torch.from_numpy(d["start"]).to(dev)[ti], t_seen=d["t_seen"])
    cache = dla.Cache(B, H, C, dk, dv, device=dev, preload=pre, merge_rule=rule, state_dtype=sdt)
    del pre

    def up(a):      # [S, steps, d] numpy -> [steps, B*H, d] bf16 on the device, tiled
        return torch.from_numpy(np.ascontiguousarray(np.swapaxes(a, 0, 1))).to(dev).to(torch.bfloat16)[:, ti]

    o, sc = _decode_steps_dev(cache, up(d["q"]), up(d["k"]), up(d["v"]), up(d["lam"]), cfg.tau, B, H)
    # every stream equals the first copy of its cache, bit for bit
    for x in [o.view(torch.int16)] + list(sc.values()):
        assert torch.equal(x, x[:, ti]), "tiled copies of one cache differ"
    o1 = o[:, :S].float().cpu().numpy().swapaxes(0, 1)
    s1 = {kk: vv[:, :S].cpu().numpy().swapaxes(0, 1) for kk, vv in sc.items()}
    compare_outputs(o1, r["o"], TOL["bf16"], "decode outputs")
    assert np.array_equal(s1["s"].view(np.uint32), r["s"].view(np.uint32))
    assert np.array_equal(s1["boundary"], r["b"])
    assert np.array_equal(s1["m_t"], r["m_t"])
    assert np.array_equal(s1["ev_i"], _merge_log(r, S, steps))
    # the first step has no previous key: s = 1 opens a state and forces a merge
    assert np.all(s1["s"][:, 0] == 1.0) and np.all(s1["ev_i"][:, 0] >= 0)
    # the whole final cache of the distinct streams against the oracle
    fin = cache.read(streams=range(S))
    tol = STATE_TOL_BF16_STORAGE if sdt == "bf16" else 1e-4
    assert np.array_equal(fin["m"], r["fin_m"]) and np.array_equal(fin["t_seen"], r["fin_t_seen"])
    for i in range(S):
        m = int(r["fin_m"][i])
        assert fin["start"][i, :m].tolist() == r["fin_start"][i, :m].tolist()
        assert fin["info"][i, :m].tolist() == r["fin_I"][i, :m].tolist()
        assert fin["count"][i, :m].tolist() == r["fin_n"][i, :m].tolist()
        assert mat_rel_err(fin["S"][i, :m], r["fin_S"][i, :m]) <= tol
        assert mat_rel_err(fin["S"][i, m - 1:m], r["fin_S"][i, m - 1:m]) <= 1e-4
    assert np.array_equal(fin["k_prev"], r["fin_k_prev"]) and np.array_equal(fin["s_prev"], r["fin_s_prev"])
    if BH > S:
        # the last tile's final cache equals the first one's
        last = cache.read(streams=range(BH - S, BH))
        for key in ("m", "info", "count", "start", "t_seen", "s_prev", "k_prev"):
            assert np.array_equal(last[key], fin[key]), key
        assert np.array_equal(last["S"].view(np.uint32), fin["S"].view(np.uint32))
    say(f"batched decode B={B} H={H}: ok, merges/stream {r['n_ev'].mean():.1f}")
