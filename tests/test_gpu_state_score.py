"""GPU parity of the state information score (a cache with score rule
"state"; reading notes "Dynamic Linear Attention | Chlience Paper Archive",
section 5.1) against the oracle: prefill on both chunk kernels, prefill
continuing a cache, and decode steps after a prefill.

The GPU reads the current state through fp16 halves on MFMA and the oracle in
fp64, so the scores agree to about 1e-6, not bit for bit: the tests take
inputs whose every boundary decision has a margin to tau above 1e-4 and whose
every capacity merge has a relative key gap above 1e-4 (asserted on the
oracle's schedule), and then require the boundaries, merges, segment ids,
state counts and starts to be exact, the scores within 2e-5, the
information sums within that per token, the outputs and final states within
their gates; the GPU's own schedule must also be exactly what the greedy rule
makes of its own scores (the independent checker)."""
import dataclasses
from fractions import Fraction

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_common import (STATE_TOL, STATE_TOL_BF16_STORAGE, TOL, compare_schedule, compare_states, gpu_prefill,
                              gpu_prefill_pieces, oracle_threads, say, torch_mod)
from tests.helpers import mat_rel_err

pytestmark = pytest.mark.gpu
S_TOL = 2e-5
MARGIN = 1e-4


def compare_outputs(o_gpu, o_ref, tol, label="", mask=None):
    """The per-row error of the other parity tests, with a floor under each
    row's scale: 5e-2 of the median row maximum.  With values that follow the
    key segments, a state is close to rank one (n v k^T), and a query nearly
    orthogonal to its key direction gives an output row near zero (down to
    three orders of magnitude below the others on these inputs), whose
    relative error measures cancellation, not the kernels."""
    o_gpu = np.asarray(o_gpu, np.float64)
    o_ref = np.asarray(o_ref, np.float64)
    if mask is not None:
        o_gpu, o_ref = o_gpu[mask], o_ref[mask]
    g = o_gpu.reshape(-1, o_gpu.shape[-1])
    r = o_ref.reshape(-1, o_ref.shape[-1])
    if len(r) == 0:
        return 0.0
    scale = np.abs(r).max(1)
    den = np.maximum(scale, 5e-2 * np.median(scale))
    den = np.where(den == 0, 1.0, den)
    err = float((np.abs(g - r).max(1) / den).max())
    assert err <= tol, f"{label}: outputs max row rel err {err:.3e} > {tol}"
    return err


def _first_unpinned(r, tau, C, merge_rule):
    """Per stream, the first token whose decision is not pinned by the
    oracle: a score within MARGIN of tau, or a capacity merge whose two best
    keys are within MARGIN (relative); T if there is none.  Up to there the
    GPU must reproduce the oracle's schedule exactly (several schedules are
    correct past such a near tie)."""
    S_, T = r["s"].shape
    out = np.full(S_, T, np.int64)
    for i in range(S_):
        q = oracle.fixed_point(r["s"][i])
        starts, m_prev = [], 0
        for t in range(T):
            if m_prev > 0 and abs(float(r["s"][i, t]) - tau) <= MARGIN:
                out[i] = t
                break
            if r["b"][i, t]:
                starts.append(t)
                if len(starts) > C:
                    ends = starts[1:] + [t + 1]
                    I = [int(q[a:e].sum()) for a, e in zip(starts, ends)]
                    n = [e - a for a, e in zip(starts, ends)]
                    if merge_rule == "sum":
                        keys = [Fraction(I[j] + I[j + 1]) for j in range(len(I) - 1)]
                    else:
                        keys = [Fraction(I[j] + I[j + 1], n[j] + n[j + 1]) for j in range(len(I) - 1)]
                    order = sorted(range(len(keys)), key=lambda j: (keys[j], j))
                    # (with C = 1 there is one pair: no tie)
                    if len(keys) > 1 and float(keys[order[1]] - keys[order[0]]) <= MARGIN * float(keys[order[0]]):
                        out[i] = t
                        break
                    del starts[order[0] + 1]
            m_prev = int(r["m_t"][i, t])
    return out


def _valid_schedule(d, i, sc, tau, C, merge_rule, o=None, rows=None):
    """The GPU's own schedule of stream i is what the rules make of its own
    scores (independent checker), and its scores and sampled outputs are the
    closed form and the slot-weighted sum on that schedule."""
    n = int(sc["n_ev"][i])
    events = list(zip(sc["ev_t"][i, :n].tolist(), sc["ev_i"][i, :n].tolist()))
    oracle.check_schedule(sc["s"][i], tau, C, sc["boundary"][i], events, m_t=sc["m_t"][i],
                          merge_rule=merge_rule, score_rule="state")
    T = d["k"].shape[1]
    sets = oracle.start_sets(T, sc["boundary"][i], events)
    ref = oracle.state_scores_closed_form(d["v"][i], d["k"][i], sets)
    assert np.abs(ref - sc["s"][i]).max() <= S_TOL, f"stream {i}: scores off their closed form"
    if o is not None:
        bf = oracle.brute_force(d["q"][i], d["k"][i], d["v"][i], d["lam"][i], sets, rows=rows)
        compare_outputs(o[i, rows], bf[rows], TOL["bf16"], f"stream {i} on its own schedule")
    return sets


def _check(d, C, tau, io, label, merge_rule="sum", state_dtype="f32", B=None, H=None):
    say(f"state score {label}: S={d['k'].shape[0]} T={d['k'].shape[1]} dk={d['k'].shape[2]} dv={d['v'].shape[2]} "
        f"C={C} tau={tau} io={io} merge={merge_rule} states={state_dtype}")
    r = oracle.run(d["q"], d["k"], d["v"], d["lam"], C, tau, nthreads=oracle_threads(), merge_rule=merge_rule,
                   score_rule="state")
    p = _first_unpinned(r, tau, C, merge_rule)
    o, sc, fin = gpu_prefill(d["q"], d["k"], d["v"], d["lam"], C, tau, io, B=B, H=H, merge_rule=merge_rule,
                             state_dtype=state_dtype, score_rule="state")
    S_, T = r["s"].shape
    tol = TOL["bf16"] if state_dtype == "bf16" else TOL[io]
    tol_state = STATE_TOL_BF16_STORAGE if state_dtype == "bf16" else STATE_TOL
    pinned = [i for i in range(S_) if p[i] == T]
    if pinned:
        sub = lambda x: {k: (v[pinned] if isinstance(v, np.ndarray) and v.shape[:1] == (S_,) else v)
                         for k, v in x.items()}
        rr = sub(r)
        rr["events"] = [r["events"][i] for i in pinned]
        compare_schedule(rr, sub(sc), sub(fin), label, s_tol=S_TOL)
        compare_states(rr, sub(fin), tol=tol_state, label=label)
        compare_outputs(o[pinned], r["o"][pinned], tol, label)
    for i in range(S_):
        # up to the first unpinned decision: the oracle's schedule exactly
        n = p[i]
        assert np.array_equal(sc["boundary"][i, :n], r["b"][i, :n]), f"{label}: boundaries differ ({i})"
        assert np.array_equal(sc["m_t"][i, :n], r["m_t"][i, :n]), f"{label}: state counts differ ({i})"
        assert np.abs(sc["s"][i, :n] - r["s"][i, :n]).max(initial=0.0) <= S_TOL, f"{label}: scores differ ({i})"
        compare_outputs(o[i, :n], r["o"][i, :n], tol, f"{label} stream {i} before {n}")
        rows = None if n == T else sorted(set(range(n, T, max(1, (T - n) // 12))) | {T - 1})
        sets = _valid_schedule(d, i, sc, tau, C, merge_rule, o=None if n == T else o, rows=rows)
        if n < T:
            # the final states: the sums over the GPU's own final token ranges
            P = sets[-1]
            m = len(P)
            assert int(fin["m"][i]) == m and fin["start"][i, :m].tolist() == list(P)
            ends = list(P[1:]) + [T]
            V, K = d["v"][i].astype(np.float64), d["k"][i].astype(np.float64)
            ref = np.stack([V[a:e].T @ K[a:e] for a, e in zip(P, ends)])
            assert mat_rel_err(fin["S"][i, :m], ref) <= tol_state, f"{label}: final states ({i})"
    say(f"state score {label}: ok, pinned streams {len(pinned)}/{S_}, boundaries {int(r['b'].sum())}, "
        f"merges {int(r['n_ev'].sum())}")
    return r


@pytest.fixture(params=["register", "streamed"])
def prefill_path(request):
    import dynamic_state_memory_amd as dla
    dla.dla_set_prefill_path(dla.DLA_PATH_STREAMED if request.param == "streamed" else dla.DLA_PATH_AUTO, 0)
    yield request.param
    dla.dla_set_prefill_path(dla.DLA_PATH_AUTO, 0)


CASES = [
    # (workload, d_k, d_v, C, T, segment means, merge rule, state dtype)
    ("gdn_1p3b_t32k_bf16", 128, 256, 8, 1500, (20, 90), "sum", "f32"),
    ("mamba2_780m_bf16", 128, 64, 6, 2100, (25,), "density", "f32"),
    ("long_t131k_bf16", 128, 128, 5, 1300, (30,), "sum", "bf16"),
    ("long_t131k_bf16", 64, 128, 4, 999, (15,), "sum", "f32"),
    ("long_t131k_bf16", 256, 64, 6, 777, (18,), "density", "f32"),
    ("gdn_1p3b_t32k_bf16", 64, 256, 7, 640, (20,), "sum", "f32"),
    # capacities 1 to 3: the scan's runs of merges into the newest pair with
    # one state (no pair before it) and two (no older pair)
    ("long_t131k_bf16", 128, 128, 1, 900, (12,), "sum", "f32"),
    ("mamba2_780m_bf16", 128, 64, 2, 1100, (15,), "sum", "f32"),
    ("mamba2_780m_bf16", 128, 64, 3, 1000, (10,), "sum", "f32"),
]


@pytest.mark.parametrize("name,dk,dv,C,T,means,rule,sdt", CASES)
def test_state_score_prefill(name, dk, dv, C, T, means, rule, sdt, prefill_path):
    torch_mod()
    cfg = dataclasses.replace(workloads.CONFIGS[name], dk=dk, dv=dv, C=C, seg_means=means)
    d = workloads.prefill_inputs(cfg, streams=[0, 1, 2], T=T, values="regime")
    r = _check(d, C, 0.6, "bf16", f"{name} dk={dk} dv={dv} {prefill_path}", merge_rule=rule, state_dtype=sdt)
    assert r["n_ev"].sum() > 0


def test_state_score_fp32_io():
    torch_mod()
    cfg = dataclasses.replace(workloads.CONFIGS["tiny_fp32"], H=2, C=4, seg_means=(20,))
    d = workloads.prefill_inputs(cfg, streams=[0, 1], values="regime")
    _check(d, 4, 0.6, "f32", "tiny fp32")


def test_state_score_random_values_every_token_opens():
    """The workloads' independent random values: every per-token state is
    nearly orthogonal to the current state (I near sqrt 2), so every token
    opens a state and merges."""
    torch_mod()
    cfg = workloads.CONFIGS["gdn_1p3b_t32k_bf16"]
    d = workloads.prefill_inputs(cfg, streams=[0, 1], T=400)
    r = _check(d, cfg.C, 0.6, "bf16", "random values")
    assert r["b"].all() and r["n_ev"].min() == 400 - cfg.C


def test_state_score_full_launch_sampled():
    """The Mamba-2-780M-shaped layer at its full batch (B=4, H=24) over 2048
    tokens with regime values: whole schedule and final cache, outputs at
    sampled tokens."""
    torch_mod()
    cfg = dataclasses.replace(workloads.CONFIGS["mamba2_780m_bf16"], seg_means=(40,), C=12)
    d = workloads.prefill_inputs(cfg, T=2048, values="regime")
    S, T = d["k"].shape[:2]
    r = oracle.run(d["q"], d["k"], d["v"], d["lam"], cfg.C, 0.6, nthreads=oracle_threads(), score_rule="state",
                   outputs=False)
    p = _first_unpinned(r, 0.6, cfg.C, "sum")
    rng = np.random.default_rng(5)
    want = np.zeros((S, T), bool)
    for i in range(S):
        want[i, rng.choice(T, 16, replace=False)] = True
        want[i, [0, 63, 64, T - 1]] = True
    ro = oracle.run(d["q"], d["k"], d["v"], d["lam"], cfg.C, 0.6, nthreads=oracle_threads(), score_rule="state",
                    want=want, final_states=False)
    say("state score full launch: GPU")
    o, sc, fin = gpu_prefill(d["q"], d["k"], d["v"], d["lam"], cfg.C, 0.6, "bf16", B=cfg.B, H=cfg.H,
                             score_rule="state")
    pinned = p == T
    assert pinned.mean() > 0.5, "most streams of the launch are pinned"
    for i in range(S):
        n = p[i]
        assert np.array_equal(sc["boundary"][i, :n], r["b"][i, :n]) and np.array_equal(sc["m_t"][i, :n], r["m_t"][i, :n])
        assert np.abs(sc["s"][i, :n] - r["s"][i, :n]).max(initial=0.0) <= S_TOL
        w = want[i].copy()
        w[n:] = False
        compare_outputs(o[i][w], ro["o"][i][w], TOL["bf16"], f"full launch stream {i}")
        if pinned[i]:
            m = int(r["fin_m"][i])
            assert fin["start"][i, :m].tolist() == r["fin_start"][i, :m].tolist()
            assert mat_rel_err(fin["S"][i, :m], r["fin_S"][i, :m]) <= STATE_TOL
        else:
            _valid_schedule(d, i, sc, 0.6, cfg.C, "sum")


# (seeds whose every decision has a margin: see _first_unpinned)
@pytest.mark.parametrize("rule,sdt,seed", [("sum", "f32", 101), ("density", "bf16", 128)])
def test_state_score_prefill_continues_the_cache(rule, sdt, seed):
    torch_mod()
    cfg = dataclasses.replace(workloads.CONFIGS["long_t131k_bf16"], C=5, seg_means=(20,))
    ends = (300, 301, 700, 1100)
    d = workloads.prefill_inputs(cfg, streams=[0, 1, 2], T=ends[-1], values="regime", seed=seed)
    r = oracle.run(d["q"], d["k"], d["v"], d["lam"], cfg.C, 0.6, nthreads=oracle_threads(), merge_rule=rule,
                   score_rule="state")
    assert (_first_unpinned(r, 0.6, cfg.C, rule) == ends[-1]).all(), "inputs with every decision pinned"
    say(f"state score prefill pieces {ends} ({rule}, {sdt})")
    o, scheds, fin = gpu_prefill_pieces(d["q"], d["k"], d["v"], d["lam"], cfg.C, 0.6, "bf16", ends,
                                        merge_rule=rule, state_dtype=sdt, score_rule="state")
    b = np.concatenate([x["boundary"] for x in scheds], 1)
    s = np.concatenate([x["s"] for x in scheds], 1)
    assert np.array_equal(b, r["b"]) and np.abs(s - r["s"]).max() <= S_TOL
    compare_outputs(o, r["o"], TOL["bf16"], "pieces")
    tol = STATE_TOL_BF16_STORAGE if sdt == "bf16" else STATE_TOL
    for i in range(3):
        m = int(r["fin_m"][i])
        assert fin["start"][i, :m].tolist() == r["fin_start"][i, :m].tolist()
        assert mat_rel_err(fin["S"][i, :m], r["fin_S"][i, :m]) <= tol


@pytest.mark.parametrize("name,dk,dv,io,rule,sdt,seed", [("long_t131k_bf16", 128, 128, "bf16", "sum", "f32", None),
                                                         ("gdn_1p3b_t32k_bf16", 128, 256, "bf16", "density", "f32", 117),
                                                         ("mamba2_780m_bf16", 128, 64, "bf16", "sum", "bf16", None),
                                                         ("tiny_fp32", 64, 64, "f32", "sum", "f32", None)])
def test_state_score_decode_after_prefill(name, dk, dv, io, rule, sdt, seed):
    """Prefill, then decode steps with the state score: the decode step scores
    each token against the current state it reads first."""
    torch = torch_mod()
    import dynamic_state_memory_amd as dla
    from tests.test_gpu_decode import _decode_steps, _merge_log
    # (C = 8: every step's lam row 16-byte aligned)
    cfg = dataclasses.replace(workloads.CONFIGS[name], H=max(workloads.CONFIGS[name].H, 2), dk=dk, dv=dv, C=8,
                              seg_means=(20,))
    T, j = 900, 150
    d = workloads.prefill_inputs(cfg, streams=[0, 1], T=T, values="regime", seed=seed)
    r = oracle.run(d["q"], d["k"], d["v"], d["lam"], cfg.C, 0.6, nthreads=oracle_threads(), merge_rule=rule,
                   score_rule="state")
    assert (_first_unpinned(r, 0.6, cfg.C, rule) == T).all(), "inputs with every decision pinned"
    say(f"state score decode {name} ({rule}, {sdt}): prefill {T - j} + {j} steps")
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    cache = dla.Cache(1, 2, cfg.C, dk, dv, device=dev, merge_rule=rule, state_dtype=sdt, score_rule="state")

    def up(a, d_):
        return torch.from_numpy(np.ascontiguousarray(a[:, :T - j])).to(dev).to(dt).reshape(1, 2, T - j, d_)

    o1 = dla.prefill(up(d["q"], dk), up(d["k"], dk), up(d["v"], dv), up(d["lam"], cfg.C), 0.6, cache)
    torch.cuda.synchronize()
    o1 = o1.float().cpu().numpy().reshape(2, T - j, dv)
    o2, sc = _decode_steps(cache, d["q"][:, T - j:], d["k"][:, T - j:], d["v"][:, T - j:], d["lam"][:, T - j:],
                           0.6, io, 1, 2)
    tol = TOL["bf16"] if sdt == "bf16" else TOL[io]
    compare_outputs(o1, r["o"][:, :T - j], tol, "prefill part")
    compare_outputs(o2, r["o"][:, T - j:], tol, "decode part")
    assert np.abs(sc["s"] - r["s"][:, T - j:]).max() <= S_TOL
    assert np.array_equal(sc["boundary"], r["b"][:, T - j:])
    assert np.array_equal(sc["m_t"], r["m_t"][:, T - j:])
    assert np.array_equal(sc["ev_i"], _merge_log(r, 2, T)[:, T - j:])
    fin = cache.read()
    stol = STATE_TOL_BF16_STORAGE if sdt == "bf16" else STATE_TOL
    for i in range(2):
        m = int(r["fin_m"][i])
        assert fin["start"][i, :m].tolist() == r["fin_start"][i, :m].tolist()
        assert mat_rel_err(fin["S"][i, :m], r["fin_S"][i, :m]) <= stol
