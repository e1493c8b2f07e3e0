"""The register-resident sweep split along the sequence.

A sweep grid that fills at most half of the device's block slots (few
streams, narrow values) is run as up to four block sets per stream: set s
takes the chunks before its range for their state updates only, then sweeps
its range in full.  The updates and merges are the same operations in the
same order as in the unsplit sweep, so outputs and final caches must equal
the unsplit sweep's bit for bit (DLA_PATH_UNSPLIT turns the split off), and
both must be one pass of the oracle."""
import dataclasses

import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_common import (TOL, compare_outputs, compare_schedule, compare_states, gpu_prefill,
                              gpu_prefill_pieces, oracle_threads, say, torch_mod)

pytestmark = pytest.mark.gpu

CASES = [
    # (workload, streams, T, C, segment means, merge rule): 8 to 24 blocks per
    # unsplit grid, 2 to 4 block sets
    ("long_t131k_bf16", [0, 1], 4096, 32, None, "sum"),
    ("long_t131k_bf16", [2], 2001, 32, (24,), "density"),
    ("mamba2_780m_bf16", [0, 1, 2], 1500, 16, (12, 90), "sum"),
    ("gdn_1p3b_t32k_bf16", [3], 3137, 32, None, "sum"),
    ("mamba2_780m_bf16", [4], 530, 8, (6,), "sum"),
]


def _both(d, C, tau, merge_rule, score_rule="cosine"):
    import dynamic_state_memory_amd as dla
    a = gpu_prefill(d["q"], d["k"], d["v"], d["lam"], C, tau, "bf16", merge_rule=merge_rule, score_rule=score_rule)
    dla.dla_set_prefill_path(dla.DLA_PATH_UNSPLIT, 0)
    try:
        b = gpu_prefill(d["q"], d["k"], d["v"], d["lam"], C, tau, "bf16", merge_rule=merge_rule,
                        score_rule=score_rule)
    finally:
        dla.dla_set_prefill_path(dla.DLA_PATH_AUTO, 0)
    return a, b


def _same(a, b, label):
    (o1, sc1, fin1), (o2, sc2, fin2) = a, b
    assert np.array_equal(o1, o2), f"{label}: outputs differ from the unsplit sweep"
    for key in sc1:
        assert np.array_equal(sc1[key], sc2[key]), f"{label}: schedule {key} differs"
    for key in fin1:
        assert np.array_equal(np.asarray(fin1[key]), np.asarray(fin2[key])), f"{label}: final cache {key} differs"


@pytest.mark.parametrize("name,streams,T,C,means,rule", CASES)
def test_split_sweep_equals_unsplit_and_oracle(name, streams, T, C, means, rule):
    torch_mod()
    cfg = dataclasses.replace(workloads.CONFIGS[name], C=C)
    if means is not None:
        cfg = dataclasses.replace(cfg, seg_means=means)
    d = workloads.prefill_inputs(cfg, streams=streams, T=T)
    label = f"split {name} S={len(streams)} T={T} C={C} {rule}"
    say(label)
    a, b = _both(d, C, cfg.tau, rule)
    _same(a, b, label)
    o, sc, fin = a
    r = oracle.run(d["q"], d["k"], d["v"], d["lam"], C, cfg.tau, nthreads=oracle_threads(), merge_rule=rule)
    compare_schedule(r, sc, fin, label)
    compare_states(r, fin, label=label)
    err = compare_outputs(o, r["o"], TOL["bf16"], label)
    say(f"{label}: ok, max row rel err {err:.2e}")


def test_split_sweep_state_score():
    """The split under the state information score (its schedule comes from
    the score kernel; the sweep is the same)."""
    torch_mod()
    cfg = dataclasses.replace(workloads.CONFIGS["mamba2_780m_bf16"], tau=0.6)
    d = workloads.prefill_inputs(cfg, streams=[0, 1], T=1600, values="regime")
    a, b = _both(d, cfg.C, cfg.tau, "sum", score_rule="state")
    _same(a, b, "split state score")


@pytest.mark.parametrize("ends,rule", [((2100, 3000), "sum"), ((700, 1400, 3000), "sum"), ((1025, 2600), "density")])
def test_split_continuing_calls(ends, rule):
    """Calls that continue a stream are split too (every block set starts
    from a copy of the cache's states): each call equals the unsplit sweep
    bit for bit, and together they are one pass of the oracle."""
    import dynamic_state_memory_amd as dla
    torch_mod()
    cfg = dataclasses.replace(workloads.CONFIGS["long_t131k_bf16"], C=32, seg_means=(40,))
    d = workloads.prefill_inputs(cfg, streams=[5, 6], T=ends[-1])
    label = f"split continuing calls {ends} {rule}"
    say(label)
    a = gpu_prefill_pieces(d["q"], d["k"], d["v"], d["lam"], cfg.C, cfg.tau, "bf16", ends, merge_rule=rule)
    dla.dla_set_prefill_path(dla.DLA_PATH_UNSPLIT, 0)
    try:
        b = gpu_prefill_pieces(d["q"], d["k"], d["v"], d["lam"], cfg.C, cfg.tau, "bf16", ends, merge_rule=rule)
    finally:
        dla.dla_set_prefill_path(dla.DLA_PATH_AUTO, 0)
    assert np.array_equal(a[0], b[0]), f"{label}: outputs differ from the unsplit sweep"
    for key in a[2]:
        assert np.array_equal(np.asarray(a[2][key]), np.asarray(b[2][key])), f"{label}: final cache {key} differs"
    o, _, fin = a
    r = oracle.run(d["q"], d["k"], d["v"], d["lam"], cfg.C, cfg.tau, nthreads=oracle_threads(), merge_rule=rule)
    compare_states(r, fin, label=label)
    err = compare_outputs(o, r["o"], TOL["bf16"], label)
    say(f"{label}: ok, max row rel err {err:.2e}")


@pytest.mark.parametrize("ends", [(3000,), (1300, 3100)])
def test_split_sweep_fixed_schedule(ends):
    """The Log-Linear fixed schedule's sweep split the same way, from position
    0 and continuing: equal to the unsplit sweep bit for bit."""
    import dynamic_state_memory_amd as dla
    torch = torch_mod()
    from tests.test_gpu_fenwick import _inputs, _run
    d = _inputs(ends[-1], [20, 21], 16)
    dev = torch.device("cuda:0")
    res = []
    for path in (dla.DLA_PATH_AUTO, dla.DLA_PATH_UNSPLIT):
        dla.dla_set_prefill_path(path, 0)
        try:
            cache = dla.Cache(1, 2, 16, 128, 64, device=dev, merge_rule="fenwick")
            outs, lo = [], 0
            for hi in ends:
                o, _ = _run({x: d[x][:, lo:hi] for x in ("q", "k", "v", "lam")}, 16, cache=cache)
                outs.append(o)
                lo = hi
            res.append((np.concatenate(outs, 1), cache.read()))
        finally:
            dla.dla_set_prefill_path(dla.DLA_PATH_AUTO, 0)
    (o1, f1), (o2, f2) = res
    assert np.array_equal(o1, o2), f"fixed schedule {ends}: outputs differ from the unsplit sweep"
    for key in f1:
        assert np.array_equal(np.asarray(f1[key]), np.asarray(f2[key])), f"fixed schedule {ends}: cache {key} differs"
    say(f"split fixed schedule {ends}: equal to the unsplit sweep")
