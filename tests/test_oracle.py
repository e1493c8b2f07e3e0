"""Pins of the CPU oracle against closed forms, library routines, brute force,
hand-derived schedules and invariants (no GPU needed)."""
import json
import os

import numpy as np
import pytest
from hypothesis import given, settings, strategies as st
from scipy.spatial.distance import cosine as scipy_cosine

import oracle
from tests.helpers import assert_close_to_sum, keys_for_scores, mat_rel_err, row_rel_err

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "schedule_cases.json")


def _rand(T, dk, dv, C, seed, S=1):
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((S, T, dk)) / np.sqrt(dk)).astype(np.float32)
    k = rng.standard_normal((S, T, dk)).astype(np.float32)
    v = (rng.standard_normal((S, T, dv)) / np.sqrt(dv)).astype(np.float32)
    lam = (1 / (1 + np.exp(-rng.standard_normal((S, T, C))))).astype(np.float32)
    return q, k, v, lam


def _regime_keys(T, dk, seg, seed, noise=0.2):
    rng = np.random.default_rng(seed)
    out = np.empty((T, dk), np.float32)
    t = 0
    while t < T:
        n = min(int(rng.geometric(1 / seg)), T - t)
        c = rng.standard_normal(dk)
        c /= np.linalg.norm(c)
        out[t:t + n] = c + noise / np.sqrt(dk) * rng.standard_normal((n, dk))
        t += n
    return out.astype(np.float32)


# ---------------------------------------------------------------- token score

# Every pin is a function with an optional ``lib`` (a handle from
# oracle.load_library); the tests below call them on the oracle itself, and
# test_oracle_mutants.py calls them on copies with a planted mistake.

def _s_pair(k0, k1, lib=None):
    k = np.stack([k0, k1]).astype(np.float32)[None]
    T, dk = 2, k.shape[2]
    q = np.zeros((1, T, dk), np.float32)
    v = np.zeros((1, T, 1), np.float32)
    lam = np.ones((1, T, 2), np.float32)
    r = oracle.run(q, k, v, lam, 2, 0.3, outputs=False, lib=lib)
    return r["s"][0]


def pin_score_closed_forms(lib=None):
    rng = np.random.default_rng(0)
    for dk in (2, 64, 128):
        k0 = rng.standard_normal(dk).astype(np.float32)
        # token 0 has no previous key: s_0 = 1
        assert _s_pair(k0, k0, lib)[0] == np.float32(1.0)
        # parallel keys (positive multiple): s ~ 0
        assert abs(_s_pair(k0, (2.5 * k0).astype(np.float32), lib)[1]) <= 1e-6
        # antiparallel: s = 2 exactly
        assert _s_pair(k0, -k0, lib)[1] == np.float32(2.0)
        # orthogonal: s = 1 exactly
        e0 = np.zeros(dk, np.float32); e0[0] = 3.0
        e1 = np.zeros(dk, np.float32); e1[1] = -0.5
        assert _s_pair(e0, e1, lib)[1] == np.float32(1.0)
        # zero key: s = 1
        assert _s_pair(k0, np.zeros(dk, np.float32), lib)[1] == np.float32(1.0)
        # invariant to scaling either key by a power of two (exact)
        k1 = rng.standard_normal(dk).astype(np.float32)
        s = _s_pair(k0, k1, lib)[1]
        assert _s_pair((4 * k0).astype(np.float32), k1, lib)[1] == s
        assert _s_pair(k0, (0.125 * k1).astype(np.float32), lib)[1] == s
        # not symmetric in its failure modes: a generic pair against scipy
        k2 = (k0 + 0.7 * rng.standard_normal(dk)).astype(np.float32)
        ref = scipy_cosine(k2.astype(np.float64), k0.astype(np.float64))
        assert abs(float(_s_pair(k0, k2, lib)[1]) - ref) <= 1e-6


def test_score_closed_forms():
    pin_score_closed_forms()


def test_score_matches_library_cosine_distance():
    rng = np.random.default_rng(1)
    for _ in range(200):
        dk = int(rng.choice([3, 64, 128]))
        k0 = rng.standard_normal(dk).astype(np.float32)
        k1 = (k0 + rng.standard_normal(dk) * rng.uniform(0, 2)).astype(np.float32)
        s = _s_pair(k0, k1)[1]
        ref = np.float32(scipy_cosine(k1.astype(np.float64), k0.astype(np.float64)))
        assert abs(float(s) - float(ref)) <= 2 * np.spacing(np.float32(max(abs(ref), 1e-3)))


# ---------------------------------------------------------- golden schedules

def _golden():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


def pin_hand_derived_schedule(case, lib=None):
    s_des = case["s_after_first"]
    T = len(s_des) + 1
    e = case["expect"]
    assert len(e["boundary"]) == T and len(e["m_t"]) == T
    k = keys_for_scores(s_des)[None]
    q, _, v, lam = _rand(T, k.shape[2], 4, case["C"], seed=7)
    rule = case.get("merge_rule", "sum")
    r = oracle.run(q, k, v, lam, case["C"], case["tau"], lib=lib, merge_rule=rule)
    assert r["s"][0].tolist() == [1.0] + [float(x) for x in s_des]
    assert r["b"][0].tolist() == e["boundary"]
    assert r["m_t"][0].tolist() == e["m_t"]
    assert [list(x) for x in r["events"][0]] == e["events"]
    m = int(r["fin_m"][0])
    assert r["fin_start"][0, :m].tolist() == e["starts"]
    assert r["fin_I"][0, :m].tolist() == [x << 30 for x in e["info_quarters"]]
    assert r["fin_n"][0, :m].tolist() == e["count"]
    # the outputs on this schedule equal the O(T^2) slot-weighted sum
    sets = oracle.start_sets(T, r["b"][0], r["events"][0])
    bf = oracle.brute_force(q[0], k[0], v[0], lam[0], sets)
    assert row_rel_err(r["o"][0], bf) < 1e-12
    # the independent checker re-derives the same merges under the case's rule
    oracle.check_schedule(r["s"][0], case["tau"], case["C"], r["b"][0], r["events"][0], r["m_t"][0],
                          merge_rule=rule)


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_hand_derived_schedules(case):
    pin_hand_derived_schedule(case)


# ----------------------------------------------------- brute force / checker

@settings(max_examples=60, deadline=None)
@given(T=st.integers(1, 70), dk=st.sampled_from([2, 4, 8]), dv=st.sampled_from([1, 3, 8]),
       C=st.integers(1, 6), tau=st.sampled_from([-1.0, 0.3, 0.9, 3.0]),
       seg=st.sampled_from([2, 8, 1000]), seed=st.integers(0, 2**31 - 1))
def test_oracle_equals_brute_force_and_greedy(T, dk, dv, C, tau, seg, seed):
    pin_brute_force_and_greedy(T, dk, dv, C, tau, seg, seed)


@settings(max_examples=40, deadline=None)
@given(T=st.integers(1, 90), dk=st.sampled_from([2, 4, 8]), dv=st.sampled_from([1, 3]),
       C=st.integers(1, 6), tau=st.sampled_from([-1.0, 0.3, 0.9]),
       seg=st.sampled_from([2, 8, 30]), seed=st.integers(0, 2**31 - 1))
def test_density_rule_equals_brute_force_and_greedy(T, dk, dv, C, tau, seg, seed):
    pin_brute_force_and_greedy(T, dk, dv, C, tau, seg, seed, merge_rule="density")


def pin_brute_force_and_greedy(T, dk, dv, C, tau, seg, seed, lib=None, merge_rule="sum"):
    q, _, v, lam = _rand(T, dk, dv, C, seed)
    k = _regime_keys(T, dk, seg, seed + 1)[None]
    r = oracle.run(q, k, v, lam, C, tau, lib=lib, merge_rule=merge_rule)
    oracle.check_schedule(r["s"][0], tau, C, r["b"][0], r["events"][0], r["m_t"][0], merge_rule=merge_rule)
    sets = oracle.start_sets(T, r["b"][0], r["events"][0])
    bf = oracle.brute_force(q[0], k[0], v[0], lam[0], sets)
    bf_abs = oracle.brute_force(np.abs(q[0]), np.abs(k[0]), np.abs(v[0]), np.abs(lam[0]), sets)
    assert_close_to_sum(r["o"][0], bf, bf_abs, 1e-12)
    # invariants of the final cache
    m = int(r["fin_m"][0])
    starts = r["fin_start"][0, :m]
    assert 1 <= m <= C and starts[0] == 0 and np.all(np.diff(starts) > 0)
    assert list(starts) == list(sets[-1])
    ends = np.append(starts[1:], T)
    assert r["fin_n"][0, :m].tolist() == (ends - starts).tolist()
    qs = oracle.fixed_point(r["s"][0])
    assert r["fin_I"][0, :m].tolist() == [int(qs[a:b].sum()) for a, b in zip(starts, ends)]
    # every state is the sum of the outer products of its own tokens
    for i, (a, b) in enumerate(zip(starts, ends)):
        ref = v[0, a:b].astype(np.float64).T @ k[0, a:b].astype(np.float64)
        assert np.allclose(r["fin_S"][0, i], ref, rtol=1e-12, atol=1e-12)


def test_checker_catches_planted_mistakes():
    """Mutating a correct schedule must make the checker fail."""
    T, C, tau = 300, 4, 0.3
    q, _, v, lam = _rand(T, 8, 2, C, 11)
    k = _regime_keys(T, 8, 6, 12)[None]
    r = oracle.run(q, k, v, lam, C, tau)
    ev = r["events"][0]
    assert len(ev) >= 3
    oracle.check_schedule(r["s"][0], tau, C, r["b"][0], ev)
    bad = [list(e) for e in ev]
    bad[1][1] = (bad[1][1] + 1) % C          # wrong pair
    with pytest.raises(AssertionError):
        oracle.check_schedule(r["s"][0], tau, C, r["b"][0], [tuple(e) for e in bad])
    with pytest.raises(AssertionError):     # a merge dropped
        oracle.check_schedule(r["s"][0], tau, C, r["b"][0], ev[:1] + ev[2:])
    b = r["b"][0].copy()
    i = int(np.flatnonzero(b == 0)[0])
    b[i] = 1                                 # a boundary invented
    with pytest.raises(AssertionError):
        oracle.check_schedule(r["s"][0], tau, C, b, ev)


def test_rules_differ_and_checker_tells_them_apart():
    """On regime-structured keys the two merge rules give different
    schedules, and the checker rejects each schedule under the other rule."""
    T, C, tau = 400, 4, 0.3
    q, _, v, lam = _rand(T, 8, 2, C, 21)
    k = _regime_keys(T, 8, 10, 22)[None]
    rs = oracle.run(q, k, v, lam, C, tau, merge_rule="sum")
    rd = oracle.run(q, k, v, lam, C, tau, merge_rule="density")
    assert rs["b"][0].tolist() == rd["b"][0].tolist()     # the boundary rule is shared
    assert rs["events"][0] != rd["events"][0]
    oracle.check_schedule(rd["s"][0], tau, C, rd["b"][0], rd["events"][0], merge_rule="density")
    with pytest.raises(AssertionError):
        oracle.check_schedule(rd["s"][0], tau, C, rd["b"][0], rd["events"][0], merge_rule="sum")
    with pytest.raises(AssertionError):
        oracle.check_schedule(rs["s"][0], tau, C, rs["b"][0], rs["events"][0], merge_rule="density")


# ------------------------------------------------------------- special cases

@pytest.mark.parametrize("tau,C", [(0.3, 3), (-1.0, 2), (3.0, 5), (0.9, 1)])
def test_lambda_one_gives_causal_linear_attention(tau, C):
    pin_lambda_one(tau, C)


def pin_lambda_one(tau, C, lib=None):
    T, dk, dv = 200, 16, 12
    q, _, v, _ = _rand(T, dk, dv, C, 3)
    k = _regime_keys(T, dk, 20, 4)[None]
    lam = np.ones((1, T, C), np.float32)
    r = oracle.run(q, k, v, lam, C, tau, lib=lib)
    Q, K, V = (a[0].astype(np.float64) for a in (q, k, v))
    ref = np.tril(Q @ K.T) @ V          # textbook causal linear attention
    assert row_rel_err(r["o"][0], ref) < 1e-12


@pytest.mark.parametrize("tau", [0.3, -1.0, 3.0])
def test_single_state_reduces_to_linear_attention(tau):
    pin_single_state(tau)


def pin_single_state(tau, lib=None):
    T, dk, dv = 150, 8, 8
    q, _, v, lam = _rand(T, dk, dv, 1, 5)
    k = _regime_keys(T, dk, 10, 6)[None]
    r = oracle.run(q, k, v, lam, 1, tau, lib=lib)
    assert np.all(r["m_t"][0] == 1)
    Q, K, V = (a[0].astype(np.float64) for a in (q, k, v))
    ref = lam[0, :, :1].astype(np.float64) * (np.tril(Q @ K.T) @ V)
    assert row_rel_err(r["o"][0], ref) < 1e-12


def test_every_token_own_state_is_dense_slot_weighted_product():
    pin_dense_slot_weighted()


def pin_dense_slot_weighted(lib=None):
    T, dk, dv = 40, 8, 5
    q, k, v, lam = _rand(T, dk, dv, T, 8)
    r = oracle.run(q, k, v, lam, T, -1.0, lib=lib)
    assert np.all(r["b"][0] == 1) and r["n_ev"][0] == 0
    Q, K, V, L = (a[0].astype(np.float64) for a in (q, k, v, lam))
    t = np.arange(T)
    W = np.where(t[:, None] >= t[None, :], L[t[:, None], np.clip(t[:, None] - t[None, :], 0, T - 1)], 0)
    assert row_rel_err(r["o"][0], (W * (Q @ K.T)) @ V) < 1e-12
    # one-hot lambda on slot 0 isolates the token's own state: (q_t . k_t) v_t
    lam1 = np.zeros_like(lam); lam1[..., 0] = 1
    r1 = oracle.run(q, k, v, lam1, T, -1.0, lib=lib)
    assert row_rel_err(r1["o"][0], np.sum(Q * K, 1)[:, None] * V) < 1e-12


def test_states_always_sum_to_the_prefix():
    pin_prefix_sum()


def pin_prefix_sum(lib=None):
    T, dk, dv, C = 400, 16, 8, 4
    q, _, v, lam = _rand(T, dk, dv, C, 9)
    k = _regime_keys(T, dk, 5, 10)[None]
    for Tp in (1, 17, 400):
        r = oracle.run(q[:, :Tp], k[:, :Tp], v[:, :Tp], lam[:, :Tp], C, 0.3, lib=lib)
        tot = r["fin_S"][0].sum(0)
        ref = v[0, :Tp].astype(np.float64).T @ k[0, :Tp].astype(np.float64)
        assert mat_rel_err(tot, ref) < 1e-12
        assert r["fin_m"][0] <= C


def test_continuing_a_stream_equals_one_long_call():
    """prefill(T) == prefill(T - j) followed by j more tokens from its cache."""
    T, dk, dv, C = 300, 8, 6, 5
    q, _, v, lam = _rand(T, dk, dv, C, 13, S=3)
    k = np.stack([_regime_keys(T, dk, 7, 20 + i) for i in range(3)])
    full = oracle.run(q, k, v, lam, C, 0.3)
    for j in (1, 5, 64):
        a = oracle.run(q[:, :-j], k[:, :-j], v[:, :-j], lam[:, :-j], C, 0.3)
        init = dict(m=a["fin_m"], S=a["fin_S"], I=a["fin_I"], n=a["fin_n"], start=a["fin_start"],
                    has_prev=a["fin_has_prev"], s_prev=a["fin_s_prev"], k_prev=a["fin_k_prev"],
                    t_seen=a["fin_t_seen"])
        bpart = oracle.run(q[:, -j:], k[:, -j:], v[:, -j:], lam[:, -j:], C, 0.3, init=init)
        assert np.array_equal(np.concatenate([a["o"], bpart["o"]], 1), full["o"])
        assert np.array_equal(np.concatenate([a["s"], bpart["s"]], 1), full["s"])
        assert np.array_equal(bpart["fin_S"], full["fin_S"])
        assert np.array_equal(bpart["fin_start"], full["fin_start"])
        # the checker, started from the same cache, accepts the continuation
        for i in range(3):
            m0 = int(a["fin_m"][i])
            starts = [int(x) - (T - j) for x in a["fin_start"][i, :m0]]
            oracle.check_schedule(bpart["s"][i], 0.3, C, bpart["b"][i], bpart["events"][i],
                                  bpart["m_t"][i],
                                  init=dict(starts=starts, infos=a["fin_I"][i, :m0].tolist(),
                                            s_prev=a["fin_s_prev"][i]))


def test_sampled_outputs_equal_full_outputs():
    T, dk, dv, C = 200, 8, 8, 3
    q, _, v, lam = _rand(T, dk, dv, C, 21, S=2)
    k = np.stack([_regime_keys(T, dk, 9, 30 + i) for i in range(2)])
    full = oracle.run(q, k, v, lam, C, 0.3)
    want = np.zeros((2, T), bool); want[0, [0, 5, 199]] = True; want[1, 100] = True
    part = oracle.run(q, k, v, lam, C, 0.3, want=want)
    assert np.array_equal(part["o"][want], full["o"][want])
    assert np.all(part["o"][~want] == 0)
