"""Pins of the oracle's state information score (reading notes "Dynamic
Linear Attention | Chlience Paper Archive", section 5.1): the per-token state
v_t k_t^T against the current state, both RMS-normalised, the boundary at
I_t >= tau.  Checked against the closed form through the cosine of the two
matrices (recomputed from the schedule's token ranges, not from the oracle's
bookkeeping), special cases with known values, a hand-derived schedule, the
independent schedule checker and the O(T^2) brute force.  No GPU."""
import json
import math
import os

import numpy as np
import pytest

import oracle
from tests.helpers import row_rel_err

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "state_score_cases.json")


def _regime(T, dk, dv, C, seed, seg=12.0, noise=0.05, S=1):
    """Streams whose keys and values both follow piecewise regimes."""
    rng = np.random.default_rng(seed)
    q = (rng.standard_normal((S, T, dk)) / np.sqrt(dk)).astype(np.float32)
    k = np.empty((S, T, dk), np.float32)
    v = np.empty((S, T, dv), np.float32)
    for s in range(S):
        t = 0
        while t < T:
            n = min(int(rng.geometric(1 / seg)), T - t)
            kc, vc = rng.standard_normal(dk), rng.standard_normal(dv)
            k[s, t:t + n] = kc + noise * rng.standard_normal((n, dk))
            v[s, t:t + n] = vc + noise * rng.standard_normal((n, dv))
            t += n
    lam = (1 / (1 + np.exp(-rng.standard_normal((S, T, C))))).astype(np.float32)
    return q, k, v, lam


def _closed(D, c):
    return math.sqrt(max(0.0, 2 * D * (1 - c))) / (math.sqrt(D) + 1e-6)


# Every pin takes an optional ``lib`` (a handle from oracle.load_library);
# test_oracle_mutants.py runs them on copies of the oracle with planted mistakes.

def pin_state_closed_form(T, dk, dv, C, tau, seed, merge_rule="sum", lib=None):
    q, k, v, lam = _regime(T, dk, dv, C, seed, S=2)
    r = oracle.run(q, k, v, lam, C, tau, score_rule="state", merge_rule=merge_rule, lib=lib)
    for i in range(2):
        sets = oracle.start_sets(T, r["b"][i], r["events"][i])
        ref = oracle.state_scores_closed_form(v[i], k[i], sets)
        err = np.abs(r["s"][i].astype(np.float64) - ref).max()
        assert err <= 1e-6, f"stream {i}: state scores differ from the closed form by {err:.3e}"
        oracle.check_schedule(r["s"][i], tau, C, r["b"][i], r["events"][i], m_t=r["m_t"][i],
                              merge_rule=merge_rule, score_rule="state")
        bf = oracle.brute_force(q[i], k[i], v[i], lam[i], sets)
        assert row_rel_err(r["o"][i], bf) <= 1e-12
    return r


def pin_state_special_cases(lib=None):
    dk, dv, T = 3, 4, 6
    rng = np.random.default_rng(1)
    kk = rng.standard_normal(dk).astype(np.float32)
    vv = rng.standard_normal(dv).astype(np.float32)
    D = dk * dv
    q = rng.standard_normal((1, T, dk)).astype(np.float32)

    def run(k, v, tau=0.3, C=4):
        n = len(k)
        lm = np.ones((1, n, C), np.float32)
        return oracle.run(q[:, :n], k[None].astype(np.float32), v[None].astype(np.float32), lm, C, tau,
                          score_rule="state", lib=lib)

    # identical tokens: I_0 = 2 (empty cache), then the per-token state is
    # parallel to the current one, c = 1, I = 0: a single state
    same_k, same_v = np.tile(kk, (T, 1)), np.tile(vv, (T, 1))
    r = run(same_k, same_v)
    assert r["s"][0][0] == np.float32(2.0) and np.all(np.abs(r["s"][0][1:]) <= 1e-6)
    assert r["b"][0].tolist() == [1] + [0] * (T - 1) and r["fin_m"][0] == 1
    # I = 0 is not below tau = 0: every token opens a state (equality is high;
    # token 1 scores exactly 0, a per-token state equal to the current one)
    r = run(same_k, same_v, tau=0.0, C=T)
    assert r["s"][0][1] == 0.0
    assert r["b"][0].tolist() == [1] * T
    # v_t = -v_{t-1}: each token is antiparallel to the state before it, c = -1
    alt_v = np.array([vv if t % 2 == 0 else -vv for t in range(T)])
    r = run(same_k, alt_v, C=T)
    assert r["b"][0].tolist() == [1] * T
    np.testing.assert_allclose(r["s"][0][1:], _closed(D, -1.0), rtol=2e-7)
    # orthogonal values: c = 0
    e = np.eye(dv, dtype=np.float32)
    r = run(np.tile(kk, (4, 1)), e[:4], C=4)
    np.testing.assert_allclose(r["s"][0][1:4], _closed(D, 0.0), rtol=2e-7)
    # a zero key: the per-token state is zero, its normalisation undefined: I = 2
    zk = same_k.copy()
    zk[3] = 0.0
    r = run(zk, same_v)
    assert r["s"][0][3] == np.float32(2.0) and r["b"][0][3] == 1
    # scale invariance of both matrices under positive factors
    qa, ka, va, la = _regime(40, 5, 3, 3, 7)
    r1 = oracle.run(qa, ka, va, la, 3, 0.3, score_rule="state", lib=lib)
    r2 = oracle.run(qa, ka * np.float32(4.0), va * np.float32(0.25), la, 3, 0.3, score_rule="state", lib=lib)
    assert np.abs(r1["s"] - r2["s"]).max() <= 1e-6
    assert np.array_equal(r1["b"], r2["b"]) and r1["events"] == r2["events"]
    # tau above every possible score: only the empty-cache token opens
    r = oracle.run(qa, ka, va, la, 3, 2.5, score_rule="state", lib=lib)
    assert r["b"][0].tolist() == [1] + [0] * 39


def _golden():
    return json.load(open(GOLDEN))["cases"]


def pin_state_golden(case, lib=None):
    v = np.asarray(case["v"], np.float32)[None]
    k = np.asarray(case["k"], np.float32)[None]
    T, dk = k.shape[1:]
    dv = v.shape[2]
    C = case["C"]
    q = np.ones((1, T, dk), np.float32)
    lam = np.ones((1, T, C), np.float32)
    r = oracle.run(q, k, v, lam, C, case["tau"], score_rule="state", lib=lib)
    D = dk * dv
    want = [2.0] + [_closed(D, float(eval(str(c), {"sqrt": math.sqrt}))) for c in case["cosine"][1:]]
    np.testing.assert_allclose(r["s"][0], want, rtol=0, atol=1e-6)
    ex = case["expect"]
    assert r["b"][0].tolist() == ex["boundary"]
    assert r["m_t"][0].tolist() == ex["m_t"]
    assert [list(e) for e in r["events"][0]] == ex["events"]
    m = int(r["fin_m"][0])
    assert r["fin_start"][0, :m].tolist() == ex["starts"] and r["fin_n"][0, :m].tolist() == ex["count"]


def pin_state_continuation(lib=None):
    """A call continuing a cache gives what one call over all the tokens gives."""
    T, dk, dv, C, tau = 90, 4, 3, 3, 0.3
    q, k, v, lam = _regime(T, dk, dv, C, 11)
    full = oracle.run(q, k, v, lam, C, tau, score_rule="state", lib=lib)
    h = 37
    a = oracle.run(q[:, :h], k[:, :h], v[:, :h], lam[:, :h], C, tau, score_rule="state", lib=lib)
    init = dict(m=a["fin_m"], S=a["fin_S"], I=a["fin_I"], n=a["fin_n"], start=a["fin_start"],
                has_prev=a["fin_has_prev"], s_prev=a["fin_s_prev"], k_prev=a["fin_k_prev"], t_seen=a["fin_t_seen"])
    b = oracle.run(q[:, h:], k[:, h:], v[:, h:], lam[:, h:], C, tau, init=init, score_rule="state", lib=lib)
    assert np.array_equal(np.concatenate([a["s"], b["s"]], 1), full["s"])
    assert np.array_equal(np.concatenate([a["b"], b["b"]], 1), full["b"])
    assert row_rel_err(np.concatenate([a["o"], b["o"]], 1), full["o"]) <= 1e-12


# ------------------------------------------------------------------- tests

@pytest.mark.parametrize("T,dk,dv,C,tau,seed", [(120, 4, 3, 3, 0.3, 1), (100, 6, 6, 2, 0.3, 2),
                                                (80, 8, 5, 5, 0.15, 3), (90, 3, 7, 1, 0.3, 4),
                                                (60, 5, 5, 4, -1.0, 5), (70, 4, 4, 70, 0.3, 6)])
def test_state_score_closed_form_and_schedule(T, dk, dv, C, tau, seed):
    r = pin_state_closed_form(T, dk, dv, C, tau, seed)
    if tau < 0:
        assert r["b"].all()


def test_state_score_density_rule():
    pin_state_closed_form(120, 4, 3, 3, 0.3, 8, merge_rule="density")


def test_state_score_sees_the_regimes():
    # with regime values the low scores sit inside segments: far fewer
    # boundaries than tokens, but more than one state
    r = pin_state_closed_form(200, 6, 6, 8, 0.3, 9)
    nb = int(r["b"].sum())
    assert 2 < nb < 200 * 2 // 2


def test_state_score_special_cases():
    pin_state_special_cases()


@pytest.mark.parametrize("case", _golden(), ids=[c["name"] for c in _golden()])
def test_state_score_hand_derived(case):
    pin_state_golden(case)


def test_state_score_continuation():
    pin_state_continuation()


def test_lambda_one_is_linear_attention_under_the_state_score():
    T, dk, dv, C = 60, 4, 3, 3
    q, k, v, lam = _regime(T, dk, dv, C, 12)
    r = oracle.run(q, k, v, np.ones_like(lam), C, 0.3, score_rule="state")
    ref = np.tril(q[0].astype(np.float64) @ k[0].T.astype(np.float64)) @ v[0].astype(np.float64)
    assert row_rel_err(r["o"][0], ref) <= 1e-12
