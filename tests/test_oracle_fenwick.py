"""Pins of the Fenwick-schedule oracle (oracle/fenwick.py) against constructions
other than its own formula, and planted mistakes that the pins must catch.

The independent construction is a binary counter of buckets: tokens are pushed
one at a time as buckets of one, and the two most recent buckets merge while
they have the same size ("Dynamic Linear Attention | Chlience Paper Archive",
section 2: a Fenwick-tree / log-scale decomposition into at most O(log T)
buckets; section 5.4: recent tokens fine, old ones coarse).  Its running sums
give the recurrent read o_t = sum_l lam_t^(l) S_t^(l) q_t of the same page,
which the oracle's quadratic form must reproduce.  No GPU is used."""
import importlib.util
import os
import traceback

import numpy as np
import pytest

import oracle.fenwick as FEN

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "fenwick.py")


def _counter(T):
    """Buckets of the prefix before each token, built by carries: parts[t] is
    the list of (start, size) before token t is pushed, oldest first; the last
    entry is the stack after all T tokens."""
    stack, parts = [], []
    for t in range(T + 1):
        parts.append(list(stack))
        if t == T:
            break
        stack.append((t, 1))
        while len(stack) >= 2 and stack[-1][1] == stack[-2][1]:
            (a, n), (_, m) = stack[-2], stack[-1]
            stack[-2:] = [(a, n + m)]
    return parts


def _data(S, T, dk, dv, L, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((S, T, dk)) / np.sqrt(dk)
    k = rng.standard_normal((S, T, dk))
    v = rng.standard_normal((S, T, dv)) / np.sqrt(dv)
    lam = 1 / (1 + np.exp(-rng.standard_normal((S, T, L))))
    return q, k, v, lam


def _recurrent(q, k, v, lam):
    """o_t = lam_t[0] (q_t.k_t) v_t + sum over the counter's buckets of
    lam_t[1 + log2(size)] S_bucket q_t, with bucket sums merged by addition."""
    S, T, _ = q.shape
    o = np.zeros((S, T, v.shape[2]))
    for x in range(S):
        stack = []      # (size, S)
        for t in range(T):
            acc = lam[x, t, 0] * (q[x, t] @ k[x, t]) * v[x, t]
            for size, St in stack:
                acc = acc + lam[x, t, size.bit_length()] * (St @ q[x, t])
            o[x, t] = acc
            stack.append((1, np.outer(v[x, t], k[x, t])))
            while len(stack) >= 2 and stack[-1][0] == stack[-2][0]:
                (n, A), (m, B) = stack[-2], stack[-1]
                stack[-2:] = [(n + m, A + B)]
    return o


# ---------------------------------------------------------------- the pins
# Each takes the module under test, so that planted mistakes run through them.

def pin_levels_match_counter(F):
    T = 300
    parts = _counter(T)
    L = F.level_matrix(T)
    for t in range(T):
        assert F.level(t, t) == 0 and L[t, t] == 0
        assert [(a, n) for a, n, _ in F.buckets(t)] == parts[t]
        assert [lv for _, _, lv in F.buckets(t)] == [n.bit_length() for _, n in parts[t]]
        for a, n in parts[t]:
            for s in range(a, a + n):
                assert F.level(t, s) == n.bit_length() == L[t, s], (t, s)
        assert (L[t, t + 1:] == -1).all()


def pin_bucket_count_is_logarithmic(F):
    for t in range(1, 5000):
        b = F.buckets(t)
        assert len(b) + 1 <= int(np.floor(np.log2(t))) + 2
        sizes = [n for _, n, _ in b]
        assert all(x > y for x, y in zip(sizes, sizes[1:]))      # recent tokens finer
        assert sum(sizes) == t


def pin_levels_needed(F):
    for T in list(range(1, 300)) + [512, 513, 4096, 4097]:
        L = F.level_matrix(T) if T <= 600 else None
        top = int(L.max()) if L is not None else (T - 1).bit_length()
        assert F.levels_needed(T) == top + 1, T


def pin_all_ones_is_causal_linear_attention(F):
    # lam = 1 on every level: the single-state recurrence S_t = S_{t-1} + v_t k_t^T, o_t = S_t q_t
    q, k, v, _ = _data(2, 150, 8, 6, 9, 1)
    lam = np.ones((2, 150, 9))
    S = np.cumsum(np.einsum("xti,xtj->xtij", v, k), axis=1)
    ref = np.einsum("xtij,xtj->xti", S, q)
    np.testing.assert_allclose(F.outputs(q, k, v, lam), ref, rtol=1e-10, atol=1e-10)


def pin_level0_is_the_token_itself(F):
    q, k, v, _ = _data(1, 100, 8, 6, 8, 2)
    lam = np.zeros((1, 100, 8))
    lam[..., 0] = 1.0
    ref = np.einsum("xt,xti->xti", np.einsum("xti,xti->xt", q, k), v)
    np.testing.assert_allclose(F.outputs(q, k, v, lam), ref, rtol=1e-10, atol=1e-12)


def pin_one_level_reads_one_bucket(F):
    T = 140
    q, k, v, _ = _data(1, T, 8, 6, 9, 3)
    parts = _counter(T)
    for lv in range(1, 9):
        lam = np.zeros((1, T, 9))
        lam[..., lv] = 1.0
        ref = np.zeros((1, T, 6))
        for t in range(T):
            for a, n in parts[t]:
                if n == 1 << (lv - 1):
                    ref[0, t] = v[0, a:a + n].T @ (k[0, a:a + n] @ q[0, t])
        np.testing.assert_allclose(F.outputs(q, k, v, lam), ref, rtol=1e-10, atol=1e-12, err_msg=str(lv))


def pin_recurrent_read(F):
    q, k, v, lam = _data(2, 200, 8, 6, 9, 4)
    np.testing.assert_allclose(F.outputs(q, k, v, lam), _recurrent(q, k, v, lam), rtol=1e-10, atol=1e-12)


def pin_output_rows(F):
    q, k, v, lam = _data(2, 260, 8, 6, 10, 5)
    rows = [0, 1, 2, 63, 64, 127, 128, 200, 255, 259]
    full = _recurrent(q, k, v, lam)
    np.testing.assert_allclose(F.output_rows(q, k, v, lam, rows), full[:, rows], rtol=1e-10, atol=1e-12)


def pin_final_states(F):
    for T in (1, 2, 3, 7, 64, 100, 128, 129, 255, 300):
        _, k, v, _ = _data(2, T, 5, 3, 2, T)
        fin = F.final_states(k, v, T)
        for x in range(2):
            stack = []
            for t in range(T):
                stack.append((t, 1, np.outer(v[x, t], k[x, t])))
                while len(stack) >= 2 and stack[-1][1] == stack[-2][1]:
                    (a, n, A), (_, m, B) = stack[-2], stack[-1]
                    stack[-2:] = [(a, n + m, A + B)]
            assert [(a, n) for a, n, _ in fin[x]] == [(a, n) for a, n, _ in stack], T
            for (_, _, G), (_, _, R) in zip(fin[x], stack):
                assert G.shape == R.shape == (3, 5)
                np.testing.assert_allclose(G, R, rtol=1e-10, atol=1e-12)


PINS = [pin_levels_match_counter, pin_bucket_count_is_logarithmic, pin_levels_needed,
        pin_all_ones_is_causal_linear_attention, pin_level0_is_the_token_itself,
        pin_one_level_reads_one_bucket, pin_recurrent_read, pin_output_rows, pin_final_states]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_oracle_pin(pin):
    pin(FEN)


def test_hand_worked_partition_of_13():
    # hand-worked: 13 = 8 + 4 + 1 tokens before query 13, oldest bucket first
    assert _counter(13)[13] == [(0, 8), (8, 4), (12, 1)]
    assert FEN.buckets(13) == [(0, 8, 4), (8, 4, 3), (12, 1, 1)]
    assert [FEN.level(13, s) for s in (0, 7, 8, 11, 12, 13)] == [4, 4, 3, 3, 1, 0]


# ---------------------------------------------------------------- planted mistakes

MUTANTS = [
    ("level from the difference, not the differing bits",
     "x = np.bitwise_xor(t, s)", "x = np.abs(t - s)"),
    ("levels shifted by one",
     "lv = np.frexp(x.astype(np.float64))[1].astype(np.int64)",
     "lv = np.frexp(x.astype(np.float64))[1].astype(np.int64) + 1"),
    ("the token itself not read",
     "causal = lv >= 0", "causal = lv > 0"),
    ("weights of the key's row",
     "W = np.take_along_axis(lam[x], idx, axis=1) * causal",
     "W = lam[x][np.arange(T)[None, :], idx] * causal"),
    ("scores transposed",
     "o[x] = ((q[x] @ k[x].T) * W) @ v[x]", "o[x] = ((k[x] @ q[x].T) * W) @ v[x]"),
    ("buckets newest first",
     "    return out\n\n\ndef outputs", "    return out[::-1]\n\n\ndef outputs"),
    ("bucket level off by one",
     "out.append((start, 1 << b, b + 1))", "out.append((start, 1 << b, b))"),
    ("final state transposed",
     "row.append((start, count, v[x, sl].T @ k[x, sl]))", "row.append((start, count, k[x, sl].T @ v[x, sl]))"),
    ("row outputs one level down",
     "w = lam[st, t, lv] * (k[st, : t + 1] @ q[st, t])", "w = lam[st, t, lv - 1] * (k[st, : t + 1] @ q[st, t])"),
    ("row outputs without the token itself",
     "s = np.arange(t + 1)\n", "s = np.arange(t + 1)\n        s = s[:-1]\n"),
    ("levels needed one short",
     "return max(T - 1, 0).bit_length() + 1", "return max(T - 1, 0).bit_length()"),
]


def _load_mutant(text, tmp_path, name):
    path = tmp_path / f"fenwick_{name}.py"
    path.write_text(text)
    spec = importlib.util.spec_from_file_location(f"fenwick_mutant_{name}", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(name, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, name
    mod = _load_mutant(src.replace(old, new), tmp_path, abs(hash(name)) % 10**8)
    failed = []
    for pin in PINS:
        try:
            pin(mod)
        except Exception:          # an assertion, or a crash the mistake causes
            failed.append(pin.__name__)
    assert failed, f"no pin catches: {name}"


def test_unmodified_copy_passes(tmp_path):
    mod = _load_mutant(open(SRC).read(), tmp_path, "clean")
    for pin in PINS:
        try:
            pin(mod)
        except Exception:
            pytest.fail(traceback.format_exc())
