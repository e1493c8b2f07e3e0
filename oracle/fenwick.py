"""CPU oracle of the Log-Linear fixed (Fenwick) schedule on the same read.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark use this module; the GPU library and its Python binding
never import it, and it imports nothing from them.

What it follows.  "Dynamic Linear Attention | Chlience Paper Archive",
section 2 (existing solutions, the multi-state line of work): Log-Linear
Attention splits the prefix seen by query t into at most O(log T) buckets by a
Fenwick-tree decomposition, keeps one summary S_t^(l) = sum over s in
B_t^(l) of v_s k_s^T per bucket, and reads o_t = sum_l lam_t^(l) S_t^(l) q_t.
Section 5.4 of the same page: the buckets follow time alone, fine for recent
tokens and coarse for old ones.

Reading (the page gives the formula but not the buckets):
  * B_t^(0) = {t}: the token itself, level 0;
  * for l >= 1, B_t^(l) holds the 2^(l-1) tokens s < t that agree with t on
    every bit above bit l-1 and have bit l-1 clear where t has it set, and is
    empty when bit l-1 of t is clear.  These are the binary decomposition of
    t: the largest (oldest) bucket first, sizes the powers of two in t;
  * equivalently, key s <= t sits at level 0 if s == t, else at
    1 + (index of the highest bit in which s and t differ);
  * lam_t has one weight per level, column l for B_t^(l).

Everything is float64 numpy, the plain definition written out: the quadratic
form o_t = sum_{s <= t} lam_t[level(t, s)] (q_t . k_s) v_s.
"""
from __future__ import annotations

import numpy as np


def level(t: int, s: int) -> int:
    """Level of key s in the partition seen by query t (0 <= s <= t)."""
    if s > t or s < 0:
        raise ValueError("a query sees keys 0 .. t only")
    return 0 if s == t else (t ^ s).bit_length()


def levels_needed(T: int) -> int:
    """Number of lam columns a call over tokens 0 .. T-1 can index (levels 0 .. L-1)."""
    return max(T - 1, 0).bit_length() + 1


def level_matrix(T: int) -> np.ndarray:
    """L[t, s] = level(t, s) for s <= t, -1 above the diagonal."""
    t = np.arange(T)[:, None]
    s = np.arange(T)[None, :]
    x = np.bitwise_xor(t, s)
    # frexp's exponent of a positive integer is its bit length (exact)
    lv = np.frexp(x.astype(np.float64))[1].astype(np.int64)
    lv[s > t] = -1
    return lv


def buckets(t: int):
    """The buckets of the prefix [0, t) (the keys a query at t reads besides
    itself), oldest first: a list of (start, count, level)."""
    out, start = [], 0
    for b in range(max(t, 0).bit_length() - 1, -1, -1):
        if (t >> b) & 1:
            out.append((start, 1 << b, b + 1))
            start += 1 << b
    return out


def outputs(q, k, v, lam) -> np.ndarray:
    """o[x, t] = sum_{s <= t} lam[x, t, level(t, s)] (q[x, t] . k[x, s]) v[x, s].

    q, k: [S, T, d_k]; v: [S, T, d_v]; lam: [S, T, L] with L >= levels_needed(T)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    lam = np.asarray(lam, np.float64)
    S, T, _ = q.shape
    if lam.shape[2] < levels_needed(T):
        raise ValueError("lam needs one column per level")
    lv = level_matrix(T)
    causal = lv >= 0
    idx = np.where(causal, lv, 0)
    o = np.empty((S, T, v.shape[2]))
    for x in range(S):
        W = np.take_along_axis(lam[x], idx, axis=1) * causal
        o[x] = ((q[x] @ k[x].T) * W) @ v[x]
    return o


def output_rows(q, k, v, lam, rows) -> np.ndarray:
    """The outputs of the listed tokens only, one row at a time (for long
    streams): o[x, i] for t = rows[i]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    lam = np.asarray(lam, np.float64)
    S = q.shape[0]
    o = np.empty((S, len(rows), v.shape[2]))
    for i, t in enumerate(rows):
        s = np.arange(t + 1)
        lv = np.frexp(np.bitwise_xor(s, t).astype(np.float64))[1]
        for st in range(S):
            w = lam[st, t, lv] * (k[st, : t + 1] @ q[st, t])
            o[st, i] = w @ v[st, : t + 1]
    return o


def final_states(k, v, T: int | None = None):
    """The cache after tokens 0 .. T-1: the buckets of the prefix [0, T),
    oldest first, as (start, count, S) with S = sum v_s k_s^T (d_v x d_k)."""
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    if T is None:
        T = k.shape[1]
    out = []
    for x in range(k.shape[0]):
        row = []
        for start, count, _ in buckets(T):
            sl = slice(start, start + count)
            row.append((start, count, v[x, sl].T @ k[x, sl]))
        out.append(row)
    return out
