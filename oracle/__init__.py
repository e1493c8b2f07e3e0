"""CPU oracle of the Dynamic Linear Attention (DLA) layer forward pass.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the CPU-baseline leg
of the benchmark use this package; the GPU library and its Python binding
never import it, and it imports nothing from them.

* ``run``            -- the recurrent oracle (plain C, double precision, one
                        stream per OpenMP thread), see ``dla_oracle.c``.
* ``brute_force``    -- the O(T^2) slot-weighted sum over tokens, computed
                        from a schedule's start sets (numpy, float64).
* ``check_schedule`` -- re-derives every boundary and every greedy merge
                        decision from the token information values alone.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "dla_oracle.c")
_OUT = os.path.join(_HERE, "_build", "libdla_oracle.so")
_lib = None


def build(force: bool = True, src: str = _SRC, out: str = _OUT) -> str:
    """Compile the C oracle (gcc, -O2, no floating-point contraction).

    ``src``/``out`` let a test compile a modified copy of the source (the
    planted-mistake tests); the default builds the oracle itself."""
    if not force and os.path.exists(out):
        return out
    os.makedirs(os.path.dirname(out), exist_ok=True)
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def load_library(path: str):
    """A ctypes handle on a compiled oracle library (for ``run(..., lib=)``)."""
    lib = C.CDLL(path)
    lib.dlao_run.argtypes = [C.POINTER(_Args)]
    lib.dlao_run.restype = C.c_int
    return lib


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_OUT) or os.path.getmtime(_OUT) < os.path.getmtime(_SRC):
            build()
        _lib = load_library(_OUT)
    return _lib


_p = C.c_void_p


class _Args(C.Structure):
    _fields_ = [
        ("BH", C.c_int32), ("T", C.c_int32), ("dk", C.c_int32), ("dv", C.c_int32),
        ("C", C.c_int32), ("tau", C.c_float),
        ("q", _p), ("k", _p), ("v", _p), ("lam", _p),
        ("init_m", _p), ("init_S", _p), ("init_I", _p), ("init_n", _p),
        ("init_start", _p), ("init_has_prev", _p), ("init_s_prev", _p),
        ("init_k_prev", _p), ("init_t_seen", _p), ("want_o", _p),
        ("o", _p), ("s_out", _p), ("b_out", _p), ("seg_out", _p), ("m_out", _p),
        ("ev_t", _p), ("ev_i", _p), ("n_ev", _p),
        ("fin_m", _p), ("fin_S", _p), ("fin_I", _p), ("fin_n", _p), ("fin_start", _p),
        ("fin_has_prev", _p), ("fin_s_prev", _p), ("fin_k_prev", _p),
        ("fin_t_seen", _p), ("nthreads", C.c_int32), ("merge_rule", C.c_int32),
        ("score_rule", C.c_int32),
    ]


MERGE_RULES = {"sum": 0, "density": 1}
SCORE_RULES = {"cosine": 0, "state": 1}


def _ptr(a):
    return None if a is None else a.ctypes.data_as(C.c_void_p)


def _c(a, dt):
    return np.ascontiguousarray(a, dtype=dt)


def run(q, k, v, lam, C_: int, tau: float, init: dict | None = None,
        want=None, outputs: bool = True, final_states: bool = True,
        nthreads: int | None = None, lib=None, merge_rule: str = "sum",
        score_rule: str = "cosine") -> dict:
    """Run the oracle on float32 inputs q,k [S,T,dk], v [S,T,dv], lam [S,T,C].

    ``merge_rule``: "sum" merges the adjacent pair of smallest summed
    information, "density" the pair of lowest (I_i + I_{i+1}) / (n_i + n_{i+1}).
    ``score_rule``: "cosine" scores a token by 1 - cos(k_t, k_{t-1}) and opens
    a state unless it and the token before are both below tau; "state" scores
    it by the state information score against the current state (the
    per-token state v k^T and the most recent state, each RMS-normalised,
    Frobenius distance over the normalised current state's norm + 1e-6) and
    opens a state when the score is at least tau.  The ``s`` output holds the
    score either way.

    ``init``: optional starting cache, dict with m [S], S [S,C,dv,dk] (float64
    or float32), I [S,C] int64, n [S,C] int32, start [S,C] int64, has_prev [S],
    s_prev [S], k_prev [S,dk], t_seen [S].
    ``want``: optional bool mask [S,T] of the outputs to compute (others are 0).
    ``lib``: a handle from ``load_library`` (default: the oracle itself).
    """
    q, k, v, lam = (_c(a, np.float32) for a in (q, k, v, lam))
    S_, T, dk = k.shape
    dv = v.shape[2]
    assert q.shape == (S_, T, dk) and v.shape[:2] == (S_, T) and lam.shape == (S_, T, C_)
    keep = []

    def hold(a):
        keep.append(a)
        return _ptr(a)

    a = _Args()
    a.BH, a.T, a.dk, a.dv, a.C, a.tau = S_, T, dk, dv, C_, float(tau)
    a.q, a.k, a.v, a.lam = hold(q), hold(k), hold(v), hold(lam)
    if init is not None:
        a.init_m = hold(_c(init["m"], np.int32))
        a.init_S = hold(_c(init["S"], np.float64))
        a.init_I = hold(_c(init["I"], np.int64))
        a.init_n = hold(_c(init["n"], np.int32))
        a.init_start = hold(_c(init["start"], np.int64))
        a.init_has_prev = hold(_c(init["has_prev"], np.int32))
        a.init_s_prev = hold(_c(init["s_prev"], np.float32))
        a.init_k_prev = hold(_c(init["k_prev"], np.float32))
        a.init_t_seen = hold(_c(init["t_seen"], np.int64))
    if want is not None:
        a.want_o = hold(_c(want, np.uint8))
    res = {}

    def out(name, shape, dt, field):
        arr = np.zeros(shape, dt)
        res[name] = arr
        setattr(a, field, hold(arr))

    if outputs:
        out("o", (S_, T, dv), np.float64, "o")
    out("s", (S_, T), np.float32, "s_out")
    out("b", (S_, T), np.uint8, "b_out")
    out("seg", (S_, T), np.int32, "seg_out")
    out("m_t", (S_, T), np.int32, "m_out")
    out("ev_t", (S_, max(T, 1)), np.int32, "ev_t")
    out("ev_i", (S_, max(T, 1)), np.int32, "ev_i")
    out("n_ev", (S_,), np.int32, "n_ev")
    out("fin_m", (S_,), np.int32, "fin_m")
    if final_states:
        out("fin_S", (S_, C_, dv, dk), np.float64, "fin_S")
    out("fin_I", (S_, C_), np.int64, "fin_I")
    out("fin_n", (S_, C_), np.int32, "fin_n")
    out("fin_start", (S_, C_), np.int64, "fin_start")
    out("fin_has_prev", (S_,), np.int32, "fin_has_prev")
    out("fin_s_prev", (S_,), np.float32, "fin_s_prev")
    out("fin_k_prev", (S_, dk), np.float32, "fin_k_prev")
    out("fin_t_seen", (S_,), np.int64, "fin_t_seen")
    a.nthreads = int(nthreads or os.environ.get("DLA_ORACLE_THREADS", 0) or os.cpu_count() or 1)
    a.merge_rule = MERGE_RULES[merge_rule]
    a.score_rule = SCORE_RULES[score_rule]
    rc = (lib or _load()).dlao_run(C.byref(a))
    if rc != 0:
        raise RuntimeError(f"dlao_run failed with code {rc}")
    res["events"] = [list(zip(res["ev_t"][i, :res["n_ev"][i]].tolist(),
                              res["ev_i"][i, :res["n_ev"][i]].tolist())) for i in range(S_)]
    return res


# ----------------------------------------------------------------------------
# Independent cross-checks (numpy / plain Python).  They share no code with
# dla_oracle.c and recompute what the oracle claims from first principles.
# ----------------------------------------------------------------------------

def fixed_point(s) -> np.ndarray:
    """Token information on the 2^-32 grid, round half to even (int64)."""
    return np.rint(np.ldexp(np.asarray(s, np.float64), 32)).astype(np.int64)


def start_sets(T: int, boundaries, events, init_starts=()):
    """Replay a schedule: the sorted list of live state starts after each token.

    ``boundaries``: iterable of 0/1 per token; ``events``: list of (t, i) merges
    of chronological pair (i, i+1) right after token t was appended.
    """
    starts = list(init_starts)
    ev = {}
    for t, i in events:
        ev[t] = i
    out = []
    for t in range(T):
        if boundaries[t]:
            starts.append(t)
            if t in ev:
                del starts[ev[t] + 1]
        out.append(tuple(starts))
    return out


def brute_force(q, k, v, lam, sets, rows=None) -> np.ndarray:
    """o_t = sum_{s<=t} lam_t[#{p in P_t : p > s}] (q_t . k_s) v_s for one stream.

    ``sets[t]`` is the start set P_t after token t (tokens of this call start at
    0; earlier starts may be negative).  float64.  ``rows`` limits the tokens.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    lam = np.asarray(lam, np.float64)
    T, dv = v.shape
    rows = range(T) if rows is None else rows
    out = np.zeros((T, dv))
    for t in rows:
        P = np.asarray(sets[t])
        s_idx = np.arange(t + 1)
        slot = (P[None, :] > s_idx[:, None]).sum(1)
        w = lam[t, slot]
        a = k[: t + 1] @ q[t]
        out[t] = (w * a) @ v[: t + 1]
    return out


def check_schedule(s, tau: float, C_: int, boundaries, events, m_t=None,
                   init=None, merge_rule: str = "sum", score_rule: str = "cosine") -> None:
    """Assert that a schedule is exactly what the greedy rule produces from s.

    Re-derives from the float32 token information ``s`` alone: every boundary
    (two-consecutive-low rule, s == tau counts as high), the moment of every
    merge (right after an append that exceeds C states, never otherwise), and
    every merged pair: summed information and token count of each live state
    are recomputed from the token ranges it covers, and the merged pair must
    be the earliest adjacent pair of minimal summed information ("sum") or of
    minimal information density, (I_i + I_{i+1}) / (n_i + n_{i+1}) as an exact
    fraction ("density").  With ``score_rule="state"`` the boundary rule is
    the single-token one, s_t >= tau (or an empty cache).  ``init`` (optional)
    is a starting cache: dict with
    starts (list, oldest first, relative to this call's token 0), infos (int64
    list), counts (int list; needed by "density") and s_prev (float) /
    has_prev.
    """
    from fractions import Fraction
    s = np.asarray(s, np.float32)
    T = len(s)
    qs = fixed_point(s)
    tau32 = np.float32(tau)
    starts = [] if init is None else list(init["starts"])
    base_info = {} if init is None else dict(zip(init["starts"], init["infos"]))
    base_count = {} if init is None or "counts" not in init else dict(zip(init["starts"], init["counts"]))
    assert merge_rule in ("sum", "density")
    assert merge_rule == "sum" or init is None or "counts" in init
    prev = np.float32(1.0) if init is None else np.float32(init["s_prev"])
    ev = {}
    for t, i in events:
        assert t not in ev, f"two merges after token {t}"
        ev[t] = i

    def info(a, b_end):
        # summed information of the tokens [a, b_end) of this call, plus the
        # information the starting cache holds for states that began in that
        # range before the call (their starts are negative)
        lo = max(a, 0)
        tot = int(qs[lo:b_end].sum()) if b_end > lo else 0
        return tot + sum(int(x) for p, x in base_info.items() if a <= p < b_end)

    def count(a, b_end):
        # tokens of [a, b_end) in this call plus those a starting state held
        lo = max(a, 0)
        return max(b_end - lo, 0) + sum(int(x) for p, x in base_count.items() if a <= p < b_end)

    assert score_rule in ("cosine", "state")
    for t in range(T):
        if score_rule == "state":
            expect_b = (len(starts) == 0) or bool(s[t] >= tau32)
        else:
            low = (s[t] < tau32) and (prev < tau32)
            expect_b = (len(starts) == 0) or (not low)
        assert bool(boundaries[t]) == expect_b, f"boundary mismatch at token {t}"
        if expect_b:
            starts.append(t)
            if len(starts) > C_:
                assert t in ev, f"cache exceeds C after token {t} but no merge logged"
                ends = starts[1:] + [t + 1]
                I = [info(a, e) for a, e in zip(starts, ends)]
                if merge_rule == "sum":
                    keys = [I[i] + I[i + 1] for i in range(len(I) - 1)]
                else:
                    n = [count(a, e) for a, e in zip(starts, ends)]
                    keys = [Fraction(I[i] + I[i + 1], n[i] + n[i + 1]) for i in range(len(I) - 1)]
                best = min(range(len(keys)), key=lambda i: (keys[i], i))
                assert ev[t] == best, f"token {t}: merged pair {ev[t]}, greedy gives {best}"
                del starts[best + 1]
            else:
                assert t not in ev, f"merge logged at token {t} without overflow"
        else:
            assert t not in ev, f"merge logged at non-boundary token {t}"
        assert len(starts) <= C_
        if m_t is not None:
            assert int(m_t[t]) == len(starts), f"m_t mismatch at token {t}"
        prev = s[t]


def state_scores_closed_form(v, k, sets, init_last=None, eps: float = 1e-6) -> np.ndarray:
    """State information scores of one stream recomputed from a schedule.

    For token t the current state is the most recent state after token t-1,
    the sum of v_s k_s^T over its tokens [a, t) with a the largest start in
    ``sets[t-1]``; ``init_last`` = (start, S) gives the most recent state of a
    starting cache (its start < 0), the current state of token 0.  With
    c = <v_t k_t^T, S>_F / (|v_t k_t^T|_F |S|_F) = v_t^T S k_t / (|v_t| |k_t| |S|_F),
    each RMS-normalised matrix has Frobenius norm sqrt(D) (D = d_v d_k) and
    |N(a) - N(S)|_F^2 = 2 D (1 - c), so the score is
    sqrt(2 D (1 - c)) / (sqrt(D) + eps); 2 without a current state or for a
    zero matrix.  float64; the current state is summed afresh from its token
    range, not taken from the oracle's bookkeeping.
    """
    v = np.asarray(v, np.float64)
    k = np.asarray(k, np.float64)
    T, dv = v.shape
    D = float(dv * k.shape[1])
    out = np.zeros(T)
    a, S = (None, None) if init_last is None else (init_last[0], np.array(init_last[1], np.float64))
    for t in range(T):
        if t > 0:
            a_new = max(sets[t - 1])
            if a_new == a:
                S = S + np.outer(v[t - 1], k[t - 1])
            else:
                assert a_new >= 0, "a state older than the call cannot become the most recent one"
                S = v[a_new:t].T @ k[a_new:t]
                a = a_new
        if S is None:
            out[t] = 2.0
            continue
        nv, nk, ns = np.linalg.norm(v[t]), np.linalg.norm(k[t]), np.linalg.norm(S)
        if nv * nk == 0.0 or ns == 0.0:
            out[t] = 2.0
        else:
            c = float(v[t] @ S @ k[t]) / (nv * nk * ns)
            out[t] = np.sqrt(max(0.0, 2.0 * D * (1.0 - c))) / (np.sqrt(D) + eps)
    return out
