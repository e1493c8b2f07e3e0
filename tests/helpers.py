"""Test helpers: exact-score key construction and error metrics (no DLA arithmetic)."""
from __future__ import annotations

import numpy as np


def keys_for_scores(s_after_first, dk: int = 32, seed: int = 0) -> np.ndarray:
    """Keys k_0..k_{T-1} whose consecutive cosine distances are exactly the
    requested values (each in {0, 0.25, ..., 2}).

    Every key is +-(indicator of a 4-element coordinate set); two such keys
    have dot product +-|overlap|, squared norms 4, hence cos = +-overlap/4,
    all exact in binary floating point and in bf16.
    """
    rng = np.random.default_rng(seed)
    T = len(s_after_first) + 1
    k = np.zeros((T, dk), np.float32)
    cur = list(rng.choice(dk, 4, replace=False))
    sign = 1.0
    k[0, cur] = sign
    for t, s in enumerate(s_after_first, start=1):
        c = 1.0 - float(s)
        assert abs(c * 4 - round(c * 4)) < 1e-12 and -1.0 <= c <= 1.0, s
        x = int(round(abs(c) * 4))
        if c < 0:
            sign = -sign
        keep = list(rng.choice(cur, x, replace=False)) if x else []
        pool = [i for i in range(dk) if i not in cur]
        fresh = list(rng.choice(pool, 4 - x, replace=False)) if x < 4 else []
        cur = keep + fresh
        k[t, cur] = sign
    return k


def row_rel_err(got, ref) -> float:
    """max over rows of max_j |got - ref| / max_j |ref| (rows along the last axis)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    g = got.reshape(-1, got.shape[-1])
    r = ref.reshape(-1, ref.shape[-1])
    num = np.abs(g - r).max(1)
    den = np.abs(r).max(1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max()) if len(num) else 0.0


def mat_rel_err(got, ref) -> float:
    """max over matrices (last two axes) of max |got - ref| / max |ref|."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    sh = got.shape
    g = got.reshape(-1, sh[-2] * sh[-1])
    r = ref.reshape(-1, sh[-2] * sh[-1])
    num = np.abs(g - r).max(1)
    den = np.abs(r).max(1)
    den = np.where(den == 0, 1.0, den)
    return float((num / den).max()) if len(num) else 0.0


def assert_close_to_sum(got, ref, ref_abs, rtol=1e-12):
    """|got - ref| <= rtol * max over the row of ref_abs, where ref_abs is the
    same sum taken over absolute values (a bound on the rounding error of any
    summation order, whatever the cancellation)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = np.asarray(ref_abs, np.float64).reshape(-1, got.shape[-1]).max(1)
    err = np.abs(got - ref).reshape(-1, got.shape[-1]).max(1)
    bad = err > rtol * np.maximum(scale, 1e-300)
    assert not bad.any(), f"rows {np.flatnonzero(bad)[:5]}: err {err[bad][:5]} scale {scale[bad][:5]}"
