"""Seeded synthetic inputs for the Dynamic Linear Attention (DLA) layer.

This module only draws random numbers and rounds them to the io dtype.  It
holds none of the layer's arithmetic (no score, no boundary, no merge, no
read), so both the CPU oracle and the GPU path can consume its output.

Workload recipe (one stream = one (batch, head) pair):
  * keys are piecewise-regime: the stream is cut into segments whose lengths
    are Geometric with mean mu (support 1, 2, ...; the last one is truncated),
    every segment has its own centroid drawn as N(0, I) and scaled to unit
    norm, and every key is centroid + noise;
  * noise, "relative" reading (default): 0.2 * N(0, I / d_k), i.e. a noise
    vector of norm about 0.2 around a unit centroid;
    noise, "literal" reading: 0.2 * N(0, I) per coordinate (norm 0.2*sqrt(d_k));
  * q ~ N(0, I / d_k), v ~ N(0, I / d_v); with values="regime" the values
    follow the key segments instead: a unit N(0, I) centroid per segment
    plus 0.2 * N(0, I / d_v) noise (a workload on which a score of the
    states, not only of the keys, sees the segments);
  * lambda = sigmoid(N(0, 1)), one value per (token, cache slot);
  * bf16 workloads round every fp32 draw once to bf16 (round to nearest even)
    and hand back the rounded values as float32 arrays.

Streams draw from independent child seeds of numpy's SeedSequence(seed), in
the order: segment lengths, centroids, noise, q, v, lambda.  A stream's values
therefore do not depend on how many streams are drawn or in which order.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "Config", "CONFIGS", "round_bf16", "prefill_inputs", "decode_inputs",
    "segment_lengths",
]


@dataclass(frozen=True)
class Config:
    name: str
    B: int
    H: int
    T: int            # tokens per stream (prefill) or decode steps
    dk: int
    dv: int
    C: int
    tau: float
    io: str           # "f32" or "bf16"
    seg_means: tuple  # one mean, or several means picked with equal probability
    seed: int
    kind: str = "prefill"   # "prefill" or "decode"
    init_tokens: int = 0    # decode: outer products summed into each initial state
    note: str = field(default="", compare=False)


# The five workloads.  Names describe the workload; seeds are fixed per workload.
CONFIGS = {
    "tiny_fp32": Config("tiny_fp32", 1, 1, 512, 64, 64, 8, 0.3, "f32", (64,), 1,
                        note="tiny fp32 layer, oracle finishes in seconds"),
    "mamba2_780m_bf16": Config("mamba2_780m_bf16", 4, 24, 8192, 128, 64, 16, 0.3,
                               "bf16", (256,), 2,
                               note="Mamba-2-780M-shaped layer"),
    "gdn_1p3b_t32k_bf16": Config("gdn_1p3b_t32k_bf16", 2, 16, 32768, 128, 256, 32,
                                 0.3, "bf16", (32, 2048), 3,
                                 note="Gated-DeltaNet-1.3B-shaped layer, T=32K, "
                                      "bursty segment lengths"),
    "long_t131k_bf16": Config("long_t131k_bf16", 1, 16, 131072, 128, 128, 32, 0.3,
                              "bf16", (512,), 4,
                              note="long-context prefill, T=131072"),
    "decode_b256_bf16": Config("decode_b256_bf16", 256, 16, 4096, 128, 128, 32, 0.3,
                               "bf16", (128,), 5, kind="decode", init_tokens=64,
                               note="batched decode, full caches, 4096 steps"),
}


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (ties to even); return float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    out = r.astype(np.uint32).view(np.float32)
    # NaN/Inf never occur in these workloads; keep them untouched anyway
    bad = ~np.isfinite(x)
    if bad.any():
        out = out.copy()
        out[bad] = x[bad]
    return out.reshape(x.shape)


def segment_lengths(rng: np.random.Generator, T: int, means: tuple) -> np.ndarray:
    """Geometric segment lengths (support >= 1) covering exactly T tokens."""
    out = []
    total = 0
    while total < T:
        if len(means) == 1:
            mu = means[0]
        else:
            mu = means[int(rng.integers(len(means)))]
        n = int(rng.geometric(1.0 / mu))
        n = min(n, T - total)
        out.append(n)
        total += n
    return np.asarray(out, dtype=np.int64)


def _keys(rng, T, dk, means, reading):
    lens = segment_lengths(rng, T, means)
    cent = rng.standard_normal((len(lens), dk), dtype=np.float32)
    cent /= np.linalg.norm(cent, axis=1, keepdims=True)
    noise = rng.standard_normal((T, dk), dtype=np.float32)
    if reading == "relative":
        noise *= np.float32(0.2 / np.sqrt(dk))
    elif reading == "literal":
        noise *= np.float32(0.2)
    else:
        raise ValueError(f"unknown noise reading {reading!r}")
    k = np.repeat(cent, lens, axis=0) + noise
    return k.astype(np.float32), lens


def _sigmoid(x):
    return (1.0 / (1.0 + np.exp(-x.astype(np.float64)))).astype(np.float32)


def _stream(seed_seq, T, dk, dv, C, means, reading, io, values="random"):
    rng = np.random.default_rng(seed_seq)
    k, lens = _keys(rng, T, dk, means, reading)
    q = rng.standard_normal((T, dk), dtype=np.float32) * np.float32(1.0 / np.sqrt(dk))
    if values == "regime":
        vc = rng.standard_normal((len(lens), dv), dtype=np.float32)
        vc /= np.linalg.norm(vc, axis=1, keepdims=True)
        v = (np.repeat(vc, lens, axis=0) +
             rng.standard_normal((T, dv), dtype=np.float32) * np.float32(0.2 / np.sqrt(dv))).astype(np.float32)
    elif values == "random":
        v = rng.standard_normal((T, dv), dtype=np.float32) * np.float32(1.0 / np.sqrt(dv))
    else:
        raise ValueError(f"unknown values {values!r}")
    lam = _sigmoid(rng.standard_normal((T, C), dtype=np.float32))
    if io == "bf16":
        q, k, v, lam = (round_bf16(a) for a in (q, k, v, lam))
    return q, k, v, lam, lens


def _workers(n):
    return max(1, min(n, int(os.environ.get("DLA_GEN_THREADS", os.cpu_count() or 1)), 16))


def prefill_inputs(cfg: Config | str, reading: str = "relative", streams=None,
                   T: int | None = None, seed: int | None = None, values: str = "random") -> dict:
    """Inputs of one prefill workload.

    Returns float32 arrays q,k [S,T,dk], v [S,T,dv], lam [S,T,C] where S is the
    number of streams drawn (all B*H by default, or the flat stream indices in
    ``streams``), plus the per-stream segment lengths.  ``T`` truncates the
    streams (the draw itself is unchanged up to T only through the segment
    lengths, so a truncated draw is a different, equally valid workload).
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    T = cfg.T if T is None else int(T)
    seed = cfg.seed if seed is None else seed
    BH = cfg.B * cfg.H
    idx = list(range(BH)) if streams is None else [int(i) for i in streams]
    children = np.random.SeedSequence(seed).spawn(BH)
    S = len(idx)
    q = np.empty((S, T, cfg.dk), np.float32)
    k = np.empty((S, T, cfg.dk), np.float32)
    v = np.empty((S, T, cfg.dv), np.float32)
    lam = np.empty((S, T, cfg.C), np.float32)
    lens = [None] * S

    def one(j):
        qq, kk, vv, ll, ln = _stream(children[idx[j]], T, cfg.dk, cfg.dv, cfg.C,
                                     cfg.seg_means, reading, cfg.io, values)
        q[j], k[j], v[j], lam[j], lens[j] = qq, kk, vv, ll, ln

    with _cf.ThreadPoolExecutor(_workers(S)) as ex:
        list(ex.map(one, range(S)))
    return dict(q=q, k=k, v=v, lam=lam, seg_lens=lens, streams=idx, T=T, cfg=cfg,
                reading=reading, values=values)


def decode_inputs(cfg: Config | str = "decode_b256_bf16", reading: str = "relative",
                  caches=None, steps: int | None = None, seed: int | None = None) -> dict:
    """Initial full caches plus per-step inputs of the batched decode workload.

    Every cache starts with C states, oldest first.  State i is the sum of
    ``init_tokens`` outer products v k^T (v ~ N(0, I/d_v), k ~ N(0, I/d_k),
    summed in float64 and rounded once to float32), holds ``init_tokens``
    tokens starting at token init_tokens*i, and carries an information sum
    drawn as Exp(1) and quantised to the 2^-32 grid (int64).  No previous key
    exists.  Step inputs q, k, v, lam per cache follow the prefill recipe with
    the decode segment mean.
    """
    if isinstance(cfg, str):
        cfg = CONFIGS[cfg]
    steps = cfg.T if steps is None else int(steps)
    seed = cfg.seed if seed is None else seed
    BH = cfg.B * cfg.H
    idx = list(range(BH)) if caches is None else [int(i) for i in caches]
    children = np.random.SeedSequence(seed).spawn(BH)
    S, C, dk, dv, n0 = len(idx), cfg.C, cfg.dk, cfg.dv, cfg.init_tokens
    states = np.empty((S, C, dv, dk), np.float32)
    info = np.empty((S, C), np.int64)
    q = np.empty((S, steps, dk), np.float32)
    k = np.empty((S, steps, dk), np.float32)
    v = np.empty((S, steps, dv), np.float32)
    lam = np.empty((S, steps, C), np.float32)

    def one(j):
        rng = np.random.default_rng(children[idx[j]])
        vv0 = rng.standard_normal((C, dv, n0), dtype=np.float32) * np.float32(1 / np.sqrt(dv))
        kk0 = rng.standard_normal((C, dk, n0), dtype=np.float32) * np.float32(1 / np.sqrt(dk))
        if cfg.io == "bf16":
            vv0, kk0 = round_bf16(vv0), round_bf16(kk0)
        states[j] = np.matmul(vv0.astype(np.float64),
                              np.swapaxes(kk0, 1, 2).astype(np.float64)).astype(np.float32)
        e = rng.exponential(1.0, size=C)
        info[j] = np.rint(np.ldexp(e, 32)).astype(np.int64)
        kk, _ = _keys(rng, steps, dk, cfg.seg_means, reading)
        qq = rng.standard_normal((steps, dk), dtype=np.float32) * np.float32(1 / np.sqrt(dk))
        vv = rng.standard_normal((steps, dv), dtype=np.float32) * np.float32(1 / np.sqrt(dv))
        ll = _sigmoid(rng.standard_normal((steps, C), dtype=np.float32))
        if cfg.io == "bf16":
            qq, kk, vv, ll = (round_bf16(a) for a in (qq, kk, vv, ll))
        q[j], k[j], v[j], lam[j] = qq, kk, vv, ll

    with _cf.ThreadPoolExecutor(_workers(S)) as ex:
        list(ex.map(one, range(S)))
    count = np.full((S, C), n0, np.int32)
    start = (np.arange(C, dtype=np.int64) * n0)[None, :].repeat(S, 0)
    return dict(states=states, info=info, count=count, start=start, t_seen=C * n0,
                q=q, k=k, v=v, lam=lam, caches=idx, steps=steps, cfg=cfg,
                reading=reading)
