"""Parity of the Log-Linear fixed (Fenwick) schedule on the GPU with its oracle
(oracle/fenwick.py): outputs within the gate of their io dtype, final cache --
the buckets of the prefix -- exact in its metadata and within the state gate in
its matrices.  A prefill followed by decode steps must give what the oracle
gives over all the tokens at once.  Inputs come from the seeded workload
generator with lam holding one weight per level."""
import dataclasses

import numpy as np
import pytest

import oracle.fenwick as FEN
import workloads
from tests.gpu_common import STATE_TOL, TOL, compare_outputs, say, torch_mod
from tests.helpers import mat_rel_err

pytestmark = pytest.mark.gpu


def _inputs(T, streams, C, dk=128, dv=64, base="gdn_1p3b_t32k_bf16"):
    cfg = dataclasses.replace(workloads.CONFIGS[base], C=C, dk=dk, dv=dv)
    return workloads.prefill_inputs(cfg, streams=streams, T=T)


def _run(d, C, B=1, H=None, cache=None):
    torch = torch_mod()
    import dynamic_state_memory_amd as dla
    q, k, v, lam = d["q"], d["k"], d["v"], d["lam"]
    S, T, dk = k.shape
    dv = v.shape[2]
    H = S // B if H is None else H
    dev = torch.device("cuda:0")

    def up(a, n):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(torch.bfloat16).reshape(B, H, T, n)

    if cache is None:
        cache = dla.Cache(B, H, C, dk, dv, device=dev, merge_rule="fenwick")
    ws = dla.prefill_workspace(B, H, T, C, dk, dv, dev)
    o = dla.prefill(up(q, dk), up(k, dk), up(v, dv), up(lam, C), 0.0, cache, workspace=ws)
    torch.cuda.synchronize()
    return o.float().cpu().numpy().reshape(S, T, dv), cache.read()


def _check_cache(fin, k, v, T, label, state_streams=None):
    """Metadata of every stream exact; each state matrix (of the streams in
    state_streams, default all) within the state gate."""
    S = k.shape[0]
    m = bin(T).count("1")
    assert (fin["m"] == m).all(), f"{label}: live states {fin['m']} != popcount({T}) = {m}"
    assert (fin["t_seen"] == T).all() and (fin["has_prev"] == 0).all(), label
    C = fin["order"].shape[1]
    bk = FEN.buckets(T)
    for x in range(S):
        assert list(fin["start"][x, :m]) == [a for a, _, _ in bk], f"{label}: starts of stream {x}"
        assert list(fin["count"][x, :m]) == [n for _, n, _ in bk], f"{label}: counts of stream {x}"
        assert (fin["info"][x, :m] == 0).all(), label
        order = list(fin["order"][x, :m])
        assert len(set(order)) == m and all(0 <= p < C for p in order), f"{label}: slots {order}"
    for x in (range(S) if state_streams is None else state_streams):
        ref = FEN.final_states(k[x:x + 1], v[x:x + 1], T)[0]
        for i, (_, _, R) in enumerate(ref):
            err = mat_rel_err(fin["S"][x, i], R)
            assert err <= STATE_TOL, f"{label}: stream {x} state {i} rel err {err:.2e} > {STATE_TOL}"


# T spans: a single token, partial first chunks, exact chunk multiples with
# odd and even last chunks (the carried merges at the end), ragged tails after
# odd and even chunks, and carries across 2, 4, 8 and 16 chunks
TS = [1, 2, 5, 63, 64, 65, 127, 128, 129, 192, 256, 300, 511, 512, 513, 777, 1024, 1100, 2256, 4160]


@pytest.mark.parametrize("T", TS)
def test_fenwick_prefill_matches_oracle(T):
    say(f"fenwick T={T}")
    d = _inputs(T, [0, 1, 2], 16)
    o, fin = _run(d, 16)
    ref = FEN.outputs(d["q"], d["k"], d["v"], d["lam"])
    compare_outputs(o, ref, TOL["bf16"], f"fenwick T={T}")
    _check_cache(fin, d["k"], d["v"], T, f"fenwick T={T}")


@pytest.mark.parametrize("dk,dv,C,T", [(64, 32, 8, 128), (64, 32, 12, 700), (128, 64, 32, 1500),
                                       (64, 16, 32, 64 * 17 + 9), (128, 128, 13, 4096)])
def test_fenwick_shapes_and_capacities(dk, dv, C, T):
    say(f"fenwick dk={dk} dv={dv} C={C} T={T}")
    d = _inputs(T, [3, 4], C, dk=dk, dv=dv)
    o, fin = _run(d, C, B=2, H=1)
    compare_outputs(o, FEN.outputs(d["q"], d["k"], d["v"], d["lam"]), TOL["bf16"], f"dk={dk} C={C} T={T}")
    _check_cache(fin, d["k"], d["v"], T, f"dk={dk} C={C} T={T}")


def _random_shapes(n, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        T = int(rng.integers(1, 3000))
        dk = int(rng.choice([64, 128]))
        dv = int(16 * rng.integers(1, 17))
        L = FEN.levels_needed(T)
        C = int(rng.integers(L, 33))
        S = int(rng.integers(1, 7))
        out.append((T, dk, dv, C, S))
    return out


@pytest.mark.parametrize("T,dk,dv,C,S", _random_shapes(12))
def test_fenwick_random_shapes(T, dk, dv, C, S):
    """Seeded random shapes within the supported ranges: T in [1, 3000), d_k in
    {64, 128}, d_v a multiple of 16 up to 256, C from the level count to 32,
    1 to 6 streams."""
    say(f"fenwick random T={T} dk={dk} dv={dv} C={C} S={S}")
    d = _inputs(T, list(range(S)), C, dk=dk, dv=dv)
    o, fin = _run(d, C, B=1, H=S)
    compare_outputs(o, FEN.outputs(d["q"], d["k"], d["v"], d["lam"]), TOL["bf16"], f"T={T} dk={dk} dv={dv} C={C}")
    _check_cache(fin, d["k"], d["v"], T, f"T={T} dk={dk} dv={dv} C={C}")


@pytest.mark.parametrize("ends", [(100, 300), (64, 128, 192), (1, 2, 3, 70), (63, 127, 1000), (500, 501, 1300),
                                  (777, 2100)])
def test_fenwick_prefill_continues_the_cache(ends):
    """Prefill in pieces on one cache (chunks of later pieces not aligned to
    the buckets) equals one pass of the oracle over all the tokens."""
    torch = torch_mod()
    import dynamic_state_memory_amd as dla
    say(f"fenwick pieces {ends}")
    T = ends[-1]
    d = _inputs(T, [16, 17], 16)
    cache = dla.Cache(1, 2, 16, 128, 64, device=torch.device("cuda:0"), merge_rule="fenwick")
    outs, lo = [], 0
    for hi in ends:
        o, _ = _run({x: d[x][:, lo:hi] for x in ("q", "k", "v", "lam")}, 16, cache=cache)
        outs.append(o)
        lo = hi
    compare_outputs(np.concatenate(outs, 1), FEN.outputs(d["q"], d["k"], d["v"], d["lam"]), TOL["bf16"],
                    f"pieces {ends}")
    _check_cache(cache.read(), d["k"], d["v"], T, f"pieces {ends}")


def test_fenwick_prefill_decode_prefill():
    """Prefill 300, decode 37 steps, prefill 500 more: one pass of the oracle."""
    torch = torch_mod()
    import dynamic_state_memory_amd as dla
    say("fenwick prefill + decode + prefill")
    T1, T2, T3 = 300, 37, 500
    T = T1 + T2 + T3
    d = _inputs(T, [18, 19], 16, dk=128, dv=128)
    cache = dla.Cache(1, 2, 16, 128, 128, device=torch.device("cuda:0"), merge_rule="fenwick")
    o1, _ = _run({x: d[x][:, :T1] for x in ("q", "k", "v", "lam")}, 16, cache=cache)
    o2 = _decode_steps(d, T1, T1 + T2, cache, "bf16")
    o3, _ = _run({x: d[x][:, T1 + T2:] for x in ("q", "k", "v", "lam")}, 16, cache=cache)
    compare_outputs(np.concatenate([o1, o2, o3], 1), FEN.outputs(d["q"], d["k"], d["v"], d["lam"]), TOL["bf16"],
                    "prefill + decode + prefill")
    _check_cache(cache.read(), d["k"], d["v"], T, "prefill + decode + prefill")


@pytest.fixture
def streamed_path():
    import dynamic_state_memory_amd as dla
    dla.dla_set_prefill_path(dla.DLA_PATH_STREAMED, 0)
    yield
    dla.dla_set_prefill_path(dla.DLA_PATH_AUTO, 0)


def _streamed_prefill_pieces(d, ends, C, dk, dv, io, cache):
    torch = torch_mod()
    import dynamic_state_memory_amd as dla
    dev = torch.device("cuda:0")
    dt = torch.float32 if io == "f32" else torch.bfloat16
    S = d["k"].shape[0]
    outs, lo = [], 0
    for hi in ends:
        def up(a, n):
            return torch.from_numpy(np.ascontiguousarray(a[:, lo:hi])).to(dev).to(dt).reshape(1, S, hi - lo, n)
        ws = dla.prefill_workspace(1, S, hi - lo, C, dk, dv, dev)
        o = dla.prefill(up(d["q"], dk), up(d["k"], dk), up(d["v"], dv), up(d["lam"], C), 0.0, cache, workspace=ws)
        outs.append(o.float().cpu().numpy().reshape(S, hi - lo, dv))
        lo = hi
    torch.cuda.synchronize()
    return np.concatenate(outs, 1)


@pytest.mark.parametrize("io,dk,ends,C", [("f32", 64, (300,), 16), ("f32", 64, (100, 613, 1000), 16),
                                          ("bf16", 128, (700,), 16), ("bf16", 64, (65, 400, 1100), 16),
                                          ("f32", 64, (200, 900), 48), ("bf16", 128, (500, 1300), 64),
                                          ("f32", 128, (130, 800), 16), ("bf16", 256, (90, 600), 24)])
def test_fenwick_streamed_kernel(io, dk, ends, C, streamed_path):
    """The fixed schedule on the streamed prefill kernel (fp32 io, C > 32 or
    d_k = 256; bf16 io forced there): from position 0 and continuing, one pass
    of the oracle."""
    torch = torch_mod()
    import dynamic_state_memory_amd as dla
    say(f"fenwick streamed io={io} dk={dk} ends={ends} C={C}")
    T = ends[-1]
    d = _inputs(T, [21, 22], C, dk=dk, dv=32)
    cache = dla.Cache(1, 2, C, dk, 32, device=torch.device("cuda:0"), merge_rule="fenwick")
    o = _streamed_prefill_pieces(d, ends, C, dk, 32, io, cache)
    compare_outputs(o, FEN.outputs(d["q"], d["k"], d["v"], d["lam"]), TOL[io], f"streamed {io} {ends}")
    _check_cache(cache.read(), d["k"], d["v"], T, f"streamed {io} {ends}")


def test_fenwick_streamed_position_limit(streamed_path):
    """The position limit on the streamed kernel with fp32 io: C = 4 level
    weights cover positions 0 .. 7, so 5 tokens at position 5 are refused on
    the device (NaN outputs, the cache as it was); 3 tokens are not."""
    torch = torch_mod()
    import dynamic_state_memory_amd as dla
    say("fenwick streamed prefill position limit (f32)")
    d = _inputs(10, [20], 4, dk=64, dv=16)
    cache = dla.Cache(1, 1, 4, 64, 16, device=torch.device("cuda:0"), merge_rule="fenwick")
    _streamed_prefill_pieces(d, (5,), 4, 64, 16, "f32", cache)
    before = cache.read()
    part = {x: d[x][:, 5:10] for x in ("q", "k", "v", "lam")}
    o = _streamed_prefill_pieces(part, (5,), 4, 64, 16, "f32", cache)
    assert np.isnan(o).all()
    after = cache.read()
    for key in ("m", "t_seen", "order", "start", "count", "S"):
        assert np.array_equal(before[key], after[key]), key
    part = {x: d[x][:, 5:8] for x in ("q", "k", "v", "lam")}
    o = _streamed_prefill_pieces(part, (3,), 4, 64, 16, "f32", cache)
    ref = FEN.outputs(*(d[x][:, :8] for x in ("q", "k", "v", "lam")))
    compare_outputs(o, ref[:, 5:8], TOL["f32"], "positions 5 .. 7")
    _check_cache(cache.read(), d["k"], d["v"], 8, "positions 0 .. 7")


def test_fenwick_prefill_position_limit():
    """C = 4 level weights cover positions 0 .. 7: a prefill of 5 tokens on a
    stream at position 5 is refused on the device (NaN outputs, the cache as it
    was); the same prefill of 3 tokens is not."""
    torch = torch_mod()
    import dynamic_state_memory_amd as dla
    say("fenwick prefill position limit")
    d = _inputs(10, [20], 4, dk=64, dv=16)
    cache = dla.Cache(1, 1, 4, 64, 16, device=torch.device("cuda:0"), merge_rule="fenwick")
    part = lambda lo, hi: {x: d[x][:, lo:hi] for x in ("q", "k", "v", "lam")}
    _run(part(0, 5), 4, cache=cache)
    before = cache.read()
    o, after = _run(part(5, 10), 4, cache=cache)
    assert np.isnan(o).all()
    for key in ("m", "t_seen", "order", "start", "count", "S"):
        assert np.array_equal(before[key], after[key]), key
    o, fin = _run(part(5, 8), 4, cache=cache)
    ref = FEN.outputs(*(d[x][:, :8] for x in ("q", "k", "v", "lam")))
    compare_outputs(o, ref[:, 5:8], TOL["bf16"], "positions 5 .. 7")
    _check_cache(fin, d["k"], d["v"], 8, "positions 0 .. 7")


@pytest.mark.parametrize("name,C,T", [("gdn_1p3b_t32k_bf16", 16, None), ("long_t131k_bf16", 18, 131072 - 77)])
def test_fenwick_full_size_sampled(name, C, T):
    """Full-size layers in the benchmark's launch configuration: the
    Gated-DeltaNet-1.3B-shaped one (B=2, H=16, T=32768, d_k=128, d_v=256) with
    16 level weights, and the long-context one (B=1, H=16, d=128) over 131072 -
    77 tokens with 18 (a ragged last chunk after 2047 full ones).  Outputs at
    sampled tokens of every stream within the bf16 gate, metadata of every
    stream exact, the final states of four streams within the state gate."""
    say(f"fenwick full size {name}: generating inputs")
    cfg = dataclasses.replace(workloads.CONFIGS[name], C=C)
    d = workloads.prefill_inputs(cfg, T=T)
    S, T = d["k"].shape[:2]
    say(f"fenwick full size {name}: GPU prefill")
    o, fin = _run(d, C, B=cfg.B, H=cfg.H)
    rng = np.random.default_rng(7)
    rows = sorted(set(rng.choice(T, 20, replace=False).tolist()) | {0, 1, 63, 64, 4095, 4096, 16383, T - 1})
    say(f"fenwick full size {name}: oracle rows ({len(rows)} per stream)")
    ref = FEN.output_rows(d["q"], d["k"], d["v"], d["lam"], rows)
    err = compare_outputs(o[:, rows], ref, TOL["bf16"], f"fenwick full size {name}")
    _check_cache(fin, d["k"], d["v"], T, f"fenwick full size {name}", state_streams=[0, 5, 9, S - 1])
    say(f"fenwick full size {name}: ok, sampled max row rel err {err:.2e}")


def _decode_steps(d, lo, hi, cache, io):
    """Decode tokens lo .. hi-1 of every stream one dla_decode_step at a time."""
    torch = torch_mod()
    import dynamic_state_memory_amd as dla
    B, H, C, dk, dv = cache.shape
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    dev = cache.device
    outs = []
    for t in range(lo, hi):
        def one(a, n):
            return torch.from_numpy(np.ascontiguousarray(a[:, t])).to(dev).to(dt).reshape(B, H, n)
        o = dla.decode_step(one(d["q"], dk), one(d["k"], dk), one(d["v"], dv), one(d["lam"], C), 0.0, cache)
        outs.append(o.float().cpu().numpy().reshape(B * H, 1, dv))
    torch.cuda.synchronize()
    return np.concatenate(outs, 1) if outs else np.zeros((B * H, 0, dv), np.float32)


@pytest.mark.parametrize("T0,k,dd,io,dv", [(0, 70, 64, "f32", 64), (0, 40, 128, "bf16", 128),
                                           (1, 66, 128, "bf16", 128), (64, 70, 64, "bf16", 64),
                                           (100, 60, 128, "bf16", 128), (255, 70, 64, "bf16", 64),
                                           (512, 33, 128, "bf16", 128), (1000, 50, 64, "bf16", 64),
                                           (300, 40, 128, "bf16", 64), (200, 50, 128, "bf16", 256),
                                           (0, 60, 256, "bf16", 128), (150, 30, 64, "bf16", 256),
                                           (200, 20, 256, "bf16", 64)])
def test_fenwick_decode_continues_the_stream(T0, k, dd, io, dv):
    """Prefill T0 tokens (none: decode from an empty cache), then k decode
    steps: outputs and final cache as one pass of the oracle over T0 + k
    (d_k = dd, and d_v = dv, equal or not)."""
    torch = torch_mod()
    import dynamic_state_memory_amd as dla
    say(f"fenwick decode T0={T0} k={k} d_k={dd} d_v={dv} io={io}")
    T = T0 + k
    d = _inputs(T, [11, 12], 16, dk=dd, dv=dv)
    cache = dla.Cache(1, 2, 16, dd, dv, device=torch.device("cuda:0"), merge_rule="fenwick")
    parts = []
    if T0:
        pre = {x: d[x][:, :T0] for x in ("q", "k", "v", "lam")}
        o_pre, _ = _run(pre, 16, cache=cache)
        parts.append(o_pre)
    parts.append(_decode_steps(d, T0, T, cache, io))
    o = np.concatenate(parts, 1)
    ref = FEN.outputs(d["q"], d["k"], d["v"], d["lam"])
    compare_outputs(o, ref, TOL[io], f"prefill {T0} + decode {k}")
    _check_cache(cache.read(), d["k"], d["v"], T, f"prefill {T0} + decode {k}")


def test_fenwick_decode_full_capacity():
    """C = 64, the largest capacity (no position limit within reach): decode
    from an empty cache as one pass of the oracle."""
    torch = torch_mod()
    import dynamic_state_memory_amd as dla
    say("fenwick decode C=64")
    d = _inputs(100, [14, 15], 64, dk=64, dv=64)
    cache = dla.Cache(1, 2, 64, 64, 64, device=torch.device("cuda:0"), merge_rule="fenwick")
    o = _decode_steps(d, 0, 100, cache, "f32")
    compare_outputs(o, FEN.outputs(d["q"], d["k"], d["v"], d["lam"]), TOL["f32"], "C=64")
    _check_cache(cache.read(), d["k"], d["v"], 100, "C=64")


def test_fenwick_decode_position_limit():
    """C = 4 level weights cover positions 0 .. 7; the step at position 8 is
    refused on the device: NaN outputs, the cache as it was."""
    torch = torch_mod()
    import dynamic_state_memory_amd as dla
    say("fenwick decode position limit")
    d = _inputs(9, [13], 4, dk=64, dv=64)
    cache = dla.Cache(1, 1, 4, 64, 64, device=torch.device("cuda:0"), merge_rule="fenwick")
    o = _decode_steps(d, 0, 8, cache, "f32")
    ref = FEN.outputs(*(d[x][:, :8] for x in ("q", "k", "v", "lam")))
    compare_outputs(o, ref, TOL["f32"], "positions 0 .. 7")
    before = cache.read()
    o8 = _decode_steps(d, 8, 9, cache, "f32")
    assert np.isnan(o8).all()
    after = cache.read()
    for key in ("m", "t_seen", "order", "start", "count", "S"):
        assert np.array_equal(before[key], after[key]), key
