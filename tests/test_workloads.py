"""The seeded generator: bf16 rounding, determinism and workload statistics."""
import numpy as np
import torch

import oracle
import workloads


def test_round_bf16_matches_library_conversion():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10.0 ** rng.integers(-30, 30, 100000),
                        np.array([0.0, -0.0, 1.0, 1 + 2 ** -8, 1 + 2 ** -9, 1 + 3 * 2 ** -9, 3e38], np.float32)])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(workloads.round_bf16(x).view(np.uint32), ref.view(np.uint32))


def test_streams_are_deterministic_and_independent_of_subset():
    a = workloads.prefill_inputs("mamba2_780m_bf16", streams=[3, 7], T=300)
    b = workloads.prefill_inputs("mamba2_780m_bf16", streams=[7], T=300)
    assert np.array_equal(a["k"][1], b["k"][0]) and np.array_equal(a["lam"][1], b["lam"][0])
    c = workloads.prefill_inputs("mamba2_780m_bf16", streams=[3, 7], T=300)
    assert all(np.array_equal(a[x], c[x]) for x in ("q", "k", "v", "lam"))
    # bf16 workloads hold bf16 values
    assert np.array_equal(workloads.round_bf16(a["q"]), a["q"])


def test_segment_statistics_and_readings():
    cfg = workloads.CONFIGS["mamba2_780m_bf16"]
    d = workloads.prefill_inputs(cfg, streams=range(4), T=8192)
    lens = np.concatenate(d["seg_lens"])
    assert sum(d["seg_lens"][0]) == 8192
    assert 200 < lens[:-1].mean() < 320            # Geometric(mean 256)
    r = oracle.run(d["q"], d["k"], d["v"], d["lam"], cfg.C, cfg.tau, outputs=False,
                   final_states=False)
    low = (r["s"] < cfg.tau).mean()
    assert low > 0.97                               # relative noise: within-segment s ~ 0.04
    nseg = sum(len(x) for x in d["seg_lens"])
    # every regime change opens a state and so does the token after it
    assert abs(int(r["b"].sum()) - 2 * nseg) <= 8
    lit = workloads.prefill_inputs(cfg, reading="literal", streams=[0], T=2048)
    r2 = oracle.run(lit["q"], lit["k"], lit["v"], lit["lam"], cfg.C, cfg.tau, outputs=False,
                    final_states=False)
    assert (r2["s"] < cfg.tau).mean() < 0.01        # literal noise: every token is a boundary


def test_mixed_segment_means():
    d = workloads.prefill_inputs("gdn_1p3b_t32k_bf16", streams=[0, 1], T=32768)
    lens = np.concatenate([x[:-1] for x in d["seg_lens"]])
    assert (lens < 200).mean() > 0.3 and (lens > 500).mean() > 0.3


def test_decode_initial_cache():
    d = workloads.decode_inputs(caches=[0, 4095], steps=16)
    cfg = d["cfg"]
    assert d["states"].shape == (2, cfg.C, cfg.dv, cfg.dk)
    assert d["info"].dtype == np.int64 and np.all(d["info"] > 0)
    assert np.all(d["count"] == 64) and d["start"][0, 1] == 64
    # a sum of 64 outer products of N(0, 1/d) vectors has entries of variance 64/d^2
    sd = d["states"].std()
    assert 0.8 * 8 / 128 < sd < 1.2 * 8 / 128
    assert d["q"].shape == (2, 16, cfg.dk) and d["lam"].shape == (2, 16, cfg.C)
