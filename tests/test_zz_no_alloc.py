"""dla_prefill_noalloc (the library's static scratch instead of a workspace)
gives what dla_prefill gives on the same inputs, on two calls in a row, the
second one smaller, through the C ABI (also where only the workspace call
has room to split its sweep along the sequence); too large a call is refused
on the host."""
import dataclasses

import numpy as np
import pytest

import dynamic_state_memory_amd as dla
import workloads
from tests.gpu_common import say, torch_mod


def test_noalloc_refuses_calls_past_the_scratch():
    # host-side check, before any device work (fake aligned addresses)
    p = 0x100000
    c = dla.dla_cache()
    c.B, c.H, c.C, c.d_k, c.d_v = 2, 16, 32, 128, 256
    c.base = p
    c.bytes = dla.dla_cache_bytes(2, 16, 32, 128, 256)
    assert dla.dla_prefill_workspace_bytes(2, 16, 32768, 32, 128, 256) > dla.DLA_NOALLOC_SCRATCH_BYTES
    st = dla.dla_prefill_noalloc(p, p, p, p, p, 32768, 0.3, dla.DLA_BF16, c, None, None)
    assert st == dla.DLA_ERR_WORKSPACE and "static scratch" in dla.dla_last_error()


def _run(entry, q, k, v, lam, C, tau, dev, merge_rule="sum"):
    torch = torch_mod()
    B, H, T, dk = q.shape
    dv = v.shape[3]
    BH = B * H
    cache = dla.Cache(B, H, C, dk, dv, device=dev, merge_rule=merge_rule)
    sched = dict(s=torch.empty(BH, T, dtype=torch.float32, device=dev),
                 boundary=torch.empty(BH, T, dtype=torch.uint8, device=dev),
                 m_t=torch.empty(BH, T, dtype=torch.int32, device=dev),
                 ev_t=torch.empty(BH, T, dtype=torch.int32, device=dev),
                 ev_i=torch.empty(BH, T, dtype=torch.int32, device=dev),
                 n_ev=torch.empty(BH, dtype=torch.int32, device=dev))
    if merge_rule == "fenwick":
        sched = {}           # the fixed schedule has no schedule export
    if entry == "noalloc":
        o = dla.prefill_noalloc(q, k, v, lam, tau, cache, sched=sched or None)
    else:
        o = dla.prefill(q, k, v, lam, tau, cache, sched=sched or None)
    torch.cuda.synchronize()
    return o.float().cpu().numpy(), {x: y.cpu().numpy() for x, y in sched.items()}, cache.read()


@pytest.mark.gpu
@pytest.mark.parametrize("case", ["bf16_register", "f32_streamed", "bf16_fenwick", "bf16_split_fallback"])
def test_noalloc_matches_the_workspace_entry(case):
    torch = torch_mod()
    dev = torch.device("cuda:0")
    if case == "bf16_register":
        cfg, H, sizes, rule = workloads.CONFIGS["mamba2_780m_bf16"], 4, (3000, 700), "sum"
    elif case == "f32_streamed":
        cfg, H, sizes, rule = dataclasses.replace(workloads.CONFIGS["tiny_fp32"], H=2), 2, (1500, 300), "sum"
    elif case == "bf16_fenwick":
        cfg, H, sizes, rule = workloads.CONFIGS["mamba2_780m_bf16"], 2, (2500, 600), "fenwick"
    else:
        # the workspace call splits its sweep along the sequence; the split's
        # slots do not fit the static scratch, so the allocation-free call runs
        # it unsplit (the same results, bit for bit)
        cfg, H, sizes, rule = workloads.CONFIGS["long_t131k_bf16"], 16, (1100, 600), "sum"
        assert dla.dla_prefill_workspace_bytes(1, H, sizes[0], cfg.C, cfg.dk, cfg.dv) > dla.DLA_NOALLOC_SCRATCH_BYTES
    dt = torch.bfloat16 if cfg.io == "bf16" else torch.float32
    C = cfg.C if rule != "fenwick" else 13
    for n, T in enumerate(sizes):
        say(f"noalloc {case}: call {n + 1}, B=1 H={H} T={T} C={C}")
        d = workloads.prefill_inputs(cfg, streams=range(H), T=T, seed=cfg.seed + 100 + n)

        def up(a, dd):
            return torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt).reshape(1, H, T, dd)

        q, k, v = up(d["q"], cfg.dk), up(d["k"], cfg.dk), up(d["v"], cfg.dv)
        lam = up(d["lam"][..., :C], C)
        o_w, s_w, f_w = _run("workspace", q, k, v, lam, C, cfg.tau, dev, rule)
        o_n, s_n, f_n = _run("noalloc", q, k, v, lam, C, cfg.tau, dev, rule)
        # the same kernels on the same inputs: every result bit for bit
        assert np.array_equal(o_w.view(np.uint32), o_n.view(np.uint32)), f"{case} T={T}: outputs differ"
        if rule != "fenwick":
            for key in s_w:
                assert np.array_equal(s_w[key], s_n[key]), f"{case} T={T}: schedule export {key} differs"
        for key in ("m", "order", "info", "count", "start", "t_seen", "s_prev", "k_prev"):
            assert np.array_equal(f_w[key], f_n[key]), f"{case} T={T}: final cache {key} differs"
        assert np.array_equal(f_w["S"].view(np.uint32), f_n["S"].view(np.uint32)), f"{case} T={T}: states differ"
