"""Shared plumbing of the GPU parity tests: run the HIP path through the C ABI
on numpy inputs and compare what it returns with the oracle."""
from __future__ import annotations

import os
import sys

import numpy as np

from tests.helpers import mat_rel_err, row_rel_err

TOL = {"f32": 1e-4, "bf16": 2e-2}
STATE_TOL = 1e-4
# final states of a cache storing closed states in bf16: the gate of a bf16
# configuration per state matrix (max |diff| / max |ref|), the same 2e-2 as its
# outputs.  Each bf16 write rounds relative 2^-9, and a state that absorbs k
# merges is rounded k times (worst seen: 1.05e-2 after a 1200-token prefill and
# 300 decode steps under the density rule)
STATE_TOL_BF16_STORAGE = 2e-2


def say(msg: str):
    print(f"[gpu-test] {msg}", flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    if not torch.cuda.is_available():
        import pytest
        pytest.skip("no GPU")
    return torch


def oracle_threads() -> int:
    return min(os.cpu_count() or 1, 16)


def gpu_prefill(q, k, v, lam, C, tau, io, B=None, H=None, repeats=1, merge_rule="sum", state_dtype="f32",
                score_rule="cosine"):
    """q,k [S,T,dk] ... float32 numpy (already bf16-valued for bf16).  Returns
    o (float32 numpy [S,T,dv]), schedule dict, final cache dict."""
    torch = torch_mod()
    import dynamic_state_memory_amd as dla
    S, T, dk = k.shape
    dv = v.shape[2]
    B = 1 if B is None else B
    H = S // B if H is None else H
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    dev = torch.device("cuda:0")

    def up(a, d):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev).to(dt).reshape(B, H, T, d)

    tq, tk, tv, tl = up(q, dk), up(k, dk), up(v, dv), up(lam, C)
    BH = B * H
    sched = dict(s=torch.empty(BH, T, dtype=torch.float32, device=dev),
                 boundary=torch.empty(BH, T, dtype=torch.uint8, device=dev),
                 seg_id=torch.empty(BH, T, dtype=torch.int32, device=dev),
                 m_t=torch.empty(BH, T, dtype=torch.int32, device=dev),
                 ev_t=torch.empty(BH, T, dtype=torch.int32, device=dev),
                 ev_i=torch.empty(BH, T, dtype=torch.int32, device=dev),
                 n_ev=torch.empty(BH, dtype=torch.int32, device=dev))
    cache = dla.Cache(B, H, C, dk, dv, device=dev, merge_rule=merge_rule, state_dtype=state_dtype,
                      score_rule=score_rule)
    ws = dla.prefill_workspace(B, H, T, C, dk, dv, dev)
    outs = []
    for rep in range(repeats):
        if rep:
            cache.reset()        # a prefill continues the cache: start afresh each time
        o = dla.prefill(tq, tk, tv, tl, tau, cache, workspace=ws, sched=sched)
        torch.cuda.synchronize()
        outs.append(o.float().cpu().numpy().reshape(S, T, dv))
    sc = {kk: vv.cpu().numpy() for kk, vv in sched.items()}
    fin = cache.read()
    if repeats == 1:
        return outs[0], sc, fin
    return outs, sc, fin


def gpu_prefill_pieces(q, k, v, lam, C, tau, io, ends, merge_rule="sum", state_dtype="f32", score_rule="cosine"):
    """Prefill the tokens [0, ends[0]), [ends[0], ends[1]), ... of every
    stream with one dla_prefill call each, on one cache.  Returns the outputs
    (float32 [S,T,dv]), per-piece schedule dicts and the final cache dict."""
    torch = torch_mod()
    import dynamic_state_memory_amd as dla
    S, T, dk = k.shape
    dv = v.shape[2]
    dt = torch.bfloat16 if io == "bf16" else torch.float32
    dev = torch.device("cuda:0")
    cache = dla.Cache(1, S, C, dk, dv, device=dev, merge_rule=merge_rule, state_dtype=state_dtype,
                      score_rule=score_rule)
    outs, scheds, lo = [], [], 0
    for hi in ends:
        n = hi - lo

        def up(a, d):
            return torch.from_numpy(np.ascontiguousarray(a[:, lo:hi])).to(dev).to(dt).reshape(1, S, n, d)

        sched = dict(s=torch.empty(S, n, dtype=torch.float32, device=dev),
                     boundary=torch.empty(S, n, dtype=torch.uint8, device=dev),
                     m_t=torch.empty(S, n, dtype=torch.int32, device=dev),
                     ev_t=torch.empty(S, n, dtype=torch.int32, device=dev),
                     ev_i=torch.empty(S, n, dtype=torch.int32, device=dev),
                     n_ev=torch.empty(S, dtype=torch.int32, device=dev))
        o = dla.prefill(up(q, dk), up(k, dk), up(v, dv), up(lam, C), tau, cache, sched=sched)
        torch.cuda.synchronize()
        outs.append(o.float().cpu().numpy().reshape(S, n, dv))
        scheds.append({kk: vv.cpu().numpy() for kk, vv in sched.items()})
        lo = hi
    return np.concatenate(outs, 1), scheds, cache.read()


def compare_schedule(r, sc, fin, label="", s_tol=None):
    """Bit-exact comparison of a GPU prefill schedule and final metadata with
    the oracle.  With s_tol the token scores may differ by that much (the
    state score: the GPU reads the states in a different precision and order),
    the rest of the schedule stays exact."""
    S = r["s"].shape[0]
    if s_tol is None:
        bad_s = np.flatnonzero(r["s"].view(np.uint32) != sc["s"].view(np.uint32))
        assert len(bad_s) == 0, (f"{label}: {len(bad_s)} token scores differ, first at "
                                f"{np.unravel_index(bad_s[0], r['s'].shape)}")
    else:
        ds = np.abs(r["s"].astype(np.float64) - sc["s"])
        assert ds.max() <= s_tol, f"{label}: token scores differ by up to {ds.max():.3e} > {s_tol}"
    assert np.array_equal(r["b"], sc["boundary"]), f"{label}: boundaries differ"
    assert np.array_equal(r["seg"], sc["seg_id"]), f"{label}: segment ids differ"
    assert np.array_equal(r["m_t"], sc["m_t"]), f"{label}: state counts differ"
    assert np.array_equal(r["n_ev"], sc["n_ev"]), f"{label}: merge counts differ"
    for i in range(S):
        n = int(r["n_ev"][i])
        assert np.array_equal(r["ev_t"][i, :n], sc["ev_t"][i, :n]), f"{label}: merge tokens differ ({i})"
        assert np.array_equal(r["ev_i"][i, :n], sc["ev_i"][i, :n]), f"{label}: merged pairs differ ({i})"
    assert np.array_equal(r["fin_m"], fin["m"]), f"{label}: final m differs"
    for i in range(S):
        m = int(r["fin_m"][i])
        if s_tol is None:
            assert np.array_equal(r["fin_I"][i, :m], fin["info"][i, :m]), f"{label}: info differs ({i})"
        else:
            # sums of scores that may each differ by s_tol (units of 2^-32)
            bound = (np.asarray(r["fin_n"][i, :m], np.float64) * s_tol + 1e-9) * 2.0 ** 32
            assert np.all(np.abs(r["fin_I"][i, :m] - fin["info"][i, :m]) <= bound), f"{label}: info differs ({i})"
        assert np.array_equal(r["fin_n"][i, :m], fin["count"][i, :m]), f"{label}: counts differ ({i})"
        assert np.array_equal(r["fin_start"][i, :m], fin["start"][i, :m]), f"{label}: starts differ ({i})"
        assert sorted(fin["order"][i, :m].tolist()) == sorted(set(fin["order"][i, :m].tolist())), \
            f"{label}: physical slots repeat ({i})"
    if s_tol is None:
        assert np.array_equal(r["fin_s_prev"], fin["s_prev"]), f"{label}: s_prev differs"
    else:
        assert np.abs(r["fin_s_prev"] - fin["s_prev"]).max() <= s_tol, f"{label}: s_prev differs"
    assert np.array_equal(r["fin_k_prev"], fin["k_prev"]), f"{label}: k_prev differs"
    assert np.array_equal(r["fin_t_seen"], fin["t_seen"]), f"{label}: t_seen differs"


def compare_states(r, fin, tol=STATE_TOL, label=""):
    S = r["fin_m"].shape[0]
    worst = 0.0
    for i in range(S):
        m = int(r["fin_m"][i])
        worst = max(worst, mat_rel_err(fin["S"][i, :m], r["fin_S"][i, :m]))
    assert worst <= tol, f"{label}: final states max rel err {worst:.3e} > {tol}"
    return worst


def compare_outputs(o_gpu, o_ref, tol, label="", mask=None):
    if mask is not None:
        o_gpu, o_ref = o_gpu[mask], o_ref[mask]
    err = row_rel_err(o_gpu, o_ref)
    assert err <= tol, f"{label}: outputs max row rel err {err:.3e} > {tol}"
    return err
