"""The C-ABI library loads, exports what include/dla.h declares, and rejects bad
arguments on the host before anything is enqueued (no GPU needed)."""
import ctypes as C
import os
import re

import pytest

import dynamic_state_memory_amd as dla

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "dla.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(dla_[a-z_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = dla.load()
    names = _declared()
    assert {"dla_prefill", "dla_decode_step", "dla_cache_init"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert dla.dla_abi_version() == 7


def test_sizes_and_layout():
    assert dla.dla_cache_bytes(1, 1, 8, 64, 64) > 8 * 64 * 64 * 4
    assert dla.dla_cache_bytes(1, 1, 0, 64, 64) == 0
    assert dla.dla_cache_bytes(1, 1, 65, 64, 64) == 0
    assert dla.dla_cache_bytes(1, 1, 8, 96, 64) == 0
    assert dla.dla_cache_bytes(1, 1, 8, 512, 64) == 0
    assert dla.dla_cache_bytes(1, 1, 8, 256, 64) > 8 * 256 * 64 * 4
    assert dla.dla_cache_bytes(1, 1, 8, 64, 24) == 0
    L = dla.dla_cache_layout(2, 3, 32, 128, 256)
    assert L.meta_offset >= 6 * 32 * 128 * 256 * 4 and L.meta_offset % 256 == 0
    assert L.meta_stride % 256 == 0 and L.off_k_prev + 4 * 128 <= L.meta_stride
    assert dla.dla_cache_bytes(2, 3, 32, 128, 256) == L.meta_offset + 6 * L.meta_stride
    ws = dla.dla_prefill_workspace_bytes(2, 16, 32768, 32, 128, 256)
    assert ws > 32 * 32768 * 8
    assert dla.dla_prefill_workspace_bytes(2, 16, 0, 32, 128, 256) == 0
    assert dla.dla_status_str(3) == "workspace missing or too small"


def test_prefill_kernel_choice(monkeypatch):
    # the environment never changes the choice; only the explicit hook does
    monkeypatch.setenv("DLA_PREFILL_PATH", "streamed")
    monkeypatch.setenv("DLA_PREFILL_DVT", "32")
    assert dla.dla_prefill_kernel(dla.DLA_BF16, 2, 16, 32, 128, 256) == "k_prefill_rs<128,16,8>"
    assert dla.dla_prefill_kernel(dla.DLA_BF16, 4, 24, 16, 128, 64) == "k_prefill_rs<128,16,4>"
    assert dla.dla_prefill_kernel(dla.DLA_F32, 1, 1, 8, 64, 64) == "k_prefill<f32,64,16>"
    assert dla.dla_prefill_kernel(dla.DLA_F32, 1, 1, 8, 128, 64) == "k_prefill<f32,128,16>"
    assert dla.dla_prefill_kernel(dla.DLA_BF16, 1, 1, 48, 64, 64) == "k_prefill<bf16,64,16>"
    assert dla.dla_prefill_kernel(dla.DLA_BF16, 1, 1, 8, 256, 64) == "k_prefill<bf16,256,16>"
    # d_k = 256 and fp32 d_k = 128 keep 16-column slices (32 would not fit the LDS)
    assert dla.dla_prefill_kernel(dla.DLA_BF16, 8, 32, 8, 256, 256) == "k_prefill<bf16,256,16>"
    assert dla.dla_prefill_kernel(dla.DLA_BF16, 1, 1, 8, 96, 64) is None
    try:
        assert dla.dla_set_prefill_path(dla.DLA_PATH_STREAMED, 0) == dla.DLA_OK
        assert dla.dla_prefill_kernel(dla.DLA_BF16, 2, 16, 32, 128, 256) == "k_prefill<bf16,128,32>"
        assert dla.dla_set_prefill_path(dla.DLA_PATH_STREAMED, 16) == dla.DLA_OK
        assert dla.dla_prefill_kernel(dla.DLA_BF16, 2, 16, 32, 128, 256) == "k_prefill<bf16,128,16>"
        assert dla.dla_set_prefill_path(7, 0) == dla.DLA_ERR_ARG
        # the register-resident sweep without its split along the sequence:
        # the same kernel
        assert dla.dla_set_prefill_path(dla.DLA_PATH_UNSPLIT, 0) == dla.DLA_OK
        assert dla.dla_prefill_kernel(dla.DLA_BF16, 1, 16, 32, 128, 128) == "k_prefill_rs<128,16,8>"
        assert dla.dla_set_prefill_path(dla.DLA_PATH_STREAMED, 16) == dla.DLA_OK
        assert dla.dla_set_prefill_path(dla.DLA_PATH_AUTO, 24) == dla.DLA_ERR_ARG
        # (a refused call changes nothing)
        assert dla.dla_prefill_kernel(dla.DLA_BF16, 2, 16, 32, 128, 256) == "k_prefill<bf16,128,16>"
    finally:
        dla.dla_set_prefill_path(dla.DLA_PATH_AUTO, 0)
    assert dla.dla_prefill_kernel(dla.DLA_BF16, 2, 16, 32, 128, 256) == "k_prefill_rs<128,16,8>"


def test_split_sweep_workspace():
    """A sweep grid of at most 256 blocks may be split along the sequence:
    its workspace holds the slots of up to three more block sets, one per 8
    chunks beyond the first 8 (a larger grid's does not)."""
    slot_bytes = 4 * 16 * 32 * 128 * 128            # B*H = 16 streams, C = 32, d_k = d_v = 128
    ws = [dla.dla_prefill_workspace_bytes(1, 16, 64 * n, 32, 128, 128) for n in (8, 15, 16, 24, 32)]
    per_chunk = ws[1] - ws[0]                       # no split slots below 16 chunks
    assert ws[2] - ws[1] >= slot_bytes > ws[2] - ws[1] - 2 * per_chunk
    assert ws[3] - ws[2] >= slot_bytes and ws[4] - ws[3] >= slot_bytes
    big = [dla.dla_prefill_workspace_bytes(2, 16, 64 * n, 32, 128, 256) for n in (15, 16)]   # 512 blocks
    assert big[1] - big[0] < slot_bytes


def _cache(B=1, H=1, C_=8, dk=64, dv=64, base=0x10000):
    c = dla.dla_cache()
    c.B, c.H, c.C, c.d_k, c.d_v = B, H, C_, dk, dv
    c.base = base
    c.bytes = dla.dla_cache_bytes(B, H, C_, dk, dv)
    return c


def test_bad_arguments_are_rejected_on_the_host():
    # fake, aligned device addresses: validation must fail before any use
    p = 0x100000
    c = _cache()
    ws = dla.dla_prefill_workspace_bytes(1, 1, 100, 8, 64, 64)
    ok_args = dict(q=p, k=p, v=p, lam=p, o=p, T=100, tau=0.3, io=dla.DLA_F32, cache=c,
                   workspace=p, workspace_bytes=ws, sched=None, stream=None)

    def call(**kw):
        a = dict(ok_args)
        a.update(kw)
        return dla.dla_prefill(a["q"], a["k"], a["v"], a["lam"], a["o"], a["T"], a["tau"], a["io"],
                               a["cache"], a["workspace"], a["workspace_bytes"], a["sched"],
                               a["stream"])

    assert call(q=None) == dla.DLA_ERR_ARG and "non-NULL" in dla.dla_last_error()
    assert call(k=p + 4) == dla.DLA_ERR_ARG and "aligned" in dla.dla_last_error()
    assert call(T=0) == dla.DLA_ERR_ARG
    assert call(T=(1 << 24) + 1) == dla.DLA_ERR_ARG
    assert call(io=7) == dla.DLA_ERR_ARG
    assert call(tau=float("nan")) == dla.DLA_ERR_ARG
    assert call(workspace_bytes=ws - 1) == dla.DLA_ERR_WORKSPACE
    assert call(workspace=None) == dla.DLA_ERR_WORKSPACE
    assert call(cache=_cache(C_=0)) == dla.DLA_ERR_ARG
    assert call(cache=_cache(base=0)) == dla.DLA_ERR_ARG
    assert call(cache=_cache(base=0x10010)) == dla.DLA_ERR_ARG
    c_small = _cache()
    c_small.bytes -= 1
    assert call(cache=c_small) == dla.DLA_ERR_ARG
    # fp32 io stops at d_k = 128 (the streamed kernel's LDS at d_k = 256)
    assert call(cache=_cache(dk=256, dv=64), io=dla.DLA_F32,
                workspace_bytes=dla.dla_prefill_workspace_bytes(1, 1, 100, 8, 256, 64)) \
        == dla.DLA_ERR_UNSUPPORTED
    assert "LDS" in dla.dla_last_error()
    # decode: d_v outside {64, 128, 256}
    assert dla.dla_decode_step(p, p, p, p, None, 0.3, dla.DLA_BF16, c, None, None) == dla.DLA_ERR_ARG
    assert dla.dla_decode_step(p, p, p, p, p, 0.3, dla.DLA_BF16, _cache(dk=64, dv=96), None, None) \
        == dla.DLA_ERR_UNSUPPORTED
    assert dla.dla_decode_step(p, p, p, p, p, 0.3, dla.DLA_BF16, _cache(dk=64, dv=512), None, None) \
        == dla.DLA_ERR_UNSUPPORTED
    # cache init
    cc = dla.dla_cache()
    f32 = dla.DLA_F32
    assert dla.dla_cache_init(cc, 0, 1 << 20, 1, 1, 8, 64, 64, f32, None, None) == dla.DLA_ERR_ARG
    assert dla.dla_cache_init(cc, p, 16, 1, 1, 8, 64, 64, f32, None, None) == dla.DLA_ERR_ARG
    pre = dla.dla_cache_preload(9, 0, p, p, p, p, 0)
    assert dla.dla_cache_init(cc, p, 1 << 30, 1, 1, 8, 64, 64, f32, pre, None) == dla.DLA_ERR_ARG
    pre = dla.dla_cache_preload(2, 0, None, p, p, p, 0)
    assert dla.dla_cache_init(cc, p, 1 << 30, 1, 1, 8, 64, 64, f32, pre, None) == dla.DLA_ERR_ARG


def test_bf16_state_storage_layout_and_checks():
    B, H, C_, dk, dv = 2, 3, 32, 128, 256
    L32 = dla.dla_cache_layout(B, H, C_, dk, dv, dla.DLA_F32)
    L16 = dla.dla_cache_layout(B, H, C_, dk, dv, dla.DLA_BF16)
    n_states = B * H * C_ * dv * dk
    # fp32: no active region; bf16: half-size slots, then one fp32 state per stream
    assert L32.active_offset == L32.meta_offset and L32.meta_offset >= 4 * n_states
    assert L16.active_offset >= 2 * n_states and L16.active_offset % 256 == 0
    assert L16.meta_offset >= L16.active_offset + 4 * B * H * dv * dk and L16.meta_offset % 256 == 0
    assert L16.meta_offset < L32.meta_offset
    assert dla.dla_cache_bytes(B, H, C_, dk, dv, dla.DLA_BF16) == L16.meta_offset + B * H * L16.meta_stride
    assert dla.dla_cache_bytes(B, H, C_, dk, dv, 7) == 0
    p = 0x100000
    cc = dla.dla_cache()
    assert dla.dla_cache_init(cc, p, 1 << 30, 1, 1, 8, 64, 64, 7, None, None) == dla.DLA_ERR_ARG
    assert "state dtype" in dla.dla_last_error()
    # the workspace holds an fp32 copy of every state (the streamed path on a
    # bf16 cache), even when the chunk records are smaller
    assert dla.dla_prefill_workspace_bytes(1, 1, 64, 64, 128, 512) >= 4 * 64 * 128 * 512
    c = _cache()
    c.state_dtype = dla.DLA_BF16
    c.bytes = dla.dla_cache_bytes(1, 1, 8, 64, 64, dla.DLA_BF16)
    ws = dla.dla_prefill_workspace_bytes(1, 1, 100, 8, 64, 64)
    assert dla.dla_prefill(p, p, p, p, p, 100, 0.3, dla.DLA_F32, c, p, ws - 1, None, None) == dla.DLA_ERR_WORKSPACE
    c.state_dtype = 3
    assert dla.dla_prefill(p, p, p, p, p, 100, 0.3, dla.DLA_BF16, c, p, ws, None, None) == dla.DLA_ERR_ARG


def test_merge_rule_is_validated_on_the_host():
    p = 0x100000
    # the view's layout: the rule sits where the header puts it
    assert C.sizeof(dla.dla_cache) == 48 and dla.dla_cache.merge_rule.offset == 20
    assert dla.dla_cache.score_rule.offset == 28
    assert dla.dla_cache.state_dtype.offset == 24 and dla.dla_cache.base.offset == 32
    c = _cache()
    assert c.merge_rule == dla.DLA_MERGE_SUM
    assert dla.load().dla_cache_set_merge_rule(C.byref(c), 3) == dla.DLA_ERR_ARG
    assert "merge rule" in dla.dla_last_error() and c.merge_rule == dla.DLA_MERGE_SUM
    assert dla.load().dla_cache_set_merge_rule(None, 1) == dla.DLA_ERR_ARG
    dla.dla_cache_set_merge_rule(c, dla.DLA_MERGE_DENSITY)
    assert c.merge_rule == dla.DLA_MERGE_DENSITY
    # a rule set directly in the view is checked by prefill and decode
    c.merge_rule = 5
    ws = dla.dla_prefill_workspace_bytes(1, 1, 100, 8, 64, 64)
    assert dla.dla_prefill(p, p, p, p, p, 100, 0.3, dla.DLA_F32, c, p, ws, None, None) == dla.DLA_ERR_ARG
    assert "merge rule" in dla.dla_last_error()
    assert dla.dla_decode_step(p, p, p, p, p, 0.3, dla.DLA_BF16, c, None, None) == dla.DLA_ERR_ARG


def test_fenwick_rule_checks_on_the_host():
    p = 0x100000
    c = _cache()                      # C = 8: levels 0 .. 7, enough for T <= 128
    dla.dla_cache_set_merge_rule(c, dla.DLA_FENWICK)
    assert c.merge_rule == dla.DLA_FENWICK

    def pre(T, io=dla.DLA_BF16, sched=None, cache=c):
        ws = dla.dla_prefill_workspace_bytes(1, 1, T, 8, 64, 64)
        return dla.dla_prefill(p, p, p, p, p, T, 0.3, io, cache, p, ws, sched, None)

    # 129 tokens need 9 level weights
    assert pre(129) == dla.DLA_ERR_ARG and "levels" in dla.dla_last_error()
    # float32 state storage only
    cb = _cache()
    cb.state_dtype = dla.DLA_BF16
    cb.bytes = dla.dla_cache_bytes(1, 1, 8, 64, 64, dla.DLA_BF16)
    dla.dla_cache_set_merge_rule(cb, dla.DLA_FENWICK)
    assert pre(100, cache=cb) == dla.DLA_ERR_UNSUPPORTED and "float32 state" in dla.dla_last_error()
    # no schedule export
    sc = dla.dla_schedule_out()
    sc.m_t = p
    assert pre(100, sched=sc) == dla.DLA_ERR_UNSUPPORTED and "export" in dla.dla_last_error()
    # decode: float32 state storage and no schedule export either
    c64 = _cache(dk=64, dv=64)
    dla.dla_cache_set_merge_rule(c64, dla.DLA_FENWICK)
    assert dla.dla_decode_step(p, p, p, p, p, 0.3, dla.DLA_BF16, c64, sc, None) == dla.DLA_ERR_UNSUPPORTED
    assert "export" in dla.dla_last_error()
    assert dla.dla_decode_step(p, p, p, p, p, 0.3, dla.DLA_BF16, cb, None, None) == dla.DLA_ERR_UNSUPPORTED
    assert "float32 state" in dla.dla_last_error()


def test_gpu_package_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "dynamic_state_memory_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".cpp", ".h")):
                txt = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in txt.lower(), f


def test_score_rule_is_validated_on_the_host():
    p = 0x100000
    c = _cache(dk=128, dv=128)
    assert c.score_rule == dla.DLA_SCORE_COSINE
    assert dla.load().dla_cache_set_score_rule(C.byref(c), 2) == dla.DLA_ERR_ARG
    assert "score rule" in dla.dla_last_error() and c.score_rule == dla.DLA_SCORE_COSINE
    assert dla.load().dla_cache_set_score_rule(None, 1) == dla.DLA_ERR_ARG
    dla.dla_cache_set_score_rule(c, dla.DLA_SCORE_STATE)
    assert c.score_rule == dla.DLA_SCORE_STATE

    def pre(cache, io=dla.DLA_BF16, T=100):
        ws = dla.dla_prefill_workspace_bytes(cache.B, cache.H, T, cache.C, cache.d_k, cache.d_v)
        return dla.dla_prefill(p, p, p, p, p, T, 0.6, io, cache, p, ws, None, None)

    def dec(cache, io=dla.DLA_BF16):
        return dla.dla_decode_step(p, p, p, p, p, 0.6, io, cache, None, None)

    # shapes the state score does not take, refused before any launch
    for dk, dv, io in [(128, 96, dla.DLA_BF16), (256, 256, dla.DLA_BF16), (128, 256, dla.DLA_F32),
                       (256, 64, dla.DLA_F32)]:
        cc = _cache(dk=dk, dv=dv)
        dla.dla_cache_set_score_rule(cc, dla.DLA_SCORE_STATE)
        assert pre(cc, io) == dla.DLA_ERR_UNSUPPORTED, (dk, dv, io)
        if dv in (64, 128, 256):
            assert dec(cc, io) == dla.DLA_ERR_UNSUPPORTED, (dk, dv, io)
    # a cache view with an unknown rule written into it
    c.score_rule = 5
    assert pre(c) == dla.DLA_ERR_ARG and "score rule" in dla.dla_last_error()
    assert dec(c) == dla.DLA_ERR_ARG
