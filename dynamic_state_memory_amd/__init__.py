"""Dynamic Linear Attention (DLA) layer forward pass on MI355X (gfx950).

Thin Python binding of ``libdla.so`` (include/dla.h).  The functions named
``dla_*`` are the C entry points with ctypes marshalling; ``Cache``,
``prefill`` and ``decode_step`` wrap them for torch device tensors.  PyTorch
only provides device memory and the current stream: every step of the layer
runs in the library's HIP kernels, and nothing here falls back to the CPU.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

__all__ = [
    "DLA_OK", "DLA_F32", "DLA_BF16", "DLAError", "lib_path", "load",
    "dla_abi_version", "dla_cache_bytes", "dla_cache_layout", "dla_cache_init",
    "dla_prefill_workspace_bytes", "dla_prefill", "dla_prefill_noalloc", "dla_decode_step",
    "dla_status_str", "dla_last_error", "dla_set_prefill_events", "dla_set_prefill_path", "Cache", "prefill",
    "decode_step",
    "prefill_workspace", "prefill_noalloc", "DLA_MAX_C", "DLA_CHUNK", "DLA_NOALLOC_SCRATCH_BYTES",
]

DLA_OK, DLA_ERR_ARG, DLA_ERR_UNSUPPORTED, DLA_ERR_WORKSPACE, DLA_ERR_HIP = 0, 1, 2, 3, 4
DLA_F32, DLA_BF16 = 0, 1
DLA_MERGE_SUM, DLA_MERGE_DENSITY, DLA_FENWICK = 0, 1, 2
DLA_PATH_AUTO, DLA_PATH_STREAMED, DLA_PATH_UNSPLIT = 0, 1, 2
DLA_SCORE_COSINE, DLA_SCORE_STATE = 0, 1
SCORE_RULES = {"cosine": DLA_SCORE_COSINE, "state": DLA_SCORE_STATE}
MERGE_RULES = {"sum": DLA_MERGE_SUM, "density": DLA_MERGE_DENSITY, "fenwick": DLA_FENWICK}
DLA_MAX_C = 64
DLA_CHUNK = 64
DLA_NOALLOC_SCRATCH_BYTES = 64 << 20

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB = os.path.join(_PKG, "_build", "libdla.so")
_lib = None


class DLAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_STATUS.get(status, status)}: {detail}")
        self.status = status


_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "workspace", 4: "HIP error"}


class dla_cache(C.Structure):
    _fields_ = [("B", C.c_int32), ("H", C.c_int32), ("C", C.c_int32), ("d_k", C.c_int32),
                ("d_v", C.c_int32), ("merge_rule", C.c_int32), ("state_dtype", C.c_int32),
                ("score_rule", C.c_int32), ("base", C.c_void_p), ("bytes", C.c_uint64)]


class dla_cache_layout_t(C.Structure):
    _fields_ = [("states_offset", C.c_uint64), ("active_offset", C.c_uint64), ("meta_offset", C.c_uint64),
                ("meta_stride", C.c_uint64), ("off_m", C.c_uint32), ("off_has_prev", C.c_uint32),
                ("off_s_prev", C.c_uint32), ("off_t_seen", C.c_uint32), ("off_order", C.c_uint32),
                ("off_info", C.c_uint32), ("off_count", C.c_uint32), ("off_start", C.c_uint32),
                ("off_k_prev", C.c_uint32)]


class dla_cache_preload(C.Structure):
    _fields_ = [("m0", C.c_int32), ("reserved", C.c_int32), ("states", C.c_void_p),
                ("info", C.c_void_p), ("count", C.c_void_p), ("start", C.c_void_p),
                ("t_seen", C.c_int64)]


class dla_schedule_out(C.Structure):
    _fields_ = [("s", C.c_void_p), ("boundary", C.c_void_p), ("seg_id", C.c_void_p),
                ("m_t", C.c_void_p), ("ev_t", C.c_void_p), ("ev_i", C.c_void_p),
                ("n_ev", C.c_void_p)]


def lib_path() -> str:
    return _LIB


def load():
    """Load libdla.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    try:
        # load torch's HIP runtime first so that the library binds to the same one
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(_LIB):
        raise RuntimeError(f"{_LIB} is missing: build it with `python __graft_entry__.py build` "
                           "or dynamic_state_memory_amd/build.py")
    lib = C.CDLL(_LIB)
    i32, u64, vp, f32 = C.c_int32, C.c_uint64, C.c_void_p, C.c_float
    lib.dla_abi_version.restype = i32
    lib.dla_abi_version.argtypes = []
    lib.dla_cache_bytes.restype = u64
    lib.dla_cache_bytes.argtypes = [i32] * 5 + [C.c_int]
    lib.dla_cache_layout.restype = C.c_int
    lib.dla_cache_layout.argtypes = [i32] * 5 + [C.c_int, C.POINTER(dla_cache_layout_t)]
    lib.dla_cache_init.restype = C.c_int
    lib.dla_cache_init.argtypes = [C.POINTER(dla_cache), vp, u64] + [i32] * 5 + \
        [C.c_int, C.POINTER(dla_cache_preload), vp]
    lib.dla_cache_set_merge_rule.restype = C.c_int
    lib.dla_cache_set_merge_rule.argtypes = [C.POINTER(dla_cache), i32]
    lib.dla_cache_set_score_rule.restype = C.c_int
    lib.dla_cache_set_score_rule.argtypes = [C.POINTER(dla_cache), i32]
    lib.dla_prefill_workspace_bytes.restype = u64
    lib.dla_prefill_workspace_bytes.argtypes = [i32] * 6
    lib.dla_prefill.restype = C.c_int
    lib.dla_prefill.argtypes = [vp, vp, vp, vp, vp, i32, f32, C.c_int, C.POINTER(dla_cache), vp,
                                u64, C.POINTER(dla_schedule_out), vp]
    lib.dla_prefill_noalloc.restype = C.c_int
    lib.dla_prefill_noalloc.argtypes = [vp, vp, vp, vp, vp, i32, f32, C.c_int, C.POINTER(dla_cache),
                                        C.POINTER(dla_schedule_out), vp]
    lib.dla_decode_step.restype = C.c_int
    lib.dla_decode_step.argtypes = [vp, vp, vp, vp, vp, f32, C.c_int, C.POINTER(dla_cache),
                                    C.POINTER(dla_schedule_out), vp]
    lib.dla_set_prefill_path.restype = C.c_int
    lib.dla_set_prefill_path.argtypes = [i32, i32]
    lib.dla_set_prefill_events.restype = C.c_int
    lib.dla_set_prefill_events.argtypes = [vp, vp]
    lib.dla_prefill_kernel.restype = C.c_char_p
    lib.dla_prefill_kernel.argtypes = [C.c_int] + [i32] * 5
    lib.dla_status_str.restype = C.c_char_p
    lib.dla_status_str.argtypes = [C.c_int]
    lib.dla_last_error.restype = C.c_char_p
    lib.dla_last_error.argtypes = []
    _lib = lib
    return lib


# ---------------------------------------------------------------- C entry points

def dla_abi_version() -> int:
    return load().dla_abi_version()


def dla_cache_bytes(B, H, C_, d_k, d_v, state_dtype=DLA_F32) -> int:
    return load().dla_cache_bytes(B, H, C_, d_k, d_v, state_dtype)


def dla_cache_layout(B, H, C_, d_k, d_v, state_dtype=DLA_F32) -> dla_cache_layout_t:
    out = dla_cache_layout_t()
    _check(load().dla_cache_layout(B, H, C_, d_k, d_v, state_dtype, C.byref(out)))
    return out


def dla_cache_init(cache: dla_cache, base: int, nbytes: int, B, H, C_, d_k, d_v, state_dtype,
                   preload: dla_cache_preload | None, stream: int) -> int:
    return load().dla_cache_init(C.byref(cache), base, nbytes, B, H, C_, d_k, d_v, state_dtype,
                                 C.byref(preload) if preload is not None else None, stream)


def dla_cache_set_merge_rule(cache: dla_cache, rule: int) -> int:
    return _check(load().dla_cache_set_merge_rule(C.byref(cache), rule))


def dla_cache_set_score_rule(cache: dla_cache, rule: int) -> int:
    return _check(load().dla_cache_set_score_rule(C.byref(cache), rule))


def dla_prefill_workspace_bytes(B, H, T, C_, d_k, d_v) -> int:
    return load().dla_prefill_workspace_bytes(B, H, T, C_, d_k, d_v)


def dla_prefill(q, k, v, lam, o, T, tau, io, cache: dla_cache, workspace, workspace_bytes,
                sched: dla_schedule_out | None, stream) -> int:
    return load().dla_prefill(q, k, v, lam, o, T, tau, io, C.byref(cache), workspace,
                              workspace_bytes, C.byref(sched) if sched is not None else None,
                              stream)


def dla_prefill_noalloc(q, k, v, lam, o, T, tau, io, cache: dla_cache,
                        sched: dla_schedule_out | None, stream) -> int:
    return load().dla_prefill_noalloc(q, k, v, lam, o, T, tau, io, C.byref(cache),
                                      C.byref(sched) if sched is not None else None, stream)


def dla_decode_step(q, k, v, lam, o, tau, io, cache: dla_cache,
                    sched: dla_schedule_out | None, stream) -> int:
    return load().dla_decode_step(q, k, v, lam, o, tau, io, C.byref(cache),
                                  C.byref(sched) if sched is not None else None, stream)


def dla_set_prefill_path(path: int, value_columns: int = 0) -> int:
    return load().dla_set_prefill_path(path, value_columns)


def dla_set_prefill_events(before, after) -> int:
    return load().dla_set_prefill_events(before, after)


def dla_prefill_kernel(io, B, H, C_, d_k, d_v) -> str | None:
    r = load().dla_prefill_kernel(io, B, H, C_, d_k, d_v)
    return r.decode() if r is not None else None


def dla_status_str(s: int) -> str:
    return load().dla_status_str(s).decode()


def dla_last_error() -> str:
    return load().dla_last_error().decode()


def _check(status: int):
    if status != DLA_OK:
        raise DLAError(status, dla_last_error())


# ------------------------------------------------------- torch convenience layer

def _torch():
    import torch
    return torch


def _io_of(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return DLA_BF16
    if t.dtype == torch.float32:
        return DLA_F32
    raise TypeError(f"io tensors must be bfloat16 or float32, got {t.dtype}")


def _dev(t, name, shape=None, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    return t.data_ptr()


def _stream(device):
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


class Cache:
    """A device cache for B*H streams (torch uint8 buffer + dla_cache view).

    ``merge_rule``: "sum" (smallest summed information, the default) or
    "density" (lowest information density) for the capacity merges, or
    "fenwick" for the Log-Linear fixed schedule (lam weights levels, C at
    least the level count bit_length(t - 1) + 1 of the positions reached).
    ``state_dtype``: "f32" (every state float32) or "bf16" (closed states
    bfloat16, the most recent one float32).
    ``score_rule``: "cosine" (cosine of consecutive keys, the default) or
    "state" (the state information score against the current state)."""

    def __init__(self, B, H, C_, d_k, d_v, device="cuda", preload: dict | None = None,
                 merge_rule: str = "sum", state_dtype: str = "f32", score_rule: str = "cosine"):
        torch = _torch()
        if state_dtype not in ("f32", "bf16"):
            raise DLAError(DLA_ERR_ARG, f"unknown state dtype {state_dtype!r}")
        sdt = DLA_BF16 if state_dtype == "bf16" else DLA_F32
        nbytes = dla_cache_bytes(B, H, C_, d_k, d_v, sdt)
        if nbytes == 0:
            raise DLAError(DLA_ERR_ARG, f"invalid cache shape {(B, H, C_, d_k, d_v)}")
        self.buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.shape = (B, H, C_, d_k, d_v)
        self.state_dtype = state_dtype
        self.view = dla_cache()
        self.layout = dla_cache_layout(B, H, C_, d_k, d_v, sdt)
        pre = None
        self._keep = []
        if preload is not None:
            m0 = int(preload["m0"])
            st = preload["states"].to(device=device, dtype=torch.float32).contiguous()
            inf = preload["info"].to(device=device, dtype=torch.int64).contiguous()
            cnt = preload["count"].to(device=device, dtype=torch.int32).contiguous()
            sta = preload["start"].to(device=device, dtype=torch.int64).contiguous()
            self._keep = [st, inf, cnt, sta]
            pre = dla_cache_preload(m0, 0, st.data_ptr(), inf.data_ptr(), cnt.data_ptr(),
                                    sta.data_ptr(), int(preload.get("t_seen", 0)))
        _check(dla_cache_init(self.view, self.buf.data_ptr(), nbytes, B, H, C_, d_k, d_v, sdt, pre,
                              _stream(self.buf.device)))
        if merge_rule not in MERGE_RULES:
            raise DLAError(DLA_ERR_ARG, f"unknown merge rule {merge_rule!r}")
        dla_cache_set_merge_rule(self.view, MERGE_RULES[merge_rule])
        if score_rule not in SCORE_RULES:
            raise DLAError(DLA_ERR_ARG, f"unknown score rule {score_rule!r}")
        dla_cache_set_score_rule(self.view, SCORE_RULES[score_rule])

    def reset(self):
        """Make every stream empty again (same buffer, shape, merge rule and
        state dtype), so that the next prefill starts afresh."""
        B, H, C_, d_k, d_v = self.shape
        rule, score = self.view.merge_rule, self.view.score_rule
        sdt = DLA_BF16 if self.state_dtype == "bf16" else DLA_F32
        _check(dla_cache_init(self.view, self.buf.data_ptr(), self.buf.numel(), B, H, C_, d_k, d_v, sdt, None,
                              _stream(self.buf.device)))
        dla_cache_set_merge_rule(self.view, rule)
        dla_cache_set_score_rule(self.view, score)

    @property
    def device(self):
        return self.buf.device

    def read(self, streams=None) -> dict:
        """Copy the cache to the host: states in chronological order, metadata.

        ``streams``: flat stream indices (b * H + h) to copy, in that order
        (default every stream); only their bytes leave the device."""
        torch = _torch()
        torch.cuda.synchronize(self.buf.device)
        B, H, C_, dk, dv = self.shape
        BH = B * H
        sel = list(range(BH)) if streams is None else [int(x) for x in streams]
        n = len(sel)
        L = self.layout
        bf = self.state_dtype == "bf16"
        ti = torch.tensor(sel, dtype=torch.int64, device=self.buf.device)
        esz = 2 if bf else 4
        slots = self.buf[L.states_offset:L.states_offset + esz * BH * C_ * dv * dk].view(BH, -1)
        slots = slots.index_select(0, ti).cpu().numpy()
        if bf:
            # closed states: bf16 bits widened to float32; the active ones: float32 region
            u16 = slots.view(np.uint16).reshape(n, C_, dv, dk)
            states = (u16.astype(np.uint32) << 16).view(np.float32)
            act = self.buf[L.active_offset:L.active_offset + 4 * BH * dv * dk].view(BH, -1)
            active = act.index_select(0, ti).cpu().numpy().view(np.float32).reshape(n, dv, dk)
        else:
            states = slots.view(np.float32).reshape(n, C_, dv, dk)
        meta = self.buf[L.meta_offset:L.meta_offset + BH * L.meta_stride].view(BH, L.meta_stride)
        meta = meta.index_select(0, ti).cpu().numpy()

        def field(off, dt, k):
            w = np.dtype(dt).itemsize
            return np.ascontiguousarray(meta[:, off:off + w * k]).view(dt).reshape(n, k)

        m = field(L.off_m, np.int32, 1)[:, 0]
        order = field(L.off_order, np.uint8, 64)[:, :C_].astype(np.int64)
        out = dict(m=m.copy(), has_prev=field(L.off_has_prev, np.int32, 1)[:, 0].copy(),
                   s_prev=field(L.off_s_prev, np.float32, 1)[:, 0].copy(),
                   t_seen=field(L.off_t_seen, np.int64, 1)[:, 0].copy(),
                   order=order, info=field(L.off_info, np.int64, 64)[:, :C_].copy(),
                   count=field(L.off_count, np.int32, 64)[:, :C_].copy(),
                   start=field(L.off_start, np.int64, 64)[:, :C_].copy(),
                   k_prev=field(L.off_k_prev, np.float32, dk).copy())
        S = np.zeros((n, C_, dv, dk), np.float32)
        for j in range(n):
            mm = int(m[j])
            for i in range(mm):
                S[j, i] = active[j] if (bf and i == mm - 1) else states[j, order[j, i]]
        out["S"] = S
        return out


def prefill_workspace(B, H, T, C_, d_k, d_v, device="cuda"):
    torch = _torch()
    n = dla_prefill_workspace_bytes(B, H, T, C_, d_k, d_v)
    if n == 0:
        raise DLAError(DLA_ERR_ARG, "invalid prefill shape")
    return torch.empty(n, dtype=torch.uint8, device=device)


def _sched_struct(sched: dict | None):
    if not sched:
        return None
    return dla_schedule_out(*[sched[k].data_ptr() if sched.get(k) is not None else None
                              for k in ("s", "boundary", "seg_id", "m_t", "ev_t", "ev_i", "n_ev")])


def prefill(q, k, v, lam, tau: float, cache: Cache, o=None, workspace=None, sched: dict | None = None):
    """dla_prefill on torch tensors q,k [B,H,T,d_k], v [B,H,T,d_v], lam [B,H,T,C]."""
    torch = _torch()
    B, H, C_, dk, dv = cache.shape
    T = q.shape[2]
    io = _io_of(q)
    dt = q.dtype
    args = [_dev(q, "q", (B, H, T, dk), dt), _dev(k, "k", (B, H, T, dk), dt),
            _dev(v, "v", (B, H, T, dv), dt), _dev(lam, "lam", (B, H, T, C_), dt)]
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=dt, device=q.device)
    args.append(_dev(o, "o", (B, H, T, dv), dt))
    if workspace is None:
        workspace = prefill_workspace(B, H, T, C_, dk, dv, q.device)
    _check(dla_prefill(*args, T, float(tau), io, cache.view, workspace.data_ptr(),
                       workspace.numel(), _sched_struct(sched), _stream(q.device)))
    return o


def prefill_noalloc(q, k, v, lam, tau: float, cache: Cache, o=None, sched: dict | None = None):
    """dla_prefill_noalloc on torch tensors (as ``prefill``; the library's
    static scratch replaces the workspace, so nothing is allocated but ``o``
    when it is not given)."""
    torch = _torch()
    B, H, C_, dk, dv = cache.shape
    T = q.shape[2]
    io = _io_of(q)
    dt = q.dtype
    args = [_dev(q, "q", (B, H, T, dk), dt), _dev(k, "k", (B, H, T, dk), dt),
            _dev(v, "v", (B, H, T, dv), dt), _dev(lam, "lam", (B, H, T, C_), dt)]
    if o is None:
        o = torch.empty((B, H, T, dv), dtype=dt, device=q.device)
    args.append(_dev(o, "o", (B, H, T, dv), dt))
    _check(dla_prefill_noalloc(*args, T, float(tau), io, cache.view, _sched_struct(sched),
                               _stream(q.device)))
    return o


def decode_step(q, k, v, lam, tau: float, cache: Cache, o=None, sched: dict | None = None):
    """dla_decode_step on torch tensors q,k [B,H,d_k], v [B,H,d_v], lam [B,H,C]."""
    torch = _torch()
    B, H, C_, dk, dv = cache.shape
    io = _io_of(q)
    dt = q.dtype
    args = [_dev(q, "q", (B, H, dk), dt), _dev(k, "k", (B, H, dk), dt),
            _dev(v, "v", (B, H, dv), dt), _dev(lam, "lam", (B, H, C_), dt)]
    if o is None:
        o = torch.empty((B, H, dv), dtype=dt, device=q.device)
    args.append(_dev(o, "o", (B, H, dv), dt))
    _check(dla_decode_step(*args, float(tau), io, cache.view, _sched_struct(sched),
                           _stream(q.device)))
    return o
