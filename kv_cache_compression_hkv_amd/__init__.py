"""HeadKV decode-time KV-cache compression on AMD MI355X (gfx950).

Thin ctypes binding of the native C ABI in ``libhkv.so`` (declared in
include/hkv.h).  The functions carry the same names as the C entry points and do
argument marshalling only: every step of the path runs in the HIP kernels.
PyTorch provides device memory and streams (and must be imported first, so the
library binds to the HIP runtime torch already loaded).

There is no fallback: if the library is missing, importing this package fails.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_float, c_int32, c_int64, c_size_t, c_void_p
from typing import Optional

import torch  # noqa: F401  (loads the HIP runtime the library binds to)

__all__ = [
    "HkvError", "hkv_config", "hkv_state", "LOCAL", "GLOBAL", "FULL",
    "DT_BF16", "DT_F32", "make_config", "config_from_workload", "HkvCache",
    "hkv_pool_slots", "hkv_workspace_bytes", "hkv_validate", "hkv_classify",
    "hkv_classify_noalloc", "hkv_prefill",
    "hkv_append", "hkv_decode_attn", "hkv_ste_evict", "hkv_decode_step",
    "hkv_decode_step_split", "hkv_check",
    "hkv_status_string", "hkv_last_error", "LIB_PATH",
]

HERE = os.path.dirname(os.path.abspath(__file__))
# HKV_LIBRARY may name another build of the same library (e.g. a tuning variant).
LIB_PATH = os.environ.get("HKV_LIBRARY") or os.path.join(HERE, "libhkv.so")

OK, E_INVAL, E_STATE, E_CAPACITY, E_HIP, E_UNSUPPORTED = 0, -1, -2, -3, -4, -5
DT_BF16, DT_F32 = 0, 1
LOCAL, GLOBAL, FULL = 0, 1, 2


class hkv_config(ctypes.Structure):
    _fields_ = [("layers", c_int32), ("batch", c_int32), ("heads", c_int32),
                ("head_dim", c_int32), ("dtype", c_int32), ("final_len", c_int32),
                ("prefill_len", c_int32), ("local_window", c_int32), ("tau", c_float),
                ("rho_num", c_int32), ("rho_den", c_int32), ("split_dist", c_int32),
                ("w_obs", c_int32), ("evict_m", c_int32), ("full_cache", c_int32),
                ("variant", c_int32)]


class hkv_state(ctypes.Structure):
    _fields_ = [("k_pool", c_void_p), ("v_pool", c_void_p), ("pos", c_void_p),
                ("score", c_void_p), ("base", c_void_p), ("cap", c_void_p),
                ("count", c_void_p), ("budget", c_void_p), ("n_tokens", c_void_p),
                ("label", c_void_p), ("free_slots", c_void_p), ("n_free", c_void_p),
                ("qstat", c_void_p),
                ("err", c_void_p), ("workspace", c_void_p), ("workspace_bytes", c_size_t),
                ("phase", c_int32)]


class HkvError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {hkv_status_string(status)} ({status}): {hkv_last_error()}")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.POINTER
    cfgp, stp = P(hkv_config), P(hkv_state)
    sig = {
        "hkv_pool_slots": (c_size_t, [cfgp]),
        "hkv_workspace_bytes": (c_size_t, [cfgp]),
        "hkv_validate": (c_int32, [cfgp]),
        "hkv_classify": (c_int32, [cfgp, stp, c_void_p, c_void_p, c_int64, c_void_p, c_int64,
                                   c_void_p]),
        "hkv_classify_noalloc": (c_int32, [cfgp, stp, c_void_p, c_void_p, c_int64, c_void_p,
                                           c_int64, c_void_p]),
        "hkv_prefill": (c_int32, [cfgp, stp, c_void_p, c_int64, c_void_p, c_void_p, c_int64,
                                  c_void_p, c_int64, c_void_p]),
        "hkv_append": (c_int32, [cfgp, stp, c_int32, c_void_p, c_void_p, c_int64, c_int32,
                                 c_int32, c_void_p]),
        "hkv_decode_attn": (c_int32, [cfgp, stp, c_int32, c_void_p, c_int64, c_void_p, c_int64,
                                      c_int32, c_int32, c_void_p]),
        "hkv_ste_evict": (c_int32, [cfgp, stp, c_int32, c_void_p, c_int64, c_void_p, c_int32,
                                    c_int32, c_void_p]),
        "hkv_decode_step": (c_int32, [cfgp, stp, c_int32, c_void_p, c_void_p, c_int64, c_void_p,
                                      c_int64, c_void_p, c_int64, c_void_p, c_int32, c_int32,
                                      c_void_p]),
        "hkv_decode_step_split": (c_int32, [cfgp, stp, c_int32, c_void_p, c_void_p, c_int64,
                                            c_void_p, c_int64, c_void_p, c_int64, c_void_p,
                                            c_int32, c_int32, c_int32, c_void_p]),
        "hkv_check": (c_int32, [cfgp, stp, c_void_p]),
        "hkv_status_string": (ctypes.c_char_p, [c_int32]),
        "hkv_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


_lib = _load()


def _ptr(x) -> Optional[int]:
    """Device pointer of a tensor (or an int / None passed through)."""
    if x is None:
        return None
    if isinstance(x, torch.Tensor):
        return x.data_ptr()
    return int(x)


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream if torch.cuda.is_available() else None
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _call(name: str, *args) -> int:
    st = getattr(_lib, name)(*args)
    if st != OK:
        raise HkvError(st, name)
    return st


def hkv_status_string(status: int) -> str:
    return _lib.hkv_status_string(status).decode()


def hkv_last_error() -> str:
    return _lib.hkv_last_error().decode()


VARIANT_UNSTRATIFIED = 1
VARIANT_UNIFORM_BUDGET = 2


def make_config(*, layers, batch, heads, head_dim, dtype, final_len, prefill_len,
                local_window, tau, rho, split_dist, w_obs=8, evict_m=8,
                full_cache=False, variant=0) -> hkv_config:
    """Build the C config.  dtype: "bf16" or "f32"; rho: (num, den); variant:
    0 or VARIANT_* bits."""
    return hkv_config(layers, batch, heads, head_dim,
                      DT_BF16 if dtype == "bf16" else DT_F32, final_len, prefill_len,
                      local_window, float(tau), int(rho[0]), int(rho[1]), split_dist, w_obs,
                      evict_m, int(bool(full_cache)), int(variant))


def config_from_workload(w) -> hkv_config:
    """C config from a workload description with the attributes layers, batch,
    heads, head_dim, dtype, N, P, local_window, tau, rho, split_dist, w_obs,
    evict_m, full_cache, unstratified and uniform_budget."""
    variant = ((VARIANT_UNSTRATIFIED if getattr(w, "unstratified", False) else 0) |
               (VARIANT_UNIFORM_BUDGET if getattr(w, "uniform_budget", False) else 0))
    return make_config(layers=w.layers, batch=w.batch, heads=w.heads, head_dim=w.head_dim,
                       dtype=w.dtype, final_len=w.N, prefill_len=w.P,
                       local_window=w.local_window, tau=w.tau, rho=w.rho,
                       split_dist=w.split_dist, w_obs=w.w_obs, evict_m=w.evict_m,
                       full_cache=w.full_cache, variant=variant)


def hkv_pool_slots(cfg: hkv_config) -> int:
    return int(_lib.hkv_pool_slots(ctypes.byref(cfg)))


def hkv_workspace_bytes(cfg: hkv_config) -> int:
    return int(_lib.hkv_workspace_bytes(ctypes.byref(cfg)))


def hkv_validate(cfg: hkv_config) -> int:
    """Status code of the configuration (does not raise)."""
    return int(_lib.hkv_validate(ctypes.byref(cfg)))


def hkv_classify(cfg, state, k_stage, v_stage, ld_stage, q_obs, ld_qobs, stream=None):
    return _call("hkv_classify", ctypes.byref(cfg), ctypes.byref(state), _ptr(k_stage),
                 _ptr(v_stage), ld_stage, _ptr(q_obs), ld_qobs, _stream(stream))


def hkv_classify_noalloc(cfg, state, k_stage, v_stage, ld_stage, q_obs, ld_qobs, stream=None):
    return _call("hkv_classify_noalloc", ctypes.byref(cfg), ctypes.byref(state), _ptr(k_stage),
                 _ptr(v_stage), ld_stage, _ptr(q_obs), ld_qobs, _stream(stream))


def hkv_prefill(cfg, state, q_stage, ld_q, k_stage, v_stage, ld_stage, out, ld_out,
                stream=None):
    return _call("hkv_prefill", ctypes.byref(cfg), ctypes.byref(state), _ptr(q_stage), ld_q,
                 _ptr(k_stage), _ptr(v_stage), ld_stage, _ptr(out), ld_out, _stream(stream))


def hkv_append(cfg, state, t, k_new, v_new, ld_kv, s_begin, s_count, stream=None):
    return _call("hkv_append", ctypes.byref(cfg), ctypes.byref(state), t, _ptr(k_new),
                 _ptr(v_new), ld_kv, s_begin, s_count, _stream(stream))


def hkv_decode_attn(cfg, state, t, q, ld_q, out, ld_o, s_begin, s_count, stream=None):
    return _call("hkv_decode_attn", ctypes.byref(cfg), ctypes.byref(state), t, _ptr(q), ld_q,
                 _ptr(out), ld_o, s_begin, s_count, _stream(stream))


def hkv_ste_evict(cfg, state, t, q_win, ld_qw, evicted_pos_log, s_begin, s_count,
                  stream=None):
    return _call("hkv_ste_evict", ctypes.byref(cfg), ctypes.byref(state), t, _ptr(q_win),
                 ld_qw, _ptr(evicted_pos_log), s_begin, s_count, _stream(stream))


def hkv_decode_step(cfg, state, t, k_new, v_new, ld_kv, q_win, ld_qw, out, ld_o,
                    evicted_pos_log, s_begin, s_count, stream=None):
    return _call("hkv_decode_step", ctypes.byref(cfg), ctypes.byref(state), t, _ptr(k_new),
                 _ptr(v_new), ld_kv, _ptr(q_win), ld_qw, _ptr(out), ld_o,
                 _ptr(evicted_pos_log), s_begin, s_count, _stream(stream))


def hkv_decode_step_split(cfg, state, t, k_new, v_new, ld_kv, q_win, ld_qw, out, ld_o,
                          evicted_pos_log, s_begin, s_count, n_split, stream=None):
    return _call("hkv_decode_step_split", ctypes.byref(cfg), ctypes.byref(state), t,
                 _ptr(k_new), _ptr(v_new), ld_kv, _ptr(q_win), ld_qw, _ptr(out), ld_o,
                 _ptr(evicted_pos_log), s_begin, s_count, n_split, _stream(stream))


def hkv_check(cfg, state, stream=None):
    return _call("hkv_check", ctypes.byref(cfg), ctypes.byref(state), _stream(stream))


class HkvCache:
    """Device buffers of one cache state, allocated with torch (plumbing only)."""

    def __init__(self, cfg: hkv_config, device="cuda"):
        slots = hkv_pool_slots(cfg)
        if slots == 0:
            raise HkvError(hkv_validate(cfg), "hkv_pool_slots")
        S = cfg.layers * cfg.batch * cfg.heads
        dt = torch.bfloat16 if cfg.dtype == DT_BF16 else torch.float32
        dev = torch.device(device)
        self.cfg = cfg
        self.S = S
        self.slots = slots
        # one pool buffer: each slot's K row, then its V row (k_pool and v_pool
        # are views of it, as the C ABI requires)
        self.kv_pool = torch.zeros((slots, 2, cfg.head_dim), dtype=dt, device=dev)
        self.k_pool = self.kv_pool[:, 0]
        self.v_pool = self.kv_pool[:, 1]
        self.pos = torch.full((slots,), -1, dtype=torch.int32, device=dev)
        self.score = torch.zeros((slots,), dtype=torch.float32, device=dev)
        self.base = torch.zeros((S,), dtype=torch.int64, device=dev)
        self.cap = torch.zeros((S,), dtype=torch.int32, device=dev)
        self.count = torch.zeros((S,), dtype=torch.int32, device=dev)
        self.budget = torch.zeros((S,), dtype=torch.int32, device=dev)
        self.n_tokens = torch.zeros((S,), dtype=torch.int32, device=dev)
        self.label = torch.zeros((S,), dtype=torch.uint8, device=dev)
        self.free_slots = torch.zeros((S, max(1, cfg.evict_m)), dtype=torch.int32, device=dev)
        self.n_free = torch.zeros((S,), dtype=torch.int32, device=dev)
        self.qstat = torch.zeros((S, max(1, cfg.w_obs), 4), dtype=torch.float32, device=dev)
        self.err = torch.zeros((1,), dtype=torch.int32, device=dev)
        nbytes = hkv_workspace_bytes(cfg)
        self.workspace = torch.zeros((nbytes + 256,), dtype=torch.uint8, device=dev)
        ws = self.workspace.data_ptr()
        ws_aligned = (ws + 255) & ~255
        self.state = hkv_state(
            self.k_pool.data_ptr(), self.v_pool.data_ptr(), self.pos.data_ptr(),
            self.score.data_ptr(), self.base.data_ptr(), self.cap.data_ptr(),
            self.count.data_ptr(), self.budget.data_ptr(), self.n_tokens.data_ptr(),
            self.label.data_ptr(), self.free_slots.data_ptr(), self.n_free.data_ptr(),
            self.qstat.data_ptr(),
            self.err.data_ptr(), ws_aligned, nbytes, 0)
