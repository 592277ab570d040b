"""Device-side generation of the seeded inputs (GPU twin of ``hkv_inputs.gen``).

Loads ``libhkv_gen.so``; the bits equal those of the numpy definition (checked by
a GPU test on sampled streams).
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_int, c_int64, c_uint32, c_void_p

import numpy as np
import torch

from . import gen
from .configs import HkvConfig

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libhkv_gen.so")
_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run __graft_entry__.build()")
        lib = ctypes.CDLL(LIB_PATH)
        lib.hkvgen_normal.restype = c_int
        lib.hkvgen_normal.argtypes = [c_void_p, c_int, c_uint32, c_uint32, c_uint32, c_int64,
                                      c_int64, c_void_p]
        lib.hkvgen_query.restype = c_int
        lib.hkvgen_query.argtypes = [c_void_p, c_void_p, c_void_p, c_void_p, c_int, c_int,
                                     c_uint32, c_uint32, c_int64, c_int, c_int, c_int, c_int,
                                     c_void_p]
        _lib = lib
    return _lib


def torch_dtype(cfg: HkvConfig):
    return torch.bfloat16 if cfg.dtype == "bf16" else torch.float32


def device_inputs(cfg: HkvConfig, seed: int, device="cuda"):
    """K [S,N,d], V [S,N,d], Q [S,q_rows,d] on the device (stored dtype)."""
    lib = _load()
    S, N, d = cfg.S, cfg.N, cfg.head_dim
    dt = torch_dtype(cfg)
    bf = 1 if cfg.dtype == "bf16" else 0
    stream = torch.cuda.current_stream().cuda_stream
    K = torch.empty((S, N, d), dtype=dt, device=device)
    V = torch.empty((S, N, d), dtype=dt, device=device)
    Q = torch.empty((S, cfg.q_rows, d), dtype=dt, device=device)
    for tag, X in ((gen.TAG_K, K), (gen.TAG_V, V)):
        if lib.hkvgen_normal(X.data_ptr(), bf, seed, cfg.cid, tag, S, N * d, stream):
            raise RuntimeError("hkvgen_normal launch failed")
    local = gen.local_flags(cfg, seed)
    if local.all():
        anchors = np.zeros((S, 4), dtype=np.int32)
    else:
        anchors = gen.anchors_all(cfg, seed)
    local_t = torch.from_numpy(local).to(device)
    anch_t = torch.from_numpy(np.ascontiguousarray(anchors)).to(device)
    if lib.hkvgen_query(Q.data_ptr(), K.data_ptr(), local_t.data_ptr(), anch_t.data_ptr(),
                        1 if cfg.anchor_mode == "full_history" else 0, bf, seed, cfg.cid, S, N,
                        cfg.P, cfg.w_obs, d, stream):
        raise RuntimeError("hkvgen_query launch failed")
    torch.cuda.synchronize()
    return K, V, Q


def bits_of(t: torch.Tensor) -> np.ndarray:
    """Host copy of a bf16/fp32 tensor as its raw bit pattern (uint16/uint32)."""
    if t.dtype == torch.bfloat16:
        return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)
    return t.detach().cpu().view(torch.int32).numpy().view(np.uint32)


def upload_bits(bits: np.ndarray, like: torch.Tensor) -> torch.Tensor:
    """Device tensor of `like`'s dtype holding the given element bits."""
    if like.dtype == torch.bfloat16:
        host = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    else:
        host = torch.from_numpy(np.ascontiguousarray(bits).view(np.float32))
    return host.to(like.device)
