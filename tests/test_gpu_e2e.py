"""The random-weight transformer driver (bench_e2e.py) on the tiny workload:
captured graphs replay, the cache state stays consistent, and the compressed
and full-cache runs give positive throughputs."""
from __future__ import annotations

import math

import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import bench_e2e
import kv_cache_compression_hkv_amd as hk
from hkv_inputs.configs import TINY, full_cache_of
from hkv_inputs.gpu import device_inputs


def test_e2e_driver_tiny():
    print("[gpu] e2e driver tiny_f32", flush=True)
    res = bench_e2e.run(TINY, 0, 1, hk, device_inputs, full_cache_of)
    for tag in ("compressed", "full_cache"):
        r = res[tag]
        assert r["tokens_per_s"] > 0 and math.isfinite(r["ms_per_gen"])
    assert res["rest_ms"] > 0
    assert math.isfinite(res["speedup"])


def test_e2e_query_ring_matches_history():
    """The doubled ring hands the decode step the W newest queries, oldest first."""
    w = TINY
    print("[gpu] e2e query ring", flush=True)
    model = bench_e2e.Model(w, 0, torch.device("cuda"))
    drv = bench_e2e.Driver(w, model, device_inputs(w, 0), hk)
    drv._reset()
    W, d, P = w.w_obs, w.head_dim, w.P
    hist = {P - W + 1 + i: drv.Q[:, 1 + i].clone() for i in range(W - 1)}
    for t in range(P, P + 11):
        q = torch.randn(drv.per, d, device="cuda", dtype=model.dt)
        drv.qring[0][:, t % W] = q
        drv.qring[0][:, t % W + W] = q
        hist[t] = q
        start = (t + 1) % W
        win = drv.qring[0][:, start:start + W]
        for i in range(W):
            assert torch.equal(win[:, i], hist[t - W + 1 + i])
