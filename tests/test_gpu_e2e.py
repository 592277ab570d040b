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


def _replay(w, layer, seq, seed=0):
    """The driver's own activations for one (layer, sequence) group, replayed on
    the oracle: the synthetic prefill, then at every step the k, v and query
    rows the model handed to hkv_decode_step.  Every output, label, eviction
    and final layout is compared (tolerances and flag bands of the harness)."""
    import numpy as np
    from hkv_inputs import gen
    from hkv_inputs.gpu import bits_of
    from tests._parity import (GpuRecord, oracle_check_group, state_after_classify,
                               state_final)
    model = bench_e2e.Model(w, seed, torch.device("cuda"))
    drv = bench_e2e.Driver(w, model, device_inputs(w, seed), hk)
    streams = [w.stream(layer, seq, h) for h in range(w.heads)]
    first = {}
    rec = drv.record(layer, seq,
                     on_classified=lambda: first.update(state_after_classify(drv.cache, streams)))
    after = state_final(drv.cache, streams)
    to_hd = lambda x: gen.decode(bits_of(x.transpose(0, 1).contiguous()), w.dtype)
    kb, vb, qb = gen.group_inputs(w, seed, layer, seq)
    K, V, Q = gen.decode(kb, w.dtype), gen.decode(vb, w.dtype), gen.decode(qb, w.dtype)
    P, W = w.P, w.w_obs
    K[:, P:] = to_hd(rec["k"])
    V[:, P:] = to_hd(rec["v"])
    Q[:, W:] = to_hd(rec["q"])
    g = GpuRecord(outs=gen.decode(bits_of(rec["out"]), w.dtype), logs=rec["log"].cpu().numpy(),
                  **first, **after)
    rep = oracle_check_group(w, seed, layer, seq, g, arrays=(K, V, Q))
    print(f"  {w.name} group ({layer}, {seq}): outputs {rep.outputs_checked} events "
          f"{rep.events_checked} max err {rep.max_out_err:.3g} flags {rep.flagged_counts}/"
          f"{rep.flagged_labels}/{rep.flagged_evictions}", flush=True)
    assert not rep.failures, rep.failures[:8]
    assert np.isfinite(g.outs).all()
    return rep


def test_e2e_driver_oracle_replay_tiny():
    print("[gpu] e2e driver replay on the oracle: tiny_f32", flush=True)
    _replay(TINY, 0, 0)


def test_e2e_driver_oracle_replay_llamagen():
    from hkv_inputs.configs import WORKLOADS
    w = WORKLOADS["llamagen_xl_rho1_6"]
    print("[gpu] e2e driver replay on the oracle: llamagen_xl_rho1_6, last layer", flush=True)
    rep = _replay(w, w.layers - 1, 0)
    assert rep.events_checked > 0
