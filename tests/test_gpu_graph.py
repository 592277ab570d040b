"""The per-layer decode loop captured as one HIP graph: every replay, each after
an eager classification and other eager work, equals the eager run bit for bit
(outputs of every step, evicted positions of every step, final cache state)."""
from __future__ import annotations

import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import kv_cache_compression_hkv_amd as hk
from hkv_inputs.gpu import device_inputs
from tests._fixtures import small_config


def _state(cache):
    return {k: getattr(cache, k).clone() for k in
            ("count", "pos", "score", "n_free", "free_slots", "k_pool", "v_pool", "label",
             "budget", "base")}


@pytest.mark.parametrize("kw,n_split", [
    (dict(layers=3, batch=2), 0),
    (dict(layers=2, batch=2, dtype="f32", head_dim=128, heads=4, rho=(1, 6), p_local=0.0), 0),
    # the split decode step (two kernels per layer per step)
    (dict(layers=3, batch=2), 4),
    (dict(layers=2, batch=2, head_dim=128, heads=6, image_tokens=744, prefill_image=100,
          split_dist=60), 3),
])
def test_graph_replay_matches_eager(kw, n_split):
    w = small_config(**kw)
    print(f"[gpu] graph replay {w.dtype} d={w.head_dim} S={w.S} n_split={n_split}", flush=True)
    K, V, Q = device_inputs(w, 5)
    cfg = hk.config_from_workload(w)
    cache = hk.HkvCache(cfg)
    st = cache.state
    S, N, d, P, W, M = w.S, w.N, w.head_dim, w.P, w.w_obs, w.evict_m
    eb, per = w.elem_bytes, w.batch * w.heads
    out = torch.zeros((S, d), dtype=K.dtype, device=K.device)
    log = torch.full((S, M), -1, dtype=torch.int32, device=K.device)
    outs = torch.empty((w.steps, S, d), dtype=K.dtype, device=K.device)
    logs = torch.empty((w.steps, S, M), dtype=torch.int32, device=K.device)

    def classify():
        hk.hkv_classify(cfg, st, K, V, N * d, Q, w.q_rows * d)

    def loop():
        for t in range(P, N):
            kp = K.data_ptr() + t * d * eb
            vp = V.data_ptr() + t * d * eb
            qw = Q.data_ptr() + (t - W + 1 - (P - W)) * d * eb
            for l in range(w.layers):
                if n_split:
                    hk.hkv_decode_step_split(cfg, st, t, kp, vp, N * d, qw, w.q_rows * d, out, d,
                                             log, l * per, per, n_split)
                else:
                    hk.hkv_decode_step(cfg, st, t, kp, vp, N * d, qw, w.q_rows * d, out, d, log,
                                       l * per, per)
            outs[t - P].copy_(out)
            logs[t - P].copy_(log)

    classify()
    loop()
    torch.cuda.synchronize()
    hk.hkv_check(cfg, st)
    ref_outs, ref_logs, ref_state = outs.clone(), logs.clone(), _state(cache)
    assert (ref_logs >= 0).any()                        # evictions happened

    classify()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        graph.capture_begin()
        loop()
        graph.capture_end()
    torch.cuda.synchronize()

    for rep in range(3):
        outs.zero_()                                    # eager work between replays
        logs.fill_(-7)
        classify()
        graph.replay()
        torch.cuda.synchronize()
        hk.hkv_check(cfg, st)
        assert torch.equal(outs, ref_outs), f"replay {rep}: outputs differ"
        assert torch.equal(logs, ref_logs), f"replay {rep}: evictions differ"
        now = _state(cache)
        for k, v in ref_state.items():
            if k in ("pos", "score", "k_pool", "v_pool"):
                # compare the slots in use only (unused pool slots are never written)
                base, cnt = ref_state["base"].cpu(), ref_state["count"].cpu()
                for s in range(S):
                    b, c = int(base[s]), int(cnt[s])
                    assert torch.equal(now[k][b:b + c], v[b:b + c]), f"replay {rep}: {k} s{s}"
            else:
                assert torch.equal(now[k], v), f"replay {rep}: {k} differs"
