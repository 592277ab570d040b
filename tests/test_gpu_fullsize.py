"""Full-size GPU parity: every workload at its real shape, in the launch
configuration the benchmark times (one fused decode-step launch over all layers x
sequences x heads per step).  The GPU runs the whole generation; the oracle
replays a few sampled (layer, sequence) groups from the same seeded inputs and
checks labels, counts, budgets, layouts, every eviction and every output of
those groups."""
from __future__ import annotations

import numpy as np
import pytest
import torch

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

from hkv_inputs.configs import WORKLOADS, full_cache_of, variant_of
from tests._parity import gpu_generation, group_streams, oracle_check_group

SEED = 0


def sampled_groups(w, n_extra=1):
    """First and last group, plus a seeded random one."""
    rng = np.random.default_rng(1234 + w.cid)
    groups = [(0, 0), (w.layers - 1, w.batch - 1)]
    for _ in range(n_extra):
        groups.append((int(rng.integers(w.layers)), int(rng.integers(w.batch))))
    return sorted(set(groups))


CASES = ["tiny_f32", "llamagen_xl_rho1_6", "janus_pro_1b_rho1_4", "janus_pro_7b_rho1_6",
         "janus_pro_7b_rho1_8", "lumina_mgpt_768_rho1_8"]


# workloads whose sampled groups' scores are read back after every step and
# compared with the oracle's at every eviction event (lock-step)
LOCKSTEP = ("tiny_f32", "llamagen_xl_rho1_6")


@pytest.mark.parametrize("name", CASES)
def test_fullsize_parity(name):
    w = WORKLOADS[name]
    groups = sampled_groups(w, n_extra=0 if name.startswith("lumina") else 1)
    print(f"[gpu] full-size {name}: S={w.S} N={w.N} P={w.P} groups={groups}", flush=True)
    g = gpu_generation(w, SEED, group_streams(w, groups), score_trace=name in LOCKSTEP)
    torch.cuda.empty_cache()
    rep = None
    for (l, b) in groups:
        rep = oracle_check_group(w, SEED, l, b, g, rep=rep)
    labels = g.labels
    print(f"  labels local/global {(labels == 0).sum()}/{(labels == 1).sum()} outputs "
          f"{rep.outputs_checked} events {rep.events_checked} (lock-step "
          f"{rep.lockstep_events}) max err {rep.max_out_err:.3g} "
          f"score err {rep.max_score_err:.3g} flags {rep.flagged_counts}/{rep.flagged_labels}/"
          f"{rep.flagged_evictions}", flush=True)
    assert not rep.failures, rep.failures[:8]
    if name != "tiny_f32":
        assert rep.events_checked > 0
    if name in LOCKSTEP:
        assert rep.lockstep_events == rep.events_checked
    # the inputs are deterministic and no decision of these workloads falls
    # inside a flag band; any flag at all means the arithmetic moved
    assert rep.flagged_counts == rep.flagged_labels == rep.flagged_evictions == 0


@pytest.mark.parametrize("name", ["llamagen_xl_rho1_6", "janus_pro_7b_rho1_6",
                                  "lumina_mgpt_768_rho1_8"])
def test_fullsize_log_free_launch_equals_logged(name):
    """The benchmark's launch passes no eviction log; the parity runs pass one
    (which also makes each eviction write its scores).  Both give the same
    outputs at every step and the same cache state, bit for bit."""
    import kv_cache_compression_hkv_amd as hk
    from hkv_inputs.gpu import device_inputs
    w = WORKLOADS[name]
    print(f"[gpu] log-free vs logged launch {name}: S={w.S} steps={w.steps}", flush=True)
    K, V, Q = device_inputs(w, SEED)
    cfg = hk.config_from_workload(w)
    d, eb, W, N, P = w.head_dim, w.elem_bytes, w.w_obs, w.N, w.P
    groups = sampled_groups(w, n_extra=1)
    idx = torch.tensor(group_streams(w, groups), dtype=torch.long, device=K.device)

    def run(with_log):
        cache = hk.HkvCache(cfg)
        st = cache.state
        hk.hkv_classify(cfg, st, K, V, N * d, Q, w.q_rows * d)
        out = torch.zeros((w.S, d), dtype=K.dtype, device=K.device)
        log = torch.full((w.S, w.evict_m), -1, dtype=torch.int32, device=K.device) \
            if with_log else None
        outs = torch.empty((w.steps, w.S if w.S <= 12288 else idx.numel(), d), dtype=K.dtype,
                           device=K.device)
        for t in range(P, N):
            hk.hkv_decode_step(cfg, st, t, K.data_ptr() + t * d * eb, V.data_ptr() + t * d * eb,
                               N * d, Q.data_ptr() + (t - W + 1 - (P - W)) * d * eb,
                               w.q_rows * d, out, d, log, 0, w.S)
            outs[t - P] = out if outs.shape[1] == w.S else out[idx]
        hk.hkv_check(cfg, st)
        state = [x.clone() for x in (cache.pos, cache.count, cache.n_free, cache.free_slots,
                                     cache.label, cache.budget, cache.cap, cache.base)]
        del cache
        return outs, state

    a_out, a_st = run(False)
    b_out, b_st = run(True)
    torch.cuda.synchronize()
    assert torch.equal(a_out.view(torch.int16), b_out.view(torch.int16))
    for x, y in zip(a_st, b_st):
        assert torch.equal(x, y)


@pytest.mark.parametrize("name", ["llamagen_xl_rho1_6", "janus_pro_7b_rho1_6"])
def test_fullsize_full_cache(name):
    """The uncompressed baseline layout at full size (sampled group, first 96 steps)."""
    w = full_cache_of(WORKLOADS[name])
    groups = [(w.layers - 1, 0)]
    print(f"[gpu] full-size full cache {w.name}", flush=True)
    g = gpu_generation(w, SEED, group_streams(w, groups), steps=96)
    torch.cuda.empty_cache()
    rep = oracle_check_group(w, SEED, *groups[0], g, steps=96)
    print(f"  outputs {rep.outputs_checked} max err {rep.max_out_err:.3g}", flush=True)
    assert not rep.failures, rep.failures[:8]


@pytest.mark.parametrize("unstrat,uniform", [(True, False), (False, True)])
def test_fullsize_variants(unstrat, uniform):
    """The ablation variants at the LlamaGen-XL shape (sampled groups, all steps)."""
    w = variant_of(WORKLOADS["llamagen_xl_rho1_6"], unstratified=unstrat, uniform_budget=uniform)
    groups = sampled_groups(w, n_extra=0)
    print(f"[gpu] full-size variant {w.name} groups={groups}", flush=True)
    g = gpu_generation(w, SEED, group_streams(w, groups))
    torch.cuda.empty_cache()
    rep = None
    for (l, b) in groups:
        rep = oracle_check_group(w, SEED, l, b, g, rep=rep)
    print(f"  events {rep.events_checked} max err {rep.max_out_err:.3g} "
          f"flags {rep.flagged_counts}/{rep.flagged_labels}/{rep.flagged_evictions}", flush=True)
    assert not rep.failures, rep.failures[:8]
    assert rep.events_checked > 0


@pytest.mark.parametrize("name", ["llamagen_xl_rho1_6", "janus_pro_1b_rho1_4"])
def test_fullsize_per_layer_equals_folded(name):
    """One launch per layer per step (a model's loop) against one launch over
    all layers per step, at full size: each stream's work does not depend on
    which launch carries it, so every output of every step and the final
    state agree bit for bit."""
    import bench
    import kv_cache_compression_hkv_amd as hk
    from hkv_inputs.gpu import device_inputs
    w = WORKLOADS[name]
    print(f"[gpu] per-layer vs folded {name}: S={w.S} steps={w.steps}", flush=True)
    inputs = device_inputs(w, SEED)
    d, per, W = w.head_dim, w.batch * w.heads, w.w_obs
    cur = torch.cuda.current_stream()

    def state(g):
        c = g.cache
        return [t.clone() for t in (c.pos, c.count, c.n_free, c.free_slots, c.label, c.budget)]

    folded = bench.Generation(w, inputs, hk)
    cap_f = torch.empty((w.steps, w.S, d), dtype=folded.out.dtype, device=folded.out.device)
    folded.run(cur, capture=cap_f)
    torch.cuda.synchronize()
    hk.hkv_check(folded.cfg, folded.cache.state)
    st_f = state(folded)
    del folded

    layered = bench.Generation(w, inputs, hk)
    st = layered.cache.state
    hk.hkv_classify(layered.cfg, st, layered.K, layered.V, w.N * d, layered.Q, w.q_rows * d, cur)
    cap_l = torch.empty_like(cap_f)
    for t in range(w.P, w.N):
        for l in range(w.layers):
            hk.hkv_decode_step(layered.cfg, st, t, layered.kp[t], layered.vp[t], w.N * d,
                               layered.qw[t], w.q_rows * d, layered.out, d, None, l * per, per,
                               cur)
        cap_l[t - w.P].copy_(layered.out)
    torch.cuda.synchronize()
    hk.hkv_check(layered.cfg, st)
    st_l = state(layered)
    assert torch.equal(cap_f.view(torch.int16), cap_l.view(torch.int16))
    for a, b in zip(st_f, st_l):
        assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["llamagen_xl_rho1_6", "janus_pro_1b_rho1_4"])
def test_fullsize_split_step_parity(name):
    """hkv_decode_step_split at full size, one launch pair per layer as a model
    runs it: every eviction of the sampled groups is scored by the split
    workgroups (bf16) and finished by the combine kernel; labels, layouts,
    every eviction and every output agree with the oracle."""
    w = WORKLOADS[name]
    groups = sampled_groups(w)
    print(f"[gpu] full-size split step {name}: S={w.S} N={w.N} groups={groups} n_split=2",
          flush=True)
    g = gpu_generation(w, SEED, group_streams(w, groups), per_layer=True, n_split=2)
    torch.cuda.empty_cache()
    rep = None
    for (l, b) in groups:
        rep = oracle_check_group(w, SEED, l, b, g, rep=rep)
    print(f"  outputs {rep.outputs_checked} events {rep.events_checked} max err "
          f"{rep.max_out_err:.3g} flags {rep.flagged_counts}/{rep.flagged_labels}/"
          f"{rep.flagged_evictions}", flush=True)
    assert not rep.failures, rep.failures[:8]
    assert rep.events_checked > 0
    assert rep.flagged_counts == rep.flagged_labels == rep.flagged_evictions == 0
