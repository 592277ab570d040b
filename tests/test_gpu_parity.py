"""GPU parity of the HIP path (through the C ABI) against the CPU oracle, on
small workloads the oracle replays in full: several tiles, ragged tails, both
element types, both head sizes and the method's degenerate cases."""
from __future__ import annotations

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():           # collected on CPU machines, never run there
    pytest.skip("needs a GPU", allow_module_level=True)

import kv_cache_compression_hkv_amd as hk
import oracle.hkv_oracle as O
from hkv_inputs import gen
from hkv_inputs.configs import TINY
from hkv_inputs.gpu import bits_of, device_inputs
from tests._fixtures import small_config
from tests._parity import gpu_generation, group_streams, oracle_check_group

CASES = {
    # initial STE (P > B_g), bf16, head_dim 64, 6 heads x 2 layers x 2 sequences
    "bf16_d64_init_ste": small_config(layers=2, batch=2),
    # no initial STE: Global heads grow from P to their budget first
    "bf16_d128_growing": small_config(head_dim=128, rho=(1, 2), prefill_image=30, p_local=0.0),
    "f32_d64": small_config(dtype="f32", heads=5),
    "f32_d128": small_config(dtype="f32", head_dim=128, heads=3, rho=(1, 6), split_dist=40,
                            p_local=0.0),
    # near subset with one candidate: the far subset supplies the rest
    "shortfall_near": small_config(split_dist=9),
    # far subset empty: every eviction comes from the near subset
    "far_empty": small_config(split_dist=400),
    # rho = 1: Global heads never evict and equal full attention
    "rho_one": small_config(rho=(1, 1), image_tokens=90),
    # wide window: most heads Local
    "wide_window": small_config(local_window=44, p_local=1.0),
    # uncompressed baseline layout
    "full_cache": small_config(full_cache=True, image_tokens=120),
    # a full-cache layout evicts nothing: M = 0 is valid there, and its free list is empty
    "full_cache_m0": small_config(full_cache=True, image_tokens=120, evict_m=0),
    # uncompressed layout with a prefill beyond the classification's on-chip
    # limit of 1024 positions (the full layout needs no classification)
    "full_cache_long_prefill": small_config(full_cache=True, image_tokens=1200,
                                            prefill_image=1090),
    # a prefill of 1000 positions (classification tile near its 1024 limit) and
    # an initial eviction of hundreds of tokens (radix select over 1000 keys)
    "long_prefill": small_config(heads=2, image_tokens=1100, prefill_image=984, p_local=0.0),
    "long_prefill_d128": small_config(head_dim=128, heads=2, image_tokens=1100,
                                      prefill_image=984, p_local=0.0),
    # odd sizes everywhere
    "ragged": small_config(heads=7, prefix=5, image_tokens=143, prefill_image=37,
                           local_window=13, split_dist=21, rho=(2, 7)),
    # Global streams longer than the on-chip scratch (spill to the workspace)
    "long_global": small_config(heads=2, prefix=0, image_tokens=1500, prefill_image=64,
                                rho=(3, 4), split_dist=300, p_local=0.0),
    # fp32 Global streams beyond the 512-slot on-chip tile (tile, positions and
    # keys in the workspace), both head sizes
    "f32_long_global": small_config(dtype="f32", heads=2, prefix=0, image_tokens=1500,
                                    prefill_image=64, rho=(3, 4), split_dist=300, p_local=0.0),
    "f32_d128_long_global": small_config(dtype="f32", head_dim=128, heads=2, prefix=0,
                                         image_tokens=1500, prefill_image=64, rho=(3, 4),
                                         split_dist=300, p_local=0.0),
    # bf16 d128 eviction paths.  Short-stream kernel (per-head budget <= 192):
    # Global streams of 321..1280 slots (two matrix-core passes, keys on chip;
    # 3 Global heads of 6, B_g = 368) and beyond 1280 (keys in the workspace;
    # config id 44 gives 1 Global head of 8, B_g = 1436)
    "bf16_d128_twopass": small_config(head_dim=128, heads=6, image_tokens=744,
                                      prefill_image=100, split_dist=60),
    "bf16_d128_twopass_spill": small_config(cid=44, head_dim=128, heads=8, image_tokens=1504,
                                            prefill_image=100, rho=(1, 8), split_dist=60,
                                            p_local=0.9),
    # long-stream kernel (budget 225, and 1312 beyond the 1280 on-chip keys)
    "bf16_d128_long": small_config(head_dim=128, heads=2, image_tokens=884, prefill_image=120,
                                   split_dist=80, p_local=0.0),
    "bf16_d128_long_spill": small_config(head_dim=128, heads=2, prefix=0, image_tokens=1750,
                                         prefill_image=64, rho=(3, 4), split_dist=300,
                                         p_local=0.0),
    # streams of exactly 256 and 257 slots at eviction (both heads Global,
    # B_g = 248 and 249): the largest selected by one wave over all keys and the
    # smallest selected by the per-wave rounds; d64 takes its scores from the
    # attention's tile, d128 (long-stream kernel) from keys written by its
    # second matrix-core pass
    "select_256_d64": small_config(heads=2, prefix=0, image_tokens=496, prefill_image=64,
                                   rho=(1, 2), split_dist=100, p_local=0.0),
    "select_257_d64": small_config(heads=2, prefix=0, image_tokens=498, prefill_image=64,
                                   rho=(1, 2), split_dist=100, p_local=0.0),
    "select_256_d128": small_config(head_dim=128, heads=2, prefix=0, image_tokens=496,
                                    prefill_image=64, rho=(1, 2), split_dist=100, p_local=0.0),
    "select_257_d128": small_config(head_dim=128, heads=2, prefix=0, image_tokens=498,
                                    prefill_image=64, rho=(1, 2), split_dist=100, p_local=0.0),
    # observation windows W = M other than 8 (quotas 1/1, 2/2, 3/3; fewer window
    # rows in the matrix-core passes and the staged queries)
    "window2_d64": small_config(w_obs=2, evict_m=2, heads=4),
    "window4_d64": small_config(w_obs=4, evict_m=4, layers=2, batch=2),
    "window6_d64": small_config(w_obs=6, evict_m=6),
    "window4_d128": small_config(w_obs=4, evict_m=4, head_dim=128, rho=(1, 2), prefill_image=30,
                                 p_local=0.0),
    "window6_d128_long": small_config(w_obs=6, evict_m=6, head_dim=128, heads=2, image_tokens=884,
                                      prefill_image=120, split_dist=80, p_local=0.0),
    "window4_f32_d128": small_config(w_obs=4, evict_m=4, dtype="f32", head_dim=128, heads=3,
                                     rho=(1, 6), split_dist=40, p_local=0.0),
    # classification thresholds other than 0.9: mostly Local heads (tau = 0.5),
    # Global heads needing nearly the whole prefill (tau = 0.99)
    "tau_half": small_config(tau=0.5, rho=(1, 6), split_dist=20),
    "tau_099": small_config(tau=0.99, layers=2),
    # a single decode step after a classification with initial eviction
    "one_step": small_config(image_tokens=41, prefill_image=40),
    # W = 4 on streams beyond 256 slots (per-wave rounds) and beyond the on-chip
    # scratch (workspace)
    "window4_long_global": small_config(w_obs=4, evict_m=4, heads=2, prefix=0, image_tokens=1500,
                                        prefill_image=64, rho=(3, 4), split_dist=300,
                                        p_local=0.0),
    # local window longer than the prefill: every head is Local (its count is at
    # most P < w) and its ring starts part-filled, then grows to w
    "window_gt_prefill": small_config(local_window=64, rho=(1, 2)),
    "window_gt_prefill_f32_d128": small_config(dtype="f32", head_dim=128, heads=3,
                                               local_window=70, rho=(1, 2)),
    # uniform budget with floor(rho*N) above the prefill: Local rings of A slots
    # start part-filled; Global heads grow from P to A before their first eviction
    "uniform_ring_gt_prefill": small_config(rho=(1, 2), uniform_budget=True),
    "uniform_ring_gt_prefill_d128": small_config(head_dim=128, rho=(1, 2), tau=0.5,
                                                 uniform_budget=True),
    # ablation variants: eviction without the near/far split; one budget for all
    "unstratified": small_config(layers=2, batch=2, unstratified=True),
    "uniform_budget": small_config(rho=(1, 6), split_dist=20, uniform_budget=True),
    "uniform_unstrat_f32_d128": small_config(dtype="f32", head_dim=128, heads=4, rho=(1, 6),
                                             p_local=0.0, unstratified=True,
                                             uniform_budget=True),
}


def _all_groups(w):
    return [(l, b) for l in range(w.layers) for b in range(w.batch)]


NO_EVENTS = ("rho_one", "wide_window", "window_gt_prefill", "window_gt_prefill_f32_d128")


def _check_all_groups(w, name, **kw):
    """Every group of a small workload, every step; the GPU's scores compared
    with the oracle's at every eviction event (lock-step)."""
    groups = _all_groups(w)
    g = gpu_generation(w, 0, group_streams(w, groups), score_trace=True, **kw)
    rep = None
    for (l, b) in groups:
        rep = oracle_check_group(w, 0, l, b, g, rep=rep)
    print(f"  outputs {rep.outputs_checked} events {rep.events_checked} "
          f"(lock-step {rep.lockstep_events}) max err {rep.max_out_err:.3g} "
          f"score err {rep.max_score_err:.3g} flags {rep.flagged_counts}/"
          f"{rep.flagged_labels}/{rep.flagged_evictions}", flush=True)
    assert not rep.failures, rep.failures[:8]
    if name not in NO_EVENTS and not w.full_cache:
        assert rep.events_checked > 0
        assert rep.lockstep_events == rep.events_checked
    # deterministic inputs: no decision of these cases falls inside a flag band
    assert rep.flagged_counts == rep.flagged_labels == rep.flagged_evictions == 0
    return g, rep


@pytest.mark.parametrize("name", ["tiny"] + sorted(CASES))
def test_parity_small(name):
    w = TINY if name == "tiny" else CASES[name]
    print(f"[gpu] parity {name}: S={w.S} N={w.N} P={w.P} d={w.head_dim} {w.dtype}", flush=True)
    g, _ = _check_all_groups(w, name)
    if name.startswith("window_gt_prefill"):
        assert (g.labels == hk.LOCAL).all() and (g.count0 == w.P).all()
    if name.startswith("uniform_ring_gt_prefill"):
        A = w.N * w.rho[0] // w.rho[1]
        assert A > w.P and (g.labels == hk.LOCAL).any() and (g.labels == hk.GLOBAL).any()
        assert (g.cap[g.labels == hk.LOCAL] == A).all() and (g.count0 == w.P).all()


SPLIT_CASES = {
    "bf16_d128_short": small_config(head_dim=128, layers=2, rho=(1, 4), split_dist=20),
    "bf16_d128_long": small_config(head_dim=128, heads=3, image_tokens=884, prefill_image=120,
                                   split_dist=80, p_local=0.3),
}


@pytest.mark.parametrize("name", sorted(SPLIT_CASES))
def test_parity_split_calls(name):
    """hkv_append + hkv_decode_attn + hkv_ste_evict as three calls per step,
    replayed on the oracle (the standalone eviction stages its own queries)."""
    w = SPLIT_CASES[name]
    print(f"[gpu] parity split calls {name}: S={w.S} N={w.N} d={w.head_dim}", flush=True)
    _check_all_groups(w, name, mode="split")


def test_generator_twin_bits():
    for w in (TINY, small_config(layers=2, batch=2), small_config(head_dim=128, dtype="f32")):
        print(f"[gpu] generator twin {w.name} {w.dtype} d={w.head_dim}", flush=True)
        K, V, Q = device_inputs(w, 3)
        for (l, b) in _all_groups(w)[:3]:
            kb, vb, qb = gen.group_inputs(w, 3, l, b)
            s0 = w.stream(l, b, 0)
            sl = slice(s0, s0 + w.heads)
            assert np.array_equal(bits_of(K[sl]), kb)
            assert np.array_equal(bits_of(V[sl]), vb)
            assert np.array_equal(bits_of(Q[sl]), qb)


@pytest.mark.parametrize("name", sorted(SPLIT_CASES))
def test_parity_stale_query_statistics(name):
    """Separate calls with the attention left out on every fifth step: an
    eviction whose window holds such a step finds stale entries in the state's
    query-statistics ring and forms the window's statistics itself.  Its
    decisions, and the outputs of the steps that attended, still match the
    oracle."""
    w = SPLIT_CASES[name]
    print(f"[gpu] parity, attention skipped every fifth step {name}", flush=True)
    _check_all_groups(w, name, mode="split", skip_attn=lambda t: t % 5 == 3)


FUSED_CASES = {
    "bf16_d64": small_config(layers=2, batch=2, heads=8),
    "f32_d64": small_config(dtype="f32", layers=2, heads=5),
    "f32_d128": small_config(dtype="f32", head_dim=128, heads=4, rho=(1, 6), split_dist=40),
    # bf16 d128: short-stream kernel (budget <= 192) and long-stream kernel
    "bf16_d128_short": small_config(head_dim=128, layers=2, heads=6, split_dist=20),
    "bf16_d128_long": small_config(head_dim=128, heads=3, image_tokens=884, prefill_image=120,
                                   split_dist=80, p_local=0.3),
}


@pytest.mark.parametrize("name", sorted(FUSED_CASES))
def test_fused_equals_separate_calls(name):
    """hkv_decode_step gives bit-identical results to append + attn + evict."""
    w = FUSED_CASES[name]
    print(f"[gpu] fused vs separate {name}", flush=True)
    inputs = device_inputs(w, 1)
    streams = list(range(w.S))
    a = gpu_generation(w, 1, streams, mode="fused", inputs=inputs)
    b = gpu_generation(w, 1, streams, mode="split", inputs=inputs)
    assert np.array_equal(a.outs, b.outs)
    assert np.array_equal(a.logs, b.logs)
    assert a.tables_final == b.tables_final
    for x, y in zip(a.scores_final, b.scores_final):
        assert np.array_equal(x, y)


def test_determinism():
    w = small_config(layers=1, batch=3, heads=6, head_dim=128)
    print("[gpu] determinism", flush=True)
    inputs = device_inputs(w, 2)
    streams = list(range(w.S))
    a = gpu_generation(w, 2, streams, inputs=inputs)
    b = gpu_generation(w, 2, streams, inputs=inputs)
    assert np.array_equal(a.outs, b.outs) and np.array_equal(a.logs, b.logs)
    assert a.tables_final == b.tables_final


def _events_of(w, seed=0):
    K, V, Q = (gen.decode(x, w.dtype) for x in gen.group_inputs(w, seed, 0, 0))
    return O.run_group(w, K, V, Q), K, V


EVICT_CASES = {
    "bf16_d64": dict(),
    "f32_d128": dict(dtype="f32", head_dim=128),
    # bf16 d128 keys read from the state's scores: short-stream kernel (budget
    # <= 192) and long-stream kernel (budget 221)
    "bf16_d128_short": dict(head_dim=128),
    "bf16_d128_long": dict(head_dim=128, image_tokens=884, prefill_image=120, split_dist=80),
}


@pytest.mark.parametrize("name", sorted(EVICT_CASES))
def test_evict_given_identical_scores(name):
    """Load the oracle's pre-eviction state (layout and fp32-rounded scores) into
    a GPU state and run hkv_ste_evict alone: the evicted set and the layout after
    the eviction must equal the oracle's selection on the same fp32 scores, bit
    for bit."""
    kw = dict(heads=4, p_local=0.0, split_dist=20)
    kw.update(EVICT_CASES[name])
    w = small_config(**kw)
    dtype = w.dtype
    print(f"[gpu] evict given scores {name}", flush=True)
    rec, K, V = _events_of(w)
    events = rec.events[:12] + rec.events[-12:]
    assert events
    cfg = hk.config_from_workload(w)
    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
    for ev in events:
        cache = hk.HkvCache(cfg)
        s = ev.head
        c = len(ev.slot_pos)
        base = 0                        # only stream s is launched
        assert c <= cache.slots
        pos = np.array(ev.slot_pos, dtype=np.int32)
        sc32 = np.array(ev.slot_score, dtype=np.float32)
        cache.base[s] = base
        cache.cap[s] = c
        cache.count[s] = c
        cache.budget[s] = ev.budget
        cache.label[:] = hk.LOCAL
        cache.label[s] = hk.GLOBAL
        cache.pos[base:base + c] = torch.from_numpy(pos).cuda()
        cache.score[base:base + c] = torch.from_numpy(sc32).cuda()
        cache.k_pool[base:base + c] = torch.from_numpy(K[s][pos]).to(dt).cuda()
        cache.v_pool[base:base + c] = torch.from_numpy(V[s][pos]).to(dt).cuda()
        cache.state.phase = 1
        log = torch.full((w.S, w.evict_m), -7, dtype=torch.int32, device="cuda")
        hk.hkv_ste_evict(cfg, cache.state, ev.t, None, 0, log, s, 1)
        hk.hkv_check(cfg, cache.state)
        own = O.ste_select(ev.slot_pos, sc32.astype(np.float64), ev.t, w.w_obs, w.split_dist,
                           w.evict_m)
        want_pos, want_sc, want_free = O.free_evicted(ev.slot_pos, list(sc32), own)
        got_log = log[s].cpu().numpy()
        assert got_log.tolist() == [ev.slot_pos[j] for j in own]       # ascending slots
        assert int(cache.count[s]) == c                                  # no row moves
        assert int(cache.n_free[s]) == w.evict_m
        assert cache.free_slots[s].cpu().numpy().tolist() == want_free
        got_pos = cache.pos[base:base + c].cpu().numpy().tolist()
        assert got_pos == want_pos
        got_sc = cache.score[base:base + c].cpu().numpy()
        assert np.array_equal(got_sc, sc32)              # the scores it ranked
        kept = [j for j in range(c) if j not in set(own)]
        got_k = cache.k_pool[base:base + c].float().cpu().numpy()[kept]
        want_k = torch.from_numpy(K[s][pos[kept]]).to(dt).float().numpy()
        assert np.array_equal(got_k, want_k)


def test_capacity_error_reported():
    """A Global stream already at capacity: append sets the device error word,
    the kernel exits normally, hkv_check reports HKV_E_CAPACITY."""
    w = small_config(p_local=0.0)
    print("[gpu] capacity error", flush=True)
    K, V, Q = device_inputs(w, 0)
    cfg = hk.config_from_workload(w)
    cache = hk.HkvCache(cfg)
    hk.hkv_classify(cfg, cache.state, K, V, w.N * w.head_dim, Q, w.q_rows * w.head_dim)
    hk.hkv_check(cfg, cache.state)
    g = int(torch.nonzero(cache.label == hk.GLOBAL)[0])
    cache.count[g] = cache.cap[g]
    t = w.P
    d = w.head_dim
    hk.hkv_append(cfg, cache.state, t, K.data_ptr() + t * d * 2, V.data_ptr() + t * d * 2,
                  w.N * d, 0, w.S)
    with pytest.raises(hk.HkvError) as ei:
        hk.hkv_check(cfg, cache.state)
    assert ei.value.status == hk.E_CAPACITY


def test_empty_range_and_phase():
    w = small_config()
    cfg = hk.config_from_workload(w)
    cache = hk.HkvCache(cfg)
    buf = torch.zeros((w.S, w.head_dim), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(hk.HkvError) as ei:
        hk.hkv_append(cfg, cache.state, w.P, buf, buf, w.head_dim, 0, w.S)
    assert ei.value.status == hk.E_STATE
    cache.state.phase = 1
    assert hk.hkv_decode_attn(cfg, cache.state, w.P, buf, w.head_dim, buf, w.head_dim, 3, 0) == 0
    with pytest.raises(hk.HkvError):
        hk.hkv_decode_attn(cfg, cache.state, w.P, buf, w.head_dim, buf, w.head_dim, 3, w.S)


@pytest.mark.parametrize("kw", [dict(layers=3, batch=2),
                                # bf16 d128, budgets 104 and 190 (short-stream class)
                                dict(layers=2, batch=2, head_dim=128, heads=6, image_tokens=400,
                                     prefill_image=100, split_dist=60),
                                dict(layers=2, batch=2, head_dim=128, heads=6, image_tokens=744,
                                     prefill_image=100, split_dist=60)])
def test_per_layer_launches_parity(kw):
    """One decode-step launch per layer (its batch x heads streams, s_begin > 0),
    as a model runs the loop: oracle parity of every output and eviction."""
    w = small_config(**kw)
    print(f"[gpu] per-layer launches S={w.S} N={w.N} d={w.head_dim}", flush=True)
    groups = _all_groups(w)
    g = gpu_generation(w, 0, group_streams(w, groups), per_layer=True)
    rep = None
    for (l, b) in groups:
        rep = oracle_check_group(w, 0, l, b, g, rep=rep)
    print(f"  outputs {rep.outputs_checked} events {rep.events_checked} "
          f"max err {rep.max_out_err:.3g}", flush=True)
    assert not rep.failures, rep.failures[:8]
    assert rep.events_checked > 0


SPLIT_STEP_CASES = {
    # (config, n_split): every element type and head size, stream classes, the
    # d64 eviction on the keys route, workspace spill, ragged splits
    "bf16_d64": (small_config(layers=3, batch=2), 3),
    "bf16_d64_long_global": (small_config(heads=2, prefix=0, image_tokens=1500, prefill_image=64,
                                          rho=(3, 4), split_dist=300, p_local=0.0), 8),
    "bf16_d128_short": (small_config(head_dim=128, layers=2, rho=(1, 4), split_dist=20), 4),
    "bf16_d128_long": (small_config(head_dim=128, heads=3, image_tokens=884, prefill_image=120,
                                    split_dist=80, p_local=0.3), 5),
    "bf16_d128_twopass_spill": (small_config(cid=44, head_dim=128, heads=8, image_tokens=1504,
                                             prefill_image=100, rho=(1, 8), split_dist=60,
                                             p_local=0.9), 8),
    "f32_d64": (small_config(dtype="f32", heads=5), 2),
    "f32_d128": (small_config(dtype="f32", head_dim=128, heads=3, rho=(1, 6), split_dist=40,
                              p_local=0.0), 7),
    "full_cache": (small_config(full_cache=True, image_tokens=120), 4),
    "one_split": (small_config(layers=2), 1),
    "ragged": (small_config(heads=7, prefix=5, image_tokens=143, prefill_image=37,
                            local_window=13, split_dist=21, rho=(2, 7)), 6),
}


@pytest.mark.parametrize("name", sorted(SPLIT_STEP_CASES))
def test_parity_split_step_per_layer(name):
    """hkv_decode_step_split, one launch pair per layer as a model runs it,
    replayed on the oracle (every group, every step, lock-step scores)."""
    w, n_split = SPLIT_STEP_CASES[name]
    print(f"[gpu] split step per layer {name}: S={w.S} N={w.N} d={w.head_dim} "
          f"n_split={n_split}", flush=True)
    _check_all_groups(w, name, per_layer=True, n_split=n_split)


def test_split_step_rejects_bad_split():
    w = small_config()
    cfg = hk.config_from_workload(w)
    cache = hk.HkvCache(cfg)
    cache.state.phase = 1
    buf = torch.zeros((w.S, w.q_rows, w.head_dim), dtype=torch.bfloat16, device="cuda")
    for bad in (0, 9, -1):
        with pytest.raises(hk.HkvError) as e:
            hk.hkv_decode_step_split(cfg, cache.state, w.P, buf, buf, w.head_dim, buf,
                                     w.q_rows * w.head_dim, buf, w.head_dim, None, 0, w.S, bad)
        assert e.value.status == hk.E_INVAL


@pytest.mark.parametrize("dtype,head_dim,layers,batch,heads", [
    ("bf16", 128, 3, 4, 50),     # 600 streams: 512 dealt to the XCDs in chunks of 64, 88 past them
    ("bf16", 64, 3, 3, 7),       # 63 streams: contiguous runs per XCD, the first 7 runs one longer
])
def test_parity_xcd_mapping_tail(dtype, head_dim, layers, batch, heads):
    """Stream counts that the workgroup-to-XCD mapping does not divide evenly:
    every stream is still processed exactly once (first, middle and last
    groups replayed on the oracle, lock-step scores)."""
    w = small_config(dtype=dtype, head_dim=head_dim, layers=layers, batch=batch, heads=heads,
                     image_tokens=60, prefill_image=20, rho=(1, 2), split_dist=12,
                     local_window=8)
    groups = sorted({(0, 0), (layers // 2, batch // 2), (layers - 1, batch - 1)})
    print(f"[gpu] xcd mapping tail: S={w.S} d={head_dim} groups={groups}", flush=True)
    g = gpu_generation(w, 0, group_streams(w, groups), score_trace=True)
    rep = None
    for (l, b) in groups:
        rep = oracle_check_group(w, 0, l, b, g, rep=rep)
    print(f"  outputs {rep.outputs_checked} events {rep.events_checked} max err "
          f"{rep.max_out_err:.3g}", flush=True)
    assert not rep.failures, rep.failures[:8]
    assert rep.events_checked > 0 and rep.lockstep_events == rep.events_checked
    assert rep.flagged_counts == rep.flagged_labels == rep.flagged_evictions == 0
