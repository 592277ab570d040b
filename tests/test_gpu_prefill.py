"""hkv_prefill: causal attention over the prefill positions with the
classification computed from the same logits (bf16).

* Every prefill output against the oracle's fp64 causal attention, within the
  bf16 tolerance.
* The classification and initial layout through a whole decode generation
  started from hkv_prefill: labels, counts, budgets, every eviction and every
  decode output against the oracle (the same checks as hkv_classify's path).
Cases span one partial query block, several blocks with a ragged first one, both
head sizes and the uncompressed layout (attention only)."""
from __future__ import annotations

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import kv_cache_compression_hkv_amd as hk
import oracle.hkv_oracle as O
from hkv_inputs import gen
from hkv_inputs.gpu import bits_of, device_inputs, upload_bits
from tests._fixtures import small_config
from tests._parity import gpu_generation, group_streams, oracle_check_group

CASES = {
    # P = 56: one partial block of 64 queries
    "d64_p56": small_config(layers=2, batch=2),
    # P = 116: a full block and a ragged one
    "d128_p116": small_config(head_dim=128, image_tokens=584, prefill_image=100, split_dist=60),
    # P = 200: four blocks, initial eviction at classification (P > B_g)
    "d128_p200": small_config(head_dim=128, heads=3, image_tokens=400, prefill_image=184,
                              rho=(1, 4), split_dist=60),
    "d64_p137_ragged": small_config(heads=5, prefix=5, image_tokens=300, prefill_image=132,
                                    local_window=13, split_dist=21, rho=(2, 7)),
    # P = 1000, near the classification's limit of 1024 positions: sixteen
    # query blocks and a 32 KB observation tile on chip
    "d64_p1000": small_config(heads=2, image_tokens=1100, prefill_image=984),
    # the same at d128: 36 KB of static LDS plus the 32 KB tile
    "d128_p1000": small_config(head_dim=128, heads=2, image_tokens=1100, prefill_image=984),
    # uncompressed layout: attention only
    "d64_full_cache": small_config(full_cache=True, image_tokens=120),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_prefill_outputs(name):
    w = CASES[name]
    S, P, d, N = w.S, w.P, w.head_dim, w.N
    print(f"[gpu] prefill outputs {name}: S={S} P={P} d={d}", flush=True)
    K, V, _ = device_inputs(w, 0)
    qbits = gen.prefill_queries(w, 0)
    qs = upload_bits(qbits, K)
    cfg = hk.config_from_workload(w)
    cache = hk.HkvCache(cfg)
    out = torch.full((S, P, d), float("nan"), dtype=K.dtype, device=K.device)
    hk.hkv_prefill(cfg, cache.state, qs, P * d, K, V, N * d, out, P * d)
    torch.cuda.synchronize()
    hk.hkv_check(cfg, cache.state)
    got = gen.decode(bits_of(out), w.dtype)
    kb, vb, _ = gen.all_inputs(w, 0)
    Kf, Vf, Qf = gen.decode(kb, w.dtype), gen.decode(vb, w.dtype), gen.decode(qbits, w.dtype)
    err = 0.0
    for s in range(S):
        for p in range(P):
            o, _ = O.attend(Qf[s, p], Kf[s, :p + 1], Vf[s, :p + 1])
            err = max(err, float(np.abs(got[s, p] - o).max()))
    print(f"  max abs err {err:.3g}", flush=True)
    assert np.isfinite(got).all()
    assert err <= 2e-2


@pytest.mark.parametrize("name", ["d64_p56", "d128_p116", "d128_p200", "d64_p137_ragged",
                                  "d64_p1000", "d128_p1000"])
def test_prefill_classification_parity(name):
    w = CASES[name]
    print(f"[gpu] prefill classification {name}: S={w.S} P={w.P}", flush=True)
    groups = [(l, b) for l in range(w.layers) for b in range(w.batch)]
    g = gpu_generation(w, 0, group_streams(w, groups), prefill=True)
    rep = None
    for (l, b) in groups:
        rep = oracle_check_group(w, 0, l, b, g, rep=rep)
    print(f"  outputs {rep.outputs_checked} events {rep.events_checked} "
          f"flags {rep.flagged_counts}/{rep.flagged_labels}/{rep.flagged_evictions}", flush=True)
    assert not rep.failures, rep.failures[:8]
    assert rep.events_checked > 0


def test_prefill_rejects_f32_and_null():
    w = small_config(dtype="f32")
    cfg = hk.config_from_workload(w)
    cache = hk.HkvCache(cfg)
    K, V, _ = device_inputs(w, 0)
    out = torch.empty((w.S, w.P, w.head_dim), dtype=K.dtype, device=K.device)
    with pytest.raises(hk.HkvError):
        hk.hkv_prefill(cfg, cache.state, K, w.N * w.head_dim, K, V, w.N * w.head_dim, out,
                       w.P * w.head_dim)
    w2 = small_config()
    cfg2 = hk.config_from_workload(w2)
    cache2 = hk.HkvCache(cfg2)
    K2, V2, _ = device_inputs(w2, 0)
    with pytest.raises(hk.HkvError):
        hk.hkv_prefill(cfg2, cache2.state, None, w2.P * w2.head_dim, K2, V2, w2.N * w2.head_dim,
                       out, w2.P * w2.head_dim)


@pytest.mark.parametrize("name", ["llamagen_xl_rho1_6", "janus_pro_7b_rho1_6"])
def test_prefill_fullsize(name):
    """hkv_prefill at a workload's full size, in the launch the benchmark times
    (queries: seeded normal values on the device, the last W rows the
    workload's observation queries).  The first and last (layer, sequence)
    groups are checked against the oracle: every prefill output of every head,
    and each stream's count and label (a count is flagged, not failed, where
    tau lies within the oracle's rounding band at the GPU's count)."""
    from hkv_inputs.configs import WORKLOADS
    from tests._parity import _count_flag
    w = WORKLOADS[name]
    S, P, d, N, W, H = w.S, w.P, w.head_dim, w.N, w.w_obs, w.heads
    print(f"[gpu] prefill full size {name}: S={S} P={P} d={d}", flush=True)
    K, V, Q = device_inputs(w, 0)
    g = torch.Generator(device=K.device).manual_seed(7)
    qs = torch.randn((S, P, d), generator=g, device=K.device).to(K.dtype)
    qs[:, P - W:] = Q[:, :W]
    out = torch.full((S, P, d), float("nan"), dtype=K.dtype, device=K.device)
    cfg = hk.config_from_workload(w)
    cache = hk.HkvCache(cfg)
    hk.hkv_prefill(cfg, cache.state, qs, P * d, K, V, N * d, out, P * d)
    torch.cuda.synchronize()
    hk.hkv_check(cfg, cache.state)
    n_gpu = cache.n_tokens.cpu().numpy()
    lab_gpu = cache.label.cpu().numpy()
    err, flagged = 0.0, 0
    for (l, b) in [(0, 0), (w.layers - 1, w.batch - 1)]:
        kb, vb, _ = gen.group_inputs(w, 0, l, b)
        Kf, Vf = gen.decode(kb, w.dtype), gen.decode(vb, w.dtype)
        for h in range(H):
            s = w.stream(l, b, h)
            q = qs[s].float().cpu().numpy().astype(np.float64)
            o = out[s].float().cpu().numpy()
            for p in range(P):
                ref, _ = O.attend(q[p], Kf[h, :p + 1], Vf[h, :p + 1])
                err = max(err, float(np.abs(o[p] - ref).max()))
            pr = O.probs(q[P - 1], Kf[h, :P])
            n_or = O.classify_count(pr, w.tau)
            if n_or != int(n_gpu[s]):
                assert _count_flag(pr, int(n_gpu[s]), w.tau), (l, b, h, n_or, int(n_gpu[s]))
                flagged += 1
            elif O.label_of(n_or, w.local_window) != int(lab_gpu[s]):
                raise AssertionError((l, b, h, "label", n_or, int(lab_gpu[s])))
    print(f"  max abs err {err:.3g}, flagged counts {flagged}", flush=True)
    assert err <= 2e-2
