"""hkv_classify_noalloc (classification scores in the library's own per-device
buffer, no workspace, nothing allocated) against hkv_classify with a workspace:
identical state, bit for bit, on two calls in a row, the second smaller."""
from __future__ import annotations

import pytest
import torch

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("needs a GPU", allow_module_level=True)

import kv_cache_compression_hkv_amd as hk
from hkv_inputs.gpu import device_inputs
from tests._fixtures import small_config

FIELDS = ("k_pool", "v_pool", "pos", "score", "base", "cap", "count", "budget", "n_tokens",
          "label", "free_slots", "n_free", "qstat", "err")


def _bits(t):
    # bit patterns, so that equal NaN tags compare equal
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16)
    return t.view(torch.int32) if t.dtype == torch.float32 else t


def _compare(w, seed):
    K, V, Q = device_inputs(w, seed)
    cfg = hk.config_from_workload(w)
    d = w.head_dim
    ref = hk.HkvCache(cfg)
    hk.hkv_classify(cfg, ref.state, K, V, w.N * d, Q, w.q_rows * d)
    na = hk.HkvCache(cfg)
    na.state.workspace = None              # the entry point must not need it
    na.state.workspace_bytes = 0
    hk.hkv_classify_noalloc(cfg, na.state, K, V, w.N * d, Q, w.q_rows * d)
    hk.hkv_check(cfg, na.state)
    torch.cuda.synchronize()
    assert na.state.phase == 1
    for f in FIELDS:
        a, b = getattr(ref, f), getattr(na, f)
        assert torch.equal(_bits(a), _bits(b)), f
    glob = int((ref.label == hk.GLOBAL).sum())
    return glob


def test_noalloc_classify_equals_workspace_classify():
    # a larger call (initial evictions from the scratch scores), then a smaller
    # one of another element type and head size: the second reads only what it
    # wrote itself
    big = small_config(layers=4, batch=4, heads=6, prefill_image=90, image_tokens=200)
    small = small_config(dtype="f32", head_dim=128, heads=3, prefill_image=20, image_tokens=90)
    print("[gpu] no-alloc classify, large then small", flush=True)
    assert _compare(big, 0) > 0
    _compare(small, 1)
    assert _compare(big, 2) > 0


def test_noalloc_rejects_oversized():
    w = small_config(layers=64, batch=8, heads=128, prefill_image=200, image_tokens=400)
    cfg = hk.config_from_workload(w)
    assert w.S * w.P * 4 > 32 << 20
    a = 1 << 20
    st = hk.hkv_state(a, a, a, a, a, a, a, a, a, a, a, a, a, a, None, 0, 0)
    with pytest.raises(hk.HkvError) as e:
        hk.hkv_classify_noalloc(cfg, st, a, a, w.N * w.head_dim, a, w.q_rows * w.head_dim)
    assert e.value.status == hk.E_UNSUPPORTED
