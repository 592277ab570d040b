"""The seeded input generator (shared by the oracle and the GPU harness)."""
from __future__ import annotations

import numpy as np
import torch

from hkv_inputs import gen
from hkv_inputs.configs import LLAMAGEN_XL, LUMINA_MGPT_768, TINY, WORKLOADS
from tests._fixtures import GOLDEN, small_config


def test_philox_known_answers():
    rows = [l.split() for l in open(f"{GOLDEN}/philox4x32_10_kat.txt")
            if l.strip() and not l.startswith("#")]
    assert len(rows) == 3
    for r in rows:
        c0, c1, c2, c3, k0, k1, *want = (int(x, 16) for x in r)
        got = gen.philox4x32_10(c0, c1, c2, c3, k0, k1)
        assert [int(x) for x in got] == want


def test_normal_moments_and_range():
    z = gen.normals(LLAMAGEN_XL, 0, 3, gen.TAG_K, np.arange(2_000_000))
    assert abs(z.mean()) < 3e-3
    assert abs(z.var() - 1.0) < 3e-3
    assert np.abs(z).max() <= 6.0
    assert np.all(z * 65536 == np.round(z * 65536))       # multiples of 2**-16


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.normal(size=100000).astype(np.float32),
                        np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -1 - 2 ** -8, 0.0, -0.0],
                                 np.float32)])
    ours = gen.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_determinism_and_seed():
    cfg = small_config()
    a = gen.stream_inputs(cfg, 5, 0, 0, 1)
    b = gen.stream_inputs(cfg, 5, 0, 0, 1)
    c = gen.stream_inputs(cfg, 6, 0, 0, 1)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    assert not np.array_equal(a[0], c[0])


def test_shapes_and_dtypes():
    for cfg in (TINY, small_config()):
        k, v, q = gen.group_inputs(cfg, 0, 0, 0)
        assert k.shape == (cfg.heads, cfg.N, cfg.head_dim) == v.shape
        assert q.shape == (cfg.heads, cfg.q_rows, cfg.head_dim)
        assert k.dtype == (np.uint32 if cfg.dtype == "f32" else np.uint16)


def test_query_recipe():
    """Locality-biased queries: fp32/bf16 rounding of 2*mean(k_{t-3..t}) + 0.5*eps."""
    cfg = small_config()
    bias = gen.head_bias(cfg, 0)
    h = int(np.nonzero(bias[0])[0][0])
    k, v, q = gen.stream_inputs(cfg, 0, 0, 0, h)
    K = gen.decode(k, cfg.dtype)
    s = cfg.stream(0, 0, h)
    for t in (cfg.P - cfg.w_obs, cfg.P + 10, cfg.N - 1):
        eps = gen.normals(cfg, 0, s, gen.TAG_QNOISE, t * cfg.head_dim + np.arange(cfg.head_dim))
        want = 2 * K[t - 3:t + 1].mean(axis=0) + 0.5 * eps
        got = gen.decode(q[t - (cfg.P - cfg.w_obs)], cfg.dtype)
        assert np.array_equal(got, gen.decode(gen.encode(want, cfg.dtype), cfg.dtype))


def test_anchor_ranges():
    for cfg in (TINY, LLAMAGEN_XL):
        for s in range(50):
            a = gen.anchors(cfg, 0, s)
            assert len(set(a.tolist())) == 4
            assert a.min() >= 0 and a.max() <= cfg.P - 33
    cfg = LUMINA_MGPT_768
    for s in range(50):
        a = gen.anchors(cfg, 0, s)
        assert len(set(a.tolist())) == 4
        assert a.min() <= cfg.P - 40 and a.max() <= cfg.N - 33


def test_head_bias_rate():
    b = gen.head_bias(LLAMAGEN_XL.with_(layers=400), 0)
    assert abs(b.mean() - 0.6) < 0.03
    assert gen.head_bias(TINY, 0).tolist() == [[True, True, False, False]]
