"""Seeded synthetic inputs (keys, values, queries) for the HeadKV decode path.

CPU (numpy) definition.  ``hkv_inputs/csrc/hkv_gen.hip`` is a GPU twin that must
produce the same bits; nothing here is part of the method's arithmetic.

Recipe (every step is integer-exact or a single IEEE-rounded operation, so the
CPU and GPU definitions agree bit for bit):

* Random words: Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random
  numbers: as easy as 1, 2, 3", SC'11), key = (seed, workload id), counter =
  (element index, stream, tag, j).
* Standard normal: Irwin-Hall sum of twelve 16-bit uniforms taken from the six
  words of two Philox blocks (j = 0: all four words, j = 1: words 0-1),
  ``z = (sum - 12 * 32767.5) / 65536``.  Mean 0, variance 1 - 2**-32, |z| <= 6;
  z is a multiple of 2**-16 and exact in fp32.
* Keys and values: z, stored as fp32 or rounded to bf16 (round to nearest even).
  Tags: 0 = key, 1 = value, 2 = query noise, 3 = anchors, 4 = head bias.
* Queries for positions t in [P - w_obs, N - 1] (the observation window and
  every decode step), from the STORED keys:
    locality-biased head: q_t = 2 * mean(k_{t-3..t}) + 0.5 * eps_t
    global-biased head:   q_t = 2 * mean(k_a over anchors a) + 0.5 * eps_t
  evaluated in fp64 as ``(2.0 * S) / m + 0.5 * eps`` (S = exact sum of the m
  keys), rounded to fp32 (nearest even), then to bf16 for bf16 workloads.
  0.5 is the noise standard deviation (the workload text's N(0, 0.25) read as a
  variance).
* Anchors: 4 distinct positions per stream by Floyd's sampling.  "prefill" mode:
  uniform in [0, P - 33], all four used at every t.  "full_history" mode: the
  first in [0, P - 40] (valid for every observation query), three more in
  [0, N - 33]; at position t the mean runs over anchors a <= t - 32.
* Head bias: explicit per-head tuple, or Bernoulli(p_local) per (layer, head)
  shared by the batch: Local-biased iff word < floor(p_local * 2**32).
"""
from __future__ import annotations

import numpy as np

from .configs import HkvConfig

_M0 = np.uint64(0xD2511F53)
_M1 = np.uint64(0xCD9E8D57)
_W0 = 0x9E3779B9
_W1 = 0xBB67AE85
_MASK = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)

TAG_K, TAG_V, TAG_QNOISE, TAG_ANCHOR, TAG_BIAS, TAG_QPRE = 0, 1, 2, 3, 4, 5


def philox4x32_10(c0, c1, c2, c3, k0: int, k1: int):
    """Philox4x32 with 10 rounds on arrays of 32-bit counters (held in uint64)."""
    c0, c1, c2, c3 = (np.asarray(c, dtype=np.uint64) & _MASK for c in (c0, c1, c2, c3))
    c0, c1, c2, c3 = np.broadcast_arrays(c0, c1, c2, c3)
    k0 &= 0xFFFFFFFF
    k1 &= 0xFFFFFFFF
    for r in range(10):
        if r:
            k0 = (k0 + _W0) & 0xFFFFFFFF
            k1 = (k1 + _W1) & 0xFFFFFFFF
        p0 = _M0 * c0
        p1 = _M1 * c2
        c0, c1, c2, c3 = ((p1 >> _S32) ^ c1 ^ np.uint64(k0), p1 & _MASK,
                          (p0 >> _S32) ^ c3 ^ np.uint64(k1), p0 & _MASK)
    return c0, c1, c2, c3


def _key(cfg: HkvConfig, seed: int):
    return int(seed), int(cfg.cid)


def normals(cfg: HkvConfig, seed: int, stream: int, tag: int, index) -> np.ndarray:
    """z for the given element indices (float64, exact multiples of 2**-16)."""
    k0, k1 = _key(cfg, seed)
    idx = np.asarray(index, dtype=np.uint64)
    a = philox4x32_10(idx, stream, tag, 0, k0, k1)
    b = philox4x32_10(idx, stream, tag, 1, k0, k1)
    words = (a[0], a[1], a[2], a[3], b[0], b[1])
    tot = np.zeros(idx.shape, dtype=np.int64)
    m16 = np.uint64(0xFFFF)
    for w in words:
        tot += (w & m16).astype(np.int64)
        tot += (w >> np.uint64(16)).astype(np.int64)
    z2 = 2 * tot - 12 * 65535                     # = 2 * (sum - 12 * 32767.5)
    return z2.astype(np.float64) / 131072.0


def f32_to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = ((u >> np.uint64(16)) & np.uint64(1)) + np.uint64(0x7FFF)
    return (((u + r) >> np.uint64(16)) & np.uint64(0xFFFF)).astype(np.uint16)


def encode(x64: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 -> stored bits: fp32 (nearest even) -> bf16 (nearest even) for bf16."""
    x32 = np.asarray(x64, dtype=np.float64).astype(np.float32)
    if dtype == "f32":
        return x32.view(np.uint32)
    return f32_to_bf16_bits(x32)


def decode(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Stored bits -> float64 values."""
    bits = np.asarray(bits)
    if dtype == "f32":
        return bits.astype(np.uint32).view(np.float32).astype(np.float64)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def head_bias(cfg: HkvConfig, seed: int) -> np.ndarray:
    """bool [layers, heads]: True = locality-biased query generator."""
    if cfg.bias_heads is not None:
        row = np.array(cfg.bias_heads, dtype=bool)
        assert row.shape == (cfg.heads,)
        return np.tile(row, (cfg.layers, 1))
    k0, k1 = _key(cfg, seed)
    hh, ll = np.meshgrid(np.arange(cfg.heads), np.arange(cfg.layers))
    w = philox4x32_10(hh, ll, TAG_BIAS, 0, k0, k1)[0]
    thr = np.uint64(int(cfg.p_local * 4294967296.0))
    return w < thr


def _floyd(words, lo_range: int, count: int):
    """Floyd's sampling of `count` distinct values in [0, lo_range)."""
    chosen = []
    for i, j in enumerate(range(lo_range - count, lo_range)):
        t = int(words[i]) % (j + 1)
        chosen.append(j if t in chosen else t)
    return chosen


def anchors(cfg: HkvConfig, seed: int, stream: int) -> np.ndarray:
    """Sorted int array of 4 anchor positions for a global-biased stream."""
    k0, k1 = _key(cfg, seed)
    w = philox4x32_10(np.arange(4), stream, TAG_ANCHOR, 0, k0, k1)[0]
    if cfg.anchor_mode == "prefill":
        R = cfg.P - 32
        assert R >= 4, "prefill anchors need P >= 36"
        return np.array(sorted(_floyd(w, R, 4)), dtype=np.int64)
    assert cfg.anchor_mode == "full_history"
    R0 = cfg.P - 40 + 1
    assert R0 >= 1, "full-history anchors need P >= 40"
    a0 = int(w[0]) % R0
    R = cfg.N - 32 - 1            # positions [0, N-33] minus a0
    rest = [v if v < a0 else v + 1 for v in _floyd(w[1:], R, 3)]
    return np.array(sorted([a0] + rest), dtype=np.int64)


def stream_inputs(cfg: HkvConfig, seed: int, l: int, b: int, h: int, bias_row=None):
    """Bits of K [N,d], V [N,d] and Q [q_rows,d] for one stream (uint16 or uint32)."""
    N, d, P, W = cfg.N, cfg.head_dim, cfg.P, cfg.w_obs
    s = cfg.stream(l, b, h)
    local = bool((head_bias(cfg, seed) if bias_row is None else bias_row)[l, h])
    idx = np.arange(N * d, dtype=np.uint64)
    kb = encode(normals(cfg, seed, s, TAG_K, idx), cfg.dtype).reshape(N, d)
    vb = encode(normals(cfg, seed, s, TAG_V, idx), cfg.dtype).reshape(N, d)
    kf = decode(kb, cfg.dtype)
    ts = np.arange(P - W, N)
    qidx = (ts[:, None] * d + np.arange(d)[None, :]).astype(np.uint64)
    eps = normals(cfg, seed, s, TAG_QNOISE, qidx)
    if local:
        csum = np.concatenate([np.zeros((1, d)), np.cumsum(kf, axis=0)], axis=0)
        lo = np.maximum(ts - 3, 0)
        S = csum[ts + 1] - csum[lo]
        m = (ts + 1 - lo).astype(np.float64)[:, None]
    else:
        anc = anchors(cfg, seed, s)
        if cfg.anchor_mode == "prefill":
            S = np.broadcast_to(kf[anc].sum(axis=0), (len(ts), d)).copy()
            m = np.full((len(ts), 1), float(len(anc)))
        else:
            valid = anc[None, :] <= (ts[:, None] - 32)          # [T, 4]
            S = np.einsum("ta,ad->td", valid.astype(np.float64), kf[anc])
            m = valid.sum(axis=1).astype(np.float64)[:, None]
    q64 = (2.0 * S) / m + 0.5 * eps
    qb = encode(q64, cfg.dtype)
    return kb, vb, qb


def group_inputs(cfg: HkvConfig, seed: int, l: int, b: int):
    """Stacked bits for the H streams of one (layer, sequence) group."""
    bias = head_bias(cfg, seed)
    parts = [stream_inputs(cfg, seed, l, b, h, bias) for h in range(cfg.heads)]
    return tuple(np.stack([p[i] for p in parts]) for i in range(3))


def all_inputs(cfg: HkvConfig, seed: int):
    """K [S,N,d], V [S,N,d], Q [S,q_rows,d] bits for every stream (small workloads)."""
    bias = head_bias(cfg, seed)
    ks, vs, qs = [], [], []
    for l in range(cfg.layers):
        for b in range(cfg.batch):
            for h in range(cfg.heads):
                k, v, q = stream_inputs(cfg, seed, l, b, h, bias)
                ks.append(k); vs.append(v); qs.append(q)
    return np.stack(ks), np.stack(vs), np.stack(qs)


def _floyd_vec(words: np.ndarray, lo_range: int, count: int) -> np.ndarray:
    """Vectorised `_floyd` over rows of `words` ([n, >=count] uint)."""
    n = words.shape[0]
    chosen = np.zeros((n, count), dtype=np.int64)
    for i, j in enumerate(range(lo_range - count, lo_range)):
        t = (words[:, i].astype(np.int64)) % (j + 1)
        dup = (chosen[:, :i] == t[:, None]).any(axis=1) if i else np.zeros(n, bool)
        chosen[:, i] = np.where(dup, j, t)
    return chosen


def anchors_all(cfg: HkvConfig, seed: int) -> np.ndarray:
    """int32 [S, 4]: `anchors(cfg, seed, s)` for every stream."""
    k0, k1 = _key(cfg, seed)
    S = cfg.S
    ss, kk = np.meshgrid(np.arange(S), np.arange(4), indexing="ij")
    w = philox4x32_10(kk, ss, TAG_ANCHOR, 0, k0, k1)[0]          # [S, 4]
    if cfg.anchor_mode == "prefill":
        out = _floyd_vec(w, cfg.P - 32, 4)
    else:
        a0 = (w[:, 0].astype(np.int64)) % (cfg.P - 40 + 1)
        rest = _floyd_vec(w[:, 1:], cfg.N - 32 - 1, 3)
        rest = np.where(rest < a0[:, None], rest, rest + 1)
        out = np.concatenate([a0[:, None], rest], axis=1)
    return np.sort(out, axis=1).astype(np.int32)


def local_flags(cfg: HkvConfig, seed: int) -> np.ndarray:
    """uint8 [S]: 1 where the stream uses the locality-biased query generator."""
    bias = head_bias(cfg, seed)                       # [L, H]
    return np.repeat(bias[:, None, :], cfg.batch, axis=1).reshape(-1).astype(np.uint8)


def prefill_queries(cfg: HkvConfig, seed: int) -> np.ndarray:
    """Bits of the queries of every prefill position, [S, P, d]: positions
    0 .. P-W-1 standard normal (their own counter tag), the last W positions the
    workload's observation queries (Q rows 0 .. W-1), so a classification from
    this prefill sees exactly the observation queries of hkv_classify."""
    P, W, d = cfg.P, cfg.w_obs, cfg.head_dim
    out = []
    _, _, q = all_inputs(cfg, seed)
    idx = np.arange((P - W) * d, dtype=np.uint64)
    for s in range(cfg.S):
        head = encode(normals(cfg, seed, s, TAG_QPRE, idx), cfg.dtype).reshape(P - W, d)
        out.append(np.concatenate([head, q[s, :W]], axis=0))
    return np.stack(out)
