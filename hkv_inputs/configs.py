"""Workload shapes for the HeadKV decode-time path, as plain data.

This module holds raw parameters only (layer/batch/head counts, lengths, window,
compression ratio, split distance).  It derives nothing that the method computes
(no per-head budget, no capacity): the oracle and the native library each derive
those on their own.

The five named workloads are synthetic stand-ins shaped like the backbones the
HeadKV pages evaluate (page "Head-Aware Key-Value Compression for Efficient
Autoregressive Image Generation", technical summary, section "Results": Janus-Pro-1B,
Janus-Pro-7B, Lumina-mGPT-768, LlamaGen-XL).  No weights are involved: keys,
values and queries come from the seeded generator in ``hkv_inputs.gen``.

Stream index convention used everywhere: ``s = (l * batch + b) * heads + h``.
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace
from typing import Optional, Tuple


@dataclass(frozen=True)
class HkvConfig:
    name: str
    cid: int                  # workload id; enters the generator key
    layers: int
    batch: int
    heads: int
    head_dim: int
    dtype: str                # "bf16" or "f32" (storage of q, k, v, o)
    prefix: int               # text-condition prefix tokens
    image_tokens: int         # generated image tokens
    prefill_image: int        # image tokens generated before classification
    local_window: int         # w
    rho: Tuple[int, int]      # compression ratio as an exact fraction (num, den)
    split_dist: int           # D: near/far split distance for eviction
    w_obs: int = 8            # observation window (queries scoring the cache)
    evict_m: int = 8          # M: tokens evicted per eviction event
    tau: float = 0.9          # attention-mass threshold for classification
    # head bias: either an explicit per-head tuple (True = locality-biased)
    # shared by all layers, or a Bernoulli probability per (layer, head)
    bias_heads: Optional[Tuple[bool, ...]] = None
    p_local: Optional[float] = None
    anchor_mode: str = "prefill"   # "prefill" or "full_history"
    full_cache: bool = False       # baseline: no classification, no eviction
    # ablation variants (same shapes; see the method notes of the library)
    unstratified: bool = False     # eviction without the near/far split
    uniform_budget: bool = False   # every head keeps floor(rho * N) tokens

    # ---- plain shape arithmetic (no method quantities) ----
    @property
    def N(self) -> int:           # final sequence length
        return self.prefix + self.image_tokens

    @property
    def P(self) -> int:           # cached length at classification
        return self.prefix + self.prefill_image

    @property
    def S(self) -> int:           # number of (layer, sequence, head) streams
        return self.layers * self.batch * self.heads

    @property
    def steps(self) -> int:       # decode steps t = P .. N-1
        return self.N - self.P

    @property
    def q_rows(self) -> int:      # stored queries: positions P-w_obs .. N-1
        return self.N - self.P + self.w_obs

    @property
    def elem_bytes(self) -> int:
        return 2 if self.dtype == "bf16" else 4

    def stream(self, l: int, b: int, h: int) -> int:
        return (l * self.batch + b) * self.heads + h

    def with_(self, **kw) -> "HkvConfig":
        return replace(self, **kw)


# The five workloads.  Readings of the workload text (documented alongside the
# design): "prefill the first 64 tokens" of the tiny case means P = 64 out of
# N = 256 with no text prefix; every other case has N = prefix + image tokens and
# P = prefix + prefilled image tokens.
TINY = HkvConfig(
    name="tiny_f32", cid=0, layers=1, batch=1, heads=4, head_dim=64, dtype="f32",
    prefix=0, image_tokens=256, prefill_image=64, local_window=16, rho=(1, 4),
    split_dist=32, bias_heads=(True, True, False, False))

LLAMAGEN_XL = HkvConfig(
    name="llamagen_xl_rho1_6", cid=1, layers=36, batch=16, heads=20, head_dim=64,
    dtype="bf16", prefix=120, image_tokens=576, prefill_image=64, local_window=32,
    rho=(1, 6), split_dist=48, p_local=0.6)

JANUS_PRO_1B = HkvConfig(
    name="janus_pro_1b_rho1_4", cid=2, layers=24, batch=32, heads=16, head_dim=128,
    dtype="bf16", prefix=64, image_tokens=576, prefill_image=64, local_window=32,
    rho=(1, 4), split_dist=48, p_local=0.6)

JANUS_PRO_7B = HkvConfig(
    name="janus_pro_7b_rho1_6", cid=3, layers=30, batch=32, heads=32, head_dim=128,
    dtype="bf16", prefix=64, image_tokens=576, prefill_image=64, local_window=32,
    rho=(1, 6), split_dist=48, p_local=0.5)

JANUS_PRO_7B_R8 = JANUS_PRO_7B.with_(name="janus_pro_7b_rho1_8", rho=(1, 8))

# 48x48 grid with one line-end token per row: 48 * 49 = 2352 image tokens;
# a window of 98 tokens is two such rows.
LUMINA_MGPT_768 = HkvConfig(
    name="lumina_mgpt_768_rho1_8", cid=4, layers=32, batch=8, heads=32, head_dim=128,
    dtype="bf16", prefix=64, image_tokens=2352, prefill_image=128, local_window=98,
    rho=(1, 8), split_dist=196, p_local=0.5, anchor_mode="full_history")

WORKLOADS = {c.name: c for c in
             (TINY, LLAMAGEN_XL, JANUS_PRO_1B, JANUS_PRO_7B, JANUS_PRO_7B_R8,
              LUMINA_MGPT_768)}


def full_cache_of(cfg: HkvConfig) -> HkvConfig:
    """The same workload laid out as an uncompressed cache (speed baseline)."""
    return cfg.with_(name=cfg.name + "_full", full_cache=True)


def variant_of(cfg: HkvConfig, unstratified: bool = False, uniform_budget: bool = False) -> HkvConfig:
    """The same workload run as an ablation variant."""
    tag = ("_unstrat" if unstratified else "") + ("_uniform" if uniform_budget else "")
    return cfg.with_(name=cfg.name + tag, unstratified=unstratified, uniform_budget=uniform_budget)
