"""Helpers shared by the tests: golden-file parsing and small workload builders."""
from __future__ import annotations

import os

import numpy as np

from hkv_inputs.configs import HkvConfig
from hkv_inputs import gen

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def read_sections(name: str):
    """Parse `[section]` / `key = values` files into {section: {key: str}}."""
    out, cur = {}, None
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if not line:
                continue
            if line.startswith("[") and line.endswith("]"):
                cur = out.setdefault(line[1:-1], {})
                continue
            k, v = (x.strip() for x in line.split("=", 1))
            cur[k] = v
    return out


def read_kv(name: str):
    """Parse flat `key = value` files."""
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if "=" in line:
                k, v = (x.strip() for x in line.split("=", 1))
                out[k] = v
    return out


def read_rows(name: str):
    """Parse `a | b | c` rows (comments with '#')."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for raw in f:
            line = raw.split("#", 1)[0].strip()
            if line:
                rows.append([c.strip() for c in line.split("|")])
    return rows


def small_config(**kw) -> HkvConfig:
    """A small bf16 workload for oracle-side property checks."""
    base = dict(name="small", cid=10, layers=1, batch=1, heads=6, head_dim=64,
                dtype="bf16", prefix=16, image_tokens=160, prefill_image=40,
                local_window=12, rho=(1, 4), split_dist=24, p_local=0.5)
    base.update(kw)
    return HkvConfig(**base)


def group_f64(cfg: HkvConfig, seed: int = 0, l: int = 0, b: int = 0):
    k, v, q = gen.group_inputs(cfg, seed, l, b)
    return gen.decode(k, cfg.dtype), gen.decode(v, cfg.dtype), gen.decode(q, cfg.dtype)
