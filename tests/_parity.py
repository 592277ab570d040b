"""GPU-vs-oracle parity harness (test infrastructure).

The GPU runs a whole generation through the C ABI and records, for the streams
of a few sampled (layer, sequence) groups, its decisions and outputs: labels and
counts, the cache layout after classification, the evicted positions of every
step, every attention output and the final layout.  The oracle then replays each
sampled group from the same seeded inputs (regenerated on the CPU).  Where the
oracle's own fp64 decision and the GPU's fp32 decision differ only inside the
flag bands below, the GPU decision is adopted so both runs stay in step; every
other difference is a failure.

Flag bands:
  classification: the oracle's count lies within 1 of the window, or tau lies
    within EPS_C of the oracle's cumulative mass at the GPU's count or count-1;
  eviction: within a subset, the gap between the scores that separate the
    oracle's choice from the GPU's is at most EPS_S.
Output tolerance: bf16 |o_gpu - o_ref| <= 2e-2 per element; fp32
  max|o_gpu - o_ref| <= 1e-5 * max|o_ref| per (stream, step).
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

import kv_cache_compression_hkv_amd as hk
import oracle.hkv_oracle as O
from hkv_inputs import gen
from hkv_inputs.configs import HkvConfig
from hkv_inputs.gpu import bits_of, device_inputs, upload_bits

EPS_C = 1e-5
EPS_S = 1e-5
BF16_ATOL = 2e-2
F32_RTOL = 1e-5


# ------------------------------------------------------------------ GPU side
@dataclass
class GpuRecord:
    streams: List[int]
    labels: np.ndarray
    n_tokens: np.ndarray
    budget: np.ndarray
    cap: np.ndarray
    count0: np.ndarray
    tables0: List[List[int]]
    outs: np.ndarray            # [T, n, d] float64
    logs: np.ndarray            # [T, n, M]
    count_final: np.ndarray
    tables_final: List[List[int]]
    scores_final: List[np.ndarray]
    scores0: List[np.ndarray]                  # scores after classification
    score_trace: Optional[np.ndarray] = None   # [T, sum of caps]: scores after each step
    score_off: Optional[List[int]] = None      # column of each stream's first slot
    no_output: Optional[List[int]] = None      # steps whose attention was not run


def _tables(cache: hk.HkvCache, streams, counts) -> List[List[int]]:
    base = cache.base.cpu().numpy()
    pos = cache.pos
    out = []
    for s, c in zip(streams, counts):
        b = int(base[s])
        out.append(pos[b:b + int(c)].cpu().numpy().astype(int).tolist())
    return out


def group_streams(w: HkvConfig, groups: Sequence[Tuple[int, int]]) -> List[int]:
    return [w.stream(l, b, h) for (l, b) in groups for h in range(w.heads)]


def gpu_generation(w: HkvConfig, seed: int, streams: Sequence[int], *, steps=None,
                   mode: str = "fused", inputs=None, cache=None,
                   per_layer: bool = False, prefill: bool = False,
                   score_trace: bool = False, skip_attn=None, n_split: int = 0) -> GpuRecord:
    """Classification and `steps` decode steps over ALL streams, in the layer-
    folded launch configuration (one call per entry point per step), or with
    per_layer one call per layer (its batch x heads streams) as a model runs.
    With prefill the classification comes from hkv_prefill (prefill attention
    with the classification as a by-product) instead of hkv_classify.  With
    score_trace the scores of the recorded streams' slots are read back after
    every step (an eviction writes the scores it ranked when given a log), for
    a comparison at every eviction event.  In mode "split", skip_attn(t) true
    leaves out step t's attention call (its outputs are not compared).  With
    n_split > 0 the fused mode calls hkv_decode_step_split instead."""
    K, V, Q = inputs if inputs is not None else device_inputs(w, seed)
    cfg = hk.config_from_workload(w)
    cache = cache or hk.HkvCache(cfg)
    st = cache.state
    S, N, d, P, W, M = w.S, w.N, w.head_dim, w.P, w.w_obs, w.evict_m
    eb = w.elem_bytes
    if prefill:
        qs = upload_bits(gen.prefill_queries(w, seed), K)
        pout = torch.empty((S, P, d), dtype=K.dtype, device=K.device)
        hk.hkv_prefill(cfg, st, qs, P * d, K, V, N * d, pout, P * d)
    else:
        hk.hkv_classify(cfg, st, K, V, N * d, Q, w.q_rows * d)
    idx = torch.tensor(list(streams), dtype=torch.long, device=K.device)
    sl = list(streams)
    rec = state_after_classify(cache, sl)
    base0 = cache.base.cpu().numpy()
    capv = rec["cap"]
    T = w.steps if steps is None else steps
    trace = None
    if score_trace:
        offs, cols = [], []
        for s, c in zip(sl, capv):
            offs.append(sum(len(x) for x in cols))
            cols.append(torch.arange(int(base0[s]), int(base0[s]) + int(c), dtype=torch.long))
        sidx = torch.cat(cols).to(K.device)
        trace = torch.empty((T, sidx.numel()), dtype=torch.float32, device=K.device)
        rec["score_off"] = offs
    out = torch.zeros((S, d), dtype=K.dtype, device=K.device)
    log = torch.full((S, M), -1, dtype=torch.int32, device=K.device)
    skipped: List[int] = []
    outs = torch.empty((T, len(sl), d), dtype=K.dtype, device=K.device)
    logs = torch.empty((T, len(sl), M), dtype=torch.int32, device=K.device)
    for step in range(T):
        t = P + step
        kp = K.data_ptr() + t * d * eb
        vp = V.data_ptr() + t * d * eb
        qp = Q.data_ptr() + (t - (P - W)) * d * eb          # query of position t
        qw = Q.data_ptr() + (t - W + 1 - (P - W)) * d * eb  # positions t-W+1 .. t
        if mode == "fused":
            per = w.batch * w.heads if per_layer else S
            for s0 in range(0, S, per):
                if n_split:
                    hk.hkv_decode_step_split(cfg, st, t, kp, vp, N * d, qw, w.q_rows * d, out, d,
                                             log, s0, per, n_split)
                else:
                    hk.hkv_decode_step(cfg, st, t, kp, vp, N * d, qw, w.q_rows * d, out, d, log,
                                       s0, per)
        else:
            hk.hkv_append(cfg, st, t, kp, vp, N * d, 0, S)
            if skip_attn is not None and skip_attn(t):
                skipped.append(step)
            else:
                hk.hkv_decode_attn(cfg, st, t, qp, w.q_rows * d, out, d, 0, S)
            hk.hkv_ste_evict(cfg, st, t, qw, w.q_rows * d, log, 0, S)
        outs[step] = out[idx]
        logs[step] = log[idx]
        if trace is not None:
            trace[step] = cache.score[sidx]
    hk.hkv_check(cfg, st)
    if trace is not None:
        rec["score_trace"] = trace.cpu().numpy()
    rec.update(outs=gen.decode(bits_of(outs), w.dtype), logs=logs.cpu().numpy(),
               no_output=skipped or None, **state_final(cache, sl))
    return GpuRecord(**rec)


# ------------------------------------------------------------------ oracle side
@dataclass
class Report:
    failures: List[str] = field(default_factory=list)
    flagged_counts: int = 0
    flagged_labels: int = 0
    flagged_evictions: int = 0
    events_checked: int = 0
    lockstep_events: int = 0     # events whose GPU scores were compared one by one
    outputs_checked: int = 0
    max_out_err: float = 0.0
    max_score_err: float = 0.0

    def fail(self, msg: str):
        if len(self.failures) < 50:
            self.failures.append(msg)


def _count_flag(p: np.ndarray, n_gpu: int, tau: float) -> bool:
    cum = np.cumsum(p[::-1])
    vals = [cum[k - 1] for k in (n_gpu, n_gpu - 1) if 1 <= k <= len(cum)]
    return any(abs(v - tau) <= EPS_C for v in vals)


def _evict_flag(slot_pos, slot_score, t, W, D, own: List[int], gpu: List[int]) -> bool:
    """True when own and gpu differ only by swapping candidates whose scores lie
    within EPS_S of the selection boundary of their subset."""
    for sub in (0, 1):
        cands = [j for j in range(len(slot_pos))
                 if (W <= t - slot_pos[j] < D) == (sub == 0) and t - slot_pos[j] >= W]
        a = sorted(j for j in own if j in cands)
        b = sorted(j for j in gpu if j in cands)
        if a == b:
            continue
        if len(a) != len(b):
            return False
        diff = set(a) ^ set(b)
        order = sorted(cands, key=lambda j: (slot_score[j], slot_pos[j]))
        e = len(a)
        boundary = 0.5 * (slot_score[order[e - 1]] + slot_score[order[e]]) if e < len(order) else None
        if boundary is None or any(abs(slot_score[j] - boundary) > EPS_S for j in diff):
            return False
    return True


def state_after_classify(cache: hk.HkvCache, streams: Sequence[int]) -> dict:
    """The recorded streams' classification results and initial layout."""
    idx = torch.tensor(list(streams), dtype=torch.long, device=cache.label.device)
    sl = list(streams)
    cnt0 = cache.count[idx].cpu().numpy()
    base0 = cache.base.cpu().numpy()
    return dict(streams=sl, labels=cache.label[idx].cpu().numpy(),
                n_tokens=cache.n_tokens[idx].cpu().numpy(),
                budget=cache.budget[idx].cpu().numpy(), cap=cache.cap[idx].cpu().numpy(),
                count0=cnt0, tables0=_tables(cache, sl, cnt0),
                scores0=[cache.score[int(base0[s]):int(base0[s]) + int(c)].cpu().numpy()
                         for s, c in zip(sl, cnt0)])


def state_final(cache: hk.HkvCache, streams: Sequence[int]) -> dict:
    """The recorded streams' layout and scores after the last step."""
    idx = torch.tensor(list(streams), dtype=torch.long, device=cache.label.device)
    sl = list(streams)
    cntf = cache.count[idx].cpu().numpy()
    base = cache.base.cpu().numpy()
    return dict(count_final=cntf, tables_final=_tables(cache, sl, cntf),
                scores_final=[cache.score[int(base[s]):int(base[s]) + int(c)].cpu().numpy()
                              for s, c in zip(sl, cntf)])


def oracle_check_group(w: HkvConfig, seed: int, l: int, b: int, g: GpuRecord,
                       steps: Optional[int] = None, rep: Optional[Report] = None,
                       arrays=None) -> Report:
    """Replays group (l, b) on the oracle against the GPU record g.  `arrays`
    (K, V, Q as float64 [H, N, d], [H, N, d], [H, N-P+W, d]) replaces the
    seeded inputs, e.g. with the rows a model produced during decoding."""
    rep = rep or Report()
    H, P, W, D, N = w.heads, w.P, w.w_obs, w.split_dist, w.N
    if getattr(w, "unstratified", False):       # one subset holds every candidate
        D = 10 ** 9
    T = w.steps if steps is None else steps
    if arrays is None:
        kb, vb, qb = gen.group_inputs(w, seed, l, b)
        K, Vv, Q = gen.decode(kb, w.dtype), gen.decode(vb, w.dtype), gen.decode(qb, w.dtype)
    else:
        K, Vv, Q = arrays
    col = {s: i for i, s in enumerate(g.streams)}
    gi = [col[w.stream(l, b, h)] for h in range(H)]

    # classification: compare counts and labels, adopt flagged GPU labels
    override: Dict[int, int] = {}
    if not w.full_cache:
        for h in range(H):
            p = O.probs(Q[h, W - 1], K[h, :P])
            n_or = O.classify_count(p, w.tau)
            n_gpu = int(g.n_tokens[gi[h]])
            lab_gpu = int(g.labels[gi[h]])
            if n_or != n_gpu:
                if _count_flag(p, n_gpu, w.tau):
                    rep.flagged_counts += 1
                else:
                    rep.fail(f"l{l} b{b} h{h}: count oracle {n_or} gpu {n_gpu}")
            if O.label_of(n_or, w.local_window) != lab_gpu:
                if abs(n_or - w.local_window) <= 1 or _count_flag(p, n_gpu, w.tau):
                    rep.flagged_labels += 1
                else:
                    rep.fail(f"l{l} b{b} h{h}: label oracle {n_or} gpu {lab_gpu}")
                override[h] = lab_gpu
    else:
        for h in range(H):
            if int(g.labels[gi[h]]) != O.FULL:
                rep.fail(f"h{h}: full-cache label {g.labels[gi[h]]}")

    def lockstep(h, t, slot_pos, slot_score, gpu):
        """The GPU's own scores at this event: each within EPS_S of the oracle's,
        and the oracle's selection run on them gives the GPU's evicted set."""
        c = gi[h]
        if t == P - 1:                  # kept positions, in the order of the table
            got = np.asarray(g.scores0[c], dtype=np.float64)
            want = np.asarray([slot_score[p] for p in g.tables0[c]])
        else:
            if g.score_trace is None:
                return
            o = g.score_off[c]
            got = g.score_trace[t - P, o:o + len(slot_pos)].astype(np.float64)
            want = np.asarray(slot_score, dtype=np.float64)
            again = O.ste_select(slot_pos, got, t, W, D, len(gpu))
            if again != gpu:
                rep.fail(f"l{l} b{b} h{h} t{t}: selection on the GPU's scores "
                         f"{[slot_pos[j] for j in again]} != its evicted set "
                         f"{[slot_pos[j] for j in gpu]}")
        err = float(np.max(np.abs(got - want))) if got.size else 0.0
        rep.max_score_err = max(rep.max_score_err, err)
        if err > EPS_S:
            rep.fail(f"l{l} b{b} h{h} t{t}: GPU scores differ by {err:.3g}")
        rep.lockstep_events += 1

    def hook(h, t, slot_pos, slot_score, own):
        if t == P - 1:
            kept = set(g.tables0[gi[h]])
            gpu_pos = set(range(P)) - kept
        else:
            row = g.logs[t - P, gi[h]]
            gpu_pos = {int(x) for x in row if x >= 0}
        gpu = sorted(j for j in range(len(slot_pos)) if slot_pos[j] in gpu_pos)
        lockstep(h, t, slot_pos, slot_score, gpu)
        rep.events_checked += 1
        if gpu == own:
            return None
        if len(gpu) == len(own) and _evict_flag(slot_pos, slot_score, t, W, D, own, gpu):
            rep.flagged_evictions += 1
        else:
            rep.fail(f"l{l} b{b} h{h} t{t}: evicted oracle {[slot_pos[j] for j in own]} "
                     f"gpu {sorted(gpu_pos)}")
        return gpu

    rec = O.run_group(w, K, Vv, Q, label_override=override, evict_hook=hook, steps=T)

    for h in range(H):
        c = gi[h]
        lab = rec.labels[h]
        if lab == O.GLOBAL and int(g.budget[c]) != rec.budget:
            rep.fail(f"l{l} b{b} h{h}: budget oracle {rec.budget} gpu {g.budget[c]}")
        if int(g.cap[c]) != rec.caps[h]:
            rep.fail(f"l{l} b{b} h{h}: cap oracle {rec.caps[h]} gpu {g.cap[c]}")
        t0 = [p for p in rec.tables_after_classify[h]]
        if lab == O.LOCAL:
            t0 = t0[:int(g.count0[c])]
        if t0 != g.tables0[c]:
            rep.fail(f"l{l} b{b} h{h}: layout after classification differs")
        tf = rec.tables_final[h]
        if lab == O.LOCAL:
            tf = [p for p in tf[:int(g.count_final[c])]]
        if tf != g.tables_final[c]:
            rep.fail(f"l{l} b{b} h{h}: final layout differs")
        # scores written at the stream's last eviction (every ranked slot, the
        # evicted ones included; slots refilled after it were reset to 0 by their
        # append)
        evs = [ev for ev in rec.events if ev.head == h]
        if evs and lab == O.GLOBAL:
            ev = evs[-1]
            want = [0.0 if (j in ev.evicted_slots and rec.tables_final[h][j] >= 0) else x
                    for j, x in enumerate(ev.slot_score)]
            got_sc = np.asarray(g.scores_final[c][:len(want)], dtype=np.float64)
            err = float(np.max(np.abs(got_sc - np.asarray(want)))) if len(want) else 0.0
            rep.max_score_err = max(rep.max_score_err, err)
            if err > EPS_S:
                rep.fail(f"l{l} b{b} h{h}: scores at the last eviction differ by {err:.3g}")
        ref = rec.outputs[h]
        got = g.outs[:T, c]
        if g.no_output:
            keep = np.setdiff1d(np.arange(T), g.no_output)
            ref, got = ref[keep], got[keep]
        if w.dtype == "bf16":
            err = np.abs(got - ref)
            bad = err > BF16_ATOL
            rep.max_out_err = max(rep.max_out_err, float(err.max()))
            if bad.any():
                st = int(np.nonzero(bad.any(axis=1))[0][0])
                rep.fail(f"l{l} b{b} h{h}: output step {st} err {err[st].max():.3g}")
        else:
            scale = np.abs(ref).max(axis=1)
            err = np.abs(got - ref).max(axis=1) / np.maximum(scale, 1e-30)
            rep.max_out_err = max(rep.max_out_err, float(err.max()))
            if (err > F32_RTOL).any():
                st = int(np.argmax(err))
                rep.fail(f"l{l} b{b} h{h}: output step {st} rel err {err[st]:.3g}")
        rep.outputs_checked += len(ref)
    return rep
