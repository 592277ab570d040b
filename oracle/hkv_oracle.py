"""CPU oracle for the HeadKV decode-time path — TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  The product (the native library and its binding) never calls it,
and it shares no code with that product: it imports numpy and the Python
standard library and nothing else.  Its callers hand it inputs decoded from the
seeded input module ``hkv_inputs``, which holds no method arithmetic.

Everything is plain float64 numpy, one stream and one step at a time, following
the method's steps in the order the pages give them.  Citations name the pages
("Head-Aware Key-Value Compression for Efficient Autoregressive Image
Generation", the gist.science technical summaries; all five language versions
carry the same text) by section:

  [Method/1]  Methodology, step 1: cache prefilling without compression.
  [Method/2]  Methodology, step 2: head grouping.  Attention is accumulated
              backward from the current position until it reaches tau = 0.9; a
              head needing fewer tokens than the local window is Local, else
              Global; done once and reused for the whole decode.
  [Method/3L] Methodology, step 3, Local heads: sliding window of the most recent
              tokens, history dropped.
  [Method/3G] Methodology, step 3, Global heads: Stratified Token Eviction (STE):
              candidates split by distance into disjoint near and far subsets,
              each scored independently from past queries, the lowest-scoring
              tokens evicted from each (for example M/2 and M/2).
  [Contrib/2] Key contributions, item 2: asymmetric budgets, compact for Local
              heads and larger for Global heads.
  [Contrib/3] Key contributions, item 3: splitting by distance keeps informative
              distant tokens that a single importance ranking tends to drop in
              favour of local ones.
  [Problem]   Problem definition: LineAR assigns one fixed, uniform budget to
              every attention head (the allocation the uniform-budget ablation
              reproduces).
  [Lay]       The lay explainer's statement that the cache keeps 1/4, 1/6 or 1/8
              of the original memory (the compression ratio rho).

Where the pages leave a step open, the reading used here is stated at the
function.  The readings are the project's, not the pages'.

Parity-pinned by tests/test_oracle_pins.py (closed forms, invariants, textbook
special cases, brute force, hand-worked golden examples).  The following are
spec choices the pages do not fix and are therefore "parity unpinned" as to
their definition (only their internal consistency is pinned): the score formula
(sum of the last W softmax probabilities), M = W, the Global budget split, the
protected zone of the W newest tokens, the (score, position) tie-break and the
slot layout (evicted slots are freed and refilled by the next tokens).  The two
ablation variants (eviction without the near/far split; one budget for every
head) are this project's readings of the comparisons the pages draw, pinned the
same way.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Callable, Dict, List, Optional

import numpy as np

LOCAL, GLOBAL, FULL = 0, 1, 2


# --------------------------------------------------------------------------
# Attention [Method/2], [Method/3*]: one query against a set of cached tokens.
# Reading: single-query softmax attention with logits q.k / sqrt(d), one KV head
# per query head.
# --------------------------------------------------------------------------
def softmax(s: np.ndarray) -> np.ndarray:
    e = np.exp(s - s.max())
    return e / e.sum()


def probs(q: np.ndarray, K: np.ndarray) -> np.ndarray:
    """softmax_j(q.k_j / sqrt(d)) over the rows of K."""
    return softmax(K @ q / math.sqrt(q.shape[-1]))


def attend(q: np.ndarray, K: np.ndarray, V: np.ndarray):
    """o = sum_j softmax_j(q.k_j / sqrt(d)) v_j; returns (o, p)."""
    p = probs(q, K)
    return p @ V, p


# --------------------------------------------------------------------------
# Classification [Method/2]
# --------------------------------------------------------------------------
def classify_count(p_by_pos: np.ndarray, tau: float) -> int:
    """Tokens needed when the attention of the current query is accumulated
    backward from the current (last) position until the sum reaches tau.

    Reading: 'reaches' means >= tau; the count is at least 1; if rounding keeps
    the total below tau the count is the whole span.
    """
    cum = np.cumsum(p_by_pos[::-1])          # cum[k-1] = mass of the k newest
    hit = np.nonzero(cum >= tau)[0]
    return int(hit[0]) + 1 if hit.size else int(p_by_pos.size)


def label_of(n: int, window: int) -> int:
    """Local iff the count is smaller than the local window [Method/2]."""
    return LOCAL if n < window else GLOBAL


def global_budget(heads: int, per_head: int, window: int, n_local: int) -> Optional[int]:
    """Per (sequence, layer): Local heads keep `window` tokens; Global heads share
    the rest of heads * per_head equally, floor [Contrib/2], [Lay].

    per_head = floor(rho * N) with N the final length.  None if no Global head.
    """
    n_global = heads - n_local
    if n_global == 0:
        return None
    return (heads * per_head - n_local * window) // n_global


# --------------------------------------------------------------------------
# Stratified Token Eviction [Method/3G]
# --------------------------------------------------------------------------
def ste_select(slot_pos, slot_score, t: int, w_obs: int, split: int, n_evict: int) -> List[int]:
    """Slots to evict, ascending.

    Readings: candidates are slots whose distance t - pos is at least w_obs (the
    w_obs newest tokens are protected: their scores cover fewer queries); near
    subset: w_obs <= distance < split; far subset: distance >= split.  Quotas
    floor(E/2) near and E - floor(E/2) far; a subset with fewer candidates than
    its quota gives all of them and the other subset supplies the rest.  Within
    a subset the lowest (score, position) pairs go first.
    """
    cand = [j for j in range(len(slot_pos)) if t - slot_pos[j] >= w_obs]
    near = [j for j in cand if t - slot_pos[j] < split]
    far = [j for j in cand if t - slot_pos[j] >= split]
    q_near = n_evict // 2
    q_far = n_evict - q_near
    if len(near) < q_near:
        q_near, q_far = len(near), n_evict - len(near)
    elif len(far) < q_far:
        q_near, q_far = n_evict - len(far), len(far)
    if q_near > len(near) or q_far > len(far):
        raise ValueError("fewer eviction candidates than evictions")
    order = lambda j: (float(slot_score[j]), int(slot_pos[j]))
    chosen = sorted(near, key=order)[:q_near] + sorted(far, key=order)[:q_far]
    return sorted(chosen)


def unstratified_select(slot_pos, slot_score, t: int, w_obs: int, n_evict: int) -> List[int]:
    """Ablation without the near/far split [Contrib/3]: the n_evict lowest
    (score, position) candidates over all candidates, ascending slots.  Same
    protected zone as ste_select (distance < w_obs is not a candidate)."""
    cand = [j for j in range(len(slot_pos)) if t - slot_pos[j] >= w_obs]
    if len(cand) < n_evict:
        raise ValueError("fewer eviction candidates than evictions")
    order = lambda j: (float(slot_score[j]), int(slot_pos[j]))
    return sorted(sorted(cand, key=order)[:n_evict])


def free_evicted(slot_pos, slot_score, evicted: List[int]):
    """Slot layout after an eviction (reading; the pages fix no layout): the
    evicted slots become free (position -1, score 0); no other slot moves.
    Returns the new table, the new scores and the free slots, ascending."""
    pos = list(slot_pos)
    sc = list(slot_score)
    for j in evicted:
        pos[j] = -1
        sc[j] = 0.0
    return pos, sc, sorted(evicted)


def append_slot(table: List[int], free: List[int]) -> int:
    """Slot receiving the next token of a Global stream (reading): the lowest
    free slot if any, else a new slot at the end of the table."""
    if free:
        return free.pop(0)
    table.append(-1)
    return len(table) - 1


def scoring_window_starts(count: int, budget: int, n_evict: int, w_obs: int) -> bool:
    """True at the step whose query is the first of the w_obs queries that score
    the next eviction: that step writes the probabilities instead of adding
    them, so that at the eviction every score sums exactly w_obs queries."""
    return count == budget + n_evict - w_obs + 1


def window_scores(Qwin: np.ndarray, K: np.ndarray, first_pos: int) -> np.ndarray:
    """Importance of every prefill position from the w_obs last prefill queries:
    query at position i (i = first_pos .. first_pos + W - 1) attends causally to
    positions 0..i; the score of position j is the sum of the probabilities it
    receives (reading of 'scored from past query features', [Method/3G], applied
    when the cache reaches its predefined length, [Method/2])."""
    P = first_pos + Qwin.shape[0]
    score = np.zeros(P)
    for r, q in enumerate(Qwin):
        i = first_pos + r
        score[: i + 1] += probs(q, K[: i + 1])
    return score


# --------------------------------------------------------------------------
# One (sequence, layer) group end to end
# --------------------------------------------------------------------------
@dataclass
class Event:
    head: int
    t: int
    slot_pos: List[int]          # table before the eviction
    slot_score: List[float]      # scores before the eviction (float64)
    evicted_slots: List[int]     # what was applied
    oracle_slots: List[int]      # the oracle's own choice on its own scores
    budget: int


@dataclass
class GroupRecord:
    n_tokens: List[int] = field(default_factory=list)
    labels: List[int] = field(default_factory=list)
    budget: Optional[int] = None            # Global budget of the group
    caps: List[int] = field(default_factory=list)
    tables_after_classify: List[List[int]] = field(default_factory=list)
    tables_final: List[List[int]] = field(default_factory=list)
    init_events: List[Event] = field(default_factory=list)
    events: List[Event] = field(default_factory=list)
    outputs: Optional[np.ndarray] = None    # [H, steps, d]
    last_probs: List[np.ndarray] = field(default_factory=list)  # classify query


def run_group(cfg, K: np.ndarray, V: np.ndarray, Q: np.ndarray,
              label_override: Optional[Dict[int, int]] = None,
              evict_hook: Optional[Callable] = None,
              steps: Optional[int] = None) -> GroupRecord:
    """Run classification and every decode step for the H streams of one group.

    K, V: [H, N, d] float64; Q: [H, N - P + W, d] float64, row r holds the query
    of position P - W + r.  `label_override` maps head -> label to adopt;
    `evict_hook(head, t, slot_pos, slot_score, oracle_slots)` may return the
    slots to apply instead of the oracle's own choice.  `steps` limits the
    decode to the first `steps` positions after prefill.
    """
    H, N, d = K.shape
    P, W, M, w = cfg.P, cfg.w_obs, cfg.evict_m, cfg.local_window
    D, tau = cfg.split_dist, cfg.tau
    num, den = cfg.rho
    per_head = (N * num) // den
    # ablation variants: eviction without the near/far split [Contrib/3]; the
    # same budget per_head for every head (the uniform allocation the pages
    # attribute to LineAR, Problem definition) instead of [Contrib/2]
    unstratified = getattr(cfg, "unstratified", False)
    uniform = getattr(cfg, "uniform_budget", False)
    ring = per_head if uniform else w          # Local window kept
    if unstratified:
        select = lambda table, sc, t, E: unstratified_select(table, sc, t, W, E)
    else:
        select = lambda table, sc, t, E: ste_select(table, sc, t, W, D, E)
    T = N - P if steps is None else steps
    rec = GroupRecord()
    q_at = lambda h, t: Q[h, t - (P - W)]

    # ---- [Method/1] prefill, [Method/2] classification ----
    if cfg.full_cache:
        labels = [FULL] * H
        rec.n_tokens = [0] * H
    else:
        labels = []
        for h in range(H):
            p = probs(q_at(h, P - 1), K[h, :P])
            n = classify_count(p, tau)
            rec.n_tokens.append(n)
            rec.last_probs.append(p)
            labels.append(label_of(n, w))
        if label_override:
            for h, lab in label_override.items():
                labels[h] = lab
    rec.labels = list(labels)
    n_local = sum(1 for x in labels if x == LOCAL)
    if cfg.full_cache:
        B = None
    elif uniform:
        B = per_head if n_local < H else None
    else:
        B = global_budget(H, per_head, w, n_local)
    rec.budget = B

    # ---- initial per-head layout ----
    tables, scores = [], []
    for h in range(H):
        if labels[h] == FULL:
            tables.append(list(range(P)))
            scores.append([0.0] * P)
            rec.caps.append(N)
        elif labels[h] == LOCAL:
            slots = [-1] * ring
            for pos in range(max(0, P - ring), P):
                slots[pos % ring] = pos
            tables.append(slots)
            scores.append([0.0] * ring)
            rec.caps.append(ring)
        else:
            rec.caps.append(B + M)
            sc = window_scores(Q[h, :W], K[h], P - W)
            if P <= B:
                tables.append(list(range(P)))
                scores.append(list(sc))
            else:
                table = list(range(P))
                own = select(table, sc, P - 1, P - B)
                use = own
                if evict_hook is not None:
                    alt = evict_hook(h, P - 1, table, list(sc), own)
                    if alt is not None:
                        use = sorted(alt)
                rec.init_events.append(Event(h, P - 1, table, list(sc), use, own, B))
                drop = set(use)
                keep = [j for j in range(P) if j not in drop]   # ascending positions
                tables.append(keep)
                scores.append([float(sc[j]) for j in keep])
    rec.tables_after_classify = [list(t) for t in tables]

    # ---- decode steps [Method/3L], [Method/3G] ----
    free: List[List[int]] = [[] for _ in range(H)]
    out = np.zeros((H, T, d))
    for step in range(T):
        t = P + step
        for h in range(H):
            q = q_at(h, t)
            lab = labels[h]
            if lab == LOCAL:
                tables[h][t % ring] = t
            elif lab == FULL:
                tables[h].append(t)
            else:
                j = append_slot(tables[h], free[h])
                if j == len(scores[h]):
                    scores[h].append(0.0)
                tables[h][j] = t
                scores[h][j] = 0.0
            live = [j for j, pos in enumerate(tables[h]) if pos >= 0]
            pos_arr = np.array([tables[h][j] for j in live], dtype=np.int64)
            o, p = attend(q, K[h, pos_arr], V[h, pos_arr])
            out[h, step] = o
            if lab != GLOBAL:
                continue
            c = len(live)
            if scoring_window_starts(c, B, M, W):
                for j in live:
                    scores[h][j] = 0.0
            for j, pj in zip(live, p):
                scores[h][j] = float(scores[h][j]) + float(pj)
            if c == B + M:
                own = select(tables[h], scores[h], t, M)
                use = own
                if evict_hook is not None:
                    alt = evict_hook(h, t, list(tables[h]), list(scores[h]), own)
                    if alt is not None:
                        use = sorted(alt)
                rec.events.append(Event(h, t, list(tables[h]), list(scores[h]), use, own, B))
                tables[h], scores[h], free[h] = free_evicted(tables[h], scores[h], use)
    rec.outputs = out
    rec.tables_final = [list(t) for t in tables]
    return rec


def full_attention_outputs(K: np.ndarray, V: np.ndarray, Q: np.ndarray, P: int, W: int,
                           steps: int) -> np.ndarray:
    """Uncompressed causal decode attention: query t attends to positions 0..t."""
    H, N, d = K.shape
    out = np.zeros((H, steps, d))
    for h in range(H):
        for step in range(steps):
            t = P + step
            out[h, step], _ = attend(Q[h, t - (P - W)], K[h, : t + 1], V[h, : t + 1])
    return out
