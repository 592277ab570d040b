"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each `check_*` takes the oracle module so that tests/test_oracle_mutations.py can
plant a mistake in it and show that some check catches it.
"""
from __future__ import annotations

import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
from scipy.optimize import brentq

import oracle.hkv_oracle as O
from hkv_inputs.configs import TINY, WORKLOADS
from tests._fixtures import group_f64, read_kv, read_rows, read_sections, small_config


# ---------------------------------------------------------------- P1
def check_uniform_count(orc, Ls=range(1, 700)):
    """q = 0 gives uniform attention 1/L, so the count is ceil(0.9 L)
    (exact in fp64 whenever 0.9 L is not an integer)."""
    for L in Ls:
        if L % 10 == 0:
            continue
        p = orc.probs(np.zeros(16), np.random.default_rng(L).normal(size=(L, 16)))
        assert orc.classify_count(p, 0.9) == -(-9 * L // 10), L


# ---------------------------------------------------------------- P2
def geometric_keys(L: int, d: int, r: float):
    """Keys whose logit against q = sqrt(d) e0 is (distance from the newest) * ln r."""
    K = np.zeros((L, d))
    K[:, 0] = (L - 1 - np.arange(L)) * math.log(r)
    q = np.zeros(d)
    q[0] = math.sqrt(d)
    return q, K


def check_geometric_count(orc, L=64, d=64, w=16, tau=0.9):
    """p_delta ~ r**delta: count = ceil(ln(1 - tau (1 - r**L)) / ln r).  r is
    chosen so that the real-valued count sits mid-way between integers at
    w-2 .. w+1, so the strict 'fewer than the window' rule is tested exactly."""
    f = lambda r, target: math.log(1 - tau * (1 - r ** L)) / math.log(r) - target
    for n in (w - 2, w - 1, w, w + 1):
        r = brentq(f, 1e-6, 1 - 1e-9, args=(n - 0.5,))
        q, K = geometric_keys(L, d, r)
        got = orc.classify_count(orc.probs(q, K), tau)
        assert got == n, (n, got)
        assert orc.label_of(got, w) == (orc.LOCAL if n < w else orc.GLOBAL)


# ---------------------------------------------------------------- P3 (golden)
def check_classify_golden(orc):
    for name, probs, n, w, lab in read_rows("classify_worked_examples.txt"):
        p = np.array([float(x) for x in probs.split()])
        got = orc.classify_count(p, 0.9)
        assert got == int(n), name
        want = orc.LOCAL if lab == "local" else orc.GLOBAL
        assert orc.label_of(got, int(w)) == want, name


def check_classify_exact_rational(orc, trials=300):
    """Random rational distributions: the count from exact Fraction arithmetic
    (skipping draws whose cumulative mass lies within 1e-9 of tau)."""
    rng = np.random.default_rng(7)
    tau = Fraction(9, 10)
    done = 0
    for _ in range(trials):
        L = int(rng.integers(1, 30))
        ints = rng.integers(1, 50, size=L)
        tot = int(ints.sum())
        cum, n_exact, near = Fraction(0), L, False
        for k in range(1, L + 1):
            cum += Fraction(int(ints[L - k]), tot)
            if abs(float(cum - tau)) < 1e-9:
                near = True
            if cum >= tau:
                n_exact = k
                break
        if near:
            continue
        # logits ln(p) reproduce p through the softmax up to rounding
        d = 4
        K = np.zeros((L, d))
        K[:, 0] = np.log(ints / tot)
        q = np.zeros(d)
        q[0] = math.sqrt(d)
        assert orc.classify_count(orc.probs(q, K), 0.9) == n_exact
        done += 1
    assert done > trials // 2


# ---------------------------------------------------------------- P4
def check_attention_textbook(orc):
    """Attention equals torch's scaled-dot-product attention in float64."""
    import torch
    rng = np.random.default_rng(3)
    for n, d in ((1, 64), (7, 64), (130, 128), (513, 128)):
        q = rng.normal(size=d)
        K = rng.normal(size=(n, d))
        V = rng.normal(size=(n, d))
        o, p = orc.attend(q, K, V)
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.tensor(q)[None, None, None, :], torch.tensor(K)[None, None],
            torch.tensor(V)[None, None])[0, 0, 0].numpy()
        assert np.max(np.abs(o - ref)) < 1e-12
        assert abs(p.sum() - 1.0) < 1e-12


def check_rho_one_is_full(orc):
    """With rho = 1 the Global budget exceeds the sequence, nothing is evicted
    and every Global head equals full attention bit for bit."""
    cfg = small_config(rho=(1, 1))
    K, V, Q = group_f64(cfg)
    rec = orc.run_group(cfg, K, V, Q)
    full = orc.full_attention_outputs(K, V, Q, cfg.P, cfg.w_obs, cfg.steps)
    glob = [h for h in range(cfg.heads) if rec.labels[h] == orc.GLOBAL]
    assert glob and not rec.events and not rec.init_events
    for h in glob:
        assert np.array_equal(rec.outputs[h], full[h])


# ---------------------------------------------------------------- P5
def check_local_window(orc):
    """A Local head whose window covers the whole sequence equals full
    attention bit for bit; a short window holds exactly the newest w positions."""
    cfg = small_config()
    K, V, Q = group_f64(cfg)
    wide = cfg.with_(local_window=cfg.N)
    rec = orc.run_group(wide, K, V, Q, label_override={h: orc.LOCAL for h in range(cfg.heads)})
    full = orc.full_attention_outputs(K, V, Q, cfg.P, cfg.w_obs, cfg.steps)
    assert np.array_equal(rec.outputs, full)
    rec = orc.run_group(cfg, K, V, Q, label_override={h: orc.LOCAL for h in range(cfg.heads)},
                        steps=37)
    w = cfg.local_window
    t_last = cfg.P + 36
    for h in range(cfg.heads):
        assert sorted(rec.tables_after_classify[h]) == list(range(cfg.P - w, cfg.P))
        assert sorted(rec.tables_final[h]) == list(range(t_last - w + 1, t_last + 1))
        # ring layout: position p sits in slot p mod w
        assert all(p % w == j for j, p in enumerate(rec.tables_final[h]))


# ---------------------------------------------------------------- P6, P8, P9, P11
def check_budget(orc, cfg, rec):
    H, w, M = cfg.heads, cfg.local_window, cfg.evict_m
    A = (cfg.N * cfg.rho[0]) // cfg.rho[1]
    n_l = sum(1 for x in rec.labels if x == orc.LOCAL)
    n_g = H - n_l
    if n_g == 0:
        return
    kept = n_l * w + n_g * rec.budget
    assert H * A - n_g < kept <= H * A          # floor leaves fewer than n_G slots
    assert rec.budget >= A >= w
    assert sum(rec.caps) <= H * (A + M)


def check_ste_events(orc, cfg, rec):
    W, M, D = cfg.w_obs, cfg.evict_m, cfg.split_dist
    for ev in rec.events:
        t, pos = ev.t, ev.slot_pos
        assert len(pos) == ev.budget + M
        assert len(ev.evicted_slots) == M
        dist = [t - pos[j] for j in ev.evicted_slots]
        assert min(dist) >= W                   # protected zone
        n_near = sum(1 for x in dist if x < D)
        near_c = sum(1 for p in pos if W <= t - p < D)
        far_c = sum(1 for p in pos if t - p >= D)
        if near_c >= M // 2 and far_c >= M - M // 2:
            assert n_near == M // 2
        assert -1 not in pos                    # no free slot at an eviction
    # layout: the M tokens after an eviction fill its freed slots, ascending
    by_head = {}
    for ev in rec.events:
        by_head.setdefault(ev.head, []).append(ev)
    for evs in by_head.values():
        for a, b in zip(evs, evs[1:]):
            assert b.t == a.t + M
            assert [b.slot_pos[j] for j in sorted(a.evicted_slots)] == \
                list(range(a.t + 1, a.t + M + 1))


def check_score_sum(orc, cfg, rec):
    """Each of the W window queries spreads probability 1 over slots that are
    all still present, so the scores sum to W."""
    W = cfg.w_obs
    assert rec.events
    for ev in rec.events:
        s = np.array(ev.slot_score)
        assert abs(s.sum() - W) < 1e-12
        assert s.min() >= 0 and s.max() <= W


def check_score_recompute(orc, cfg, rec, K, Q):
    """The accumulated score equals the W x count causal scoring tile recomputed
    at the eviction step from the queries and keys themselves."""
    W, P = cfg.w_obs, cfg.P
    for ev in rec.events[:40]:
        pos = np.array(ev.slot_pos)
        want = np.zeros(len(pos))
        for i in range(ev.t - W + 1, ev.t + 1):
            present = pos <= i
            q = Q[ev.head, i - (P - W)]
            logits = K[ev.head, pos[present]] @ q / math.sqrt(q.size)
            e = np.exp(logits - logits.max())
            want[present] += e / e.sum()
        assert np.max(np.abs(want - np.array(ev.slot_score))) < 1e-12


def check_layout(orc, cfg, rec):
    """Global tables always hold every position not yet evicted, once."""
    for h in range(cfg.heads):
        if rec.labels[h] != orc.GLOBAL:
            continue
        gone = set()
        for ev in rec.init_events + rec.events:
            if ev.head == h:
                gone |= {ev.slot_pos[j] for j in ev.evicted_slots}
        final = [p for p in rec.tables_final[h] if p >= 0]
        assert len(set(final)) == len(final)
        assert set(final) == set(range(cfg.N)) - gone


def run_small(orc, steps=None, **kw):
    cfg = small_config(**kw)
    K, V, Q = group_f64(cfg)
    return cfg, orc.run_group(cfg, K, V, Q, steps=steps), K, Q


def check_group_invariants(orc):
    for kw in ({}, dict(rho=(1, 6), split_dist=20), dict(heads=4, p_local=0.0)):
        cfg, rec, K, Q = run_small(orc, **kw)
        check_budget(orc, cfg, rec)
        check_ste_events(orc, cfg, rec)
        check_score_sum(orc, cfg, rec)
        check_score_recompute(orc, cfg, rec, K, Q)
        check_layout(orc, cfg, rec)


# ---------------------------------------------------------------- P7 (golden + brute force)
def check_ste_golden(orc):
    for name, ex in read_sections("ste_worked_examples.txt").items():
        pos = [int(x) for x in ex["pos"].split()]
        score = [float(x) for x in ex["score"].split()]
        t, W, D, E, keep = (int(ex[k]) for k in ("t", "w_obs", "split", "evict", "keep"))
        ev = orc.ste_select(pos, score, t, W, D, E)
        assert sorted(pos[j] for j in ev) == [int(x) for x in ex["evicted_pos"].split()], name
        want_after = [int(x) for x in ex["table_after"].split()]
        if ex["mode"] == "decode":        # evicted slots freed, refilled ascending
            after, sc_after, free = orc.free_evicted(pos, score, ev)
            assert after == want_after, name
            assert all(sc_after[j] == 0.0 for j in ev)
            table = list(after)
            slots = [orc.append_slot(table, free) for _ in range(E)]
            assert slots == [int(x) for x in ex["refill"].split()], name
            assert orc.append_slot(table, free) == len(pos), name    # then the table grows
        else:                               # classification time: order-preserving
            after = [pos[j] for j in range(len(pos)) if j not in set(ev)]
            assert after == want_after, name


def check_ste_bruteforce(orc, trials=200):
    """Within each subset the evicted set is the lexicographically smallest
    k-subset of (score, position) keys; enumerated exhaustively."""
    rng = np.random.default_rng(11)
    for _ in range(trials):
        n = int(rng.integers(16, 29))
        t = 100
        W = 8
        D = int(rng.integers(W + 1, 30))
        pos = sorted(rng.choice(np.arange(0, t + 1 - W), size=n - W, replace=False).tolist())
        pos += list(range(t - W + 1, t + 1))
        score = rng.integers(0, 6, size=n).astype(float) / 8.0   # many ties
        E = 8
        ev = orc.ste_select(pos, score, t, W, D, E)
        near = [j for j in range(n) if W <= t - pos[j] < D]
        far = [j for j in range(n) if t - pos[j] >= D]
        got_near = [j for j in ev if j in near]
        got_far = [j for j in ev if j in far]
        assert len(ev) == E and len(got_near) + len(got_far) == E
        key = lambda j: (score[j], pos[j])
        for sub, got in ((near, got_near), (far, got_far)):
            if len(sub) > 12:
                continue
            best = min(itertools.combinations(sub, len(got)),
                       key=lambda c: sorted(key(j) for j in c))
            assert sorted(best) == sorted(got)
        # quotas: 4 and 4 unless a subset is short
        if len(near) >= 4 and len(far) >= 4:
            assert len(got_near) == 4
        elif len(near) < 4:
            assert len(got_near) == len(near)
        else:
            assert len(got_far) == len(far)


# ---------------------------------------------------------------- P10
def check_uniform_scores(orc):
    """All queries zero: every candidate scores sum_i 1/count_i, so the
    tie-break evicts the oldest tokens of each subset."""
    cfg = small_config(heads=3, p_local=0.0)
    K, V, Q = group_f64(cfg)
    rec = orc.run_group(cfg, K, V, np.zeros_like(Q), steps=60)
    assert rec.events
    W, D = cfg.w_obs, cfg.split_dist
    for ev in rec.events:
        pos = ev.slot_pos
        counts = [sum(1 for p in pos if p <= i) for i in range(ev.t - W + 1, ev.t + 1)]
        closed = sum(1.0 / c for c in counts)
        cand = [j for j in range(len(pos)) if ev.t - pos[j] >= W]
        for j in cand:
            assert abs(ev.slot_score[j] - closed) < 1e-12
        near = sorted(pos[j] for j in cand if ev.t - pos[j] < D)
        far = sorted(pos[j] for j in cand if ev.t - pos[j] >= D)
        got = sorted(pos[j] for j in ev.evicted_slots)
        assert got == sorted(far[:4] + near[:4])


# ---------------------------------------------------------------- initial-eviction scores
def _fraction(x: str) -> Fraction:
    return Fraction(x)


def check_window_scores_uniform(orc):
    """All window queries zero: query i gives each of positions 0..i the
    probability 1/(i+1), so position j scores sum_{i=max(j, P-W)}^{P-1} 1/(i+1)
    (a closed form that fixes causality, the window's first position and the
    number of queries)."""
    rng = np.random.default_rng(31)
    for P, W, d in ((5, 3, 4), (12, 8, 64), (40, 8, 128), (9, 1, 8), (8, 8, 16)):
        K = rng.normal(size=(P, d))
        got = orc.window_scores(np.zeros((W, d)), K, P - W)
        want = [sum(1.0 / (i + 1) for i in range(max(j, P - W), P)) for j in range(P)]
        assert got.shape == (P,)
        assert np.max(np.abs(got - np.array(want))) < 1e-12, (P, W)


def _rational_window(ex):
    """Keys (ln u_j, 0, 0, 0) and queries (2 a_r, 0, 0, 0) of a worked example."""
    u = [int(x) for x in ex["u"].split()]
    a = [int(x) for x in ex["a"].split()]
    K = np.zeros((len(u), 4))
    K[:, 0] = np.log(np.array(u, dtype=np.float64))
    Q = np.zeros((len(a), 4))
    Q[:, 0] = 2.0 * np.array(a, dtype=np.float64)
    return K, Q


def check_window_scores_golden(orc):
    """Hand-worked initial-eviction scores with rational probabilities, and one
    whole classification + initial eviction of a one-head group."""
    for name, ex in read_sections("window_scores_worked.txt").items():
        P, W = int(ex["P"]), int(ex["W"])
        K, Q = _rational_window(ex)
        got = orc.window_scores(Q, K, P - W)
        want = [float(_fraction(x)) for x in ex["score"].split()]
        assert np.max(np.abs(got - np.array(want))) < 1e-12, name
        if "evicted_pos" not in ex:
            continue
        N = int(ex["N"])
        num, den = (int(x) for x in ex["rho"].split("/"))
        from hkv_inputs.configs import HkvConfig
        cfg = HkvConfig(name=name, cid=99, layers=1, batch=1, heads=1, head_dim=4, dtype="f32",
                        prefix=0, image_tokens=N, prefill_image=P,
                        local_window=int(ex["window"]), rho=(num, den),
                        split_dist=int(ex["split"]), w_obs=W, evict_m=W)
        Kg = np.zeros((1, N, 4))
        Kg[0, :P] = K
        Qg = np.zeros((1, N - P + W, 4))
        Qg[0, :W] = Q
        rec = orc.run_group(cfg, Kg, np.zeros_like(Kg), Qg, steps=0)
        assert rec.n_tokens == [int(ex["count"])], name
        assert rec.labels == [orc.GLOBAL], name
        assert rec.budget == (N * num) // den, name
        assert len(rec.init_events) == 1, name
        ev = rec.init_events[0]
        assert sorted(ev.slot_pos[j] for j in ev.evicted_slots) == \
            [int(x) for x in ex["evicted_pos"].split()], name
        assert rec.tables_after_classify[0] == [int(x) for x in ex["table_after"].split()], name


def check_init_score_sum(orc):
    """Every initial eviction's scores sum to W: each of the W window queries
    spreads probability 1 over positions that are all present at
    classification."""
    seen = 0
    for kw in ({}, dict(rho=(1, 6), split_dist=20), dict(head_dim=128, rho=(1, 8), heads=4)):
        cfg, rec, _, _ = run_small(orc, steps=0, **kw)
        for ev in rec.init_events:
            s = np.array(ev.slot_score)
            assert abs(s.sum() - cfg.w_obs) < 1e-12
            assert s.min() >= 0 and s.max() <= cfg.w_obs
            seen += 1
    assert seen > 0


def check_window_scores(orc):
    check_window_scores_uniform(orc)
    check_window_scores_golden(orc)
    check_init_score_sum(orc)


# ---------------------------------------------------------------- ablation variants
def check_unstratified_bruteforce(orc, trials=200):
    """Without the near/far split the evicted set is the lexicographically
    smallest E-subset of all candidates' (score, position) keys, enumerated
    exhaustively; it equals the stratified choice with an unreachable split
    (empty far subset, whose quota the shortfall rule hands to the near one)."""
    rng = np.random.default_rng(23)
    for _ in range(trials):
        n = int(rng.integers(16, 21))
        t, W = 100, 8
        pos = sorted(rng.choice(np.arange(0, t + 1 - W), size=n - W, replace=False).tolist())
        pos += list(range(t - W + 1, t + 1))
        score = rng.integers(0, 5, size=n).astype(float) / 8.0   # many ties
        E = int(rng.choice([2, 4, 6, 8]))
        ev = orc.unstratified_select(pos, score, t, W, E)
        cand = [j for j in range(n) if t - pos[j] >= W]
        best = min(itertools.combinations(cand, E),
                   key=lambda c: sorted((score[j], pos[j]) for j in c))
        assert ev == sorted(best)
        assert ev == orc.ste_select(pos, score, t, W, 10 ** 9, E)


def check_variant_groups(orc):
    """Group invariants of the ablation variants: the uniform variant keeps
    exactly floor(rho*N) tokens in every head (Local rings of that size,
    Global tables back at that budget after every eviction); the unstratified
    variant evicts M candidates per event regardless of distance; scores still
    sum to W and tables stay exact; and the variants do change decisions."""
    base = dict(rho=(1, 6), split_dist=20)
    cfg0, rec0, _, _ = run_small(orc, **base)
    for unstrat, uniform in ((True, False), (False, True), (True, True)):
        cfg, rec, K, Q = run_small(orc, unstratified=unstrat, uniform_budget=uniform, **base)
        H, M, W = cfg.heads, cfg.evict_m, cfg.w_obs
        A = (cfg.N * cfg.rho[0]) // cfg.rho[1]
        if uniform:
            assert rec.budget in (None, A)
            for h in range(H):
                want_cap = A if rec.labels[h] == orc.LOCAL else A + M
                assert rec.caps[h] == want_cap
                if rec.labels[h] == orc.LOCAL:
                    t_last = cfg.N - 1
                    assert sorted(rec.tables_final[h]) == list(range(t_last - A + 1, t_last + 1))
        for ev in rec.events:
            assert len(ev.slot_pos) == ev.budget + M
            assert len(ev.evicted_slots) == M
            assert min(ev.t - ev.slot_pos[j] for j in ev.evicted_slots) >= W
        check_score_sum(orc, cfg, rec)
        check_score_recompute(orc, cfg, rec, K, Q)
        check_layout(orc, cfg, rec)
        assert [e.evicted_slots for e in rec.events] != [e.evicted_slots for e in rec0.events]


# ---------------------------------------------------------------- tests
def test_uniform_count():
    check_uniform_count(O)


def test_geometric_count():
    check_geometric_count(O)
    check_geometric_count(O, L=192, d=128, w=98)


def test_classify_golden():
    check_classify_golden(O)


def test_classify_exact_rational():
    check_classify_exact_rational(O)


def test_attention_textbook():
    check_attention_textbook(O)


def test_rho_one_is_full():
    check_rho_one_is_full(O)


def test_local_window():
    check_local_window(O)


def test_group_invariants():
    check_group_invariants(O)


def test_ste_golden():
    check_ste_golden(O)


def test_ste_bruteforce():
    check_ste_bruteforce(O)


def test_uniform_scores():
    check_uniform_scores(O)


def test_tiny_workload_runs():
    """The tiny fp32 workload: invariants hold over all 192 decode steps."""
    K, V, Q = group_f64(TINY)
    rec = O.run_group(TINY, K, V, Q)
    assert rec.outputs.shape == (4, 192, 64)
    check_budget(O, TINY, rec)
    check_ste_events(O, TINY, rec)
    check_score_sum(O, TINY, rec)
    check_layout(O, TINY, rec)


def test_pages_parameters():
    """Workloads use the tau and rho values the pages state."""
    vals = read_kv("pages_parameters.txt")
    tau = float(vals["tau"])
    rhos = {tuple(int(x) for x in r.split("/")) for r in vals["rho"].split()}
    for c in WORKLOADS.values():
        assert c.tau == tau
        assert c.rho in rhos
        assert c.evict_m % 2 == 0


def test_unstratified_bruteforce():
    check_unstratified_bruteforce(O)


def test_variant_groups():
    check_variant_groups(O)


def test_window_scores_uniform():
    check_window_scores_uniform(O)


def test_window_scores_golden():
    check_window_scores_golden(O)


def test_init_score_sum():
    check_init_score_sum(O)
