"""Plant plausible mistakes in the oracle (on the CPU) and show a pin catches each.

Every mutant is a copy of one oracle function with one deliberate error; the
test asserts that at least one of the pins in tests/test_oracle_pins.py fails
against it.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle.hkv_oracle as O
from tests import test_oracle_pins as pins


def _label_le(n, window):                      # '<=' instead of '<'
    return O.LOCAL if n <= window else O.GLOBAL


def _count_forward(p, tau):                    # accumulates from the oldest token
    cum = np.cumsum(p)
    hit = np.nonzero(cum >= tau)[0]
    return int(hit[0]) + 1 if hit.size else int(p.size)


def _count_strict(p, tau):                     # '>' instead of '>=' and off by one
    cum = np.cumsum(p[::-1])
    hit = np.nonzero(cum > tau)[0]
    return int(hit[0]) if hit.size else int(p.size)


def _probs_no_scale(q, K):                     # dropped 1/sqrt(d)
    return O.softmax(K @ q)


def _select_unstratified(slot_pos, slot_score, t, w_obs, split, n_evict):
    cand = [j for j in range(len(slot_pos)) if t - slot_pos[j] >= w_obs]
    key = lambda j: (float(slot_score[j]), int(slot_pos[j]))
    return sorted(sorted(cand, key=key)[:n_evict])


def _select_protect_off_by_one(slot_pos, slot_score, t, w_obs, split, n_evict):
    return _ORIG_SELECT(slot_pos, slot_score, t, w_obs + 1, split, n_evict)


def _select_quota_swapped(slot_pos, slot_score, t, w_obs, split, n_evict):
    cand = [j for j in range(len(slot_pos)) if t - slot_pos[j] >= w_obs]
    near = [j for j in cand if t - slot_pos[j] < split]
    far = [j for j in cand if t - slot_pos[j] >= split]
    q_far = n_evict // 2
    q_near = n_evict - q_far
    if len(near) < q_near:
        q_near, q_far = len(near), n_evict - len(near)
    elif len(far) < q_far:
        q_near, q_far = n_evict - len(far), len(far)
    key = lambda j: (float(slot_score[j]), int(slot_pos[j]))
    return sorted(sorted(near, key=key)[:q_near] + sorted(far, key=key)[:q_far])


def _select_newest_first_on_ties(slot_pos, slot_score, t, w_obs, split, n_evict):
    neg = [-p for p in slot_pos]
    cand = [j for j in range(len(slot_pos)) if t - slot_pos[j] >= w_obs]
    near = [j for j in cand if t - slot_pos[j] < split]
    far = [j for j in cand if t - slot_pos[j] >= split]
    q_near = n_evict // 2
    q_far = n_evict - q_near
    if len(near) < q_near:
        q_near, q_far = len(near), n_evict - len(near)
    elif len(far) < q_far:
        q_near, q_far = n_evict - len(far), len(far)
    key = lambda j: (float(slot_score[j]), neg[j])
    return sorted(sorted(near, key=key)[:q_near] + sorted(far, key=key)[:q_far])


def _append_highest_free(table, free):          # refills freed slots in descending order
    if free:
        return free.pop()
    table.append(-1)
    return len(table) - 1


def _free_evicted_keep_scores(slot_pos, slot_score, evicted):   # evicted scores not cleared
    pos = list(slot_pos)
    for j in evicted:
        pos[j] = -1
    return pos, list(slot_score), sorted(evicted)


def _budget_uniform(heads, per_head, window, n_local):
    return None if heads == n_local else per_head


def _budget_ceil(heads, per_head, window, n_local):
    n_g = heads - n_local
    return None if n_g == 0 else -(-(heads * per_head - n_local * window) // n_g)


_ORIG_SELECT = O.ste_select


def _unstrat_no_protection(slot_pos, slot_score, t, w_obs, n_evict):   # newest tokens eligible
    order = lambda j: (float(slot_score[j]), int(slot_pos[j]))
    return sorted(sorted(range(len(slot_pos)), key=order)[:n_evict])


def _unstrat_highest(slot_pos, slot_score, t, w_obs, n_evict):         # keeps the lowest scores
    cand = [j for j in range(len(slot_pos)) if t - slot_pos[j] >= w_obs]
    order = lambda j: (-float(slot_score[j]), int(slot_pos[j]))
    return sorted(sorted(cand, key=order)[:n_evict])


def _window_noncausal(Qwin, K, first_pos):           # every query sees the whole prefill
    P = first_pos + Qwin.shape[0]
    score = np.zeros(P)
    for q in Qwin:
        score += O.probs(q, K[:P])
    return score


def _window_last_only(Qwin, K, first_pos):           # only the newest query scores
    P = first_pos + Qwin.shape[0]
    return O.probs(Qwin[-1], K[:P])


def _window_start_off_by_one(Qwin, K, first_pos):    # queries placed one position early
    P = first_pos + Qwin.shape[0]
    score = np.zeros(P)
    for r, q in enumerate(Qwin):
        i = first_pos + r - 1
        score[: i + 1] += O.probs(q, K[: i + 1])
    return score


MUTANTS = {
    "label_le": ("label_of", _label_le),
    "count_forward": ("classify_count", _count_forward),
    "count_strict": ("classify_count", _count_strict),
    "probs_no_scale": ("probs", _probs_no_scale),
    "select_unstratified": ("ste_select", _select_unstratified),
    "select_protect_off_by_one": ("ste_select", _select_protect_off_by_one),
    "select_quota_swapped": ("ste_select", _select_quota_swapped),
    "select_newest_first_on_ties": ("ste_select", _select_newest_first_on_ties),
    "append_highest_free": ("append_slot", _append_highest_free),
    "free_keeps_scores": ("free_evicted", _free_evicted_keep_scores),
    "budget_uniform": ("global_budget", _budget_uniform),
    "budget_ceil": ("global_budget", _budget_ceil),
    "score_window_never_reset": ("scoring_window_starts", lambda *a: False),
    "score_window_late": ("scoring_window_starts",
                          lambda c, b, m, w: c == b + m - w + 2),
    "unstrat_no_protection": ("unstratified_select", _unstrat_no_protection),
    "unstrat_highest": ("unstratified_select", _unstrat_highest),
    "window_noncausal": ("window_scores", _window_noncausal),
    "window_last_only": ("window_scores", _window_last_only),
    "window_start_off_by_one": ("window_scores", _window_start_off_by_one),
}

ALL_CHECKS = [
    lambda: pins.check_uniform_count(O, range(1, 200)),
    lambda: pins.check_geometric_count(O),
    lambda: pins.check_classify_golden(O),
    lambda: pins.check_classify_exact_rational(O, trials=100),
    lambda: pins.check_attention_textbook(O),
    lambda: pins.check_rho_one_is_full(O),
    lambda: pins.check_local_window(O),
    lambda: pins.check_group_invariants(O),
    lambda: pins.check_ste_golden(O),
    lambda: pins.check_ste_bruteforce(O, trials=60),
    lambda: pins.check_uniform_scores(O),
    lambda: pins.check_unstratified_bruteforce(O, trials=60),
    lambda: pins.check_variant_groups(O),
    lambda: pins.check_window_scores(O),
]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = 0
    for chk in ALL_CHECKS:
        try:
            chk()
        except (AssertionError, ValueError):
            caught += 1
    assert caught >= 1, f"no pin catches mutant {name}"
