"""Planted mistakes in the oracle (on the CPU) must be caught by its pins.

Each case swaps one oracle function for a plausible wrong version (a flipped
sign, a dropped factor, a wrong scale, an off-by-one, the opposite tie rule)
and checks that at least one pin test then fails.  This shows the pins are
sharp enough to catch that class of error.
"""

import math

import numpy as np
import pytest

from oracle import mac_oracle as M
import tests.test_oracle_pins as P


def rope_sign_flip(x, pos, theta):
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    ang = float(pos) * M.inv_freq(x.shape[-1], theta)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c + b * s, b * c - a * s], axis=-1)


def rope_adjacent_pairs(x, pos, theta):
    x = np.asarray(x, dtype=np.float64)
    ang = float(pos) * M.inv_freq(x.shape[-1], theta)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = b * c + a * s
    return out


def merge_without_rescale(a, b):
    m = np.maximum(a.m, b.m)
    l = a.l + b.l
    with np.errstate(invalid="ignore"):
        o = (a.l[:, None] * a.o + b.l[:, None] * b.o) / l[:, None]
    return M.State(np.nan_to_num(o), m, l)


def attend_wrong_scale(qr, K, V):
    qr = np.atleast_2d(np.asarray(qr, dtype=np.float64))
    h, d = qr.shape
    if K.shape[0] == 0:
        return M.State.empty(h, d)
    z = (qr @ np.asarray(K, float).T) / d
    m = z.max(axis=1)
    e = np.exp(z - m[:, None])
    l = e.sum(axis=1)
    return M.State((e @ np.asarray(V, float)) / l[:, None], m, l)


def match_oldest_on_ties(q, ring, tau, p_new):
    dists = np.full(len(ring), np.nan)
    best, best_d = -1, np.inf
    for j, e in enumerate(ring):
        if not (0 <= e.p <= p_new):
            continue
        dj = float(np.sqrt(np.sum((q - e.q) ** 2)))
        dists[j] = dj
        if dj < best_d:
            best, best_d = j, dj
    return M.Match(best, best >= 0 and best_d < tau, best_d, dists)


def match_non_strict(q, ring, tau, p_new):
    # hit when the distance equals tau
    m = ORIG_MATCH(q, ring, tau, p_new)
    return M.Match(m.j, m.j >= 0 and m.dist <= tau, m.dist, m.dists)


def match_any_prefix(q, ring, tau, p_new):
    # candidates whose cached prefix passes the current one are not skipped
    dists = np.full(len(ring), np.nan)
    best, best_d = -1, np.inf
    for j in range(len(ring) - 1, -1, -1):
        dj = float(np.sqrt(np.sum((q - ring[j].q) ** 2)))
        dists[j] = dj
        if dj < best_d:
            best, best_d = j, dj
    return M.Match(best, best >= 0 and best_d < tau, best_d, dists)


ORIG_MATCH = M.match

MUTANTS = [
    ("rope", rope_sign_flip, [P.test_rope_matches_complex_rotation]),
    ("rope", rope_adjacent_pairs, [P.test_rope_matches_complex_rotation]),
    ("merge", merge_without_rescale, [lambda: P.test_merge_of_any_partition_equals_single_pass(1.0)]),
    ("attend", attend_wrong_scale, [P.test_attend_equals_scipy_softmax_attention]),
    ("match", match_oldest_on_ties, [P.test_match_golden_ties_and_strictness]),
    ("match", match_non_strict, [P.test_match_golden_ties_and_strictness]),
    ("match", match_any_prefix, [P.test_match_skips_entries_whose_prefix_passes_the_current_one]),
    # a hit that skips the band: fresh attention from the matched entry's
    # context end instead of its prefix end
    ("fresh_start", lambda e: e.n,
     [P.test_hit_reads_golden, lambda: P.test_brute_force_agrees_on_tiny_inputs(0)]),
    ("prefix_end", lambda n, band: max(0, n - band + 1),
     [lambda: P.test_brute_force_agrees_on_tiny_inputs(0)]),
    ("prefix_end", lambda n, band: max(0, n - band - 1),
     [P.test_hit_reads_golden]),
]


@pytest.mark.parametrize("i", range(len(MUTANTS)))
def test_planted_mistake_is_caught(i, monkeypatch):
    name, fn, pins = MUTANTS[i]
    monkeypatch.setattr(M, name, fn)
    caught = 0
    for pin in pins:
        try:
            pin()
        except AssertionError:
            caught += 1
    assert caught == len(pins), f"mutant {i} of {name} slipped through"


def test_non_strict_threshold_is_caught(monkeypatch):
    real = M.match

    def non_strict(q, ring, tau, p_new):
        mt = real(q, ring, tau, p_new)
        mt.hit = mt.j >= 0 and mt.dist <= tau
        return mt

    monkeypatch.setattr(M, "match", non_strict)
    with pytest.raises(AssertionError):
        P.test_match_golden_ties_and_strictness()
    with pytest.raises(AssertionError):
        P.test_match_repeated_query_hits_any_positive_tau()
