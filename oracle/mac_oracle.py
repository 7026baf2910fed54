"""fp64 CPU oracle of the MAC-Attention match -> amend -> complete decode step.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
path (``kv_cache_reuse_amd``), and it is deliberately plain: NumPy float64,
one definition per function, no blocking or fusion.

Source: the abstract of "MAC-Attention: a Match-Amend-Complete Scheme for Fast
and Accurate Attention Computation" (the paper page's abstract).  The abstract
states the three stages only in words:

* match:    pre-RoPE L2 matching of the current query against a short local
            window of recent queries;
* amend:    the reused attention is rectified by recomputing a small band of
            keys near the match boundary;
* complete: the rectified result is fused with fresh attention over the KV
            tail by a numerically stable merge;
* on a miss the step is ordinary full decode attention; on a hit its cost does
  not depend on the context length.

Everything else is a reading of that text, fixed here:

D1  each decode step first appends its token's key/value at index n-1, then
    the query at position n-1 attends to keys [0, n) (itself included).
D2  rotary embedding is rotate-half: dims (i, i+d/2) rotate by the angle
    pos * theta**(-2i/d), angles in float64.  Keys arrive already rotated.
D3  the partial state over a key set S is m = max z, l = sum exp(z - m),
    o = sum exp(z - m) v / l with z = <rope(q), k> / sqrt(d); the empty state
    is (o = 0, m = -inf, l = 0).
D4  merge: m = max(m1, m2), w_i = l_i exp(m_i - m), l = w1 + w2,
    o = (w1 o1 + w2 o2) / l.  Two empty states merge to the empty state.
D5  each (sequence, query head) keeps a ring of the last W steps' entries
    (q_pre, o, m, l, p, n).  Every step pushes one entry, hit or miss.
D6  match: dist_j = ||q_pre - entry_j.q||_2; j* = argmin, exact ties go to the
    most recent entry; hit iff the ring has a candidate and dist_j* < tau
    (strict).  A NaN distance is never chosen.  An entry is a candidate only if
    0 <= entry.p <= p_new (always true for entries this recurrence pushed).
D7  an entry caches the state of its own query over the prefix [0, p) with
    p = max(0, n_entry - B): every key but the last B of its context.
D8  s = entry_j*.p on a hit, else 0; p_new = max(0, n - B).  Fresh attention
    covers [s, n): the band [p_j*, n_j*) (amend) and the tail [n_j*, n)
    (complete).
D9  A = state([s, p_new)), C = state([p_new, n)); prefix = merge(reused, A)
    on a hit, else A; out = merge(prefix, C).o; the pushed entry is
    (q_pre, prefix, p_new, n).
D10 a miss (s = 0) is exactly dense softmax attention over [0, n).
D11 keys read for one (sequence, head, step) = n - s; on a hit this is
    (n - n_j*) + min(B, n_j*), independent of n.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

NEG_INF = -np.inf


# ---------------------------------------------------------------------------
# D2: rotary position embedding, rotate-half pairing
# ---------------------------------------------------------------------------

def inv_freq(d: int, theta: float) -> np.ndarray:
    """theta ** (-2 i / d) for i in [0, d/2), float64."""
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / float(d))


def rope(x: np.ndarray, pos: int, theta: float) -> np.ndarray:
    """Rotate the pairs (x_i, x_{i+d/2}) of the last axis by pos * inv_freq_i."""
    x = np.asarray(x, dtype=np.float64)
    h = x.shape[-1] // 2
    ang = float(pos) * inv_freq(x.shape[-1], theta)
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


# ---------------------------------------------------------------------------
# D3 / D4: partial softmax states and their merge
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class State:
    """Partial softmax state of H query rows: o [H, d], m [H], l [H]."""
    o: np.ndarray
    m: np.ndarray
    l: np.ndarray

    @staticmethod
    def empty(h: int, d: int) -> "State":
        return State(np.zeros((h, d)), np.full(h, NEG_INF), np.zeros(h))

    @property
    def lse(self) -> np.ndarray:
        with np.errstate(divide="ignore"):
            return self.m + np.log(self.l)


def attend(qr: np.ndarray, K: np.ndarray, V: np.ndarray) -> State:
    """D3: state of the rotated query rows ``qr`` [H, d] over keys K [L, d]
    with values V [L, d]; scores are scaled by 1/sqrt(d), base e."""
    qr = np.atleast_2d(np.asarray(qr, dtype=np.float64))
    h, d = qr.shape
    if K.shape[0] == 0:
        return State.empty(h, d)
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    z = (qr @ K.T) / math.sqrt(d)                    # [H, L]
    m = z.max(axis=1)
    e = np.exp(z - m[:, None])
    l = e.sum(axis=1)
    o = (e @ V) / l[:, None]
    return State(o, m, l)


def merge(a: State, b: State) -> State:
    """D4: log-sum-exp merge of two states of the same rows.  A row is empty
    iff its m is -inf; NaN in either input propagates to the result."""
    ea, eb = a.m == NEG_INF, b.m == NEG_INF
    m = np.maximum(a.m, b.m)
    with np.errstate(invalid="ignore", over="ignore"):
        wa = np.where(ea, 0.0, a.l * np.exp(a.m - m))
        wb = np.where(eb, 0.0, b.l * np.exp(b.m - m))
        l = wa + wb
        o = (wa[:, None] * a.o + wb[:, None] * b.o) / l[:, None]
    both = ea & eb
    o = np.where(both[:, None], 0.0, o)
    l = np.where(both, 0.0, l)
    m = np.where(both, NEG_INF, m)
    return State(o, m, l)


def merge_all(states: Sequence[State]) -> State:
    """Left fold of D4 in the given (ascending key) order."""
    acc = states[0]
    for s in states[1:]:
        acc = merge(acc, s)
    return acc


def dense(qr: np.ndarray, K: np.ndarray, V: np.ndarray) -> np.ndarray:
    """Plain softmax attention output over every key (reference for D10)."""
    return attend(qr, K, V).o


# ---------------------------------------------------------------------------
# D5-D9: ring entries, match, composition
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Entry:
    q: np.ndarray     # pre-RoPE query [d] (the dtype-rounded value, in fp64)
    o: np.ndarray     # prefix output [d]
    m: float
    l: float
    p: int            # prefix end: the state covers keys [0, p)
    n: int            # context length the entry's query saw

    def state(self) -> State:
        return State(self.o[None, :].copy(), np.array([self.m]),
                     np.array([self.l]))


@dataclasses.dataclass
class Match:
    j: int            # index into the ring (oldest first), -1 if none
    hit: bool
    dist: float       # distance of j* (+inf when there is no candidate)
    dists: np.ndarray  # distance to every ring entry (nan for non-candidates)


def match(q: np.ndarray, ring: Sequence[Entry], tau: float, p_new: int) -> Match:
    """D6: L2 distance of pre-RoPE q to each ring entry, argmin with ties to
    the most recent entry, strict threshold."""
    dists = np.full(len(ring), np.nan)
    best, best_d = -1, np.inf
    for j in range(len(ring) - 1, -1, -1):          # most recent first
        e = ring[j]
        if not (0 <= e.p <= p_new):
            continue
        dj = float(np.sqrt(np.sum((q - e.q) ** 2)))
        dists[j] = dj
        if dj < best_d:                              # strict: ties keep the newer
            best, best_d = j, dj
    hit = best >= 0 and best_d < tau
    return Match(best, bool(hit), best_d, dists)


def fresh_start(entry: Entry) -> int:
    """D8: on a hit, fresh attention starts where the matched entry's cached
    prefix ends, so the band [entry.p, entry.n) is recomputed (amend) before
    the tail [entry.n, n) (complete)."""
    return entry.p


def prefix_end(n: int, band: int) -> int:
    """D7/D8: the cached prefix of a query that saw n keys ends B keys early."""
    return max(0, n - band)


def compose(qr: np.ndarray, K: np.ndarray, V: np.ndarray,
            reused: Optional[State], s: int, p_new: int,
            n: int) -> Tuple[State, State]:
    """D8/D9 for the rows ``qr`` [H, d] sharing one key range.

    Fresh attention covers [s, p_new) (A) and [p_new, n) (C).  Returns
    (prefix, full) where prefix = merge(reused, A) (or A when ``reused`` is
    None) and full = merge(prefix, C); full.o is the step's output."""
    A = attend(qr, K[s:p_new], V[s:p_new])
    C = attend(qr, K[p_new:n], V[p_new:n])
    prefix = A if reused is None else merge(reused, A)
    return prefix, merge(prefix, C)


@dataclasses.dataclass
class StepResult:
    out: np.ndarray        # [Hq, d]
    hit: np.ndarray        # [Hq] bool
    match_n: np.ndarray    # [Hq] n of the matched entry, -1 on a miss
    dist: np.ndarray       # [Hq] distance of the best candidate (+inf if none)
    second: np.ndarray     # [Hq] distance of the runner-up candidate (+inf)
    s: np.ndarray          # [Hq] start of the fresh range
    keys_read: np.ndarray  # [Hq] n - s  (D11)
    p_new: int
    n: int
    entries: List[Entry]   # the pushed entries, per head


class MacOracle:
    """The step-by-step recurrence for a batch of sequences.

    ``step(b, q_pre, K, V, n)`` runs one decode step of sequence ``b`` whose
    cache holds ``n`` keys after this step's append.  ``K``/``V`` are that
    sequence's [Hkv, >= n, d] arrays (natural layout; float32 or float64).
    ``force`` maps a query head to a (hit, ring index) decision that replaces
    the oracle's own; tests use it only where the distance is within the
    stated tolerance of tau, or two candidates are within it of each other.
    """

    def __init__(self, batch: int, n_q_heads: int, n_kv_heads: int,
                 head_dim: int, window: int, band: int, tau: float,
                 rope_theta: float):
        assert n_q_heads % n_kv_heads == 0
        self.batch, self.hq, self.hkv, self.d = batch, n_q_heads, n_kv_heads, head_dim
        self.G = n_q_heads // n_kv_heads
        self.W, self.B, self.tau, self.theta = window, band, float(tau), rope_theta
        self.rings: List[List[List[Entry]]] = [
            [[] for _ in range(n_q_heads)] for _ in range(batch)]

    @classmethod
    def for_workload(cls, w) -> "MacOracle":
        return cls(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.window,
                   w.band, w.tau, w.rope_theta)

    def push(self, b: int, h: int, e: Entry) -> None:
        """D5: append, then evict the oldest beyond W entries."""
        ring = self.rings[b][h]
        ring.append(e)
        while len(ring) > self.W:
            ring.pop(0)

    def step(self, b: int, q_pre: np.ndarray, K: np.ndarray, V: np.ndarray,
             n: int, force: Optional[Dict[int, Tuple[bool, int]]] = None
             ) -> StepResult:
        hq, d = self.hq, self.d
        q_pre = np.asarray(q_pre, dtype=np.float64).reshape(hq, d)
        pos = n - 1
        p_new = prefix_end(n, self.B)
        qr = rope(q_pre, pos, self.theta)

        res = StepResult(np.zeros((hq, d)), np.zeros(hq, bool),
                         np.full(hq, -1, np.int64), np.full(hq, np.inf),
                         np.full(hq, np.inf), np.zeros(hq, np.int64),
                         np.zeros(hq, np.int64), p_new, n, [None] * hq)
        chosen: List[Optional[Entry]] = [None] * hq
        for h in range(hq):
            ring = self.rings[b][h]
            mt = match(q_pre[h], ring, self.tau, p_new)
            hit, j = mt.hit, mt.j
            if force is not None and h in force:
                hit, j = force[h]
                hit = bool(hit) and j >= 0
            finite = np.sort(mt.dists[~np.isnan(mt.dists)])
            res.dist[h] = mt.dist
            res.second[h] = finite[1] if finite.size > 1 else np.inf
            if hit:
                chosen[h] = ring[j]
                res.hit[h] = True
                res.match_n[h] = ring[j].n
                res.s[h] = fresh_start(ring[j])
        res.keys_read[:] = n - res.s

        # fresh attention per KV group; query heads that share a start s are
        # stacked into one call (each row's arithmetic is unchanged)
        for g in range(self.hkv):
            Kg, Vg = K[g], V[g]
            heads = list(range(g * self.G, (g + 1) * self.G))
            by_s: Dict[Tuple[int, bool], List[int]] = {}
            for h in heads:
                by_s.setdefault((int(res.s[h]), chosen[h] is not None),
                                []).append(h)
            for (s, _), hs in by_s.items():
                reused = None
                if chosen[hs[0]] is not None:
                    reused = State(
                        np.stack([chosen[h].o for h in hs]),
                        np.array([chosen[h].m for h in hs]),
                        np.array([chosen[h].l for h in hs]))
                    assert all(chosen[h] is not None for h in hs)
                else:
                    assert all(chosen[h] is None for h in hs)
                prefix, full = compose(qr[hs], Kg, Vg, reused, s, p_new, n)
                for i, h in enumerate(hs):
                    res.out[h] = full.o[i]
                    res.entries[h] = Entry(q_pre[h].copy(), prefix.o[i].copy(),
                                           float(prefix.m[i]),
                                           float(prefix.l[i]), p_new, n)
        for h in range(hq):
            self.push(b, h, res.entries[h])
        return res


    def seed(self, b: int, q_hist: np.ndarray, K: np.ndarray, V: np.ndarray,
             n_now: int) -> None:
        """Ring seeding from a prefill.

        Reading of the match stage's window (MAC-Attention abstract) as the
        last W decode steps leaves it empty after a prefill.  Seeding replays
        the last len(q_hist) positions of sequence b, whose cache holds n_now
        keys, oldest first, as decode steps that do not match: each pushes the
        entry a miss at that position would push (the exact prefix state of
        its own query over [0, max(0, position + 1 - B)))."""
        q_hist = np.asarray(q_hist, dtype=np.float64).reshape(-1, self.hq, self.d)
        m = q_hist.shape[0]
        assert 0 <= m <= self.W and m <= n_now
        no_match = {h: (False, -1) for h in range(self.hq)}
        for j in range(m):
            self.step(b, q_hist[j], K, V, n_now - m + j + 1, force=no_match)


# ---------------------------------------------------------------------------
# decisions as a function of the query stream alone
# ---------------------------------------------------------------------------

def decisions_only(q64: np.ndarray, window: int, tau: float):
    """Hit/miss of every (step, sequence, head) of a stream q64 [T, b, H, d].

    Because every step pushes its own query (D5) and every pushed entry is a
    candidate (D6), the decision at step t depends only on q_t and the W
    queries before it.  Returns (hit [T, b, H] bool, age [T, b, H] int: steps
    back to the matched entry, 0 on a miss, dist [T, b, H])."""
    T = q64.shape[0]
    best = np.full(q64.shape[:-1], np.inf)
    age = np.zeros(q64.shape[:-1], dtype=np.int64)
    for k in range(1, window + 1):                   # k = 1 is the most recent
        if k >= T:
            break
        dk = np.sqrt(np.sum((q64[k:] - q64[:-k]) ** 2, axis=-1))
        better = dk < best[k:]                       # strict: keep the newer
        best[k:] = np.where(better, dk, best[k:])
        age[k:] = np.where(better, k, age[k:])
    hit = best < tau
    return hit, np.where(hit, age, 0), best


def run(w, inputs, K64=None, V64=None, steps: Optional[int] = None,
        seqs: Optional[Sequence[int]] = None):
    """Run the recurrence over a generated workload (synth.Inputs).

    Returns a list over steps of {b: StepResult}.  ``K64``/``V64`` may hold
    pre-converted float64 (or float32) copies of the caches."""
    orc = MacOracle.for_workload(w)
    K = inputs.k.float().numpy() if K64 is None else K64
    V = inputs.v.float().numpy() if V64 is None else V64
    T = inputs.q64.shape[0] if steps is None else steps
    seqs = range(w.batch) if seqs is None else seqs
    out = []
    for t in range(T):
        row = {}
        for b in seqs:
            n = int(inputs.contexts[b]) + t + 1
            row[b] = orc.step(b, inputs.q64[t, b], K[b], V[b], n)
        out.append(row)
    return out, orc
