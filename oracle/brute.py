"""Pure-Python brute force of the MAC-Attention decode step, for tiny inputs.

TEST INFRASTRUCTURE ONLY (same rules as ``mac_oracle``).  This is a second,
independently structured statement of the same definitions (D1-D11 in
``mac_oracle``): plain loops over Python floats with the ``math`` module, the
rotary embedding as an explicit 2x2 rotation per pair, and every attention
output written as one weighted average over its key set instead of a fold of
partial states.  A hit's output is the weighted average in which the reused
entry counts as one pseudo-key of weight l_e * exp(m_e) and value o_e (that is
what merging its state means), the recomputed keys [s, n) count with weight
exp(z_k) each.  All weights are taken relative to one common maximum.
"""

from __future__ import annotations

import math
from typing import List, Optional


def rotate(x: List[float], pos: int, theta: float) -> List[float]:
    d = len(x)
    h = d // 2
    out = [0.0] * d
    for i in range(h):
        ang = pos * theta ** (-2.0 * i / d)
        c, s = math.cos(ang), math.sin(ang)
        # [out_i, out_{i+h}] = [[c, -s], [s, c]] @ [x_i, x_{i+h}]
        out[i] = c * x[i] - s * x[i + h]
        out[i + h] = s * x[i] + c * x[i + h]
    return out


def dot(a, b) -> float:
    acc = 0.0
    for x, y in zip(a, b):
        acc += x * y
    return acc


def weighted_average(terms):
    """terms: list of (log_weight, weight_multiplier, vector).  Returns
    (average vector, max log weight, sum of weights relative to that max) or
    None if there are no terms."""
    terms = [t for t in terms if t[1] != 0.0]
    if not terms:
        return None
    mx = max(t[0] for t in terms)
    d = len(terms[0][2])
    num = [0.0] * d
    den = 0.0
    for lw, mult, vec in terms:
        w = mult * math.exp(lw - mx)
        den += w
        for i in range(d):
            num[i] += w * vec[i]
    return [x / den for x in num], mx, den


class BruteMac:
    """Rings and the recurrence over Python lists; one sequence per list."""

    def __init__(self, batch, n_q_heads, n_kv_heads, head_dim, window, band,
                 tau, rope_theta):
        self.hq, self.hkv, self.d = n_q_heads, n_kv_heads, head_dim
        self.G = n_q_heads // n_kv_heads
        self.W, self.B, self.tau, self.theta = window, band, tau, rope_theta
        # entry = dict(q, o, m, l, p, n); newest last
        self.rings = [[[] for _ in range(n_q_heads)] for _ in range(batch)]

    def step(self, b, q_pre, K, V, n):
        """q_pre: [Hq][d] floats; K, V: [Hkv][L][d] floats (L >= n).
        Returns per head dicts with out, hit, match_n, s, keys_read."""
        results = []
        pushes = []
        p_new = n - self.B if n - self.B > 0 else 0
        for h in range(self.hq):
            g = h // self.G
            q = list(q_pre[h])
            ring = self.rings[b][h]
            # match: scan all entries, keep the smallest distance; on equal
            # distances prefer the later (more recent) entry
            best = None
            best_d = float("inf")
            for idx, e in enumerate(ring):
                if e["p"] < 0 or e["p"] > p_new:
                    continue
                dd = math.sqrt(sum((q[i] - e["q"][i]) ** 2 for i in range(self.d)))
                if dd != dd:
                    continue
                if dd <= best_d:
                    best, best_d = idx, dd
            hit = best is not None and best_d < self.tau
            s = ring[best]["p"] if hit else 0
            qr = rotate(q, n - 1, self.theta)
            scale = 1.0 / math.sqrt(self.d)
            z = {k: dot(qr, K[g][k]) * scale for k in range(s, n)}

            reused_term = []
            if hit:
                e = ring[best]
                if e["l"] > 0.0:
                    reused_term = [(e["m"], e["l"], e["o"])]
            # prefix: reused pseudo-key plus keys [s, p_new)
            pre_terms = reused_term + [(z[k], 1.0, V[g][k]) for k in range(s, p_new)]
            pre = weighted_average(pre_terms)
            full = weighted_average(reused_term + [(z[k], 1.0, V[g][k])
                                                   for k in range(s, n)])
            out = full[0] if full is not None else [0.0] * self.d
            if pre is None:
                entry = dict(q=q, o=[0.0] * self.d, m=float("-inf"), l=0.0,
                             p=p_new, n=n)
            else:
                entry = dict(q=q, o=pre[0], m=pre[1], l=pre[2], p=p_new, n=n)
            pushes.append(entry)
            results.append(dict(out=out, hit=hit,
                                match_n=ring[best]["n"] if hit else -1,
                                s=s, keys_read=n - s, entry=entry))
        for h, e in enumerate(pushes):
            ring = self.rings[b][h]
            ring.append(e)
            while len(ring) > self.W:
                del ring[0]
        return results
