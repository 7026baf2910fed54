"""Parity check of recorded GPU steps against the fp64 oracle, per KV group.

The oracle runs per KV group (b, g): the G query heads of that group form an
independent problem (their own rings, their own keys), so groups can be
replayed separately, and in parallel processes.

Decision parity: hit/miss and the matched entry's context length must agree
exactly, except where the oracle's best distance lies within 1e-4 * tau of
tau, or (both sides hitting) the GPU's entry is within 1e-4 * tau of the
oracle's best: there the GPU's decision is accepted, logged, and the oracle
follows it so that both rings stay comparable.

Nothing here touches the GPU: the inputs are recorded GPU outputs (numpy
arrays) and the seeded workload draws.
"""

from __future__ import annotations

import atexit
import dataclasses
import multiprocessing as mp
import os
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from oracle import mac_oracle as M

OUT_TOL = 2e-3          # max |out_gpu - out_oracle|
BORDER_REL = 1e-4       # borderline band around tau, relative


@dataclasses.dataclass
class Report:
    steps: int = 0
    heads: int = 0
    hits: int = 0
    borderline: List[tuple] = dataclasses.field(default_factory=list)
    max_err: float = 0.0
    max_dist_err: float = 0.0
    mismatches: List[tuple] = dataclasses.field(default_factory=list)
    groups: int = 0

    def ok(self, tol=OUT_TOL) -> bool:
        return not self.mismatches and self.max_err <= tol

    def add(self, o: "Report") -> "Report":
        self.steps += o.steps
        self.heads += o.heads
        self.hits += o.hits
        self.borderline += o.borderline
        self.max_err = max(self.max_err, o.max_err)
        self.max_dist_err = max(self.max_dist_err, o.max_dist_err)
        self.mismatches += o.mismatches
        self.groups += o.groups
        return self


def check_group(w, b: int, g: int, ctx_b: int, q64: np.ndarray, Kg: np.ndarray, Vg: np.ndarray,
                out: Dict[int, np.ndarray], match_n: Dict[int, np.ndarray],
                dist: Dict[int, np.ndarray], T: int, tol: float = OUT_TOL,
                seed_q64: Optional[np.ndarray] = None, collect=None) -> Report:
    """Replay the oracle for KV group (b, g) over steps 0..T-1 and compare the
    recorded GPU steps.

    q64 [T, G, d]: the group's pre-RoPE queries; Kg, Vg [>= ctx_b + T, d]:
    its keys and values (float64 or float32); out / match_n / dist map a
    step to the GPU's [G, d] / [G] / [G] results of the group's heads (steps
    missing there are replayed without comparing; exact decision checks need
    every step).  seed_q64 [n, G, d]: queries the rings were seeded with."""
    G = w.group
    rep = Report(groups=1)
    tau = float(w.tau)
    orc = M.MacOracle(1, G, 1, w.head_dim, w.window, w.band, tau, w.rope_theta)
    Kg, Vg = Kg[None], Vg[None]
    h0 = g * G
    if seed_q64 is not None:
        orc.seed(0, seed_q64, Kg, Vg, ctx_b)
    for t in range(T):
        n = ctx_b + t + 1
        p_new = max(0, n - w.band)
        q = q64[t]
        have = t in out
        force = {}
        if have:
            for i in range(G):
                h = h0 + i
                mt = M.match(q[i], orc.rings[0][i], tau, p_new)
                g_n = int(match_n[t][i])
                g_hit = g_n >= 0
                o_n = orc.rings[0][i][mt.j].n if mt.hit else -1
                # distance of the GPU-reported best candidate
                gd = float(dist[t][i])
                if np.isfinite(mt.dist):
                    rep.max_dist_err = max(rep.max_dist_err, abs(gd - mt.dist) / max(1.0, mt.dist))
                if g_hit == mt.hit and g_n == o_n:
                    continue
                border = abs(mt.dist - tau) <= BORDER_REL * tau
                j_gpu = -1
                if g_hit:
                    js = [j for j, e in enumerate(orc.rings[0][i]) if e.n == g_n]
                    j_gpu = js[0] if js else -1
                    if j_gpu >= 0 and mt.hit:
                        dj = mt.dists[j_gpu]
                        border = border or abs(dj - mt.dist) <= BORDER_REL * tau
                    if j_gpu >= 0 and not mt.hit:
                        dj = mt.dists[j_gpu]
                        border = border or abs(dj - tau) <= BORDER_REL * tau
                if border and (not g_hit or j_gpu >= 0):
                    rep.borderline.append((b, h, t, mt.dist, g_n, o_n))
                    force[i] = (g_hit, j_gpu)
                else:
                    rep.mismatches.append((b, h, t, "decision", g_n, o_n, mt.dist, gd))
        r = orc.step(0, q, Kg, Vg, n, force=force or None)
        if collect is not None:
            collect[(b, g, t)] = (r.out.copy(), r.match_n.copy())
        if have:
            got = out[t]
            err = np.abs(got.astype(np.float64) - r.out)
            e = float(np.nanmax(err)) if err.size else 0.0
            if (np.isnan(got) != np.isnan(r.out)).any():
                rep.mismatches.append((b, g, t, "nan-pattern"))
            rep.max_err = max(rep.max_err, e)
            if e > tol:
                rep.mismatches.append((b, g, t, "out", e))
            rep.steps += 1
            rep.heads += G
            rep.hits += int(r.hit.sum())
    return rep


def group_slices(w, gpu, b: int, g: int):
    """The GPU results of group (b, g)'s heads, per recorded step."""
    hs = slice(g * w.group, (g + 1) * w.group)
    return ({t: o[b, hs] for t, o in gpu.out.items()},
            {t: m[b, hs] for t, m in gpu.match_n.items()},
            {t: d[b, hs] for t, d in gpu.dist.items()})


def check_groups(w, inp, gpu, groups: Sequence[Tuple[int, int]],
                 steps: Optional[Sequence[int]] = None, K64=None, V64=None,
                 tol: float = OUT_TOL, seed_q64=None, collect=None) -> Report:
    """check_group over `groups` in this process; `gpu` holds [batch, Hq, ...]
    results per step, `inp` the workload's draws (synth.Inputs)."""
    T = max(gpu.out) + 1 if steps is None else max(steps) + 1
    G = w.group
    rep = Report()
    for (b, g) in groups:
        heads = list(range(g * G, (g + 1) * G))
        Kg = K64[b, g] if K64 is not None else inp.k[b, g].double().numpy()
        Vg = V64[b, g] if V64 is not None else inp.v[b, g].double().numpy()
        o, m, d = group_slices(w, gpu, b, g)
        sq = seed_q64[:, b, heads] if seed_q64 is not None else None
        rep.add(check_group(w, b, g, int(inp.contexts[b]), inp.q64[:, b, heads], Kg, Vg, o, m, d,
                            T, tol=tol, seed_q64=sq, collect=collect))
    return rep


# ---------------------------------------------------------------------------
# the same replay in worker processes
# ---------------------------------------------------------------------------

_POOL = None


def _worker_init():
    # one BLAS thread per worker: the workers are the parallelism
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _replay(task):
    from synth.streams import make_kv_group
    w, b, g, contexts, kv_steps, layer, q64, o, m, d, T, tol = task
    k, v, _ = make_kv_group(w, contexts, kv_steps, b, g, layer)
    return check_group(w, b, g, int(contexts[b]), q64, k.double().numpy(), v.double().numpy(),
                       o, m, d, T, tol=tol)


def _pool(workers: int):
    global _POOL
    if _POOL is None:
        # spawned (not forked) workers: a fork of a process that uses the GPU
        # would carry its device handles along
        env = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS",
                                               "MKL_NUM_THREADS")}
        for k in env:
            os.environ[k] = "1"
        try:
            _POOL = mp.get_context("spawn").Pool(workers, initializer=_worker_init)
        finally:
            for k, val in env.items():
                if val is None:
                    os.environ.pop(k, None)
                else:
                    os.environ[k] = val
        atexit.register(_POOL.terminate)
    return _POOL


def default_workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(12, n))


def check_groups_parallel(w, inp, gpu, groups: Sequence[Tuple[int, int]], layer: int = 0,
                          tol: float = OUT_TOL, workers: Optional[int] = None,
                          progress=None) -> Report:
    """check_groups with one task per group in a pool of spawned workers.
    Each worker draws its group's keys and values again from the workload's
    seeds (synth.make_kv_group with the same layer and step count as `inp`),
    so only queries and GPU results travel.  Groups are independent, so the
    report equals the serial one."""
    T = max(gpu.out) + 1
    kv_steps = int(inp.q.shape[0])
    G = w.group
    tasks = []
    for (b, g) in groups:
        o, m, d = group_slices(w, gpu, b, g)
        q = np.ascontiguousarray(inp.q64[:, b, g * G:(g + 1) * G])
        tasks.append((w, b, g, np.asarray(inp.contexts), kv_steps, layer, q, o, m, d, T, tol))
    pool = _pool(workers or default_workers())
    rep = Report()
    for i, r in enumerate(pool.imap_unordered(_replay, tasks)):
        rep.add(r)
        if progress is not None:
            progress(i + 1, len(tasks), rep)
    return rep
