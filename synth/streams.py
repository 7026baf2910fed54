"""Workload shapes and seeded draws for the MAC-Attention decode step.

The MAC-Attention abstract (page "MAC-Attention: a Match-Amend-Complete
Scheme ...", abstract) prints no query or key distributions; its quality
suites (LongBench v2 and RULER at 120K, LongGenBench at 16K continuous
generation) are stood in for by the five synthetic shapes below:

* ``tiny``     - 1 sequence, 4 query heads over 1 KV head, d=64, fp32, 2K keys
* ``8b_32k``   - Llama-3-8B shaped: 32 query / 8 KV heads, d=128, bf16, 32K keys
* ``8b_128k``  - the same shape at 131072 keys (the headline shape)
* ``paged_b8`` - 8 sequences with contexts uniform in [16384, 65536], 16-key pages
* ``70b_128k`` - 4 sequences, 64 query / 8 KV heads, 131072 keys, 1% outlier keys x8
* ``gen_16k``  - 1 sequence, 8B shape, 16384-key prefill, 2048 generated tokens

Query stream (pre-RoPE), per sequence b: ``q_0 ~ N(0, I)``; for t >= 1 a single
Bernoulli(p) per (b, t) decides a jump, which redraws the whole token's query
(all heads) as ``N(0, I)``; otherwise ``q_t = rho q_{t-1} + sqrt(1 - rho^2) eps``
with eps ~ N(0, I) elementwise.  The recurrence runs in float64 on unrounded
values; each ``q_t`` is then rounded to the workload dtype (round to nearest
even) and that rounded value is what both the oracle and the GPU read.

Keys are drawn directly as post-rotation N(0, 1) vectors: a rotation of an
i.i.d. standard Gaussian vector is again i.i.d. standard Gaussian, so this is
the same distribution as drawing pre-rotation keys and rotating them, without
putting rotary arithmetic into the generator.  Values are N(0, 1).  In the
70B shape a Bernoulli(0.01) per (sequence, token, KV head) multiplies that
whole key vector by 8 (values are left alone).

Seeds: ``SeedSequence([1000 + index, layer])`` per workload, spawned in a
fixed order: q innovations, jumps, keys, values, outliers, page table,
contexts, per-head rho.  Nothing here depends on the GPU.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

# ---------------------------------------------------------------------------
# workload table
# ---------------------------------------------------------------------------

# tau for the 8B/32K shape: chosen so that about 80% of (sequence, head, step)
# match decisions hit on its query stream; found by bisection with the
# oracle's query-only decision function (oracle/calibrate_tau.py) and checked
# by a CPU test that re-runs the oracle on the stream.
TAU_8B_32K = 3.9066


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int                 # 1..5, selects the seed
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str                 # "f32" or "bf16"
    context: int               # prefill keys per sequence (ignored if ctx_range)
    steps: int                 # decode steps
    rope_theta: float
    rho: float                 # AR(1) coefficient (ignored if rho_range)
    p_jump: float              # per-token jump probability
    window: int                # W
    band: int                  # B
    tau: float
    page_size: int = 0         # 0 = contiguous cache, else keys per page
    ctx_range: Optional[tuple] = None   # (lo, hi) inclusive, per sequence
    rho_range: Optional[tuple] = None   # (lo, hi) uniform, per query head
    rho_per_kv: bool = False   # rho_range drawn per KV head, shared by its query heads
    outlier_p: float = 0.0
    outlier_scale: float = 1.0
    period: int = 0            # >0: q_t repeats q_{t-period} exactly (tests)

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads

    @property
    def bytes_per_elem(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


_TAU_HALF_SQRT_D128 = 0.5 * math.sqrt(128.0)

WORKLOADS = {
    "tiny": Workload(
        name="tiny", index=1, batch=1, n_q_heads=4, n_kv_heads=1, head_dim=64,
        dtype="f32", context=2048, steps=64, rope_theta=1e4, rho=0.95,
        p_jump=0.2, window=16, band=64, tau=0.5 * math.sqrt(64.0)),
    "8b_32k": Workload(
        name="8b_32k", index=2, batch=1, n_q_heads=32, n_kv_heads=8,
        head_dim=128, dtype="bf16", context=32768, steps=256, rope_theta=5e5,
        rho=0.95, p_jump=0.1, window=32, band=256, tau=TAU_8B_32K),
    "8b_128k": Workload(
        name="8b_128k", index=3, batch=1, n_q_heads=32, n_kv_heads=8,
        head_dim=128, dtype="bf16", context=131072, steps=512,
        rope_theta=5e5, rho=0.95, p_jump=1.0, window=32, band=256,
        tau=_TAU_HALF_SQRT_D128),
    "paged_b8": Workload(
        name="paged_b8", index=4, batch=8, n_q_heads=32, n_kv_heads=8,
        head_dim=128, dtype="bf16", context=65536, steps=128, rope_theta=5e5,
        rho=0.95, p_jump=0.1, window=32, band=128, tau=_TAU_HALF_SQRT_D128,
        page_size=16, ctx_range=(16384, 65536)),
    "70b_128k": Workload(
        name="70b_128k", index=5, batch=4, n_q_heads=64, n_kv_heads=8,
        head_dim=128, dtype="bf16", context=131072, steps=256,
        rope_theta=5e5, rho=0.9, p_jump=0.1, window=64, band=256,
        tau=_TAU_HALF_SQRT_D128, rho_range=(0.8, 0.99), outlier_p=0.01,
        outlier_scale=8.0),
    # long continuous generation from a 16K prefill (the shape of the
    # pages' 16K continuous-generation suite), for the drift of the reused
    # states along chains of hits
    "gen_16k": Workload(
        name="gen_16k", index=6, batch=1, n_q_heads=32, n_kv_heads=8,
        head_dim=128, dtype="bf16", context=16384, steps=2048, rope_theta=5e5,
        rho=0.95, p_jump=0.05, window=32, band=256, tau=_TAU_HALF_SQRT_D128),
}

# jump probabilities of the headline hit-rate sweep (about 0/50/80/95% hits)
SWEEP_P_JUMP = (1.0, 0.5, 0.2, 0.05)


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return w.replace(**overrides) if overrides else w


# ---------------------------------------------------------------------------
# seeded draws
# ---------------------------------------------------------------------------

def _children(w: Workload, layer: int):
    ss = np.random.SeedSequence([1000 + w.index, layer])
    names = ("q", "jump", "k", "v", "outlier", "pages", "ctx", "rho")
    return dict(zip(names, ss.spawn(len(names))))


def _round(x: np.ndarray, dtype: str) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(torch.float32 if dtype == "f32" else torch.bfloat16)


def contexts(w: Workload, layer: int = 0) -> np.ndarray:
    """Prefill length of each sequence."""
    if w.ctx_range is None:
        return np.full(w.batch, w.context, dtype=np.int64)
    rng = np.random.default_rng(_children(w, layer)["ctx"])
    lo, hi = w.ctx_range
    return rng.integers(lo, hi, size=w.batch, endpoint=True).astype(np.int64)


def rho_per_head(w: Workload, layer: int = 0) -> np.ndarray:
    """AR(1) coefficient of each query head: w.rho, or drawn uniformly from
    w.rho_range per query head (or per KV head, shared by its query heads)."""
    if w.rho_range is None:
        return np.full(w.n_q_heads, w.rho, dtype=np.float64)
    rng = np.random.default_rng(_children(w, layer)["rho"])
    lo, hi = w.rho_range
    if w.rho_per_kv:
        return np.repeat(rng.uniform(lo, hi, size=w.n_kv_heads), w.group)
    return rng.uniform(lo, hi, size=w.n_q_heads)


def even_jumps(p: float, start: int, count: int) -> np.ndarray:
    """A jump schedule at rate p with the jumps evenly spaced: token i jumps
    iff floor((i + 1) p) > floor(i p), for i in [start, start + count).  Any
    run of n consecutive tokens then holds floor(n p) or ceil(n p) jumps."""
    i = np.arange(start, start + count, dtype=np.float64)
    return np.floor((i + 1) * p) > np.floor(i * p)


def make_q_stream(w: Workload, p_jump: Optional[float] = None, layer: int = 0,
                  steps: Optional[int] = None, jumps: Optional[np.ndarray] = None):
    """Pre-RoPE query stream.

    Returns ``(q, q64)``: ``q`` is a CPU tensor ``[T, batch, Hq, d]`` in the
    workload dtype and ``q64`` the float64 numpy copy of the same rounded
    values.  ``jumps`` ([T] or [T, batch] bool) replaces the Bernoulli(p)
    jump draws by a given schedule.
    """
    p = w.p_jump if p_jump is None else p_jump
    T = w.steps if steps is None else steps
    ch = _children(w, layer)
    eps = np.random.default_rng(ch["q"]).standard_normal(
        (T, w.batch, w.n_q_heads, w.head_dim))
    u = np.random.default_rng(ch["jump"]).random((T, w.batch))
    if jumps is None:
        jump_at = u < p
    else:
        jump_at = np.broadcast_to(np.asarray(jumps, dtype=bool).reshape(T, -1), (T, w.batch))
    rho = rho_per_head(w, layer)[None, :, None]
    c = np.sqrt(1.0 - rho * rho)
    q = np.empty_like(eps)
    q[0] = eps[0]
    for t in range(1, T):
        ar = rho * q[t - 1] + c * eps[t]
        jump = jump_at[t][:, None, None]
        q[t] = np.where(jump, eps[t], ar)
    if w.period > 0:
        for t in range(w.period, T):
            q[t] = q[t - w.period]
    qt = _round(q, w.dtype)
    return qt, qt.to(torch.float64).numpy()


@dataclasses.dataclass
class Inputs:
    workload: Workload
    q: torch.Tensor            # [T, batch, Hq, d] dtype (pre-RoPE)
    q64: np.ndarray            # same values, float64
    k: torch.Tensor            # [batch, Hkv, Lmax, d] dtype, post-RoPE keys
    v: torch.Tensor            # [batch, Hkv, Lmax, d] dtype
    contexts: np.ndarray       # [batch] prefill length
    page_table: Optional[np.ndarray]   # [batch, max_pages] int32, -1 = unused
    n_pages: int               # pages in the pool (paged workloads)
    outlier: Optional[np.ndarray]      # [batch, Hkv, Lmax] bool

    @property
    def total_len(self) -> np.ndarray:
        return self.contexts + self.q.shape[0]


def make_kv_group(w: Workload, ctx: np.ndarray, steps: int, b: int, g: int, layer: int = 0):
    """Keys and values of one (sequence, KV head) for prefill plus every
    decode step: ([n, d] dtype tensor, [n, d] dtype tensor, [n] bool outlier
    flags or None) with n = ctx[b] + steps.  Each group draws from seeds of
    its own, so a group can be drawn without the others."""
    ch = _children(w, layer)
    i = b * w.n_kv_heads + g
    n = int(ctx[b]) + steps
    kk = np.random.default_rng(ch["k"].spawn(w.batch * w.n_kv_heads)[i]).standard_normal(
        (n, w.head_dim), dtype=np.float32)
    flag = None
    if w.outlier_p > 0:
        oss = ch["outlier"].spawn(w.batch * w.n_kv_heads)[i]
        flag = np.random.default_rng(oss).random(n) < w.outlier_p
        kk[flag] *= np.float32(w.outlier_scale)
    vv = np.random.default_rng(ch["v"].spawn(w.batch * w.n_kv_heads)[i]).standard_normal(
        (n, w.head_dim), dtype=np.float32)
    return _round(kk, w.dtype), _round(vv, w.dtype), flag


def make_kv(w: Workload, ctx: np.ndarray, steps: int, layer: int = 0):
    """Keys and values for prefill plus every decode step, natural layout."""
    L = int(ctx.max()) + steps
    shape = (w.batch, w.n_kv_heads, L, w.head_dim)
    k = torch.zeros(shape, dtype=w.torch_dtype())
    v = torch.zeros(shape, dtype=w.torch_dtype())
    outl = np.zeros((w.batch, w.n_kv_heads, L), dtype=bool) if w.outlier_p > 0 else None
    for b in range(w.batch):
        n = int(ctx[b]) + steps
        for g in range(w.n_kv_heads):
            kk, vv, flag = make_kv_group(w, ctx, steps, b, g, layer)
            k[b, g, :n] = kk
            v[b, g, :n] = vv
            if outl is not None:
                outl[b, g, :n] = flag
    return k, v, outl


def make_page_table(w: Workload, ctx: np.ndarray, steps: int, layer: int = 0):
    """Seeded random page table: each sequence's pages are a random slice of a
    permuted pool just large enough for prefill plus all decode steps."""
    ps = w.page_size
    per = [-(-(int(c) + steps) // ps) for c in ctx]
    pool = int(sum(per))
    perm = np.random.default_rng(_children(w, layer)["pages"]).permutation(pool)
    table = np.full((w.batch, max(per)), -1, dtype=np.int32)
    off = 0
    for b, n in enumerate(per):
        table[b, :n] = perm[off:off + n]
        off += n
    return table, pool


def make_inputs(w: Workload, p_jump: Optional[float] = None, layer: int = 0,
                steps: Optional[int] = None) -> Inputs:
    T = w.steps if steps is None else steps
    ctx = contexts(w, layer)
    q, q64 = make_q_stream(w, p_jump, layer, T)
    k, v, outl = make_kv(w, ctx, T, layer)
    table, pool = (None, 0)
    if w.page_size:
        table, pool = make_page_table(w, ctx, T, layer)
    return Inputs(w, q, q64, k, v, ctx, table, pool, outl)
