"""Benchmark of the MAC-Attention decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--layers L]

Workload: the Llama-3-8B decode-attention shape at a 131072-key context
(batch 1, 32 query / 8 KV heads, d = 128, bf16 K/V, W = 32, B = 256,
tau = 0.5 sqrt(128)).  One step is one pass of the whole hot path for one
token: append k/v, then match -> split-K attention -> merge (one attention
layer).  L layer copies (own caches, rings and streams) are visited in turn
so that consecutive steps do not find the previous step's KV in the 256 MB
last-level cache.  Every layer copy's ring is seeded with the queries of
the last W prefill positions before the first step, and the jumps of the
query stream (a redrawn query, so a miss) fall on evenly spaced tokens at
the point's rate: the timed steps hold exactly the jump rate's share of
misses whatever their number.

Printed: one JSON line.  `value` is the effective KV bandwidth of the miss
path (every step misses: jump probability 1), i.e. algorithmic bytes / time;
`sweep` holds the hit-rate sweep (jump probability 1, 0.5, 0.2, 0.05) with
us/token, effective and dense-equivalent GB/s and the measured hit rates;
`flatness` the hit-step latency at contexts 8K..128K; `latency_classes`
per-step p10/p50/p90 at jump probability 0.2 split by the step's decisions
(every head hit, every head missed, mixed); `configs` the other workloads
(8B shape at 32K keys, the ragged paged batch of 8, the 70B shape and its
rho-per-KV-head supplement): miss path with the step kernel's achieved
bandwidth, the workload's own stream and the all-hit step; `seeding` the
cost of seeding the rings from the prefill (1 and W positions); `calls`
the miss and all-hit steps as two calls (mac_append_kv, mac_decode_step)
against the fused call, and mac_append_kv alone; `drift` the
largest |out_MAC - out_dense| on a 16K continuous-generation stream by
reuse-chain depth, over tau and B; `multilayer` every layer of a token in
one graph (32 layers, 16K keys); `mqa` 32 query heads over one KV head at
128K keys; `read_ceiling` the rate of a plain streaming-read kernel on the
same device; `roofline` the step kernel's achieved bandwidth from HIP events
around its launches; `cpu_baseline` the fp64 oracle timed on a bounded
sample of the same workload on the host cores, with per-class and
single-thread figures on the 8B 32K stream.
"""

from __future__ import annotations

import argparse
import copy
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
METRIC = ("decode-attention µs/token + effective KV GB/s (% HBM peak) at 128K, "
          "hit-rate sweep")
PROFILE_TRAFFIC = os.path.join(ROOT, "profiles", "traffic_step_kernel_8b_128k.json")
# sources the step kernel is compiled from: the stored counter figures are
# only valid for the kernel they were taken on
KERNEL_SRCS = [os.path.join(ROOT, "kv_cache_reuse_amd", "csrc", f)
               for f in ("step.hip", "match.h", "mac_dev.h", "rows_map.h")]
ROOFLINE_KERNEL = "mac::step_kernel<bf16,128,contiguous>"
COPY_CAL_BYTES = 512 * 1024 * 1024


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


# ---------------------------------------------------------------------------
# algorithmic bytes of one step, from the step's decisions
# ---------------------------------------------------------------------------

def step_bytes(w, n_ctx, match_n, ring_count):
    """Algorithmic HBM bytes of one decode step.

    n_ctx: [batch] keys after the append; match_n: [batch, Hq] (-1 = miss);
    ring_count: [batch, Hq] entries the ring held before the step.
    Returns (total bytes, KV bytes, keys read) where keys read sums, over
    KV groups, n - min over the group's heads of the fresh-range start."""
    bpe, d, G, B = w.bytes_per_elem, w.head_dim, w.group, w.band
    keys = 0
    for b in range(w.batch):
        n = int(n_ctx[b])
        for g in range(w.n_kv_heads):
            mn = match_n[b, g * G:(g + 1) * G]
            s = np.where(mn >= 0, np.maximum(0, mn - B), 0)
            keys += n - int(s.min())
    kv = keys * 2 * d * bpe
    hq = w.batch * w.n_q_heads
    hits = int((match_n >= 0).sum())
    ring_q = int(np.minimum(ring_count, w.window).sum()) * (d * bpe + 8)
    reused = hits * (d * 4 + 8)
    entry = hq * (d * bpe + d * 4 + 16)
    qo = hq * (d * bpe + d * 4)                       # q in, out
    append = w.batch * w.n_kv_heads * 2 * d * bpe * 2  # read k/v_new, write cache
    return kv + ring_q + reused + entry + qo + append, kv, keys


# ---------------------------------------------------------------------------
# one timed point
# ---------------------------------------------------------------------------

class Layer:
    def __init__(self, w, inp, n_steps, max_context, kv_layout=0):
        import torch
        from kv_cache_reuse_amd import binding as B
        self.w, self.inp = w, inp
        if w.page_size:
            # paged cache: the stream's page table (16-token pages from a
            # shared, shuffled pool)
            cfg = B.config_from_workload(w, n_pages=int(inp.n_pages),
                                         max_pages_per_seq=int(inp.page_table.shape[1]),
                                         kv_layout=kv_layout)
            self.sess = B.MacSession(cfg, page_table=inp.page_table)
        else:
            cfg = B.config_from_workload(w, max_context=max_context, kv_layout=kv_layout)
            self.sess = B.MacSession(cfg)
        dev = torch.device("cuda")
        self.K = inp.k.to(dev)
        self.V = inp.v.to(dev)
        self.ctx = [int(c) for c in inp.contexts]
        self.q = inp.q.to(dev)
        self.n_steps = n_steps
        self.t = 0
        bidx = torch.arange(w.batch, device=dev)
        T = inp.q.shape[0]
        pos = torch.tensor(self.ctx, device=dev)[:, None] + torch.arange(T, device=dev)[None]
        # per-step appended k/v, gathered once: [T, batch, Hkv, d]
        self.k_new = self.K[bidx[:, None], :, pos].permute(1, 0, 2, 3).contiguous()
        self.v_new = self.V[bidx[:, None], :, pos].permute(1, 0, 2, 3).contiguous()
        hq = w.n_q_heads
        self.match_n = torch.empty((T, w.batch, hq), dtype=torch.int32, device=dev)
        self.out = torch.empty((T, w.batch, hq, w.head_dim), dtype=torch.float32, device=dev)

    def prefill(self, upto=None):
        for b in range(self.w.batch):
            n = self.ctx[b] if upto is None else upto
            self.sess.prefill(b, self.K[b, :, :n], self.V[b, :, :n])

    def step(self, stream=None, separate=False):
        from kv_cache_reuse_amd import binding as B
        t = self.t
        s = self.sess
        st = s._s() if stream is None else stream
        if separate:
            # mac_append_kv, then mac_decode_step: two library calls
            B.mac_append_kv(s.ctx, s.k_cache.data_ptr(), s.v_cache.data_ptr(), s._pt(),
                            self.k_new[t].data_ptr(), self.v_new[t].data_ptr(), st)
            B.mac_decode_step(s.ctx, self.q[t].data_ptr(), s.k_cache.data_ptr(),
                              s.v_cache.data_ptr(), s._pt(), self.out[t].data_ptr(),
                              self.match_n[t].data_ptr(), 0, st)
        else:
            # append + match + split-K attention + merge: one library call
            B.mac_decode_step_append(s.ctx, self.q[t].data_ptr(), self.k_new[t].data_ptr(),
                                     self.v_new[t].data_ptr(), s.k_cache.data_ptr(),
                                     s.v_cache.data_ptr(), s._pt(), self.out[t].data_ptr(),
                                     self.match_n[t].data_ptr(), 0, st)
        self.t += 1

    def append_only(self, stream):
        """mac_append_kv of the next token alone (no decode)."""
        from kv_cache_reuse_amd import binding as B
        t = self.t
        s = self.sess
        B.mac_append_kv(s.ctx, s.k_cache.data_ptr(), s.v_cache.data_ptr(), s._pt(),
                        self.k_new[t].data_ptr(), self.v_new[t].data_ptr(), stream)
        self.t += 1


def layer_inputs(w, p_jump, per_layer, layer, inputs_cache, seed_hist=0, jumps=None):
    """Inputs of one layer copy: the workload's draws for `per_layer` decode
    steps (keys and values cached per (workload, layer, per_layer)), with a
    query stream of seed_hist + per_layer tokens whose first seed_hist are
    the last prefill positions (seeded into the ring before decoding).
    `jumps` [per_layer] bool: an explicit jump schedule for the decode
    tokens (none in the seeded history)."""
    from synth.streams import make_inputs, make_q_stream
    key = (w.name, w.batch, w.n_kv_heads, layer, per_layer)
    if inputs_cache is not None and key in inputs_cache:
        base = inputs_cache[key]
    else:
        base = make_inputs(w, p_jump=p_jump, layer=layer, steps=per_layer)
        if inputs_cache is not None:
            inputs_cache[key] = base
    sched = None
    if jumps is not None:
        sched = np.concatenate([np.zeros(seed_hist, bool), np.asarray(jumps, bool)])
    q, q64 = make_q_stream(w, p_jump=p_jump, layer=layer, steps=seed_hist + per_layer,
                           jumps=sched)
    inp = base.__class__(**{**base.__dict__, "q": q[seed_hist:], "q64": q64[seed_hist:]})
    return inp, (q[:seed_hist] if seed_hist else None)


def make_layers(w, p_jump, per_layer, layers, inputs_cache, context=None, prefill_upto=None,
                seed_hist=0, jumps=None, kv_layout=0):
    """`layers` layer copies, prefilled (and, with seed_hist > 0, their rings
    seeded with the queries of the last seed_hist prefill positions).
    jumps: [layers][per_layer] bool schedules, or None for Bernoulli(p)."""
    import torch
    Ls = []
    for l in range(layers):
        inp, hist = layer_inputs(w, p_jump, per_layer, l, inputs_cache, seed_hist,
                                 None if jumps is None else jumps[l])
        if prefill_upto is not None:
            inp = inp.__class__(**{**inp.__dict__, "contexts": np.full(w.batch, prefill_upto)})
        mc = int(inp.contexts.max()) + per_layer if context is None else context
        L = Layer(w, inp, per_layer, max_context=mc, kv_layout=kv_layout)
        L.hist = hist
        Ls.append(L)
    for L in Ls:
        L.prefill()
        if L.hist is not None:
            L.sess.seed(L.hist.to(torch.device("cuda")).contiguous())
    return Ls


def layer_jump_schedules(p, steps, warmup, layers, per_layer):
    """Evenly spaced jumps at rate p over the timed steps (and, separately,
    over the warm-up), dealt to the layer copies in the round-robin order the
    steps visit them: the timed steps then hold floor or ceil of p * steps
    jumps whatever their number."""
    from synth.streams import even_jumps
    J = np.concatenate([even_jumps(p, 0, warmup), even_jumps(p, 0, steps)])
    out = []
    for l in range(layers):
        m = np.zeros(per_layer, bool)
        mine = J[l::layers]
        m[:len(mine)] = mine
        out.append(m)
    return out


def run_point(w, p_jump, steps, warmup, layers, kernel_timing=False, graph=True,
              context=None, prefill_upto=None, inputs_cache=None, per_step=False,
              seeded=False, kv_layout=0, separate=False):
    """warmup + steps decode steps, round-robin over `layers` layer copies.

    The warmup runs eagerly.  With `graph` the timed steps are captured into
    one HIP graph (through torch.cuda.CUDAGraph, on the capture stream) and
    the graph is replayed exactly once inside the timed region; otherwise
    they are launched eagerly.  `kernel_timing` (eager only) brackets every
    split-K attention launch with HIP events on the step's stream.  With
    `per_step` (eager) every step is bracketed by events too and the
    durations come back as the fifth value.  `seeded`: every layer's ring is
    seeded with W prefill queries and the jumps follow the evenly spaced
    schedule (so that a short run sees the jump rate p exactly)."""
    import torch
    from kv_cache_reuse_amd import binding as B
    per_layer = (steps + warmup + layers - 1) // layers + 1
    jumps = layer_jump_schedules(p_jump, steps, warmup, layers, per_layer) if seeded else None
    Ls = make_layers(w, p_jump, per_layer, layers, inputs_cache, context, prefill_upto,
                     seed_hist=w.window if seeded else 0, jumps=jumps, kv_layout=kv_layout)
    torch.cuda.synchronize()
    order = [i % layers for i in range(warmup + steps)]
    for i in order[:warmup]:
        Ls[i].step(separate=separate)
    torch.cuda.synchronize()
    starts = [L.t for L in Ls]
    use_graph = graph and not kernel_timing and not per_step
    g = None
    if use_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            cs = torch.cuda.current_stream().cuda_stream
            for i in order[warmup:]:
                Ls[i].step(stream=cs, separate=separate)
        torch.cuda.synchronize()
    if kernel_timing:
        for L in Ls:
            B.mac_profile_enable(L.sess.ctx, True)
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    marks = []
    e0.record(stream)
    if use_graph:
        g.replay()
    else:
        for i in order[warmup:]:
            if per_step:
                ea = torch.cuda.Event(enable_timing=True)
                eb = torch.cuda.Event(enable_timing=True)
                ea.record(stream)
                Ls[i].step(separate=separate)
                eb.record(stream)
                marks.append((i, Ls[i].t - 1, ea, eb))
            else:
                Ls[i].step(separate=separate)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    step_us = [(i, t, 1e3 * ea.elapsed_time(eb)) for i, t, ea, eb in marks]
    kms, klaunch = 0.0, 0
    if kernel_timing:
        for L in Ls:
            a, n = B.mac_profile_read(L.sess.ctx)
            kms += a
            klaunch += n
            B.mac_profile_enable(L.sess.ctx, False)
    recs = []
    mns = []
    hist = w.window if seeded else 0
    for li, L in enumerate(Ls):
        mn = L.match_n[:L.t].cpu().numpy()
        mns.append(mn)
        for t in range(starts[li], L.t):
            n_ctx = L.inp.contexts + t + 1
            cnt = np.full((w.batch, w.n_q_heads), min(t + hist, w.window))
            recs.append((n_ctx, mn[t], cnt))
    classes = [(("all_hit" if (mns[i][t] >= 0).all() else
                 "all_miss" if (mns[i][t] < 0).all() else "mixed"), us)
               for i, t, us in step_us]
    # one record per timed step (per_step): decisions, bytes and time
    steplog = []
    for (i, t, us), (cls, _) in zip(step_us, classes):
        mn = mns[i][t]
        n_ctx = Ls[i].inp.contexts + t + 1
        cnt = np.full((w.batch, w.n_q_heads), min(t + hist, w.window))
        tot, _, keys = step_bytes(w, n_ctx, mn, cnt)
        g = (mn >= 0).reshape(w.batch, w.n_kv_heads, w.group).all(axis=2)
        steplog.append({"layer": int(i), "step": int(t), "n": [int(x) for x in n_ctx],
                        "class": cls, "us": float(us), "hit_rate": float((mn >= 0).mean()),
                        "group_all_hit": float(g.mean()), "matched_n": mn.tolist(),
                        "kv_keys": int(keys), "bytes": int(tot)})
    del g
    for L in Ls:
        L.sess.close()
    del Ls
    torch.cuda.empty_cache()
    if per_step:
        return ms, recs, kms, klaunch, classes, steplog
    return ms, recs, kms, klaunch


def latency_classes(w, p_jump, steps, warmup, layers, inputs_cache, seeded=False, log_path=None):
    """Per-step latency (HIP events around each eager step) by the step's
    decisions: every head hit, every head missed, or mixed.  With log_path,
    one JSON line per timed step is appended there (workload, layer copy,
    step, context lengths, decision class, µs, head and group hit rates, the
    matched context length of every head (-1 on a miss), KV keys read and
    algorithmic bytes)."""
    out = run_point(w, p_jump, steps, warmup, layers, graph=False, inputs_cache=inputs_cache,
                    per_step=True, seeded=seeded)
    if log_path:
        with open(log_path, "a") as fh:
            for rec in out[5]:
                fh.write(json.dumps({"workload": w.name, "p_jump": p_jump, **rec}) + "\n")
    res = {}
    for cls in ("all_hit", "mixed", "all_miss"):
        v = np.array([us for c, us in out[4] if c == cls])
        if len(v):
            res[cls] = {"steps": int(len(v)), "p10_us": float(np.percentile(v, 10)),
                        "p50_us": float(np.percentile(v, 50)),
                        "p90_us": float(np.percentile(v, 90))}
    return res


def seeding_cost(w, cache):
    """Time mac_seed_ring at the headline shape for the last prefill
    position and for a full window (each position is one miss-path step),
    and report whether the first decode step after it hits."""
    import torch
    from synth.streams import make_q_stream
    res = []
    for n_hist in (1, w.window):
        Ls = make_layers(w, 0.0, 4, 1, cache)
        L = Ls[0]
        q, _ = make_q_stream(w, p_jump=0.0, layer=7, steps=n_hist + 1)
        dev = torch.device("cuda")
        hist = q[:n_hist].to(dev).contiguous()
        L.q = q[n_hist:].to(dev).contiguous()
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        L.sess.seed(hist)
        e1.record(stream)
        L.step()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        first_hit = float((L.match_n[0] >= 0).float().mean().item())
        res.append({"n_hist": n_hist, "ms": ms, "us_per_position": 1e3 * ms / n_hist,
                    "first_step_hit_rate": first_hit})
        log(f"  seed {n_hist} positions: {ms:.3f} ms, first decode step hit rate {first_hit:.2f}")
        L.sess.close()
        del Ls, L
        torch.cuda.empty_cache()
    return res


def chain_depths(match_n, contexts):
    """Reuse-chain depth of the entry each (step, sequence, head) pushes: 0
    after a miss, else one more than the depth of the entry it reused (found
    by its context length).  match_n: [T, batch, Hq]; rings start empty."""
    T, nb, hq = match_n.shape
    depth = np.zeros((T, nb, hq), np.int64)
    for b in range(nb):
        for h in range(hq):
            by_n = {}
            for t in range(T):
                m = int(match_n[t, b, h])
                d = by_n[m] + 1 if m >= 0 else 0
                depth[t, b, h] = d
                by_n[int(contexts[b]) + t + 1] = d
    return depth


def drift_run(w, steps, inputs=None):
    """Run one query stream through two sessions on the same KV: the MAC
    configuration of `w`, and W = 0, which never matches and so computes
    plain attention over every key.  Returns per (step, sequence, head) the
    largest |out_MAC - out_dense| over the head dimension, the MAC side's
    matched context lengths, and the inputs."""
    import torch
    from kv_cache_reuse_amd import binding as B
    from synth.streams import make_inputs
    inp = make_inputs(w, steps=steps) if inputs is None else inputs
    dev = torch.device("cuda")
    mc = int(inp.contexts.max()) + steps
    sess = [B.MacSession(B.config_from_workload(x, max_context=mc))
            for x in (w, w.replace(window=0))]
    K, V = inp.k.to(dev), inp.v.to(dev)
    for s_ in sess:
        for b in range(w.batch):
            n0 = int(inp.contexts[b])
            s_.prefill(b, K[b, :, :n0], V[b, :, :n0])
    q = inp.q.to(dev)
    bidx = torch.arange(w.batch, device=dev)
    ctx_t = torch.tensor([int(c) for c in inp.contexts], device=dev)
    dmax = torch.empty((steps, w.batch, w.n_q_heads), dtype=torch.float32, device=dev)
    match_n = torch.empty((steps, w.batch, w.n_q_heads), dtype=torch.int32, device=dev)
    for t in range(steps):
        pos = ctx_t + t
        k_new = K[bidx, :, pos].contiguous()
        v_new = V[bidx, :, pos].contiguous()
        o_mac, m_mac, _ = sess[0].decode_append(q[t], k_new, v_new)
        o_den, _, _ = sess[1].decode_append(q[t], k_new, v_new, match_ctx=False, dist=False)
        dmax[t] = (o_mac - o_den).abs().amax(dim=-1)
        match_n[t] = m_mac
    torch.cuda.synchronize()
    res = dmax.cpu().numpy(), match_n.cpu().numpy(), inp
    for s_ in sess:
        s_.close()
    torch.cuda.empty_cache()
    return res


DEPTH_BUCKETS = ((0, 0), (1, 1), (2, 3), (4, 7), (8, 15), (16, 31), (32, 1 << 30))


def drift_summary(dmax, match_n, contexts):
    depth = chain_depths(match_n, contexts)
    rows = []
    for lo, hi in DEPTH_BUCKETS:
        sel = (depth >= lo) & (depth <= hi)
        if sel.any():
            rows.append({"depth": [lo, hi if hi < (1 << 30) else None], "count": int(sel.sum()),
                         "max": float(dmax[sel].max()), "mean": float(dmax[sel].mean())})
    return {"hit_rate": float((match_n >= 0).mean()), "max_drift": float(dmax.max()),
            "max_depth": int(depth.max()), "by_depth": rows}


def drift_sweep(steps):
    """Drift of MAC from dense attention along chains of hits on a 16K
    continuous-generation stream, for tau in {0.30, 0.32, 0.35, 0.5} sqrt(d)
    (consecutive queries of the stream lie about 0.32 sqrt(d) apart) and B in
    {64, 256, 1024}."""
    from synth.streams import workload
    base = workload("gen_16k")
    out = []
    for f in (0.30, 0.32, 0.35, 0.5):
        for band in (64, 256, 1024):
            w = base.replace(tau=f * math.sqrt(base.head_dim), band=band)
            dmax, mn, inp = drift_run(w, steps)
            s = drift_summary(dmax, mn, inp.contexts)
            s.update({"tau_over_sqrt_d": f, "band": band})
            out.append(s)
            deep = s["by_depth"][-1]
            log(f"  tau {f:.2f} sqrt(d), B {band}: hit {s['hit_rate']:.3f}, max drift "
                f"{s['max_drift']:.2e}, deepest chain {s['max_depth']} "
                f"(depth {deep['depth'][0]}+: max {deep['max']:.2e})")
    return out


def multilayer(layers=32, tokens=32):
    """Every layer of a token in one HIP graph: `layers` layer copies of the
    16K-context 8B shape (own caches and rings), visited in order for each
    token, `tokens` tokens captured in one graph and replayed once.  Reports
    the time per token across all layers and per layer step."""
    from synth.streams import workload
    w = workload("gen_16k")
    out = []
    cache = {}
    for p in (0.05, 1.0):
        steps = layers * tokens
        ms, recs, _, _ = run_point(w, p, steps, layers * 2, layers, inputs_cache=cache,
                                   seeded=True)
        st = summarize(w, ms, recs, steps)
        out.append({"p_jump": p, "layers": layers, "tokens": tokens,
                    "us_per_token_all_layers": 1e3 * ms / tokens,
                    "us_per_layer_step": 1e3 * ms / steps, "hit_rate": st["hit_rate"]})
        log(f"  {layers} layers, p={p}: {1e3 * ms / tokens:.0f} us per token "
            f"({1e3 * ms / steps:.2f} us per layer step, hit {st['hit_rate']:.3f})")
    return out


# One MQA layer's cache is 67 MB: eight copies (537 MB) keep the steps from
# finding their keys in the 256 MB last-level cache.
MQA_LAYERS = 8


def mqa(steps, warmup, cache=None):
    """MQA at the headline context: 32 query heads over one KV head (one
    32-head group: a match launch, then one pass over the tiles for all its
    heads).  Miss path (graph-replayed steps, and the attention kernel timed
    by HIP events in an eager run) and the all-hit step."""
    from synth.streams import workload
    w = workload("8b_128k", n_kv_heads=1)
    # step time from the graph replay; the step kernel's duration from an
    # eager run with HIP events around it
    ms, recs, _, _ = run_point(w, 1.0, steps, warmup, MQA_LAYERS, inputs_cache=cache)
    st = summarize(w, ms, recs, steps)
    _, recs_k, kms, kl = run_point(w, 1.0, steps, warmup, MQA_LAYERS, kernel_timing=True,
                                   inputs_cache=cache)
    keys = sum(step_bytes(w, *r)[2] for r in recs_k)
    kbytes = keys * 2 * w.head_dim * w.bytes_per_elem / max(kl, 1)
    msh, rh, _, _ = run_point(w, 0.0, steps, warmup, MQA_LAYERS, inputs_cache=cache, seeded=True)
    sh = summarize(w, msh, rh, steps)
    res = {"workload": "8b_128k with 1 KV head: 32 query heads in one group (a match launch, then "
                       f"one pass over the tiles for all 32 heads); {MQA_LAYERS} layer copies "
                       "visited in turn",
           "miss_us_per_step": st["us_per_step"], "miss_kernel_us": 1e3 * kms / max(kl, 1),
           "miss_kernel_GBps": kbytes / (kms / 1e3 / max(kl, 1)) / 1e9,
           "hit_us_per_step": sh["us_per_step"], "hit_rate": sh["hit_rate"]}
    log(f"  MQA miss: {res['miss_us_per_step']:.1f} us/step (kernel {res['miss_kernel_us']:.1f} us, "
        f"{res['miss_kernel_GBps']:.0f} GB/s of KV); all-hit {res['hit_us_per_step']:.2f} us/step")
    return res


CONFIG_POINTS = {
    # key: (workload, overrides, layer copies visited in turn, description)
    "8b_32k": ("8b_32k", {}, 4,
               "8b_32k: batch 1, 32 query / 8 KV heads, d 128, bf16 K/V, 32768-key context, "
               "W 32, B 256, tau calibrated to 80 % head hits, jump probability 0.1"),
    "paged_b8": ("paged_b8", {}, 2,
                 "paged_b8: batch 8, contexts 16K-64K keys (ragged), 32 query / 8 KV heads, "
                 "d 128, bf16 K/V, paged cache (16-token pages), W 32, B 128, jump probability 0.1"),
    "70b_128k": ("70b_128k", {}, 1,
                 "70b_128k: batch 4, 64 query / 8 KV heads (G 8), d 128, bf16 K/V with 1 % "
                 "outlier keys x8, 131072-key context, W 64, B 256, rho U[0.8, 0.99] per query "
                 "head, jump probability 0.1"),
    "70b_128k_rho_per_kv": ("70b_128k", dict(rho_per_kv=True), 1,
                            "70b_128k with rho drawn per KV head (shared by its 8 query heads)"),
}


def config_point(key, steps, warmup, cache, miss=True, classes=False, streams=True,
                 log_path=None):
    """One workload of the configs: its miss path (every token jumps), graph-
    replayed, with the step kernel timed by HIP events in an eager run (that
    kernel's roofline at this shape); its own query stream (its jump
    probability as an evenly spaced schedule, rings seeded with W prefill
    queries); and the step when every head hits (no jumps)."""
    from synth.streams import workload
    name, kw, layers, desc = CONFIG_POINTS[key]
    w = workload(name, **kw)
    res = {"workload": desc, "layers_rotated": layers}
    if miss:
        ms, recs, _, _ = run_point(w, 1.0, steps, warmup, layers, inputs_cache=cache, seeded=True)
        st = summarize(w, ms, recs, steps)
        _, recs_k, kms, kl = run_point(w, 1.0, steps, warmup, layers, kernel_timing=True,
                                       inputs_cache=cache, seeded=True)
        keys = sum(step_bytes(w, *r)[2] for r in recs_k)
        kbytes = keys * 2 * w.head_dim * w.bytes_per_elem / max(kl, 1)
        kus = 1e3 * kms / max(kl, 1)
        res["miss"] = {"us_per_step": st["us_per_step"], "eff_GBps": st["eff_GBps"],
                       "pct_hbm_peak": st["pct_hbm_peak"], "kernel_us": kus,
                       "kernel_bytes_per_launch": kbytes, "kernel_GBps": kbytes / kus / 1e3,
                       "kernel_frac_hbm_peak": kbytes / kus / 1e3 / HBM_PEAK_GBPS,
                       "launches": kl}
        log(f"  {key} miss: {st['us_per_step']:.1f} us/step ({st['eff_GBps']:.0f} GB/s), step "
            f"kernel {kus:.1f} us = {kbytes / kus / 1e3:.0f} GB/s "
            f"({100 * kbytes / kus / 1e3 / HBM_PEAK_GBPS:.1f} % of 8 TB/s)")
    for label, p in ((("stream", w.p_jump), ("all_hit", 0.0)) if streams else ()):
        msp, rp, _, _ = run_point(w, p, steps, warmup, layers, inputs_cache=cache, seeded=True)
        sp = summarize(w, msp, rp, steps)
        res[label] = {"p_jump": p, "us_per_step": sp["us_per_step"],
                      "us_per_token": sp["us_per_token"], "eff_GBps": sp["eff_GBps"],
                      "dense_equiv_GBps": sp["dense_equiv_GBps"], "hit_rate": sp["hit_rate"],
                      "group_all_hit": sp["group_all_hit"]}
        log(f"  {key} p={p}: {sp['us_per_step']:.1f} us/step (hit {sp['hit_rate']:.3f}, group "
            f"all-hit {sp['group_all_hit']:.3f}, dense-equivalent {sp['dense_equiv_GBps']:.0f} GB/s)")
    if classes:
        res["latency_classes"] = latency_classes(w, w.p_jump, steps, warmup, layers, cache,
                                                 seeded=True, log_path=log_path)
        for k, v in res["latency_classes"].items():
            log(f"  {key} {k}: {v['steps']} steps, p10/p50/p90 {v['p10_us']:.1f} / "
                f"{v['p50_us']:.1f} / {v['p90_us']:.1f} us")
    return res


def read_ceiling():
    """HBM read rate of a plain streaming-read kernel (libmac_bw.so) over a
    2 GiB buffer (8x the last-level cache): the best of a few grid sizes,
    with default and with non-temporal loads, each timed with HIP events."""
    import ctypes
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "kv_cache_reuse_amd", "libmac_bw.so"))
    lib.mac_bw_read.restype = ctypes.c_int
    lib.mac_bw_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p,
                                ctypes.c_uint32, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    nbytes = 2 << 30
    buf = torch.ones(nbytes // 2, dtype=torch.bfloat16, device="cuda")
    sink = torch.zeros(16384, dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    best = {0: (0.0, 0), 1: (0.0, 0)}
    for nt in (0, 1):
        for blocks in (512, 1024, 2048, 4096, 8192, 16384):
            for rep_ in range(4):
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                st = lib.mac_bw_read(buf.data_ptr(), nbytes, sink.data_ptr(), 0x9e3779b9, blocks,
                                     nt, stream.cuda_stream)
                e1.record(stream)
                torch.cuda.synchronize()
                if st != 0:
                    raise RuntimeError(f"mac_bw_read failed with HIP error {st}")
                if rep_ > 0:
                    gbps = nbytes / (e0.elapsed_time(e1) / 1e3) / 1e9
                    best[nt] = max(best[nt], (gbps, blocks))
    del buf
    torch.cuda.empty_cache()
    top = max(best.values())
    return {"GBps": top[0], "blocks": top[1], "bytes": nbytes,
            "pct_hbm_peak": 100.0 * top[0] / HBM_PEAK_GBPS,
            "default_loads_GBps": best[0][0], "nontemporal_loads_GBps": best[1][0]}


def summarize(w, ms, recs, steps):
    tot = kv = keys = 0
    hits = []
    grp_all = []
    dense = 0
    for n_ctx, mn, cnt in recs:
        a, b_, k = step_bytes(w, n_ctx, mn, cnt)
        tot += a
        kv += b_
        keys += k
        hits.append((mn >= 0).mean())
        g = (mn >= 0).reshape(w.batch, w.n_kv_heads, w.group).all(axis=2)
        grp_all.append(g.mean())
        dense += int(n_ctx.sum()) * w.n_kv_heads * 2 * w.head_dim * w.bytes_per_elem
    sec = ms / 1e3
    return {
        "hit_rate": float(np.mean(hits)),
        "group_all_hit": float(np.mean(grp_all)),
        "us_per_token": 1e3 * ms / steps / w.batch,
        "us_per_step": 1e3 * ms / steps,
        "eff_GBps": tot / sec / 1e9,
        "kv_GBps": kv / sec / 1e9,
        "pct_hbm_peak": 100.0 * tot / sec / 1e9 / HBM_PEAK_GBPS,
        "dense_equiv_GBps": dense / sec / 1e9,
        "bytes_per_step": tot / steps,
        "kv_keys_per_step": keys / steps,
    }


# ---------------------------------------------------------------------------
# cpu baseline: the oracle on a bounded sample
# ---------------------------------------------------------------------------

def cpu_baseline(w, sample_steps):
    from threadpoolctl import threadpool_limits, threadpool_info
    from oracle import mac_oracle as M
    from synth.streams import make_inputs
    cores = len(os.sched_getaffinity(0))
    inp = make_inputs(w, p_jump=1.0, steps=sample_steps)
    K = inp.k.float().numpy()
    V = inp.v.float().numpy()
    orc = M.MacOracle.for_workload(w)
    with threadpool_limits(limits=cores):
        used = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        t0 = time.perf_counter()
        recs = []
        for t in range(sample_steps):
            n = int(inp.contexts[0]) + t + 1
            r = orc.step(0, inp.q64[t, 0], K[0], V[0], n)
            recs.append((np.array([n]), r.match_n.reshape(1, -1).astype(np.int64),
                         np.full((1, w.n_q_heads), min(t, w.window))))
        sec = time.perf_counter() - t0
    tot = sum(step_bytes(w, *r)[0] for r in recs)
    return {
        "value": tot / sec / 1e9, "unit": "GB/s", "cores": int(used), "kind": "oracle",
        "sample": (f"{sample_steps} decode steps of the {w.name} stream at jump probability 1 "
                   f"(all misses, every KV group, {int(inp.contexts[0])}-key context), "
                   f"fp64 NumPy oracle; {sec:.1f} s, {sec / sample_steps * 1e6:.0f} us/step"),
        "us_per_step": sec / sample_steps * 1e6,
    }


def cpu_classes(sample_steps, single_steps):
    """The oracle per decision class on the 8b_32k stream, whose calibrated
    tau makes steps where every head hits, some heads hit and every head
    misses all occur.  Rings seeded with W prefill queries (untimed, the
    oracle's own seeding).  Each step timed alone: us/step and algorithmic
    GB/s per class on all host threads, and the mean of a shorter sample on
    one thread."""
    from threadpoolctl import threadpool_info, threadpool_limits
    from oracle import mac_oracle as M
    from synth.streams import make_inputs, make_q_stream, workload
    w = workload("8b_32k")
    W = w.window
    cores = len(os.sched_getaffinity(0))
    T = max(sample_steps, single_steps)
    inp = make_inputs(w, steps=T)
    _, q64 = make_q_stream(w, steps=W + T)
    K = inp.k.float().numpy()
    V = inp.v.float().numpy()
    n0 = int(inp.contexts[0])

    seeded = M.MacOracle.for_workload(w)
    with threadpool_limits(limits=cores):
        seeded.seed(0, q64[:W, 0], K[0], V[0], n0)

    def run(steps, threads):
        orc = copy.deepcopy(seeded)
        out = []
        with threadpool_limits(limits=threads):
            used = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
            for t in range(steps):
                n = n0 + t + 1
                t0 = time.perf_counter()
                r = orc.step(0, q64[W + t, 0], K[0], V[0], n)
                sec = time.perf_counter() - t0
                mn = r.match_n.reshape(1, -1).astype(np.int64)
                b = step_bytes(w, np.array([n]), mn, np.full((1, w.n_q_heads), W))[0]
                cls = "all_hit" if r.hit.all() else "all_miss" if not r.hit.any() else "mixed"
                out.append((cls, sec, b))
        return out, used

    rows, used = run(sample_steps, cores)
    per = {}
    for cls in ("all_hit", "mixed", "all_miss"):
        sel = [(sec, b) for c, sec, b in rows if c == cls]
        if sel:
            sec = sum(x for x, _ in sel)
            per[cls] = {"steps": len(sel), "us_per_step": 1e6 * sec / len(sel),
                        "GBps": sum(b for _, b in sel) / sec / 1e9}
    one, used1 = run(single_steps, 1)
    sec1 = sum(x for _, x, _ in one)
    return {
        "per_class": {"workload": "8b_32k stream (jump probability 0.1, tau for 80 % head "
                                  "hits), rings seeded; each step timed alone",
                      "threads": int(used), "classes": per},
        "single_thread": {"workload": "8b_32k stream, the same steps", "threads": int(used1),
                          "steps": single_steps, "us_per_step": 1e6 * sec1 / single_steps,
                          "GBps": sum(b for _, _, b in one) / sec1 / 1e9},
    }


def kernel_sha256():
    h = hashlib.sha256()
    for path in KERNEL_SRCS:
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def kernel_traffic():
    """HBM traffic of the step kernel from the committed counter summary,
    or None if the kernel source changed since the counters were taken."""
    if not os.path.exists(PROFILE_TRAFFIC):
        return None
    with open(PROFILE_TRAFFIC) as f:
        tr = json.load(f)
    if tr.get("kernel_sha256") != kernel_sha256():
        return None
    return tr.get("bytes_per_launch")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256)
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--layers", type=int, default=2)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-flatness", action="store_true")
    ap.add_argument("--no-latency", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true")
    ap.add_argument("--no-seed", action="store_true")
    ap.add_argument("--no-drift", action="store_true")
    ap.add_argument("--no-multilayer", action="store_true")
    ap.add_argument("--no-mqa", action="store_true")
    ap.add_argument("--no-batch", action="store_true")
    ap.add_argument("--no-c2", action="store_true")
    ap.add_argument("--no-c5", action="store_true")
    ap.add_argument("--no-layout", action="store_true")
    ap.add_argument("--no-calls", action="store_true")
    ap.add_argument("--step-log", type=str, default="",
                    help="append one JSON line per timed step of the latency-class runs here")
    ap.add_argument("--drift-steps", type=int, default=2048)
    ap.add_argument("--cpu-steps", type=int, default=50)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--points", type=str, default="")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first copy 512 MiB device-to-device (counter calibration)")
    ap.add_argument("--config-only", type=str, default="",
                    help="run only this config point (for profiling its kernels) and print it")
    ap.add_argument("--miss-only", action="store_true",
                    help="with --config-only: the miss path only")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the decode step "
              "is measured on one device; sharding is design-only.", file=sys.stderr)
        sys.exit(2)

    import torch
    from synth.streams import SWEEP_P_JUMP, workload
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    w = workload("8b_128k")
    cache = {}
    if args.copy_calibration:
        # a plain device copy of known size, for scaling hardware byte counters
        src = torch.empty(COPY_CAL_BYTES // 2, dtype=torch.bfloat16, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: {COPY_CAL_BYTES} bytes read and written")
        del src, dst

    if args.config_only:
        key = args.config_only
        if key not in CONFIG_POINTS:
            print(f"unknown config point {key}; one of {sorted(CONFIG_POINTS)}", file=sys.stderr)
            sys.exit(2)
        log(f"config point {key} only")
        res = config_point(key, args.steps, args.warmup, cache,
                           miss=key != "70b_128k_rho_per_kv", streams=not args.miss_only)
        print(json.dumps({"config_only": key, **res}), flush=True)
        return

    # ---- headline: miss path (jump probability 1)
    log(f"headline: {w.name} p_jump=1 steps={args.steps} warmup={args.warmup} layers={args.layers}")
    ms, recs, _, _ = run_point(w, 1.0, args.steps, args.warmup, args.layers,
                               inputs_cache=cache, seeded=True)
    head = summarize(w, ms, recs, args.steps)
    log(f"headline (graph): {head['us_per_token']:.1f} us/token, {head['eff_GBps']:.0f} GB/s")
    ms_e, recs_e, _, _ = run_point(w, 1.0, args.steps, args.warmup, args.layers, graph=False,
                                   inputs_cache=cache, seeded=True)
    head_eager = summarize(w, ms_e, recs_e, args.steps)
    log(f"headline (eager): {head_eager['us_per_token']:.1f} us/token, "
        f"{head_eager['eff_GBps']:.0f} GB/s")

    # ---- step kernel timing (HIP events around each launch, on its stream)
    log("kernel timing pass")
    ms_k, recs_k, kms, klaunch = run_point(w, 1.0, args.steps, args.warmup, args.layers,
                                           kernel_timing=True, inputs_cache=cache, seeded=True)
    keys = sum(step_bytes(w, *r)[2] for r in recs_k)
    kern_bytes = keys * 2 * w.head_dim * w.bytes_per_elem / max(klaunch, 1)
    kern_sec = kms / 1e3 / max(klaunch, 1)
    achieved = kern_bytes / kern_sec / 1e9
    roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBPS, "traffic": kernel_traffic(),
                "kernel": ROOFLINE_KERNEL,
                "avg_launch_us": kern_sec * 1e6, "bytes_per_launch": kern_bytes,
                "launches": klaunch}
    # HBM traffic over the algorithmic bytes (1.0: no byte fetched twice)
    roofline["traffic_over_algorithmic"] = (roofline["traffic"] / kern_bytes
                                            if roofline["traffic"] else None)
    log(f"kernel: {kern_sec * 1e6:.1f} us/launch, {achieved:.0f} GB/s")

    # ---- the same step kernel on caches in the natural row layout
    layout_ab = None
    if not args.no_layout:
        _, recs_r, kms_r, kl_r = run_point(w, 1.0, args.steps, args.warmup, args.layers,
                                           kernel_timing=True, inputs_cache=cache, seeded=True,
                                           kv_layout=1)
        keys_r = sum(step_bytes(w, *r)[2] for r in recs_r)
        bytes_r = keys_r * 2 * w.head_dim * w.bytes_per_elem / max(kl_r, 1)
        us_r = 1e3 * kms_r / max(kl_r, 1)
        msh_t, rh_t, _, _ = run_point(w, 0.0, args.steps, args.warmup, args.layers,
                                      inputs_cache=cache, seeded=True)
        msh_r, rh_r, _, _ = run_point(w, 0.0, args.steps, args.warmup, args.layers,
                                      inputs_cache=cache, seeded=True, kv_layout=1)
        layout_ab = {"workload": "8b_128k miss path (step kernel, HIP events) and all-hit step",
                     "tiles_kernel_us": kern_sec * 1e6, "rows_kernel_us": us_r,
                     "rows_kernel_GBps": bytes_r / us_r / 1e3,
                     "tiles_all_hit_us_per_step": summarize(w, msh_t, rh_t, args.steps)["us_per_step"],
                     "rows_all_hit_us_per_step": summarize(w, msh_r, rh_r, args.steps)["us_per_step"]}
        log(f"layout A/B: step kernel tiles {kern_sec * 1e6:.1f} us, rows {us_r:.1f} us; all-hit "
            f"step tiles {layout_ab['tiles_all_hit_us_per_step']:.2f} us, rows "
            f"{layout_ab['rows_all_hit_us_per_step']:.2f} us")

    # ---- mac_append_kv and mac_decode_step as two calls against the fused
    # call, and mac_append_kv alone
    calls = None
    if not args.no_calls:
        ms_s, rec_s, _, _ = run_point(w, 1.0, args.steps, args.warmup, args.layers,
                                      inputs_cache=cache, seeded=True, separate=True)
        msh_s, rh_s, _, _ = run_point(w, 0.0, args.steps, args.warmup, args.layers,
                                      inputs_cache=cache, seeded=True, separate=True)
        msh_f, rh_f, _, _ = run_point(w, 0.0, args.steps, args.warmup, args.layers,
                                      inputs_cache=cache, seeded=True)
        k_app, us_app = append_alone(w, args.steps, args.warmup, args.layers, cache)
        calls = {"workload": "8b_128k: miss path and all-hit step, graph-replayed; "
                             "mac_append_kv alone over the same layer copy",
                 "fused_miss_us_per_token": head["us_per_token"],
                 "separate_miss_us_per_token": summarize(w, ms_s, rec_s, args.steps)["us_per_token"],
                 "fused_all_hit_us_per_step": summarize(w, msh_f, rh_f, args.steps)["us_per_step"],
                 "separate_all_hit_us_per_step": summarize(w, msh_s, rh_s, args.steps)["us_per_step"],
                 "append_us": us_app, "append_calls": k_app}
        log(f"calls: miss step fused {calls['fused_miss_us_per_token']:.2f} / separate "
            f"{calls['separate_miss_us_per_token']:.2f} us; all-hit fused "
            f"{calls['fused_all_hit_us_per_step']:.2f} / separate "
            f"{calls['separate_all_hit_us_per_step']:.2f} us; mac_append_kv alone {us_app:.2f} us")

    # ---- hit-rate sweep
    sweep = []
    pts = [float(x) for x in args.points.split(",")] if args.points else list(SWEEP_P_JUMP)
    if not args.no_sweep:
        for p in pts:
            if p == 1.0:
                s = dict(head)
            else:
                log(f"sweep point p_jump={p}")
                msp, rp, _, _ = run_point(w, p, args.steps, args.warmup, args.layers,
                                          inputs_cache=cache, seeded=True)
                s = summarize(w, msp, rp, args.steps)
                mse, re_, _, _ = run_point(w, p, args.steps, args.warmup, args.layers,
                                           graph=False, inputs_cache=cache, seeded=True)
                s["us_per_token_eager"] = summarize(w, mse, re_, args.steps)["us_per_token"]
            if p == 1.0:
                s["us_per_token_eager"] = head_eager["us_per_token"]
            s["p_jump"] = p
            sweep.append(s)
            log(f"  p={p}: hit {s['hit_rate']:.3f} (group {s['group_all_hit']:.3f}) "
                f"{s['us_per_token']:.1f} us/token (eager {s['us_per_token_eager']:.1f})")

    # ---- hit-step latency over context length (no jumps: every step hits)
    flat_steps = []
    if not args.no_flatness:
        flat_steps = hit_step_latency(w, cache)

    # ---- per-step latency by decision class (eager, events around each step)
    lat = None
    if not args.no_latency:
        log("latency classes: p_jump=0.2, eager per-step events")
        lat = latency_classes(w, 0.2, args.steps, args.warmup, args.layers, cache, seeded=True,
                              log_path=args.step_log or None)
        for k, v in lat.items():
            log(f"  {k}: {v['steps']} steps, p10/p50/p90 {v['p10_us']:.1f} / {v['p50_us']:.1f} / "
                f"{v['p90_us']:.1f} us")

    # ---- ring seeding from the prefill
    seed = None
    if not args.no_seed:
        log("ring seeding at 131072 keys")
        seed = seeding_cost(w, cache)

    # ---- drift from dense attention along chains of hits (16K generation)
    drift = None
    if not args.no_drift:
        log(f"drift: gen_16k, {args.drift_steps} steps per point")
        drift = drift_sweep(args.drift_steps)

    # ---- every layer of a token in one graph (16K context, 32 layers)
    multi = None
    if not args.no_multilayer:
        log("multi-layer graph: gen_16k shape, 32 layers")
        multi = multilayer()

    # ---- the other configs: 8B at 32K, the ragged paged batch, the 70B shape
    configs = {}
    cfg_keys = [k for k in CONFIG_POINTS
                if not (k == "8b_32k" and args.no_c2) and not (k == "paged_b8" and args.no_batch)
                and not (k.startswith("70b") and args.no_c5)]
    for key in cfg_keys:
        log(f"config point {key}")
        configs[key] = config_point(key, min(args.steps, 64), min(args.warmup, 8),
                                    cache if key != "paged_b8" else {},
                                    miss=key != "70b_128k_rho_per_kv", classes=key == "8b_32k",
                                    log_path=args.step_log or None)
        if key.startswith("70b"):
            cache = {k: v for k, v in cache.items() if not k[0].startswith("70b")}

    # ---- MQA / groups wider than the 16-head tile
    mq = None
    if not args.no_mqa:
        log("MQA: 32 query heads over 1 KV head at 131072 keys")
        mq = mqa(min(args.steps, 128), args.warmup, {})

    # ---- streaming-read ceiling of this device, same run
    ceil = None
    if not args.no_ceiling:
        ceil = read_ceiling()
        roofline["pct_of_read_ceiling"] = 100.0 * achieved / ceil["GBps"]
        log(f"read ceiling: {ceil['GBps']:.0f} GB/s ({ceil['pct_hbm_peak']:.1f} % of peak; default "
            f"loads {ceil['default_loads_GBps']:.0f}, non-temporal {ceil['nontemporal_loads_GBps']:.0f}); "
            f"step kernel at {roofline['pct_of_read_ceiling']:.1f} % of it")

    cpu = None
    if not args.no_cpu:
        log(f"cpu baseline: oracle, {args.cpu_steps} steps")
        cpu = cpu_baseline(w, args.cpu_steps)
        log(f"cpu baseline: {cpu['value']:.3f} GB/s on {cpu['cores']} threads")
        cpu.update(cpu_classes(48, 12))
        for k, v in cpu["per_class"]["classes"].items():
            log(f"  oracle {k}: {v['steps']} steps, {v['us_per_step']:.0f} us/step")
        log(f"  oracle on one thread: {cpu['single_thread']['us_per_step']:.0f} us/step")

    line = {
        "metric": METRIC,
        "value": head["eff_GBps"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["us_per_step"] / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "8b_128k: decode attention, batch 1, 32 query / 8 KV heads, "
                               "d 128, bf16 K/V, 131072-key context, W 32, B 256, "
                               "tau 0.5*sqrt(128), miss path (jump probability 1)",
                   "batch": 1, "context": 131072, "layers_rotated": args.layers},
        "launch": "timed steps captured in one HIP graph, replayed once",
        "us_per_token": head["us_per_token"],
        "us_per_token_eager": head_eager["us_per_token"],
        "eager_GBps": head_eager["eff_GBps"],
        "pct_hbm_peak": head["pct_hbm_peak"],
        "sweep": sweep,
        "flatness": flat_steps,
        "latency_classes": lat,
        "seeding": seed,
        "drift": drift,
        "multilayer": multi,
        "mqa": mq,
        "configs": configs,
        "layout_ab": layout_ab,
        "calls": calls,
        "read_ceiling": ceil,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


def append_alone(w, steps, warmup, layers, cache):
    """mac_append_kv alone: the calls a layer copy of the headline point can
    take (its decode-step inputs), captured in one HIP graph and replayed
    once.  Returns (calls, us per call)."""
    import torch
    per_layer = (steps + warmup + layers - 1) // layers + 1
    L = make_layers(w, 1.0, per_layer, 1, cache)[0]
    k = per_layer - 1
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        cs = torch.cuda.current_stream().cuda_stream
        for _ in range(k):
            L.append_only(cs)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    stream = torch.cuda.current_stream()
    e0.record(stream)
    g.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / k
    del g
    L.sess.close()
    return k, us


def hit_step_latency(w, cache, steps=128):
    """Latency of steps in which every head hits, per context length.

    Uses a query stream with no jumps (jump probability 0): after the first
    step every head matches its previous query, so each timed step reads the
    band and tail only.  The configured capacity is the same at every context
    (131072 + 512 keys), so the launch grid is identical; only the prefill
    length changes.  Steps are graph-replayed; the mean per step is reported
    with the fraction of (head, step) decisions that hit."""
    out = []
    for n0 in (8192, 16384, 32768, 65536, 131072):
        ms, recs, _, _ = run_point(w, 0.0, steps, 8, 1, inputs_cache=cache,
                                   prefill_upto=n0, context=131072 + 512)
        st = summarize(w, ms, recs, steps)
        out.append({"context": n0, "us_per_step": st["us_per_step"],
                    "hit_rate": st["hit_rate"], "group_all_hit": st["group_all_hit"],
                    "kv_keys_per_step": st["kv_keys_per_step"]})
        log(f"  context {n0}: {st['us_per_step']:.2f} us/step, hit {st['hit_rate']:.3f}")
    return out


if __name__ == "__main__":
    main()
