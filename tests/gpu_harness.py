"""Shared GPU-test plumbing: run a synthetic workload through libmac and
record its outputs for the comparison with the fp64 oracle
(tests/oracle_check.py, re-exported here)."""

from __future__ import annotations

import dataclasses
import sys
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

from tests.oracle_check import (BORDER_REL, OUT_TOL, Report, check_groups,  # noqa: F401
                                check_groups_parallel)


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


@dataclasses.dataclass
class GpuRun:
    out: Dict[int, np.ndarray]        # step -> [batch, Hq, d] float32
    match_n: Dict[int, np.ndarray]    # step -> [batch, Hq] int32
    dist: Dict[int, np.ndarray]       # step -> [batch, Hq] float32
    session: object


def make_session(w, inp, steps: int, max_slices: int = 0, paged: Optional[bool] = None,
                 capacity: Optional[int] = None, workspace=None, kv_layout: int = 0):
    from kv_cache_reuse_amd import binding as B
    paged = bool(w.page_size) if paged is None else paged
    if paged:
        table = inp.page_table
        if capacity:   # more table columns, never read: positions past every context
            pages = -(-capacity // 16)
            if pages > table.shape[1]:
                table = np.pad(table, ((0, 0), (0, pages - table.shape[1])))
        cfg = B.config_from_workload(w.replace(page_size=16), n_pages=int(inp.n_pages),
                                     max_pages_per_seq=int(table.shape[1]),
                                     max_slices=max_slices, kv_layout=kv_layout)
    else:
        table = None
        cfg = B.config_from_workload(w.replace(page_size=0),
                                     max_context=capacity or int(inp.contexts.max()) + steps,
                                     max_slices=max_slices, kv_layout=kv_layout)
    return B.MacSession(cfg, page_table=table, workspace=workspace)


def write_rows(sess, w, K, V, ctx):
    """Write tokens [0, ctx[b]) of every sequence straight into natural-row
    caches (contiguous [batch][Hkv][max_context][d], or paged
    [n_pages][Hkv][16][d] through the page table), then bind the context
    again with those lengths (mac_resume keeps the ring, empty here)."""
    from kv_cache_reuse_amd import binding as B
    cfg = sess.cfg
    assert cfg.kv_layout == B.MAC_KV_ROWS
    d, hkv = cfg.head_dim, cfg.n_kv_heads
    for b in range(w.batch):
        n = ctx[b]
        if cfg.page_size:
            pages = sess.page_table[b, : -(-n // 16)].long()
            kc = sess.k_cache.view(cfg.n_pages, hkv, 16, d)
            vc = sess.v_cache.view(cfg.n_pages, hkv, 16, d)
            kp = torch.zeros((pages.numel() * 16, hkv, d), dtype=K.dtype, device=K.device)
            vp = torch.zeros_like(kp)
            kp[:n] = K[b, :, :n].transpose(0, 1)
            vp[:n] = V[b, :, :n].transpose(0, 1)
            kc[pages] = kp.view(-1, 16, hkv, d).transpose(1, 2)
            vc[pages] = vp.view(-1, 16, hkv, d).transpose(1, 2)
        else:
            kc = sess.k_cache.view(cfg.batch, hkv, cfg.max_context, d)
            vc = sess.v_cache.view(cfg.batch, hkv, cfg.max_context, d)
            kc[b, :, :n] = K[b, :, :n]
            vc[b, :, :n] = V[b, :, :n]
    sess.seq_lens.copy_(torch.tensor(ctx, dtype=torch.int32, device=sess.seq_lens.device))
    torch.cuda.synchronize()
    B.mac_destroy(sess.ctx)
    sess.ctx = B.mac_resume(cfg, sess.ring.data_ptr(), sess.workspace.data_ptr(),
                            sess.seq_lens.data_ptr(), ctx, sess._s())


def step_inputs(w, inp, dev):
    """The step inputs on the device: q [T, batch, Hq, d] and the appended
    keys and values [T, batch, Hkv, d] of every step."""
    K = inp.k.to(dev)
    V = inp.v.to(dev)
    T = inp.q.shape[0]
    bidx = torch.arange(w.batch, device=dev)
    pos = torch.tensor([int(c) for c in inp.contexts], device=dev)[:, None] + \
        torch.arange(T, device=dev)[None]
    k_new = K[bidx[:, None], :, pos].permute(1, 0, 2, 3).contiguous()
    v_new = V[bidx[:, None], :, pos].permute(1, 0, 2, 3).contiguous()
    return K, V, inp.q.to(dev).contiguous(), k_new, v_new


def prefill(sess, w, inp, K, V):
    for b in range(w.batch):
        n0 = int(inp.contexts[b])
        sess.prefill(b, K[b, :, :n0], V[b, :, :n0])


def run_layers(w, inps, steps: Optional[int] = None, capacity: Optional[int] = None,
               share_workspace: bool = False, graph: bool = False) -> List[GpuRun]:
    """Several contexts of one config (say the layers of a model), each with
    its own caches, rings and inputs, stepped in order for every token on one
    stream with fused append+decode calls.  `share_workspace`: every context
    uses the first one's workspace.  `graph`: all steps of all contexts are
    captured in one HIP graph, which is replayed once; each (step, context)
    writes outputs of its own, checked after the replay."""
    from kv_cache_reuse_amd import binding as B
    T = inps[0].q.shape[0] if steps is None else steps
    dev = torch.device("cuda")
    sessions, staged = [], []
    for inp in inps:
        ws = sessions[0].workspace if (share_workspace and sessions) else None
        sess = make_session(w, inp, T, capacity=capacity, workspace=ws)
        K, V, q, kn, vn = step_inputs(w, inp, dev)
        prefill(sess, w, inp, K, V)
        sessions.append(sess)
        staged.append((q, kn, vn))
    hq = w.n_q_heads
    outs = [torch.empty((T, w.batch, hq, w.head_dim), dtype=torch.float32, device=dev)
            for _ in inps]
    mns = [torch.empty((T, w.batch, hq), dtype=torch.int32, device=dev) for _ in inps]
    dss = [torch.empty((T, w.batch, hq), dtype=torch.float32, device=dev) for _ in inps]
    torch.cuda.synchronize()

    def all_steps(stream):
        for t in range(T):
            for i, sess in enumerate(sessions):
                q, kn, vn = staged[i]
                B.mac_decode_step_append(sess.ctx, q[t].data_ptr(), kn[t].data_ptr(),
                                         vn[t].data_ptr(), sess.k_cache.data_ptr(),
                                         sess.v_cache.data_ptr(), sess._pt(),
                                         outs[i][t].data_ptr(), mns[i][t].data_ptr(),
                                         dss[i][t].data_ptr(), stream)

    if graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            all_steps(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        del g
    else:
        all_steps(sessions[0]._s())
        torch.cuda.synchronize()
    runs = []
    for i, sess in enumerate(sessions):
        o, m, d = outs[i].cpu().numpy(), mns[i].cpu().numpy(), dss[i].cpu().numpy()
        runs.append(GpuRun({t: o[t] for t in range(T)}, {t: m[t] for t in range(T)},
                           {t: d[t] for t in range(T)}, sess))
    return runs


def run_gpu(w, inp, steps: Optional[int] = None, record=None, max_slices: int = 0,
            paged: Optional[bool] = None, q_override=None, poison: bool = False,
            fused: bool = False, seed_q=None, capacity: Optional[int] = None,
            kv_layout: int = 0, direct_prefill: bool = False) -> GpuRun:
    """Prefill every sequence, optionally seed the rings with the queries
    `seed_q` [n, batch, Hq, d] of the last n prefill positions, then
    `steps` x (append, decode).  `record` selects the steps whose outputs are
    copied back (default: all)."""
    T = inp.q.shape[0] if steps is None else steps
    dev = torch.device("cuda")
    sess = make_session(w, inp, T, max_slices=max_slices, paged=paged, capacity=capacity,
                        kv_layout=kv_layout)
    if poison:                       # stale NaN in every slot not yet written
        sess.k_cache.fill_(float("nan"))
        sess.v_cache.fill_(float("nan"))
    K = inp.k.to(dev)
    V = inp.v.to(dev)
    ctx = [int(c) for c in inp.contexts]
    if direct_prefill:
        # natural rows: the caller writes the prefill into the caches itself
        # (as a KV manager that owns the pool would) and starts the context
        # with those lengths
        write_rows(sess, w, K, V, ctx)
    else:
        for b in range(w.batch):
            sess.prefill(b, K[b, :, :ctx[b]], V[b, :, :ctx[b]])
    if seed_q is not None:
        sess.seed(seed_q.to(dev).contiguous())
    q_all = (inp.q if q_override is None else q_override).to(dev)
    bidx = torch.arange(w.batch, device=dev)
    ctx_t = torch.tensor(ctx, device=dev)
    res = GpuRun({}, {}, {}, sess)
    for t in range(T):
        pos = ctx_t + t
        k_new = K[bidx, :, pos].contiguous()          # [batch, Hkv, d]
        v_new = V[bidx, :, pos].contiguous()
        if fused:
            out, mc, ds = sess.decode_append(q_all[t].contiguous(), k_new, v_new)
        else:
            sess.append(k_new, v_new)
            out, mc, ds = sess.decode(q_all[t].contiguous())
        if record is None or t in record:
            res.out[t] = out.float().cpu().numpy().copy()
            res.match_n[t] = mc.cpu().numpy().copy()
            res.dist[t] = ds.cpu().numpy().copy()
    torch.cuda.synchronize()
    return res
