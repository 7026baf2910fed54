"""The natural (row) KV layout on the GPU: the same steps as the library's
tile layout, bitwise, for every kernel variant, and caches written directly
by the caller (needs an MI355X)."""

import math

import numpy as np
import pytest
import torch

from synth.streams import make_inputs, workload
from tests.gpu_harness import check_groups, run_gpu, say
from tests.test_gpu_parity import all_groups, assert_report

pytestmark = pytest.mark.gpu

ROWS = 1

CASES = {
    # name: (workload, overrides, run_gpu options)
    "narrow": ("8b_32k", dict(context=2100, steps=24), {}),
    "narrow_ragged_capacity": ("8b_32k", dict(context=1000, steps=21), {}),  # max_context 1021
    "paged": ("paged_b8", dict(ctx_range=(700, 2300), steps=20), {}),
    "paged_rounds": ("paged_b8", dict(ctx_range=(700, 2300), steps=20, p_jump=0.15),
                     dict(capacity=30000)),
    "contig_rounds": ("paged_b8", dict(page_size=0, ctx_range=(700, 2300), steps=20, p_jump=0.15),
                      dict(capacity=30000)),
    "g8": ("70b_128k", dict(batch=2, context=1500, steps=16), {}),
    "mqa_g32": ("8b_32k", dict(n_kv_heads=1, context=2500, steps=16), {}),
    "mqa_g64_paged": ("paged_b8", dict(batch=2, n_q_heads=64, n_kv_heads=1, ctx_range=(500, 1200),
                                       steps=12), {}),
    "d64": ("8b_32k", dict(head_dim=64, context=1500, steps=16, tau=4.0), {}),
    # fp32 caches: every fp32 instantiation of the step kernel
    "f32_d128": ("tiny", dict(head_dim=128, n_q_heads=8, n_kv_heads=2, context=900, steps=16,
                              tau=0.5 * math.sqrt(128)), {}),
    "f32_d128_g8": ("tiny", dict(head_dim=128, n_q_heads=16, n_kv_heads=2, context=1100,
                                 steps=12, tau=0.5 * math.sqrt(128)), {}),
    "f32_d64_mqa": ("tiny", dict(n_q_heads=32, n_kv_heads=1, context=1300, steps=12), {}),
    "f32_d64_paged": ("paged_b8", dict(dtype="f32", head_dim=64, batch=2, ctx_range=(400, 1100),
                                       steps=12, tau=0.5 * math.sqrt(64)), {}),
    "f32_paged_g8": ("paged_b8", dict(dtype="f32", batch=2, n_q_heads=32, n_kv_heads=4,
                                      ctx_range=(300, 900), steps=12), {}),
    "f32_rounds": ("paged_b8", dict(dtype="f32", page_size=0, ctx_range=(700, 1500), steps=12,
                                    p_jump=0.15), dict(capacity=30000)),
}


@pytest.mark.parametrize("name", list(CASES))
def test_rows_equal_tiles_bitwise(name):
    # the row layout changes only where each value comes from, not the
    # arithmetic: every output, decision and distance must match the tile
    # layout's bit for bit, and the oracle
    base, kw, opts = CASES[name]
    w = workload(base, **kw)
    inp = make_inputs(w)
    say(f"[rows:{name}] {w}")
    tiles = run_gpu(w, inp, fused=True, poison=True, **opts)
    rows = run_gpu(w, inp, fused=True, poison=True, kv_layout=ROWS, **opts)
    for t in tiles.out:
        np.testing.assert_array_equal(rows.out[t], tiles.out[t])
        np.testing.assert_array_equal(rows.match_n[t], tiles.match_n[t])
        np.testing.assert_array_equal(rows.dist[t], tiles.dist[t])
    for b in range(w.batch):
        n = int(inp.contexts[b]) + w.steps
        k, v = rows.session.read_kv(b, 0, n)
        torch.cuda.synchronize()
        assert torch.equal(k.cpu(), inp.k[b, :, :n]) and torch.equal(v.cpu(), inp.v[b, :, :n])
    rep = check_groups(w, inp, rows, all_groups(w))
    assert_report(rep, f"rows:{name}")


@pytest.mark.parametrize("name", ["narrow", "narrow_ragged_capacity", "paged", "paged_rounds",
                                  "mqa_g32", "f32_d128", "f32_d64_paged"])
def test_rows_written_by_the_caller(name):
    # the prefill goes straight into the natural-row caches through torch
    # indexing (no library call), as a KV manager that owns the pool would
    # write it; the decode steps then append through the library
    base, kw, opts = CASES[name]
    w = workload(base, **kw)
    inp = make_inputs(w)
    say(f"[rows direct:{name}] {w}")
    gpu = run_gpu(w, inp, fused=True, kv_layout=ROWS, direct_prefill=True, **opts)
    rep = check_groups(w, inp, gpu, all_groups(w))
    assert_report(rep, f"rows_direct:{name}")
    # and the decode steps' tokens are rows of the caller's view too
    cfg = gpu.session.cfg
    if not cfg.page_size:
        kc = gpu.session.k_cache.view(cfg.batch, cfg.n_kv_heads, cfg.max_context, cfg.head_dim)
        for b in range(w.batch):
            n = int(inp.contexts[b]) + w.steps
            assert torch.equal(kc[b, :, :n].cpu(), inp.k[b, :, :n])
