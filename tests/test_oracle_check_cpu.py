"""CPU checks of the parity machinery the GPU tests use: results the oracle
itself produced pass, planted output and decision errors are caught, and the
parallel per-group replay reports exactly what the serial one does."""

import types

import numpy as np
import pytest
import torch

from oracle import mac_oracle as M
from synth.streams import make_inputs, make_kv_group, workload
from tests.oracle_check import check_groups, check_groups_parallel


def oracle_as_gpu(w, inp):
    """The oracle's own results, shaped and rounded like recorded GPU steps."""
    res, _ = M.run(w, inp)
    run = types.SimpleNamespace(out={}, match_n={}, dist={})
    for t, row in enumerate(res):
        run.out[t] = np.stack([row[b].out for b in range(w.batch)]).astype(np.float32)
        run.match_n[t] = np.stack([row[b].match_n for b in range(w.batch)]).astype(np.int32)
        run.dist[t] = np.stack([row[b].dist for b in range(w.batch)]).astype(np.float32)
    return run


def small():
    return workload("paged_b8", head_dim=16, ctx_range=(40, 90), steps=24, window=6, band=20,
                    batch=3, n_q_heads=8, n_kv_heads=2, tau=0.5 * 4.0, p_jump=0.2)


def groups(w):
    return [(b, g) for b in range(w.batch) for g in range(w.n_kv_heads)]


def test_kv_of_one_group_equals_the_batch_draw():
    for w in (small(), workload("70b_128k", batch=2, context=300, steps=5)):
        inp = make_inputs(w)
        for b in range(w.batch):
            for g in range(w.n_kv_heads):
                k, v, flag = make_kv_group(w, inp.contexts, inp.q.shape[0], b, g)
                n = int(inp.contexts[b]) + inp.q.shape[0]
                assert torch.equal(k, inp.k[b, g, :n]) and torch.equal(v, inp.v[b, g, :n])
                if flag is not None:
                    assert (flag == inp.outlier[b, g, :n]).all()


def test_the_oracles_own_results_pass_and_planted_errors_fail():
    w = small()
    inp = make_inputs(w)
    gpu = oracle_as_gpu(w, inp)
    rep = check_groups(w, inp, gpu, groups(w))
    assert rep.ok() and rep.hits > 0 and not rep.borderline
    assert rep.steps == w.steps * w.batch * w.n_kv_heads
    # an output element off by more than the tolerance
    bad = oracle_as_gpu(w, inp)
    bad.out[5][1, 3, 7] += 3e-3
    rep = check_groups(w, inp, bad, groups(w))
    assert not rep.ok() and any(m[3] == "out" for m in rep.mismatches)
    # a hit reported as a miss (away from the threshold)
    t, b, h = next((t, b, h) for t in range(w.steps) for b in range(w.batch)
                   for h in range(w.n_q_heads) if gpu.match_n[t][b, h] >= 0
                   and abs(gpu.dist[t][b, h] - w.tau) > 0.1)
    bad = oracle_as_gpu(w, inp)
    bad.match_n[t][b, h] = -1
    rep = check_groups(w, inp, bad, groups(w))
    assert any(m[3] == "decision" for m in rep.mismatches)


def test_parallel_replay_equals_the_serial_one():
    w = small()
    inp = make_inputs(w)
    gpu = oracle_as_gpu(w, inp)
    gpu.out[7][2, 5, 0] += 1e-3          # inside the tolerance, shows in max_err
    a = check_groups(w, inp, gpu, groups(w))
    bpar = check_groups_parallel(w, inp, gpu, groups(w), workers=2)
    assert (a.steps, a.heads, a.hits, a.groups) == (bpar.steps, bpar.heads, bpar.hits, bpar.groups)
    assert a.max_err == bpar.max_err and a.max_dist_err == bpar.max_dist_err
    assert sorted(a.mismatches) == sorted(bpar.mismatches) == []
