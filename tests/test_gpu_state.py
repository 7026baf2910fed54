"""GPU checks of the state a context carries between steps, against the fp64
oracle: several layer contexts stepped in one HIP graph, contexts sharing one
workspace, and a context resumed from a checkpoint (needs an MI355X).
"""

import numpy as np
import pytest
import torch

from synth.streams import make_inputs, workload
from tests.gpu_harness import (GpuRun, check_groups, make_session, prefill, run_layers, say,
                               step_inputs)
from tests.test_gpu_parity import all_groups, assert_report

pytestmark = pytest.mark.gpu


LAYERED = {
    # the 8B shape, one round of workgroups, each layer with its own workspace
    "8b_32k_4_layers": ("8b_32k", dict(context=2100, steps=16, p_jump=0.2), 4, None, False),
    # a ragged paged batch whose launches take two rounds of workgroups (the
    # later rounds read the plan start slice 0 publishes), 4 layers sharing
    # one workspace
    "paged_rounds_4_layers": ("paged_b8", dict(ctx_range=(700, 2300), steps=12, p_jump=0.15),
                              4, 30000, True),
    # G = 8 (the 70B shape's grouping)
    "70b_5_layers": ("70b_128k", dict(batch=1, context=1500, steps=10), 5, None, True),
}


@pytest.mark.parametrize("name", list(LAYERED))
def test_layers_in_one_graph_match_the_oracle(name):
    # every layer of every token captured in one HIP graph, replayed once;
    # each layer (own caches, rings and query stream) is checked against
    # its own oracle replay
    base, kw, layers, capacity, share = LAYERED[name]
    w = workload(base, **kw)
    inps = [make_inputs(w, layer=l) for l in range(layers)]
    say(f"[graph:{name}] {layers} layers, shared workspace {share}: {w}")
    runs = run_layers(w, inps, capacity=capacity, share_workspace=share, graph=True)
    for l, (inp, run) in enumerate(zip(inps, runs)):
        rep = check_groups(w, inp, run, all_groups(w))
        assert_report(rep, f"graph:{name}:layer{l}")


def test_contexts_sharing_a_workspace_in_lockstep():
    # two contexts of one config step in turn on one stream with one
    # workspace: their rings advance together, so a plan start the one
    # publishes carries the tag the other's next step looks for; the merge
    # clears it after each step, and each context must match its oracle
    w = workload("paged_b8", ctx_range=(700, 2300), steps=24, p_jump=0.1)
    inps = [make_inputs(w, layer=l) for l in range(2)]
    say(f"[shared workspace] {w}")
    runs = run_layers(w, inps, capacity=30000, share_workspace=True)
    assert runs[0].session.workspace.data_ptr() == runs[1].session.workspace.data_ptr()
    for l, (inp, run) in enumerate(zip(inps, runs)):
        rep = check_groups(w, inp, run, all_groups(w))
        assert_report(rep, f"shared_ws:layer{l}")


def _steps(sess, q, kn, vn, t0, t1, res):
    for t in range(t0, t1):
        out, mc, ds = sess.decode_append(q[t], kn[t], vn[t])
        res.out[t] = out.cpu().numpy().copy()
        res.match_n[t] = mc.cpu().numpy().copy()
        res.dist[t] = ds.cpu().numpy().copy()


@pytest.mark.parametrize("paged", [True, False])
def test_resume_from_a_checkpoint_is_bitwise(paged):
    # run T1 steps, take byte copies of the ring, caches, page table and
    # lengths, and continue twice: the original context, and a new one bound
    # to the copies with mac_resume.  The new context's workspace starts out
    # filled with plan words that carry the tag of the next step and a
    # plausible plan start: mac_resume must clear them, or the later-round
    # workgroups of the next step (a miss) would leave with work undone.
    w = workload("paged_b8", page_size=16 if paged else 0, ctx_range=(700, 2300), steps=24,
                 p_jump=0.1)
    inp = make_inputs(w)
    T, T1 = w.steps, 10
    g = torch.Generator().manual_seed(77)
    q = inp.q.clone()
    q[T1] = torch.randn(q[T1].shape, generator=g, dtype=torch.float64).to(q.dtype)
    inp.q, inp.q64 = q, q.double().numpy()
    dev = torch.device("cuda")
    a = make_session(w, inp, T, capacity=30000)
    assert a.cfg.max_slices == 0
    K, V, qd, kn, vn = step_inputs(w, inp, dev)
    prefill(a, w, inp, K, V)
    run_a = GpuRun({}, {}, {}, a)
    _steps(a, qd, kn, vn, 0, T1, run_a)
    ck = a.checkpoint()
    _steps(a, qd, kn, vn, T1, T, run_a)

    from kv_cache_reuse_amd import binding as B
    ws = torch.empty(B.mac_workspace_bytes(a.cfg), dtype=torch.uint8, device=dev)
    ws.view(torch.int64).fill_((T1 << 32) | 500)
    b = B.MacSession(a.cfg, page_table=ck.get("page_table"), workspace=ws, resume_from=ck)
    run_b = GpuRun({}, {}, {}, b)
    _steps(b, qd, kn, vn, T1, T, run_b)
    torch.cuda.synchronize()
    say(f"[resume paged={paged}] step {T1} heads missing: {(run_a.match_n[T1] < 0).sum()}")
    assert (run_a.match_n[T1] < 0).all(), "the first step after the checkpoint should miss"
    for t in range(T1, T):
        np.testing.assert_array_equal(run_b.out[t], run_a.out[t])
        np.testing.assert_array_equal(run_b.match_n[t], run_a.match_n[t])
        np.testing.assert_array_equal(run_b.dist[t], run_a.dist[t])
    assert torch.equal(b.seq_lens, a.seq_lens)
    assert torch.equal(b.ring, a.ring)
    rep = check_groups(w, inp, run_a, all_groups(w))
    assert_report(rep, f"resume:{paged}")
