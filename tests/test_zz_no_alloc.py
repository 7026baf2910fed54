"""mac_decode_step_append_noalloc through the C ABI against
mac_decode_step_append (needs an MI355X).

The no-allocation entry point keeps the step's scratch in the library's
static device array, shared by every call on the GPU.  Two contexts of
different sizes are stepped in turn with it, so every call finds the
previous call's contents in the array (the second call of each pair has the
smaller input), and every call must equal bitwise the same step of a twin
context stepped through the workspace entry point.
"""

import pytest
import torch

from synth.streams import make_inputs, workload
from tests.gpu_harness import GpuRun, check_groups, make_session, prefill, say, step_inputs

pytestmark = pytest.mark.gpu


def _twins(w, inp, T, capacity=None, no_workspace=False):
    from kv_cache_reuse_amd import binding as B
    dev = torch.device("cuda")
    ref = make_session(w, inp, T, capacity=capacity)
    if no_workspace:
        table = ref.page_table.cpu().numpy() if ref.page_table is not None else None
        new = B.MacSession(ref.cfg, page_table=table, no_workspace=True)
        assert new.workspace is None
    else:
        new = make_session(w, inp, T, capacity=capacity)
    K, V, q, kn, vn = step_inputs(w, inp, dev)
    prefill(ref, w, inp, K, V)
    prefill(new, w, inp, K, V)
    return ref, new, (q, kn, vn)


def test_noalloc_equals_the_workspace_entry_point():
    # large: a ragged paged batch of 8 whose launch takes two rounds of
    # workgroups (64 KV groups, 8 slices each); small: one 8B-shaped
    # sequence (8 groups), created without a workspace
    wa = workload("paged_b8", ctx_range=(700, 2300), steps=20, p_jump=0.15)
    wb = workload("8b_32k", context=900, steps=20, p_jump=0.2)
    ia, ib = make_inputs(wa), make_inputs(wb)
    T = wa.steps
    ref_a, new_a, sa = _twins(wa, ia, T, capacity=30000)
    ref_b, new_b, sb = _twins(wb, ib, T, no_workspace=True)
    assert new_a.cfg.max_slices == 0
    runs = {"a": GpuRun({}, {}, {}, new_a), "b": GpuRun({}, {}, {}, new_b)}
    torch.cuda.synchronize()
    for t in range(T):
        for key, ref, new, (q, kn, vn) in (("a", ref_a, new_a, sa), ("b", ref_b, new_b, sb)):
            o_ref, m_ref, d_ref = ref.decode_append(q[t], kn[t], vn[t])
            o, m, d = new.decode_append_noalloc(q[t], kn[t], vn[t])
            torch.cuda.synchronize()
            assert torch.equal(o, o_ref), (key, t)
            assert torch.equal(m, m_ref), (key, t)
            assert torch.equal(d, d_ref), (key, t)
            r = runs[key]
            r.out[t], r.match_n[t], r.dist[t] = (o.cpu().numpy().copy(), m.cpu().numpy().copy(),
                                                 d.cpu().numpy().copy())
    # (rings are not compared as bytes: slots not yet written and padding
    # hold whatever the allocator left there)
    for ref, new, w, inp in ((ref_a, new_a, wa, ia), (ref_b, new_b, wb, ib)):
        assert torch.equal(new.seq_lens, ref.seq_lens)
        for b in range(w.batch):       # the written keys (unwritten slots hold garbage)
            n = int(inp.contexts[b]) + T
            k1, v1 = new.read_kv(b, 0, n)
            k2, v2 = ref.read_kv(b, 0, n)
            torch.cuda.synchronize()
            assert torch.equal(k1, k2) and torch.equal(v1, v2)
    # and both against the oracle
    for key, w, inp in (("a", wa, ia), ("b", wb, ib)):
        groups = [(b, g) for b in range(w.batch) for g in range(w.n_kv_heads)]
        rep = check_groups(w, inp, runs[key], groups)
        say(f"[noalloc {key}] steps={rep.steps} hits={rep.hits} max_err={rep.max_err:.2e} "
            f"borderline={len(rep.borderline)}")
        assert rep.ok() and rep.hits > 0


def test_noalloc_refuses_what_the_scratch_cannot_hold():
    from kv_cache_reuse_amd import binding as B
    # 64 KV groups x 512 slices x 4 heads of 128 fp32 partial dims: 64 MiB
    w = workload("paged_b8", page_size=0, ctx_range=(100, 200), steps=2)
    inp = make_inputs(w)
    big = make_session(w, inp, 2, max_slices=512)
    dev = torch.device("cuda")
    K, V, q, kn, vn = step_inputs(w, inp, dev)
    prefill(big, w, inp, K, V)
    torch.cuda.synchronize()
    with pytest.raises(B.MacError) as e:
        big.decode_append_noalloc(q[0], kn[0], vn[0])
    assert e.value.status == B.MAC_ERR_CAPACITY
    assert "static scratch" in str(e.value)
    # refused before any device call: the context still works
    out, mc, _ = big.decode_append(q[0], kn[0], vn[0])
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and (mc.cpu() == -1).all()
    # a context without a workspace steps only through the noalloc entry point
    ref, new, (q2, kn2, vn2) = _twins(workload("8b_32k", context=300, steps=2),
                                      make_inputs(workload("8b_32k", context=300, steps=2)), 2,
                                      no_workspace=True)
    with pytest.raises(B.MacError) as e:
        new.decode_append(q2[0], kn2[0], vn2[0])
    assert e.value.status == B.MAC_ERR_INVALID_ARG
    o, _, _ = new.decode_append_noalloc(q2[0], kn2[0], vn2[0])
    o_ref, _, _ = ref.decode_append(q2[0], kn2[0], vn2[0])
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref)
