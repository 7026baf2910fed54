"""GPU parity of libmac against the fp64 oracle (needs an MI355X).

Small shapes (several 16-token tiles, ragged tails, every KV group) are
checked on every step; the full-size shapes run in the launch configuration
the benchmark uses (fused append and decode) and are checked on every KV
group and every step, the oracle replaying the groups in parallel worker
processes.
"""

import math

import numpy as np
import pytest
import torch

from synth.streams import make_inputs, workload

pytestmark = pytest.mark.gpu

from tests.gpu_harness import (OUT_TOL, check_groups, check_groups_parallel, run_gpu,  # noqa: E402
                               say)


def all_groups(w):
    return [(b, g) for b in range(w.batch) for g in range(w.n_kv_heads)]


def assert_report(rep, name, min_hits=1):
    say(f"[{name}] steps={rep.steps} heads={rep.heads} hits={rep.hits} "
        f"max_err={rep.max_err:.3e} dist_err={rep.max_dist_err:.2e} "
        f"borderline={len(rep.borderline)} mismatches={rep.mismatches[:5]}")
    assert not rep.mismatches, rep.mismatches[:10]
    assert rep.max_err <= OUT_TOL
    assert rep.max_dist_err <= 1e-5
    assert rep.hits >= min_hits


SMALL = {
    "tiny_full": ("tiny", {}),
    "8b_32k_ragged": ("8b_32k", dict(context=3001, steps=40)),
    "8b_128k_p05": ("8b_128k", dict(context=5003, steps=48, p_jump=0.5)),
    "8b_128k_p005": ("8b_128k", dict(context=4099, steps=48, p_jump=0.05)),
    "paged_b8_small": ("paged_b8", dict(ctx_range=(700, 2300), steps=32)),
    "70b_small": ("70b_128k", dict(batch=2, context=3333, steps=32)),
    "band0": ("8b_32k", dict(context=1000, steps=24, band=0, p_jump=0.2)),
    "window0": ("8b_32k", dict(context=1000, steps=12, window=0)),
    "band_over_ctx": ("tiny", dict(context=40, steps=40, band=500)),
    "ctx1": ("tiny", dict(context=1, steps=40, band=8, window=4)),
    "periodic_tail": ("8b_32k", dict(context=2100, steps=40, period=5, window=8, band=64,
                                     tau=0.5 * math.sqrt(128))),
    "d64_bf16": ("8b_32k", dict(head_dim=64, context=1500, steps=24, tau=0.5 * math.sqrt(64))),
    "d128_f32": ("tiny", dict(head_dim=128, n_q_heads=8, n_kv_heads=2, context=900, steps=24,
                              tau=0.5 * math.sqrt(128))),
    # groups wider than the 16-head matrix tile: split into equal chunks
    "mqa_g32": ("8b_32k", dict(n_kv_heads=1, context=2500, steps=24)),
    "mqa_g64": ("8b_32k", dict(n_q_heads=64, n_kv_heads=1, context=1800, steps=16)),
    "g20": ("8b_32k", dict(n_q_heads=40, n_kv_heads=2, context=1200, steps=16)),
    "mqa_paged": ("paged_b8", dict(batch=2, n_kv_heads=1, ctx_range=(500, 1200), steps=12)),
    # wide-path match over windows of two and three rounds of slots (the
    # matched entry's state then comes from a later round)
    "mqa_w64": ("8b_32k", dict(n_kv_heads=1, context=1300, steps=80, window=64, p_jump=0.2)),
    "g20_w100": ("8b_32k", dict(n_q_heads=40, n_kv_heads=2, context=900, steps=120, window=100,
                               p_jump=0.2)),
    # every remaining (dtype, d, paged, wide) instantiation of the step kernel
    "f32_d128_wide": ("tiny", dict(head_dim=128, n_q_heads=16, n_kv_heads=2, context=1100, steps=16,
                                   tau=0.5 * math.sqrt(128))),
    "f32_d64_mqa": ("tiny", dict(n_q_heads=32, n_kv_heads=1, context=1300, steps=16)),
    "f32_paged": ("paged_b8", dict(dtype="f32", batch=2, ctx_range=(400, 1100), steps=12)),
    "f32_d64_paged_wide": ("paged_b8", dict(dtype="f32", head_dim=64, batch=2, n_q_heads=32,
                                            n_kv_heads=4, ctx_range=(300, 900), steps=12,
                                            tau=0.5 * math.sqrt(64))),
    "d64_bf16_paged_wide": ("paged_b8", dict(head_dim=64, batch=2, n_q_heads=32, n_kv_heads=2,
                                             ctx_range=(500, 1300), steps=12, tau=0.5 * math.sqrt(64))),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_small_shapes_every_step(name):
    base, kw = SMALL[name]
    w = workload(base, **kw)
    say(f"[{name}] {w}")
    inp = make_inputs(w)
    gpu = run_gpu(w, inp)
    rep = check_groups(w, inp, gpu, all_groups(w))
    min_hits = 0 if (w.window == 0) else 1
    assert_report(rep, name, min_hits)


@pytest.mark.parametrize("max_slices", [100, 600, 1024])
def test_merge_over_many_slices(max_slices):
    # more slices per group than one merge wave folds: several waves per
    # query head (100: four waves, the last one partly filled) and, above
    # 512 slices, two rounds of loads per wave; the context fills every
    # slice on a miss
    w = workload("8b_32k", n_q_heads=4, n_kv_heads=2, context=66000, steps=12, p_jump=0.3)
    say(f"[slices{max_slices}] {w}")
    inp = make_inputs(w)
    gpu = run_gpu(w, inp, max_slices=max_slices)
    rep = check_groups(w, inp, gpu, all_groups(w))
    assert_report(rep, f"slices{max_slices}")


@pytest.mark.parametrize("fused,page_size,capacity", [(False, 0, 30000), (True, 0, 30000),
                                                       (False, 16, 30000), (True, 16, 30000),
                                                       (True, 0, 70000), (False, 16, 70000),
                                                       (True, 16, 70000)])
def test_two_rounds_every_step(fused, page_size, capacity):
    # a capacity far above the contexts gives the default launch more
    # rounds of workgroups (4 slices per group in the first round; 8 slices
    # in all at capacity 30000, 16 at 70000): the slice-0 workgroups publish
    # their plan start and later-round workgroups with an empty slice leave
    # early on hit steps.  The ragged contexts give the later rounds' ids a
    # sequence order (longest first) other than the batch order.
    w = workload("paged_b8", page_size=page_size, ctx_range=(700, 2300), steps=24, p_jump=0.1)
    say(f"[rounds fused={fused} page_size={page_size} capacity={capacity}] {w}")
    inp = make_inputs(w)
    gpu = run_gpu(w, inp, capacity=capacity, fused=fused)
    assert gpu.session.cfg.max_slices == 0
    rep = check_groups(w, inp, gpu, all_groups(w))
    assert_report(rep, f"rounds:{fused}:{page_size}:{capacity}")


@pytest.mark.parametrize("fused,page_size", [(False, 0), (True, 0), (True, 16)])
def test_wide_groups_in_two_rounds(fused, page_size):
    # groups of 8 query heads (the 70B shape) with a capacity that gives the
    # launch three rounds of workgroups (the later rounds run every match
    # and take their slices of the plan)
    w = workload("70b_128k", batch=2, page_size=page_size, context=2000, steps=24)
    if page_size:
        w = w.replace(ctx_range=(1500, 2500))
    say(f"[wide rounds fused={fused} page_size={page_size}] {w}")
    inp = make_inputs(w)
    gpu = run_gpu(w, inp, capacity=140000, fused=fused)   # 16 groups: 3 rounds of 16 slices
    assert gpu.session.cfg.max_slices == 0
    rep = check_groups(w, inp, gpu, all_groups(w))
    assert_report(rep, f"wide_rounds:{fused}:{page_size}")


@pytest.mark.parametrize("batch", [16, 17])
def test_later_rounds_at_the_order_limits(batch):
    # 16 sequences fill every entry of the later rounds' sequence order; 17
    # go without one (batch order).  With 128 or 136 groups the default
    # launch has 2 slices per group in the first round and 8 in all, so a
    # hit's band and tail get one slice.
    w = workload("paged_b8", batch=batch, page_size=16, ctx_range=(300, 1500), steps=16, p_jump=0.15)
    say(f"[order limits batch={batch}] {w}")
    inp = make_inputs(w)
    gpu = run_gpu(w, inp, capacity=30000)
    rep = check_groups(w, inp, gpu, all_groups(w))
    assert_report(rep, f"order_limits:{batch}")


@pytest.mark.parametrize("name,period", [("8b_32k", 3), ("70b_128k", 3), ("tiny", 2)])
def test_exact_ties_take_the_newest_entry(name, period):
    # q_t repeats q_{t-period} exactly, so several ring entries lie at
    # distance 0 from the query: the newest must win on both sides.  With a
    # period of 3 (or 2) the tied entries sit in ring slots of both
    # parities, so for narrow groups they fall to the two waves that split a
    # head's slots, and the cross-wave combine decides.  The harness would
    # accept either entry of an exact tie as borderline; here none may occur.
    kw = dict(context=700, steps=30, period=period, window=8, band=64)
    if name != "tiny":
        kw["batch"] = 1
    w = workload(name, **kw)
    say(f"[ties {name} period {period}] {w}")
    inp = make_inputs(w)
    gpu = run_gpu(w, inp)
    rep = check_groups(w, inp, gpu, all_groups(w))
    assert_report(rep, f"ties_{name}", min_hits=(w.steps - 2 * period) * w.batch * w.n_q_heads)
    assert not rep.borderline, rep.borderline[:5]


@pytest.mark.parametrize("name", ["ctx1", "8b_32k_ragged", "paged_b8_small", "d64_bf16"])
def test_stale_cache_slots_do_not_leak(name):
    # unwritten cache slots hold NaN; they sit past the end of each sequence
    # inside its last 16-token tile and must not reach any output
    base, kw = SMALL[name]
    w = workload(base, **kw)
    inp = make_inputs(w, steps=min(w.steps, 20))
    say(f"[poison:{name}]")
    gpu = run_gpu(w, inp, poison=True)
    rep = check_groups(w, inp, gpu, all_groups(w))
    assert_report(rep, f"poison:{name}", 0)


@pytest.mark.parametrize("name", ["tiny_full", "8b_128k_p05", "paged_b8_small", "70b_small",
                                  "ctx1", "mqa_g32", "mqa_paged", "f32_d128_wide",
                                  "d64_bf16_paged_wide"])
def test_fused_append_decode_every_step(name):
    base, kw = SMALL[name]
    w = workload(base, **kw)
    inp = make_inputs(w)
    say(f"[fused:{name}]")
    gpu = run_gpu(w, inp, fused=True, poison=True)
    rep = check_groups(w, inp, gpu, all_groups(w))
    assert_report(rep, f"fused:{name}", 0 if w.window == 0 else 1)


def test_fused_equals_separate_calls_bitwise():
    w = workload("paged_b8", ctx_range=(600, 1400), steps=20)
    inp = make_inputs(w)
    a = run_gpu(w, inp, fused=True)
    b = run_gpu(w, inp, fused=False)
    for t in a.out:
        np.testing.assert_array_equal(a.out[t], b.out[t])
        np.testing.assert_array_equal(a.match_n[t], b.match_n[t])
        np.testing.assert_array_equal(a.dist[t], b.dist[t])
    for bb in range(w.batch):
        n = int(inp.contexts[bb]) + w.steps
        ka, va = a.session.read_kv(bb, 0, n)
        kb, vb = b.session.read_kv(bb, 0, n)
        torch.cuda.synchronize()
        assert torch.equal(ka, kb) and torch.equal(va, vb)
        assert torch.equal(ka.cpu(), inp.k[bb, :, :n])
    assert torch.equal(a.session.seq_lens.cpu(), b.session.seq_lens.cpu())


def test_paged_equals_contiguous_bitwise():
    w = workload("paged_b8", ctx_range=(500, 1500), steps=16)
    inp = make_inputs(w)
    say("[paged_vs_contig] paged")
    a = run_gpu(w, inp, max_slices=8, paged=True)
    say("[paged_vs_contig] contiguous")
    b = run_gpu(w, inp, max_slices=8, paged=False)
    for t in a.out:
        np.testing.assert_array_equal(a.out[t], b.out[t])
        np.testing.assert_array_equal(a.match_n[t], b.match_n[t])


def test_runs_are_bitwise_deterministic():
    w = workload("8b_32k", context=2500, steps=16)
    inp = make_inputs(w)
    a = run_gpu(w, inp)
    b = run_gpu(w, inp)
    for t in a.out:
        np.testing.assert_array_equal(a.out[t], b.out[t])
        np.testing.assert_array_equal(a.dist[t], b.dist[t])


def test_kv_roundtrip_is_exact():
    for name, kw in (("8b_32k", dict(context=1000, steps=4)),
                     ("paged_b8", dict(ctx_range=(300, 800), steps=4)),
                     ("tiny", dict(context=333, steps=4))):
        w = workload(name, **kw)
        inp = make_inputs(w)
        gpu = run_gpu(w, inp, steps=2)
        sess = gpu.session
        for b in range(w.batch):
            n = int(inp.contexts[b]) + 2
            k, v = sess.read_kv(b, 0, n)
            torch.cuda.synchronize()
            assert torch.equal(k.cpu(), inp.k[b, :, :n])
            assert torch.equal(v.cpu(), inp.v[b, :, :n])


def test_nan_query_poisons_only_its_head():
    w = workload("8b_32k", context=700, steps=10)
    inp = make_inputs(w)
    q = inp.q.clone()
    q[6, 0, 5, 17] = float("nan")
    inp.q = q
    inp.q64 = q.double().numpy()
    gpu = run_gpu(w, inp)
    assert np.isnan(gpu.out[6][0, 5]).all()
    assert gpu.match_n[6][0, 5] == -1
    rep = check_groups(w, inp, gpu, all_groups(w))
    assert_report(rep, "nan_head", 0)


# Keys whose scale grows along the sequence (about 26x at 1500 keys,
# scores up to about 100 in log2 units), with two slices per KV group, so
# that each streaming wave walks a dozen tiles or more of rising scale: a
# head's tile maximum keeps passing the softmax reference the step kernels
# hold by more than 2^8, and the lazy rescale (a ballot, then the cross-row
# maximum and the accumulators' rescale) runs several times in every wave.
# One case keeps the default slice count (many short slices), so partial
# states with references of every size meet in the merge and the ring.
RAMP = {
    "ramp_narrow": ("8b_32k", dict(context=1500, steps=24, p_jump=0.3), 2),
    "ramp_narrow_default_slices": ("8b_32k", dict(context=1500, steps=24, p_jump=0.3), 0),
    "ramp_g8": ("70b_128k", dict(batch=2, context=1300, steps=16, outlier_p=0.0), 2),
    "ramp_mqa_wide": ("8b_32k", dict(n_kv_heads=1, context=1700, steps=16, p_jump=0.3), 2),
    "ramp_paged": ("paged_b8", dict(batch=2, ctx_range=(900, 1600), steps=12), 2),
    "ramp_f32": ("tiny", dict(context=1400, steps=24), 2),
}


@pytest.mark.parametrize("name", list(RAMP))
def test_growing_key_scale_every_step(name):
    base, kw, slices = RAMP[name]
    w = workload(base, **kw)
    inp = make_inputs(w)
    L = inp.k.shape[2]
    ramp = 1.0 + torch.arange(L, dtype=torch.float32) / 60.0
    inp.k = (inp.k.float() * ramp[None, None, :, None]).to(inp.k.dtype)
    gpu = run_gpu(w, inp, max_slices=slices)
    rep = check_groups(w, inp, gpu, all_groups(w))
    assert_report(rep, name)


# ---------------------------------------------------------------------------
# full sizes, launch configuration of the benchmark, every KV group and step
# ---------------------------------------------------------------------------

FULL = {
    # name: (workload, overrides, decode steps[, run_gpu options])
    "8b_32k": ("8b_32k", dict(), 256),
    "8b_128k_p1": ("8b_128k", dict(p_jump=1.0), 512),
    "8b_128k_p05": ("8b_128k", dict(p_jump=0.5), 512),
    "8b_128k_p02": ("8b_128k", dict(p_jump=0.2), 512),
    "8b_128k_p005": ("8b_128k", dict(p_jump=0.05), 512),
    "paged_b8": ("paged_b8", dict(), 128),
    "70b_128k": ("70b_128k", dict(), 256),
    # the labelled supplement: rho drawn per KV head (shared by its 8 query
    # heads), so that whole groups hit and take the band-and-tail path
    "70b_128k_rho_per_kv": ("70b_128k", dict(rho_per_kv=True), 256),
    "8b_128k_mqa": ("8b_128k", dict(n_kv_heads=1, p_jump=0.2), 48),
    # natural-row caches (kv_layout 1) in the same launch configuration
    "8b_32k_rows": ("8b_32k", dict(), 256, dict(kv_layout=1)),
}


@pytest.mark.parametrize("name", list(FULL))
def test_full_size_every_group(name):
    base, kw, steps, *opts = FULL[name]
    opts = opts[0] if opts else {}
    w = workload(base, **kw, steps=steps)
    say(f"[full:{name}] generating {w}")
    inp = make_inputs(w)
    say(f"[full:{name}] gpu run, {steps} steps {opts}")
    gpu = run_gpu(w, inp, fused=True, **opts)
    groups = all_groups(w)
    say(f"[full:{name}] oracle replay of {len(groups)} KV groups x {steps} steps")

    def progress(i, n, rep):
        if i == n or i % max(1, n // 8) == 0:
            say(f"[full:{name}]   {i}/{n} groups, max_err {rep.max_err:.2e}, "
                f"mismatches {len(rep.mismatches)}")

    rep = check_groups_parallel(w, inp, gpu, groups, progress=progress)
    assert rep.groups == len(groups) and rep.steps == len(groups) * steps
    hit_rate = rep.hits / rep.heads
    say(f"[full:{name}] head hit rate {hit_rate:.3f}, borderline decisions {len(rep.borderline)}")
    # (every token jumps at p = 1: no step can hit)
    assert_report(rep, f"full:{name}", min_hits=0 if w.p_jump >= 1.0 else 1)


# ---------------------------------------------------------------------------
# ring seeding from the prefill
# ---------------------------------------------------------------------------

SEEDED = {
    "8b_32k_seed_w": ("8b_32k", dict(context=2100, steps=24), 32),
    "paged_seed_half": ("paged_b8", dict(ctx_range=(700, 1500), steps=16), 16),
    "70b_seed": ("70b_128k", dict(batch=2, context=1200, steps=12), 64),
    "tiny_seed_short_ctx": ("tiny", dict(context=10, steps=20, band=8, window=16), 10),
}


@pytest.mark.parametrize("name", list(SEEDED))
def test_seeded_ring_every_step(name):
    # the last n prefill positions are replayed into the rings; the decode
    # queries continue the same stream, so the first decode step already hits
    base, kw, n_hist = SEEDED[name]
    w = workload(base, **kw)
    full = make_inputs(w, steps=n_hist + w.steps)
    hist, hist64 = full.q[:n_hist], full.q64[:n_hist]
    inp = full.__class__(**{**full.__dict__, "q": full.q[n_hist:], "q64": full.q64[n_hist:]})
    say(f"[seed:{name}] n_hist={n_hist} {w}")
    gpu = run_gpu(w, inp, seed_q=hist)
    rep = check_groups(w, inp, gpu, all_groups(w), seed_q64=hist64)
    assert_report(rep, f"seed:{name}")
    assert (gpu.match_n[0] >= 0).any(), "no hit on the first step after seeding"
    lens = gpu.session.seq_lens.cpu().numpy()
    np.testing.assert_array_equal(lens, inp.contexts + w.steps)


# ---------------------------------------------------------------------------
# HIP graph replay
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name,capacity,stale", [("8b_32k_ragged", None, False),
                                                  ("paged_b8_small", None, False),
                                                  ("mqa_g32", None, False),
                                                  ("f32_d128_wide", None, False),
                                                  ("paged_b8_small", 70000, True)])
def test_graph_replays_equal_eager_steps(name, capacity, stale):
    # one fused decode step is captured once and replayed for every token,
    # its input buffers refilled by eager copies between replays; every
    # replay must equal the eagerly launched step bitwise (the kernels read
    # the lengths and ring counts on the device, so each replay advances).
    # `stale`: a launch of four rounds captured before the prefill, so the
    # later rounds' sequence order it holds is the batch order, not the
    # order of the lengths the eager steps used: the results must not change
    from kv_cache_reuse_amd import binding as B
    from tests.gpu_harness import make_session
    base, kw = SMALL[name]
    w = workload(base, **{**kw, "steps": 12})
    inp = make_inputs(w)
    ref = run_gpu(w, inp, fused=True, capacity=capacity)
    T = w.steps
    dev = torch.device("cuda")
    sess = make_session(w, inp, T, capacity=capacity)
    K, V = inp.k.to(dev), inp.v.to(dev)
    ctx = [int(c) for c in inp.contexts]
    assert not stale or len(set(ctx)) > 1
    bidx = torch.arange(w.batch, device=dev)
    ctx_t = torch.tensor(ctx, device=dev)
    q_all = inp.q.to(dev)
    q_buf = torch.empty_like(q_all[0])
    k_buf = torch.empty((w.batch, w.n_kv_heads, w.head_dim), dtype=q_all.dtype, device=dev)
    v_buf = torch.empty_like(k_buf)
    g = torch.cuda.CUDAGraph()

    def capture():
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            B.mac_decode_step_append(sess.ctx, q_buf.data_ptr(), k_buf.data_ptr(), v_buf.data_ptr(),
                                     sess.k_cache.data_ptr(), sess.v_cache.data_ptr(), sess._pt(),
                                     sess.out.data_ptr(), sess.match_ctx.data_ptr(),
                                     sess.dist.data_ptr(), torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()

    if stale:
        capture()
    for b in range(w.batch):
        sess.prefill(b, K[b, :, :ctx[b]], V[b, :, :ctx[b]])
    if not stale:
        capture()
    torch.cuda.synchronize()
    for t in range(T):
        pos = ctx_t + t
        q_buf.copy_(q_all[t])
        k_buf.copy_(K[bidx, :, pos])
        v_buf.copy_(V[bidx, :, pos])
        g.replay()
        torch.cuda.synchronize()
        np.testing.assert_array_equal(sess.out.cpu().numpy(), ref.out[t])
        np.testing.assert_array_equal(sess.match_ctx.cpu().numpy(), ref.match_n[t])
        np.testing.assert_array_equal(sess.dist.cpu().numpy(), ref.dist[t])
    np.testing.assert_array_equal(sess.seq_lens.cpu().numpy(), inp.contexts + T)
    del g
