"""Pins of the fp64 oracle against facts fixed outside the oracle itself.

Each test checks the oracle against something it does not compute itself:
a closed form (complex-number rotation, the rotation group's relative-position
property), a library routine (scipy's softmax and logsumexp), a hand-derived
fixture (tests/golden/closed_forms.json), an invariant of the definitions
(partition invariance of the merge, constant reads on a hit, dense attention
whenever nothing can be reused), or the pure-Python brute force, which states
the same definitions with a different structure.
"""

import json
import math
import os

import numpy as np
import pytest
from scipy.special import logsumexp, softmax

from oracle import brute
from oracle import mac_oracle as M
from synth.streams import make_inputs, make_q_stream, workload

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# rotary embedding (D2)
# ---------------------------------------------------------------------------

def test_rope_position_zero_is_identity():
    x = np.random.default_rng(0).standard_normal((5, 64))
    np.testing.assert_array_equal(M.rope(x, 0, 1e4), x)


def test_rope_matches_complex_rotation():
    # rotate-half RoPE = multiply z_i = x_i + i x_{i+d/2} by exp(i pos theta^(-2i/d))
    rng = np.random.default_rng(1)
    d, theta = 128, 5e5
    for pos in (1, 7, 4097, 131071):
        x = rng.standard_normal(d)
        z = x[: d // 2] + 1j * x[d // 2:]
        freqs = np.array([theta ** (-2.0 * i / d) for i in range(d // 2)])
        zr = z * np.exp(1j * pos * freqs)
        want = np.concatenate([zr.real, zr.imag])
        # angles up to 1.3e5 rad: an ulp of the frequency moves sin/cos by ~1e-11
        np.testing.assert_allclose(M.rope(x, pos, theta), want, rtol=0, atol=1e-10)


def test_rope_relative_position_property():
    # <R(a) q, R(b) k> = <R(a - b) q, k>: rotations compose additively
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal(64), rng.standard_normal(64)
    for a, b in ((10, 3), (5000, 4999), (77, 0)):
        lhs = M.rope(q, a, 1e4) @ M.rope(k, b, 1e4)
        rhs = M.rope(q, a - b, 1e4) @ k
        assert abs(lhs - rhs) < 1e-9


def test_rope_preserves_norm_and_matches_brute():
    rng = np.random.default_rng(3)
    for d in (4, 8, 64):
        x = rng.standard_normal(d)
        y = M.rope(x, 1234, 1e4)
        assert abs(np.linalg.norm(y) - np.linalg.norm(x)) < 1e-12
        np.testing.assert_allclose(y, brute.rotate(list(x), 1234, 1e4), atol=1e-12)


# ---------------------------------------------------------------------------
# partial states and merge (D3, D4)
# ---------------------------------------------------------------------------

def test_attend_equals_scipy_softmax_attention():
    rng = np.random.default_rng(4)
    d, L = 64, 300
    qr, K, V = rng.standard_normal((3, d)), rng.standard_normal((L, d)), rng.standard_normal((L, d))
    st = M.attend(qr, K, V)
    z = qr @ K.T / math.sqrt(d)
    np.testing.assert_allclose(st.o, softmax(z, axis=1) @ V, atol=1e-13)
    np.testing.assert_allclose(st.lse, logsumexp(z, axis=1), atol=1e-12)


@pytest.mark.parametrize("scale", [1.0, 8.0, 30.0])
def test_merge_of_any_partition_equals_single_pass(scale):
    rng = np.random.default_rng(5)
    d, L = 32, 200
    qr = rng.standard_normal((2, d))
    K = rng.standard_normal((L, d)) * scale
    V = rng.standard_normal((L, d))
    whole = M.attend(qr, K, V)
    for trial in range(20):
        cuts = np.sort(rng.integers(0, L + 1, size=rng.integers(1, 8)))
        edges = [0, *cuts.tolist(), L]          # repeated cuts give empty parts
        parts = [M.attend(qr, K[a:b], V[a:b]) for a, b in zip(edges[:-1], edges[1:])]
        if trial % 2:                            # a different association
            acc = parts[-1]
            for p in reversed(parts[:-1]):
                acc = M.merge(p, acc)
        else:
            acc = M.merge_all(parts)
        np.testing.assert_allclose(acc.o, whole.o, atol=1e-12)
        np.testing.assert_allclose(acc.lse, whole.lse, atol=1e-10)
        assert np.all(np.isfinite(acc.o))


def test_merge_empty_is_identity_and_symmetric():
    rng = np.random.default_rng(6)
    qr, K, V = rng.standard_normal((2, 16)), rng.standard_normal((9, 16)), rng.standard_normal((9, 16))
    a = M.attend(qr, K[:4], V[:4])
    b = M.attend(qr, K[4:], V[4:])
    e = M.State.empty(2, 16)
    for got in (M.merge(a, e), M.merge(e, a)):
        np.testing.assert_array_equal(got.o, a.o)
        np.testing.assert_array_equal(got.m, a.m)
        np.testing.assert_array_equal(got.l, a.l)
    ee = M.merge(e, e)
    assert np.all(ee.m == -np.inf) and np.all(ee.l == 0) and np.all(ee.o == 0)
    ab, ba = M.merge(a, b), M.merge(b, a)
    np.testing.assert_allclose(ab.o, ba.o, atol=1e-15)


def test_merge_golden_closed_form():
    g = golden()["merge_two_states"]
    a = M.State(np.array([g["o1"]]), np.array([g["m1"]]), np.array([g["l1"]]))
    b = M.State(np.array([g["o2"]]), np.array([math.log(g["exp_m2"])]), np.array([g["l2"]]))
    got = M.merge(a, b)
    np.testing.assert_allclose(got.o[0], g["o"], atol=1e-15)
    assert abs(got.l[0] - g["l"]) < 1e-15


# ---------------------------------------------------------------------------
# match (D6)
# ---------------------------------------------------------------------------

def _ring(qs, p=0, n=10):
    return [M.Entry(np.asarray(q, float), np.zeros(len(q)), 0.0, 1.0, p, n + i)
            for i, q in enumerate(qs)]


def test_match_golden_ties_and_strictness():
    g = golden()["match"]
    ring = _ring(g["ring"])
    for case in g["cases"]:
        mt = M.match(np.asarray(g["q"], float), ring, case["tau"], p_new=5)
        assert mt.j == case["j"] and mt.hit == case["hit"]
        assert abs(mt.dist - case["dist"]) < 1e-15


def test_match_repeated_query_hits_any_positive_tau():
    q = np.random.default_rng(7).standard_normal(8)
    ring = _ring([q + 1.0, q, q + 2.0])
    for tau in (1e-300, 1e-3, 10.0):
        mt = M.match(q, ring, tau, p_new=0)
        assert mt.hit and mt.j == 1 and mt.dist == 0.0
    assert not M.match(q, ring, 0.0, p_new=0).hit           # strict: tau = 0 never hits
    assert not M.match(q, [], 10.0, p_new=0).hit            # empty ring


def test_match_nan_is_never_chosen():
    q = np.zeros(4)
    ring = _ring([[np.nan, 0, 0, 0], [3.0, 0, 0, 0]])
    mt = M.match(q, ring, 10.0, p_new=0)
    assert mt.j == 1 and mt.hit and mt.dist == 3.0
    mt = M.match(np.full(4, np.nan), ring, 10.0, p_new=0)
    assert mt.j == -1 and not mt.hit and mt.dist == np.inf


def test_match_skips_entries_whose_prefix_passes_the_current_one():
    q = np.zeros(4)
    ring = [M.Entry(np.zeros(4), np.zeros(4), 0.0, 1.0, 50, 60),
            M.Entry(np.ones(4) * 0.1, np.zeros(4), 0.0, 1.0, 10, 20)]
    mt = M.match(q, ring, 1.0, p_new=30)
    assert mt.j == 1 and mt.hit


# ---------------------------------------------------------------------------
# the recurrence
# ---------------------------------------------------------------------------

def small(**kw):
    base = dict(head_dim=16, context=120, steps=40, window=6, band=20)
    base.update(kw)
    return workload("tiny", **base)


def run_dense_check(w, p_jump=None):
    inp = make_inputs(w, p_jump=p_jump)
    res, _ = M.run(w, inp)
    K, V = inp.k.double().numpy(), inp.v.double().numpy()
    G = w.group
    hits = 0
    for t, row in enumerate(res):
        for b, r in row.items():
            n = int(inp.contexts[b]) + t + 1
            for h in range(w.n_q_heads):
                qr = M.rope(inp.q64[t, b, h], n - 1, w.rope_theta)
                z = K[b, h // G, :n] @ qr / math.sqrt(w.head_dim)
                want = softmax(z) @ V[b, h // G, :n]
                np.testing.assert_allclose(r.out[h], want, atol=1e-12)
            hits += int(r.hit.sum())
    return hits


def test_tau_zero_is_dense_attention():
    assert run_dense_check(small(tau=0.0)) == 0


def test_window_zero_is_dense_attention():
    assert run_dense_check(small(window=0)) == 0


def test_band_covering_the_context_is_dense_even_on_hits():
    hits = run_dense_check(small(band=10_000))
    assert hits > 0


def test_entry_after_a_miss_is_dense_prefix_state():
    w = small(p_jump=1.0)
    inp = make_inputs(w)
    res, _ = M.run(w, inp)
    K, V = inp.k.double().numpy(), inp.v.double().numpy()
    checked = 0
    for t, row in enumerate(res):
        r = row[0]
        for h in np.nonzero(~r.hit)[0]:
            e = r.entries[h]
            qr = M.rope(inp.q64[t, 0, h], r.n - 1, w.rope_theta)
            z = K[0, 0, :e.p] @ qr / math.sqrt(w.head_dim)
            np.testing.assert_allclose(e.o, softmax(z) @ V[0, 0, :e.p], atol=1e-12)
            assert abs(e.m + math.log(e.l) - logsumexp(z)) < 1e-10
            checked += 1
    assert checked > 10


def test_exact_reused_prefix_turns_a_hit_into_dense_attention():
    # a hit reuses a state over [0, s); if that state were the current query's
    # own, the composition must give dense attention over [0, n)
    rng = np.random.default_rng(8)
    d, n, B = 32, 500, 64
    K, V = rng.standard_normal((n, d)), rng.standard_normal((n, d))
    qr = rng.standard_normal((3, d))
    for s in (0, 1, 200, n - B - 5, n - B):
        exact = M.attend(qr, K[:s], V[:s])
        prefix, full = M.compose(qr, K, V, exact, s, n - B, n)
        z = qr @ K.T / math.sqrt(d)
        np.testing.assert_allclose(full.o, softmax(z, axis=1) @ V, atol=1e-12)
        zp = z[:, : n - B]
        np.testing.assert_allclose(prefix.lse, logsumexp(zp, axis=1), atol=1e-10)


def test_hit_reads_are_constant_in_context_length():
    counts = {}
    for ctx in (2048, 131072):
        w = small(head_dim=8, context=ctx, steps=60, window=8, band=32,
                  p_jump=0.2)
        inp = make_inputs(w)
        res, _ = M.run(w, inp)
        got = []
        for t, row in enumerate(res):
            r = row[0]
            for h in range(w.n_q_heads):
                if r.hit[h]:
                    delta = r.n - r.match_n[h]
                    assert r.keys_read[h] == delta + min(w.band, r.match_n[h])
                    assert 1 <= delta <= w.window
                else:
                    assert r.keys_read[h] == r.n
                got.append((t, h, bool(r.hit[h]), int(r.keys_read[h]) if r.hit[h] else -1))
        counts[ctx] = got
    assert counts[2048] == counts[131072]            # same decisions, same reads
    assert sum(1 for x in counts[2048] if x[2]) > 20


def test_query_only_decisions_agree_with_the_recurrence():
    for w in (small(p_jump=0.3, batch=2, n_q_heads=4, n_kv_heads=2),
              small(period=3, window=4, steps=30)):
        inp = make_inputs(w)
        res, _ = M.run(w, inp)
        hit, age, best = M.decisions_only(inp.q64, w.window, w.tau)
        for t, row in enumerate(res):
            for b, r in row.items():
                np.testing.assert_array_equal(r.hit, hit[t, b])
                np.testing.assert_allclose(r.dist, best[t, b], rtol=1e-15)
                want_n = np.where(hit[t, b], r.n - age[t, b], -1)
                np.testing.assert_array_equal(r.match_n, want_n)


BRUTE_CASES = [
    dict(head_dim=4, context=8, steps=40, window=4, band=3, batch=1, n_q_heads=2, n_kv_heads=1),
    dict(head_dim=4, context=1, steps=40, window=4, band=0, batch=2, n_q_heads=4, n_kv_heads=2),
    dict(head_dim=8, context=5, steps=40, window=1, band=100, batch=1, n_q_heads=2, n_kv_heads=2),
    dict(head_dim=4, context=6, steps=42, window=4, band=3, period=3, batch=1, n_q_heads=2, n_kv_heads=1),
    dict(head_dim=4, context=3, steps=45, window=4, band=5, p_jump=0.5, batch=1, n_q_heads=4, n_kv_heads=1),
]


@pytest.mark.parametrize("case", range(len(BRUTE_CASES)))
def test_brute_force_agrees_on_tiny_inputs(case):
    kw = dict(BRUTE_CASES[case])
    kw.setdefault("tau", 0.5 * math.sqrt(kw["head_dim"]))
    w = workload("tiny", **kw)
    inp = make_inputs(w)
    K, V = inp.k.double().numpy(), inp.v.double().numpy()
    orc = M.MacOracle.for_workload(w)
    bf = brute.BruteMac(w.batch, w.n_q_heads, w.n_kv_heads, w.head_dim, w.window,
                        w.band, w.tau, w.rope_theta)
    hits = 0
    for t in range(w.steps):
        for b in range(w.batch):
            n = int(inp.contexts[b]) + t + 1
            r = orc.step(b, inp.q64[t, b], K[b], V[b], n)
            rb = bf.step(b, inp.q64[t, b].tolist(), K[b].tolist(), V[b].tolist(), n)
            for h in range(w.n_q_heads):
                x = rb[h]
                assert bool(r.hit[h]) == x["hit"]
                assert int(r.match_n[h]) == x["match_n"]
                assert int(r.keys_read[h]) == x["keys_read"]
                np.testing.assert_allclose(r.out[h], x["out"], atol=1e-12)
                e, xe = r.entries[h], x["entry"]
                assert (e.p, e.n) == (xe["p"], xe["n"])
                if xe["l"] > 0:
                    np.testing.assert_allclose(e.o, xe["o"], atol=1e-12)
                    assert abs((e.m + math.log(e.l)) - (xe["m"] + math.log(xe["l"]))) < 1e-10
                else:
                    assert e.l == 0 and e.m == -np.inf
                hits += int(r.hit[h])
    assert hits > 0


def test_nan_query_misses_and_poisons_only_its_head():
    w = small(steps=12, n_q_heads=4, n_kv_heads=2)
    inp = make_inputs(w)
    K, V = inp.k.double().numpy(), inp.v.double().numpy()
    orc = M.MacOracle.for_workload(w)
    for t in range(w.steps):
        q = inp.q64[t, 0].copy()
        if t == 8:
            q[1, 3] = np.nan
        r = orc.step(0, q, K[0], V[0], int(inp.contexts[0]) + t + 1)
        if t == 8:
            assert not r.hit[1]
            assert np.all(np.isnan(r.out[1]))
            assert np.all(np.isfinite(np.delete(r.out, 1, axis=0)))


def test_calibrated_tau_gives_eighty_percent_hits():
    w = workload("8b_32k")
    _, q64 = make_q_stream(w)
    hit, _, _ = M.decisions_only(q64, w.window, w.tau)
    assert abs(hit.mean() - 0.80) <= 0.01


def test_hit_rate_sweep_points():
    # the jump probabilities of the headline sweep give about 0/50/80/95% hits
    w = workload("8b_128k")
    want = {1.0: (0.0, 0.0), 0.5: (0.40, 0.60), 0.2: (0.72, 0.88), 0.05: (0.90, 1.0)}
    for p, (lo, hi) in want.items():
        _, q64 = make_q_stream(w, p_jump=p)
        rate = M.decisions_only(q64, w.window, w.tau)[0].mean()
        assert lo <= rate <= hi, (p, rate)


def test_hit_reads_golden():
    for c in golden()["hit_reads"]["cases"]:
        w = workload("tiny", head_dim=4, context=c["n_e"] - 1, steps=2,
                     window=2, band=c["band"], tau=1.0, period=1)
        # the second step repeats the first query, so it hits the entry of
        # context n_e; extend the context so that the step sees n keys
        w = w.replace(context=c["n_e"] - 1)
        inp = make_inputs(w, steps=c["n"] - c["n_e"] + 1)
        K, V = inp.k.double().numpy(), inp.v.double().numpy()
        orc = M.MacOracle.for_workload(w)
        q0 = inp.q64[0, 0]
        r = orc.step(0, q0, K[0], V[0], c["n_e"])
        r = orc.step(0, q0, K[0], V[0], c["n"])
        assert r.hit.all() and (r.match_n == c["n_e"]).all()
        assert (r.keys_read == c["keys_read"]).all()


# ---------------------------------------------------------------------------
# ring seeding from a prefill
# ---------------------------------------------------------------------------

def test_seeded_entries_are_exact_prefix_states():
    # each seeded entry is the scipy softmax attention of its own rotated
    # query over [0, max(0, position + 1 - B)), with p and n of that position
    w = small(band=8, window=6)
    inp = make_inputs(w, steps=w.window)
    N = int(inp.contexts[0])
    K, V = inp.k.double().numpy(), inp.v.double().numpy()
    orc = M.MacOracle.for_workload(w)
    hist = inp.q64[:w.window, 0]
    orc.seed(0, hist, K[0], V[0], N)
    for h in range(w.n_q_heads):
        ring = orc.rings[0][h]
        assert len(ring) == w.window
        for j, e in enumerate(ring):
            pos = N - w.window + j
            assert (e.p, e.n) == (max(0, pos + 1 - w.band), pos + 1)
            g = h // w.group
            qr = M.rope(hist[j, h], pos, w.rope_theta)
            z = K[0, g, :e.p] @ qr / math.sqrt(w.head_dim)
            np.testing.assert_allclose(e.o, softmax(z) @ V[0, g, :e.p], atol=1e-12)
            assert abs(e.m + math.log(e.l) - logsumexp(z)) < 1e-10
            np.testing.assert_array_equal(e.q, hist[j, h])


def test_decode_after_seeding_matches_the_newest_seeded_query():
    # the first decode query repeats the last prefill query: distance 0, the
    # newest entry (context N) wins, and only the band and the tail are read
    w = small(band=8, window=6)
    inp = make_inputs(w, steps=w.window)
    N = int(inp.contexts[0])
    K, V = inp.k.double().numpy(), inp.v.double().numpy()
    orc = M.MacOracle.for_workload(w)
    orc.seed(0, inp.q64[:w.window, 0], K[0], V[0], N)
    r = orc.step(0, inp.q64[w.window - 1, 0], K[0], V[0], N + 1)
    assert r.hit.all()
    assert (r.match_n == N).all()
    assert (r.dist == 0).all()
    assert (r.keys_read == (N + 1) - max(0, N - w.band)).all()


def test_seeding_nothing_leaves_the_ring_empty():
    w = small()
    inp = make_inputs(w, steps=2)
    orc = M.MacOracle.for_workload(w)
    orc.seed(0, inp.q64[:0, 0], inp.k[0].double().numpy(), inp.v[0].double().numpy(),
             int(inp.contexts[0]))
    assert all(len(r) == 0 for r in orc.rings[0])


def test_reuse_chain_depths():
    # 0 after a miss, else one more than the reused entry's depth
    import bench
    mn = np.array([-1, 1001, 1002, -1, 1004, 1002]).reshape(-1, 1, 1)
    d = bench.chain_depths(mn, np.array([1000]))[:, 0, 0]
    assert d.tolist() == [0, 1, 2, 0, 1, 2]   # the entry of context 1002 has depth 1


def test_a_miss_is_dense_attention_in_the_oracle():
    # the drift of MAC from dense attention is zero (to rounding) on misses
    w = small(p_jump=0.3)
    inp = make_inputs(w)
    res, _ = M.run(w, inp)
    K, V = inp.k.double().numpy(), inp.v.double().numpy()
    misses = 0
    for t, row in enumerate(res):
        r = row[0]
        qr = M.rope(inp.q64[t, 0], r.n - 1, w.rope_theta)
        for h in np.nonzero(~r.hit)[0]:
            g = h // w.group
            np.testing.assert_allclose(r.out[h], M.dense(qr[h:h + 1], K[0, g, :r.n],
                                                         V[0, g, :r.n])[0], atol=1e-12)
            misses += 1
    assert misses > 5
