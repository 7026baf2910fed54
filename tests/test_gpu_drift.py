"""Drift of MAC from dense attention along chains of hits (GPU, against the
oracle).  The benchmark's drift runner decodes one stream twice on the same
KV, with the MAC configuration and with W = 0 (never a match, so plain
attention over every key), and reports max |out_MAC - out_dense| per head.
Here the same quantity is computed from the fp64 oracle's MAC outputs and
its dense attention and compared."""

import math

import numpy as np
import pytest

import bench
from oracle import mac_oracle as M
from synth.streams import workload
from tests.gpu_harness import OUT_TOL, GpuRun, check_groups, say

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("tau_f,band", [(0.5, 256), (0.75, 64)])
def test_drift_matches_the_oracle(tau_f, band):
    w = workload("gen_16k", context=1500, steps=96,
                 tau=tau_f * math.sqrt(128), band=band)
    say(f"[drift] tau {tau_f} sqrt(d), B {band}")
    dmax, match_n, inp = bench.drift_run(w, w.steps)
    # the oracle replays the MAC stream (following the GPU only at
    # borderline decisions) and gives dense attention at every step
    gpu = GpuRun({t: np.zeros((1, w.n_q_heads, w.head_dim), np.float32) for t in range(w.steps)},
                 {t: match_n[t] for t in range(w.steps)},
                 {t: np.full((1, w.n_q_heads), np.nan, np.float32) for t in range(w.steps)}, None)
    got = {}
    rep = check_groups(w, inp, gpu, [(0, g) for g in range(w.n_kv_heads)], collect=got,
                       tol=float("inf"))
    assert not [m for m in rep.mismatches if m[3] == "decision"], rep.mismatches[:5]
    K, V = inp.k.double().numpy(), inp.v.double().numpy()
    G = w.group
    worst = 0.0
    hit_steps = 0
    for t in range(w.steps):
        n = int(inp.contexts[0]) + t + 1
        qr = M.rope(inp.q64[t, 0], n - 1, w.rope_theta)
        for g in range(w.n_kv_heads):
            mac_o, mn = got[(0, g, t)]
            dense_o = M.dense(qr[g * G:(g + 1) * G], K[0, g, :n], V[0, g, :n])
            d_orc = np.abs(mac_o - dense_o).max(axis=1)
            d_gpu = dmax[t, 0, g * G:(g + 1) * G]
            worst = max(worst, float(np.abs(d_gpu - d_orc).max()))
            # a head that missed runs the dense plan exactly
            miss = mn < 0
            assert (d_gpu[miss] == 0).all(), (t, g)
            hit_steps += int((~miss).sum())
    say(f"[drift] hits {hit_steps}, max drift {dmax.max():.3e}, |gpu - oracle| {worst:.2e}")
    assert worst <= 2 * OUT_TOL
    assert hit_steps > 0
    depth = bench.chain_depths(match_n, inp.contexts)
    assert depth.max() >= 2
