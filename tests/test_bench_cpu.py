"""CPU checks of bench.py: its algorithmic byte count (the roofline's
numerator) against the closed forms of the method's reads, and its refusal
of more than one GPU."""

import os
import subprocess
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth.streams import workload  # noqa: E402


def _step(w, n, match_n, ring_count):
    return bench.step_bytes(w, np.array([n]), np.asarray(match_n).reshape(1, -1),
                            np.full((1, w.n_q_heads), ring_count))


def test_miss_reads_every_key_of_every_group():
    w = workload("8b_128k")
    n = 131073
    total, kv, keys = _step(w, n, np.full(w.n_q_heads, -1), w.window)
    assert keys == w.n_kv_heads * n
    assert kv == keys * 2 * w.head_dim * w.bytes_per_elem
    # the rest: ring rows, q in / out, the entry, the appended token; no reused state
    hq, d, bpe = w.n_q_heads, w.head_dim, w.bytes_per_elem
    rest = hq * w.window * (d * bpe + 8) + hq * (d * bpe + d * 4 + 16) + hq * (d * bpe + d * 4) \
        + w.n_kv_heads * 2 * d * bpe * 2
    assert total == kv + rest


def test_hit_reads_band_and_tail_whatever_the_context():
    # a match one step old: the tail is 1 key and the band B keys (the
    # constant-cost hit of the method), at 2K and at 128K keys alike
    w = workload("8b_128k")
    for n in (2048, 131073):
        _, _, keys = _step(w, n, np.full(w.n_q_heads, n - 1), w.window)
        assert keys == w.n_kv_heads * (1 + w.band)


def test_one_missing_head_makes_its_group_read_everything():
    w = workload("8b_128k")
    n = 50000
    mn = np.full(w.n_q_heads, n - 1)
    mn[5] = -1                       # head 5 is in group 1 (G = 4)
    _, _, keys = _step(w, n, mn, w.window)
    assert keys == (w.n_kv_heads - 1) * (1 + w.band) + n


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
