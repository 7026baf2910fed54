"""Find tau for the 8B/32K workload so that about 80% of match decisions hit.

TEST INFRASTRUCTURE: calls only the oracle's query-only decision function on
the seeded query stream and prints the threshold; the value is stored as
``TAU_8B_32K`` in ``synth/streams.py`` and re-checked by a CPU test.

    python -m oracle.calibrate_tau
"""

import numpy as np

from oracle.mac_oracle import decisions_only
from synth.streams import workload, make_q_stream


def hit_rate(q64, window, tau):
    hit, _, _ = decisions_only(q64, window, tau)
    return float(hit.mean())


def main(target=0.80):
    w = workload("8b_32k")
    _, q64 = make_q_stream(w)
    lo, hi = 0.0, 4.0 * np.sqrt(w.head_dim)
    for _ in range(60):
        mid = 0.5 * (lo + hi)
        if hit_rate(q64, w.window, mid) < target:
            lo = mid
        else:
            hi = mid
    tau = round(hi, 4)
    print(f"tau={tau:.4f} hit_rate={hit_rate(q64, w.window, tau):.4f}")


if __name__ == "__main__":
    main()
