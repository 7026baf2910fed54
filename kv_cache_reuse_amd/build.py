"""Build the libraries in-tree for gfx950 with hipcc.

    python -m kv_cache_reuse_amd.build

libmac.so is the decode path (C ABI in include/mac.h); libmac_bw.so is the
streaming-read probe the benchmark measures the bandwidth ceiling with.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
LIBS = {
    "libmac.so": ["csrc/step.hip", "csrc/wide.hip", "csrc/kv_ring.hip", "csrc/mac_api.hip"],
    "libmac_bw.so": ["csrc/bw_probe.hip"],
}
SOURCES = LIBS["libmac.so"]
OUT = os.path.join(HERE, "libmac.so")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
    # the compiler must not form packed fp32 instructions (v_pk_*_f32)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(verbose: bool = False) -> str:
    for name, sources in LIBS.items():
        _build_one(os.path.join(HERE, name), sources, verbose)
    return OUT


def _build_one(out: str, sources, verbose: bool) -> None:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc, *FLAGS, "-o", tmp, *[os.path.join(HERE, s) for s in sources]]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    noise = "packed-fp32-ops"
    msgs = [l for l in (r.stdout + r.stderr).splitlines() if noise not in l]
    if r.returncode != 0:
        sys.stderr.write("\n".join(msgs) + "\n")
        raise RuntimeError(f"hipcc failed with status {r.returncode}")
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, out)


if __name__ == "__main__":
    print(build(verbose=True))
