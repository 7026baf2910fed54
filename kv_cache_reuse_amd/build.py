"""Build the libraries in-tree for gfx950 with hipcc.

    python -m kv_cache_reuse_amd.build

libmac.so is the decode path (C ABI in include/mac.h); libmac_bw.so is the
streaming-read probe the benchmark measures the bandwidth ceiling with.
"""

import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
LIBS = {
    "libmac.so": ["csrc/step.hip", "csrc/merge.hip", "csrc/wide.hip", "csrc/kv_ring.hip",
                  "csrc/mac_api.hip"],
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


def _run(cmd, verbose: bool) -> None:
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


def _build_one(out: str, sources, verbose: bool) -> None:
    """Each source compiles to an object of its own, in parallel, then one
    link."""
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    objdir = os.path.join(HERE, "_build", os.path.basename(out))
    os.makedirs(objdir, exist_ok=True)
    objs = [os.path.join(objdir, os.path.basename(s) + ".o") for s in sources]
    compile_flags = [f for f in FLAGS if f != "-shared"]
    jobs = [[hipcc, *compile_flags, "-c", "-o", o, os.path.join(HERE, s)]
            for s, o in zip(sources, objs)]
    workers = max(1, min(len(jobs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 1))))
    with ThreadPoolExecutor(max_workers=workers) as pool:
        for f in [pool.submit(_run, j, verbose) for j in jobs]:
            f.result()
    tmp = out + ".tmp"
    _run([hipcc, "--offload-arch=gfx950", "-fPIC", "-shared", "-o", tmp, *objs], verbose)
    os.replace(tmp, out)


if __name__ == "__main__":
    print(build(verbose=True))
