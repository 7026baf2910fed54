"""CPU checks of the C ABI: the library loads, exports every entry point
include/mac.h declares, and rejects bad arguments before any HIP call.  Also
compiles and runs the host check of the kernels' integer logic."""

import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def B():
    import kv_cache_reuse_amd.binding as B
    return B


def declared_symbols():
    with open(os.path.join(ROOT, "include", "mac.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(mac_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported(B):
    names = declared_symbols()
    assert len(names) >= 12
    for n in names:
        assert hasattr(B.library(), n), n
    assert set(names) == set(B.EXPORTED)


def valid_cfg(B, **kw):
    c = B.MacConfig()
    c.batch, c.n_q_heads, c.n_kv_heads, c.head_dim = 1, 32, 8, 128
    c.dtype = B.MAC_DTYPE_BF16
    c.max_context, c.window, c.band, c.tau, c.rope_theta = 4096, 32, 256, 5.0, 5e5
    for k, v in kw.items():
        setattr(c, k, v)
    return c


BAD = [
    (dict(batch=0), 1), (dict(n_kv_heads=0), 1), (dict(n_q_heads=30), 1),
    # a group must split into equal parts of at most 32 heads (bf16) or 16 (fp32)
    (dict(n_q_heads=8 * 33), 2), (dict(n_q_heads=8 * 17, dtype=0), 2),
    (dict(head_dim=96), 2), (dict(dtype=7), 2),
    (dict(kv_layout=2), 1),
    (dict(window=-1), 1), (dict(band=-3), 1), (dict(tau=-1.0), 1),
    (dict(tau=float("nan")), 1), (dict(rope_theta=0.0), 1),
    (dict(rope_theta=float("inf")), 1), (dict(max_slices=1), 1),
    (dict(max_context=0), 1), (dict(page_size=8), 2),
    (dict(page_size=16, max_pages_per_seq=0, n_pages=4), 1),
]


@pytest.mark.parametrize("i", range(len(BAD)))
def test_bad_configs_are_rejected(B, i):
    kw, status = BAD[i]
    cfg = valid_cfg(B, **kw)
    assert B.mac_ring_bytes(cfg) == 0
    assert B.mac_workspace_bytes(cfg) == 0
    assert B.mac_kv_cache_bytes(cfg) == 0
    out = ctypes.c_void_p()
    host = (ctypes.c_int32 * cfg.batch if cfg.batch > 0 else ctypes.c_int32 * 1)()
    st = B.library().mac_init(ctypes.byref(cfg), 0x10000, 0x20000, 0x30000,
                              ctypes.cast(host, ctypes.c_void_p), None, ctypes.byref(out))
    assert st == status, B.mac_last_error()
    assert out.value is None
    assert B.mac_last_error()


def test_wide_groups_are_accepted(B):
    # bf16 groups of 17-32 heads run as one group, 33-64 as two equal ones
    for hq in (8 * 17, 8 * 32, 8 * 64, 8 * 48):
        assert B.mac_workspace_bytes(valid_cfg(B, n_q_heads=hq)) > 0
    assert B.mac_workspace_bytes(valid_cfg(B, n_q_heads=8 * 34)) > 0


def test_sizes_of_a_valid_config(B):
    cfg = valid_cfg(B)
    kv = B.mac_kv_cache_bytes(cfg)
    assert kv == 8 * (4096 // 16) * 16 * 128 * 2
    ring = B.mac_ring_bytes(cfg)
    assert ring >= 32 * 33 * (128 * 2 + 128 * 4 + 16)
    assert B.mac_workspace_bytes(cfg) > 0
    paged = valid_cfg(B, page_size=16, max_pages_per_seq=300, n_pages=1000)
    assert B.mac_kv_cache_bytes(paged) == 1000 * 8 * 16 * 128 * 2
    # natural rows: [batch][Hkv][max_context][d] exactly, pages as for tiles
    rows = valid_cfg(B, kv_layout=B.MAC_KV_ROWS, max_context=4097)
    assert B.mac_kv_cache_bytes(rows) == 8 * 4097 * 128 * 2
    tiles = valid_cfg(B, max_context=4097)
    assert B.mac_kv_cache_bytes(tiles) == 8 * 4112 * 128 * 2
    paged_rows = valid_cfg(B, page_size=16, max_pages_per_seq=300, n_pages=1000,
                           kv_layout=B.MAC_KV_ROWS)
    assert B.mac_kv_cache_bytes(paged_rows) == B.mac_kv_cache_bytes(paged)
    # fp32 rows too
    rows32 = valid_cfg(B, kv_layout=B.MAC_KV_ROWS, max_context=4097, dtype=B.MAC_DTYPE_F32)
    assert B.mac_kv_cache_bytes(rows32) == 8 * 4097 * 128 * 4


@pytest.mark.parametrize("name,capacity,slices", [
    ("8b_128k", 131200, 32),      # 8 groups: one round of 32 slices per group
    ("paged_b8", 20000, 4),       # 64 groups: one round of 4
    ("paged_b8", 30000, 8),       # two rounds
    ("paged_b8", 50000, 16),      # ceil(50000 / 16384) = 4 rounds
    ("paged_b8", 70000, 16),      # capped at 4 rounds
])
def test_default_slice_count(B, name, capacity, slices):
    # the workspace holds the split-K partial states of every slice, so the
    # default slice count shows as the size of an explicit one
    from synth.streams import workload
    w = workload(name).replace(page_size=0)
    default = B.mac_workspace_bytes(B.config_from_workload(w, max_context=capacity))
    assert default == B.mac_workspace_bytes(B.config_from_workload(w, max_context=capacity,
                                                                   max_slices=slices))
    assert default != B.mac_workspace_bytes(B.config_from_workload(w, max_context=capacity,
                                                                   max_slices=slices + 1))


def test_pointer_and_capacity_errors_come_before_device_calls(B):
    lib = B.library()
    cfg = valid_cfg(B)
    out = ctypes.c_void_p()
    host = (ctypes.c_int32 * 1)(0)
    hp = ctypes.cast(host, ctypes.c_void_p)
    assert lib.mac_init(ctypes.byref(cfg), None, 0x20000, 0x30000, hp, None, ctypes.byref(out)) == 1
    assert "ring" in B.mac_last_error()
    assert lib.mac_init(ctypes.byref(cfg), 0x10008, 0x20000, 0x30000, hp, None, ctypes.byref(out)) == 1
    assert "aligned" in B.mac_last_error()
    assert lib.mac_init(ctypes.byref(cfg), 0x10000, 0x20000, 0x30000, None, None, ctypes.byref(out)) == 1
    host[0] = 4097
    assert lib.mac_init(ctypes.byref(cfg), 0x10000, 0x20000, 0x30000, hp, None, ctypes.byref(out)) == 3
    host[0] = -1
    assert lib.mac_init(ctypes.byref(cfg), 0x10000, 0x20000, 0x30000, hp, None, ctypes.byref(out)) == 3
    assert lib.mac_init(ctypes.byref(cfg), 0x10000, 0x20000, 0x30000, hp, None, None) == 1


def test_null_context_calls(B):
    lib = B.library()
    assert lib.mac_append_kv(None, 16, 16, None, 16, 16, None) == 1
    assert lib.mac_decode_step(None, 16, 16, 16, None, 16, None, None, None) == 1
    assert lib.mac_prefill_kv(None, 16, 16, None, 0, 16, 16, 1, None) == 1
    assert lib.mac_read_kv(None, 16, 16, None, 0, 0, 1, 16, 16, None) == 1
    assert lib.mac_query_cache_push(None, 16, 16, 16, 16, 16, 16, None, None) == 1
    assert lib.mac_seed_ring(None, 16, 1, 16, 16, None, None) == 1
    assert lib.mac_profile_enable(None, 1) == 1
    assert lib.mac_destroy(None) == 0


def test_host_integer_logic(tmp_path):
    exe = str(tmp_path / "host_logic_test")
    src = os.path.join(ROOT, "tests", "cpp", "host_logic.cpp")
    r = subprocess.run(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O1", "-std=c++17",
                        "-x", "hip", src, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and "OK" in r.stdout, r.stdout[-2000:]


def test_device_error_poisons_the_context(tmp_path):
    # the C ABI linked against launchers that fail on request (no GPU):
    # MAC_ERR_DEVICE from the failing call, MAC_ERR_STATE from every later
    # call on that context, other contexts unaffected
    exe = str(tmp_path / "state_stub_test")
    srcs = [os.path.join(ROOT, "kv_cache_reuse_amd", "csrc", "mac_api.hip"),
            os.path.join(ROOT, "tests", "cpp", "state_stub.cpp")]
    r = subprocess.run(["/opt/rocm/bin/hipcc", "--offload-arch=gfx950", "-O1", "-std=c++17",
                        *srcs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0 and "OK" in r.stdout, r.stdout[-2000:] + r.stderr[-2000:]
