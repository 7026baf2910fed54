"""CPU checks of the built gfx950 code object: every kernel of libmac keeps
its arrays in registers (no private segment, no vector-register spills), and
the kernels that run two waves per SIMD fit that occupancy's register file.

The code object is taken out of the library the build wrote (its
.hip_fatbin section, then the gfx950 bundle) and its metadata note read."""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "kv_cache_reuse_amd", "libmac.so")
LLVM = "/opt/rocm/llvm/bin"


MAGIC = b"__CLANG_OFFLOAD_BUNDLE__"


def kernel_metadata(tmp_path):
    """Kernel records of every code object in the library: each source file
    of the library adds its own offload bundle to the .hip_fatbin section."""
    tools = [os.path.join(LLVM, t) for t in ("llvm-objcopy", "clang-offload-bundler", "llvm-readelf")]
    if not all(os.path.exists(t) for t in tools):
        pytest.skip("ROCm LLVM tools not found")
    if not os.path.exists(LIB):
        pytest.skip("libmac.so is not built")
    objcopy, bundler, readelf = tools
    fat = tmp_path / "fat.bin"
    subprocess.run([objcopy, f"--dump-section=.hip_fatbin={fat}", LIB, str(tmp_path / "lib.so")],
                   check=True, capture_output=True)
    data = fat.read_bytes()
    starts = []
    i = data.find(MAGIC)
    while i >= 0:
        starts.append(i)
        i = data.find(MAGIC, i + 1)
    kernels = {}
    for k, a in enumerate(starts):
        e = starts[k + 1] if k + 1 < len(starts) else len(data)
        piece = tmp_path / f"bundle{k}.bin"
        piece.write_bytes(data[a:e])
        co = tmp_path / f"gfx950_{k}.co"
        subprocess.run([bundler, "--type=o", f"--input={piece}", "--unbundle",
                        "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={co}"],
                       check=True, capture_output=True)
        if co.stat().st_size == 0:
            continue
        notes = subprocess.run([readelf, "--notes", str(co)], check=True, capture_output=True,
                               text=True).stdout
        cur = None
        for line in notes.splitlines():
            m = re.match(r"\s*-?\s*\.(\w+):\s+(\S+)", line)
            if not m:
                continue
            key, val = m.groups()
            if key == "agpr_count":          # first field of each kernel's record
                cur = {"agpr_count": int(val)}
            elif cur is not None and key in ("name", "private_segment_fixed_size", "vgpr_count",
                                             "vgpr_spill_count", "max_flat_workgroup_size"):
                cur[key] = val if key == "name" else int(val)
                if key == "name":
                    kernels[val] = cur
    return kernels


def test_every_source_file_code_object_is_read(tmp_path):
    # each source file's kernels come in a bundle of their own: the step,
    # wide-path and set-up kernels must all be among the records read
    ks = kernel_metadata(tmp_path)
    for part in ("step_kernel", "merge_kernel", "wide_step_kernel", "match_kernel",
                 "append_kernel"):
        assert any(part in n for n in ks), part


def test_no_kernel_uses_scratch(tmp_path):
    ks = kernel_metadata(tmp_path)
    assert len(ks) >= 40
    for name, k in ks.items():
        assert k.get("private_segment_fixed_size", 0) == 0, (name, k)
        assert k.get("vgpr_spill_count", 0) == 0, (name, k)


def test_two_wave_kernels_fit_their_register_file(tmp_path):
    # a SIMD holds 512 registers per lane: workgroups of 8 waves on 4 SIMDs
    # run two waves per SIMD, so each may use at most 256 (VGPRs and AGPRs)
    ks = kernel_metadata(tmp_path)
    for name, k in ks.items():
        if k.get("max_flat_workgroup_size", 0) == 512:
            assert k["vgpr_count"] + k["agpr_count"] <= 256, (name, k)
