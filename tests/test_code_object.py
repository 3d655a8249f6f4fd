"""Properties of the built gfx950 code objects (host only, no GPU).

Every kernel in libsv.so must run without scratch memory: a spill to memory
or a stack-allocated array turns the hot loops' register traffic into memory
traffic (an order of magnitude slower), and the compiler gives no error for it.
The kernel descriptors' metadata (AMDGPU code object notes) states each
kernel's private segment size.  (Vector registers spilled to the accumulation
registers need no memory and are allowed.)
"""
import os
import re
import shutil
import subprocess

import pytest

import draft_token_verification_sv_amd as sv

LLVM = "/opt/rocm/llvm/bin"


def _kernel_notes(tmp_path):
    lib = sv.library_path
    if not lib or not os.path.exists(lib):
        pytest.skip("library not built")
    objdump, readelf = os.path.join(LLVM, "llvm-objdump"), os.path.join(LLVM, "llvm-readelf")
    if not (os.path.exists(objdump) and os.path.exists(readelf)):
        pytest.skip("llvm tools not found")
    copy = tmp_path / "libsv.so"
    shutil.copy(lib, copy)
    subprocess.run([objdump, "--offloading", str(copy)], check=True, capture_output=True, cwd=tmp_path)
    cos = sorted(p for p in tmp_path.iterdir() if p.name.endswith("gfx950"))
    assert cos, "no gfx950 code object in the library"
    kernels = {}
    for co in cos:
        text = subprocess.run([readelf, "--notes", str(co)], check=True, capture_output=True, text=True).stdout
        # the kernel list: one YAML mapping per kernel, keys in any order
        for block in re.split(r"\n\s+- \.", text):
            name = re.search(r"\.name:\s+(\S+)", "." + block)
            if not name or "kernel" not in name.group(1):
                continue
            fields = dict(re.findall(r"\.(private_segment_fixed_size|vgpr_spill_count|sgpr_spill_count):\s+(\d+)",
                                     "." + block))
            kernels[name.group(1)] = {k: int(v) for k, v in fields.items()}
    return kernels


def test_kernels_use_no_scratch(tmp_path):
    kernels = _kernel_notes(tmp_path)
    assert any("attn_dma_kernel" in k for k in kernels), sorted(kernels)[:5]
    assert all("private_segment_fixed_size" in v for v in kernels.values())
    bad = {k: v for k, v in kernels.items() if v["private_segment_fixed_size"] != 0}
    assert not bad, bad
