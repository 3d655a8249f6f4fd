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


@pytest.mark.parametrize("debug", [False, True], ids=["release", "debug"])
@pytest.mark.parametrize("source,kernel,variants",
                         [("attn_q4.hip", "attn_q4c_kernel", 6),      # 3 tile counts x (contiguous, paged)
                          ("attn_q4w.hip", "attn_q4w_kernel", 5)])    # 3 contiguous, 2 paged
def test_cooperative_kernel_owns_its_accumulation_registers(tmp_path, source, kernel, variants, debug):
    """The cooperative 4-bit attention kernels keep values of their own in
    a0..a95 through inline assembly alone (the four-wave kernel its O
    accumulators; the eight-wave kernel its O accumulators in a0..a47 and its
    query fragments in a48..a95); the compiler must not place any value of its
    own there (a spill or copy into them would corrupt O or the scores without
    an error).  Compiled to assembly with the library's flags, every reference
    to a0..a95 in those kernels must sit inside an inline-assembly block."""
    import importlib.util
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    spec = importlib.util.spec_from_file_location("sv_build", os.path.join(root, "draft_token_verification_sv_amd",
                                                                           "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    if not os.path.exists(mod.HIPCC):
        pytest.skip("hipcc not found")
    src = os.path.join(mod.CSRC, source)
    out = tmp_path / (source + ".s")
    flags = [f for f in mod.FLAGS if f not in ("-Wall",)] + mod.EXTRA.get(source, []) + (["-DSV_DEBUG"] if debug else [])
    subprocess.run([mod.HIPCC, *flags, "--cuda-device-only", "-S", src, "-o", str(out)], check=True,
                   capture_output=True)
    lines = out.read_text().split("\n")
    starts = [i for i, l in enumerate(lines) if re.match(r"^_Z\S*" + kernel + r"\S*:", l)]
    assert len(starts) == variants, len(starts)
    pinned = re.compile(r"\ba(\d+)\b|\ba\[(\d+):(\d+)\]")
    for s0 in starts:
        in_asm, bad, n_asm = False, [], 0
        for l in lines[s0:]:
            t = l.strip()
            if t.startswith(".Lfunc_end"):
                break
            if t.startswith(";;#ASMSTART"):
                in_asm = True
                continue
            if t.startswith(";;#ASMEND"):
                in_asm = False
                continue
            code = t.split(";")[0]
            for m in pinned.finditer(code):
                lo = int(m.group(1) if m.group(1) is not None else m.group(2))
                if lo < 96:
                    if in_asm:
                        n_asm += 1
                    else:
                        bad.append(t)
        assert n_asm > 0
        assert not bad, (lines[s0], bad[:5])
