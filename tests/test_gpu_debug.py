"""The SV_DEBUG library on the GPU: broken device-side inputs are recorded in
the precondition word that sv_check_device_errors returns, and the kernels
still finish normally with the documented behaviour (a parent that is not an
earlier node ends the path, a page outside the pool reads zeros, ctx_lens
are clamped, out-of-range accept lengths skip the compaction).

The debug library is loaded by the binding when SV_DEBUG=1 is set before the
import, so the calls run in one child process that prints each step's
result as it goes; this process only checks them.
"""
import json
import os
import subprocess
import sys

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r'''
import json, sys
import numpy as np, torch
sys.path.insert(0, ROOT)
sys.path.insert(0, ROOT + "/tests")
import draft_token_verification_sv_amd as sv
import workloads
from sv_harness import DeviceCase
assert sv.debug_build and sv.library_path.endswith("libsv_debug.so")

def report(name, **kw):
    print(json.dumps(dict(step=name, **kw)), flush=True)

cfg = workloads.small_variant(workloads.CONFIGS["C3"], ctx=100, vocab=500)
case = workloads.make_case(cfg, seed=5, capacity_pad=4)
dc = DeviceCase(case)
report("clean_start", bits=sv.check_device_errors())
out, lse = dc.attn()
acc, path, tok, am = dc.accept()
report("clean_calls", bits=sv.check_device_errors(), finite=bool(torch.isfinite(out.float()).all()))

bad = case.parent.copy()
bad[0, 5] = 7                                   # not an earlier node
dc.parent.copy_(torch.from_numpy(bad))
out, lse = dc.attn()
report("bad_parent_attn", bits=sv.check_device_errors(), finite=bool(torch.isfinite(out.float()).all()))
acc, path, tok, am = dc.accept()
report("bad_parent_accept", bits=sv.check_device_errors())
dc.parent.copy_(torch.from_numpy(case.parent))

ctx = dc.ctx.clone()
dc.ctx.fill_(int(case.ctx_lens.max()) + 3)      # above max_ctx: clamped
out, lse = dc.attn()
report("ctx_over_max", bits=sv.check_device_errors())
dc.ctx.copy_(ctx)

acc, path, tok, am = dc.accept()
acc_bad = torch.full_like(acc, cfg.n_nodes)    # accept length out of range
sv.kv_compact(dc.kv, dc.ctx, dc.max_ctx, path, acc_bad)
report("bad_accept_len", bits=sv.check_device_errors())

pcfg = workloads.small_variant(workloads.CONFIGS["C5"], ctx=40, ctx_hi=90, vocab=500)
pcase = workloads.make_case(pcfg, seed=6, capacity_pad=2)
pt = pcase.page_table.copy()
pt[1, 1] = pcase.k.shape[0] + 3                 # outside the pool
pdc = DeviceCase(pcase)
pdc.pt.copy_(torch.from_numpy(pt))
out, lse = pdc.attn()
report("bad_page_attn", bits=sv.check_device_errors(), finite=bool(torch.isfinite(out.float()).all()))
report("after_clear", bits=sv.check_device_errors())

# 4-bit head-dim-256 cache, paged, 48 packed rows: the eight-wave kernel
qcfg = workloads.Config("q4 paged", 2, 24, 4, 256, 8, "bf16", "q4", "f32", 500, 300, ctx_hi=340, paged=True,
                        q_std=0.5, kv_std=0.5)
qcase = workloads.make_case(qcfg, seed=7, capacity_pad=2)
qdc = DeviceCase(qcase)
out, lse = qdc.attn()
report("clean_q4", bits=sv.check_device_errors(), finite=bool(torch.isfinite(out.float()).all()))
qpt = qcase.page_table.copy()
qpt[1, 2] = qcase.k.shape[0] + 5                # outside the pool
qdc.pt.copy_(torch.from_numpy(qpt))
out, lse = qdc.attn()
report("bad_page_attn_q4", bits=sv.check_device_errors(), finite=bool(torch.isfinite(out.float()).all()))
'''


def test_debug_library_records_preconditions():
    env = dict(os.environ, SV_DEBUG="1")
    lib = os.path.join(ROOT, "draft_token_verification_sv_amd", "libsv_debug.so")
    assert os.path.exists(lib), "build it with draft_token_verification_sv_amd/build.py --debug"
    print("[debug lib] child process: bad parent, ctx, accept length, page", flush=True)
    r = subprocess.run([sys.executable, "-u", "-c", f"ROOT = {ROOT!r}\n" + CHILD], env=env, capture_output=True,
                       text=True, timeout=300)
    print(r.stdout[-4000:], r.stderr[-4000:], flush=True)
    assert r.returncode == 0
    steps = {d["step"]: d for d in (json.loads(l) for l in r.stdout.splitlines() if l.startswith("{"))}
    PARENT, PAGE, CTX, PATH = 1, 2, 4, 8
    assert steps["clean_start"]["bits"] == 0
    assert steps["clean_calls"]["bits"] == 0 and steps["clean_calls"]["finite"]
    assert steps["bad_parent_attn"]["bits"] == PARENT and steps["bad_parent_attn"]["finite"]
    assert steps["bad_parent_accept"]["bits"] == PARENT
    assert steps["ctx_over_max"]["bits"] == CTX
    assert steps["bad_accept_len"]["bits"] == PATH
    assert steps["bad_page_attn"]["bits"] == PAGE and steps["bad_page_attn"]["finite"]
    assert steps["after_clear"]["bits"] == 0
    assert steps["clean_q4"]["bits"] == 0 and steps["clean_q4"]["finite"]
    assert steps["bad_page_attn_q4"]["bits"] == PAGE and steps["bad_page_attn_q4"]["finite"]
