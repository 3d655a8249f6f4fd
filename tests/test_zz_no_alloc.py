"""sv_verify_attn_noalloc against sv_verify_attn through the C ABI.

The allocation-free entry point runs the same plan and kernels as
sv_verify_attn with its split partials in the library's static per-GPU
buffer, so its results must equal sv_verify_attn's bit for bit: two calls in
a row (the second with a smaller input, over the buffer the first left
behind), plus the oracle's tolerance on both, and a plan that needs more than
the buffer rejected before anything runs.
"""
import ctypes

import numpy as np
import pytest
import torch

import workloads
from sv_harness import DeviceCase, Guarded, check_attention, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import draft_token_verification_sv_amd as m
    return m


def _noalloc(sv, dc, window=0):
    B, N, Hq = dc.q.shape[:3]
    out = Guarded(tuple(dc.q.shape), dc.q.dtype, dc.q.device)
    lse = Guarded((B, N, Hq), torch.float32, dc.q.device)
    d = dc.kv.desc()
    rc = sv.lib.sv_verify_attn_noalloc(ctypes.byref(d), B, N, Hq, dc.ctx.data_ptr(), dc.max_ctx, dc.q.data_ptr(),
                                       sv.SV_BF16 if dc.q.dtype == torch.bfloat16 else sv.SV_F32,
                                       dc.parent.data_ptr(), ctypes.c_float(0.0), window, out.t.data_ptr(),
                                       lse.t.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert rc == 0, sv.lib.sv_error_string(rc)
    out.check("out", "noalloc")
    lse.check("lse", "noalloc")
    return out.t, lse.t


CALLS = [
    # (label, config, make_case kwargs, window): the first large, the second smaller
    ("4-bit block of 16, 6000 keys", workloads.small_variant(workloads.CONFIGS["C4"], ctx=6000), {}, 0),
    ("tree of 22, 700 keys, peaked", workloads.small_variant(workloads.CONFIGS["C3"], ctx=700),
     {"variant": "peaked"}, 0),
]


def test_noalloc_matches_workspace_entry_point(sv):
    for label, cfg, kw, window in CALLS:
        say(f"[noalloc] {label}")
        case = workloads.make_case(cfg, seed=19, **kw)
        dc = DeviceCase(case)
        o_ref, l_ref = dc.attn(window=window)
        o, l = _noalloc(sv, dc, window)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(l, l_ref), label
        check_attention(case, o, l)


def test_noalloc_batch_then_single(sv):
    """A paged batch (dynamic schedule, per-sequence table in the buffer),
    then a single short sequence."""
    for label, cfg in [("paged batch of 8", workloads.small_variant(workloads.CONFIGS["C5"], ctx=200, ctx_hi=3000)),
                       ("one chain of 8, 300 keys", workloads.small_variant(workloads.CONFIGS["C2"], ctx=300))]:
        say(f"[noalloc] {label}")
        case = workloads.make_case(cfg, seed=23)
        dc = DeviceCase(case)
        o_ref, l_ref = dc.attn()
        o, l = _noalloc(sv, dc)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(l, l_ref), label
        check_attention(case, o, l)


def test_noalloc_rejects_plans_beyond_the_buffer(sv):
    """A plan whose partials exceed the static buffer returns SV_EWORKSPACE
    before anything is launched (outputs untouched)."""
    cfg = workloads.Config("big batch", 64, 32, 8, 128, 16, "bf16", "bf16", "f32", 50, 30000, paged=True)
    d = sv._KvDesc()
    d.dtype, d.n_kv_heads, d.head_dim, d.page_size = sv.SV_BF16, 8, 128, 16
    d.capacity, d.max_pages_per_seq = 200000, (30000 + 16 + 15) // 16
    d.k, d.v, d.page_table = 1 << 40, (1 << 40) + (1 << 30), 1 << 41
    need = sv.lib.sv_verify_attn_workspace_size(ctypes.byref(d), cfg.batch, cfg.n_nodes, cfg.n_q_heads, 30000)
    assert need > sv.NOALLOC_SCRATCH_BYTES
    P = ctypes.c_void_p(1 << 40)
    rc = sv.lib.sv_verify_attn_noalloc(ctypes.byref(d), cfg.batch, cfg.n_nodes, cfg.n_q_heads, P, 30000, P,
                                       sv.SV_BF16, P, ctypes.c_float(0.0), 0, P, None, None)
    assert rc == -3
