"""GPU parity with page ids outside the pool.

A page id outside [0, capacity) reads as zero rows and is never written (the
paged-cache convention of the library, after xdnf.cn's 16-token pages,
section 2).  The device runs on the pool as given, with one page-table entry
of a used range pointing past the pool; the oracle runs on a copy of the
pool with one extra all-zero page appended, the same entry pointing at it.
Both must agree: attention on every kernel family that reads paged caches,
and compaction (standalone and fused with acceptance) whose moving source
row sits on such a page.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads
from sv_harness import DeviceCase, check_attention, q4_key_rounding, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import draft_token_verification_sv_amd as m
    return m


def _with_zero_page(case, b, page_idx):
    """(device case, oracle case): the device page table sends entry
    [b][page_idx] past the pool; the oracle's pool gains a zero page there."""
    P = case.k.shape[0]
    dev_pt = case.page_table.copy()
    dev_pt[b, page_idx] = P + 7
    ref_pt = case.page_table.copy()
    ref_pt[b, page_idx] = P

    def grow(a):
        return np.concatenate([a, np.zeros((1,) + a.shape[1:], dtype=a.dtype)], axis=0)
    ref = dataclasses.replace(case, k=grow(case.k), v=grow(case.v),
                              k_scale=None if case.k_scale is None else grow(case.k_scale),
                              v_scale=None if case.v_scale is None else grow(case.v_scale),
                              page_table=ref_pt, capacity=P + 1)
    dev = dataclasses.replace(case, page_table=dev_pt)
    return dev, ref


ATTN = [
    # (label, Hq, Hkv, D, N, q, kv, tree, ctx, tuning): one kernel family each
    ("pipelined bf16 D128", 16, 4, 128, 4, "bf16", "bf16", "chain", 300, None),
    ("cooperative q4 D256", 24, 4, 256, 16, "bf16", "q4", "chain", 700, None),
    ("pipelined q4 D256", 24, 4, 256, 16, "bf16", "q4", "chain", 700, {"attn_q4_kernel": "pipelined"}),
    ("eight-wave q4 D256", 24, 4, 256, 8, "bf16", "q4", "chain", 700, {"attn_q4_kernel": "wide"}),
    ("staged q4 D128", 16, 4, 128, 4, "bf16", "q4", "ddtree", 300, None),
    ("vector fp32 D64", 4, 2, 64, 3, "f32", "f32", "chain", 200, None),
]


@pytest.mark.parametrize("c", ATTN, ids=[a[0] for a in ATTN])
def test_attention_page_outside_pool(sv, c):
    label, Hq, Hkv, D, N, qd, kvd, tree, ctx, tuning = c
    say(f"[bad page attn] {label}")
    cfg = workloads.Config(label, 2, Hq, Hkv, D, N, qd, kvd, "f32", 50, ctx, ctx_hi=ctx + 40, tree=tree,
                           paged=True, q_std=0.5, kv_std=0.5,
                           draft_rule="tree" if tree == "ddtree" else "geometric")
    case = workloads.make_case(cfg, seed=91, capacity_pad=2, variant="peaked")
    dev_case, ref_case = _with_zero_page(case, 1, 3)              # positions 48..63 of sequence 1
    out, lse = DeviceCase(dev_case).attn(tuning=tuning)
    torch.cuda.synchronize()
    ref = oracle.verify_attention(ref_case)
    kernel = (tuning or {}).get("attn_q4_kernel", "cooperative")
    check_attention(ref_case, out, lse, ref=ref, key_rounding=q4_key_rounding(ref_case, kernel))
    # the zero page changed the answer (the check has power)
    plain = oracle.verify_attention(case)
    assert np.nanmax(np.abs(plain[0] - ref[0])) > 1e-3


def _compaction_case(kvd, D):
    """Batch of 2, 16-token pages; sequence 0 accepts a sibling branch whose
    first moving source (position 16) sits on its page 1."""
    cfg = workloads.Config("bad-page compaction", 2, 8, 2, D, 6, "bf16", kvd, "bf16", 300, 14, tree="ddtree",
                           paged=True, q_std=0.5, kv_std=0.5, draft_rule="tree")
    case = workloads.make_case(cfg, seed=92, capacity_pad=2)
    case.ctx_lens = np.array([14, 14], dtype=np.int32)
    case.parent[0] = np.array([-1, 0, 0, 2, 3, 1], dtype=np.int32)
    return case


@pytest.mark.parametrize("kvd,D", [("bf16", 128), ("q4", 256)])
@pytest.mark.parametrize("fused", [False, True])
def test_compaction_source_outside_pool(sv, kvd, D, fused):
    say(f"[bad page compact] {kvd} D{D} fused={fused}")
    case = _compaction_case(kvd, D)
    dev_case, ref_case = _with_zero_page(case, 0, 1)              # positions 16..31 of sequence 0
    # sequence 0 accepts nodes 2 and 3: path (0, 2, 3), rows 15 <- 16, 16 <- 17
    am = np.zeros((2, 6), dtype=np.int32)
    drafts = case.draft_ids.copy()
    drafts[0] = [0, 101, 102, 103, 104, 105]
    am[0, 0] = 102            # root's argmax = node 2's draft
    am[0, 2] = 103            # node 2's argmax = node 3's draft
    am[0, 3] = 7
    am[1, :] = 9              # sequence 1 accepts nothing
    V = case.cfg.vocab
    logits = np.full((2, 6, V), -3.0, dtype=np.float32)
    for b in range(2):
        for i in range(6):
            logits[b, i, am[b, i]] = 5.0
    case.logits = logits
    dev_case = dataclasses.replace(dev_case, logits=logits, draft_ids=drafts, parent=case.parent)
    ref_case = dataclasses.replace(ref_case, logits=logits, draft_ids=drafts, parent=case.parent)
    ref_case.cfg = dataclasses.replace(ref_case.cfg, logits_dtype="f32")
    dev_case.cfg = ref_case.cfg
    dc = DeviceCase(dev_case)
    r_am, r_acc, r_path, r_tok = oracle.greedy_accept(logits.astype(np.float64), drafts, case.parent)
    assert int(r_acc[0]) == 2 and list(r_path[0][:3]) == [0, 2, 3]
    if fused:
        acc, path, tok, _, new_lens = sv.greedy_accept_compact(dc.logits, dc.drafts, dc.parent, dc.kv, dc.ctx,
                                                               dc.max_ctx)
    else:
        acc, path, tok, _ = sv.greedy_accept(dc.logits, dc.drafts, dc.parent)
        new_lens = sv.kv_compact(dc.kv, dc.ctx, dc.max_ctx, path, acc)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(acc.cpu().numpy(), r_acc)
    arrs = [ref_case.k[None], ref_case.v[None]]
    if kvd == "q4":
        arrs += [ref_case.k_scale[None], ref_case.v_scale[None]]
    exp, r_new, _ = oracle.compact_cache(arrs, ctx_lens=case.ctx_lens, path=r_path, accept_len=r_acc,
                                         page_table=ref_case.page_table, page_size=16)
    P = case.k.shape[0]
    for e, got in zip(exp, dc.cache_arrays_host()):
        np.testing.assert_array_equal(got, e[0][:P])             # the pool; the zero page is the oracle's own
    np.testing.assert_array_equal(new_lens.cpu().numpy(), r_new)
    # row 15 (page 0, a real page) now holds the zero row read from page 1
    pg0 = int(case.page_table[0, 0])
    k_host = dc.cache_arrays_host()[0]
    assert not np.any(k_host[pg0, :, 15])
