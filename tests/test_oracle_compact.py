"""Pins for the oracle's KV compaction (CPU only)."""
import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_compaction():
    with open(os.path.join(GOLDEN, "compact_example.json")) as f:
        c = json.load(f)
    cache = np.array(c["before"], dtype=np.float32)[None, None, None, :, None]  # [L,B,H,pos,D]
    path = np.array([c["path"] + [-1]])
    (out,), new_lens, moves = oracle.compact_cache([cache], ctx_lens=[c["ctx"]], path=path,
                                                   accept_len=[c["accept_len"]])
    np.testing.assert_array_equal(out[0, 0, 0, :, 0], c["after"])
    assert new_lens[0] == c["new_len"]


def test_compacted_decode_equals_masked_decode():
    """Decode attention over the compacted cache equals attention over the
    uncompacted cache restricted to the cache plus positions ctx + path."""
    rng = np.random.default_rng(0)
    for trial in range(20):
        ctx = int(rng.integers(0, 30))
        n = int(rng.integers(1, 12))
        D, H = 8, 2
        parent = np.array([-1] + [int(rng.integers(0, i)) for i in range(1, n)])
        # pick a random accepted node and its root path
        end = int(rng.integers(0, n))
        path = []
        j = end
        while j >= 0:
            path.append(j)
            j = parent[j] if j > 0 else -1
        path = path[::-1]
        a = len(path) - 1
        K = rng.standard_normal((1, 1, H, ctx + n + 3, D))
        V = rng.standard_normal((1, 1, H, ctx + n + 3, D))
        pth = np.full((1, n), -1)
        pth[0, :a + 1] = path
        (K2, V2), new_lens, _ = oracle.compact_cache([K, V], ctx_lens=[ctx], path=pth, accept_len=[a])
        q = rng.standard_normal((1, H, D))
        L = int(new_lens[0])
        out_c, _ = oracle.verify_attention_seq(q, K2[0, 0][:, :L], V2[0, 0][:, :L], L - 1, [-1], 0.5)
        rows = list(range(ctx)) + [ctx + p for p in path]
        out_m, _ = oracle.verify_attention_seq(q, K[0, 0][:, rows], V[0, 0][:, rows], len(rows) - 1, [-1], 0.5)
        np.testing.assert_allclose(out_c, out_m, rtol=1e-13, atol=1e-14)
        # rows past ctx + a untouched, rows before ctx untouched
        np.testing.assert_array_equal(K2[..., L:, :], K[..., L:, :])
        np.testing.assert_array_equal(K2[..., :ctx, :], K[..., :ctx, :])


def test_chain_compaction_moves_nothing_and_overlap_reads_first():
    rng = np.random.default_rng(1)
    K = rng.standard_normal((2, 1, 1, 20, 4))
    n = 6
    path = np.arange(n)[None]
    (K2,), nl, _ = oracle.compact_cache([K], ctx_lens=[10], path=path, accept_len=[n - 1])
    np.testing.assert_array_equal(K2, K)
    assert nl[0] == 10 + n
    # overlapping moves: path [0, 1, 3, 4] with a read-before-write hazard on 3 <- 4
    path = np.array([[0, 1, 3, 4, -1, -1]])
    (K3,), _, _ = oracle.compact_cache([K], ctx_lens=[10], path=path, accept_len=[3])
    np.testing.assert_array_equal(K3[:, 0, 0, 12], K[:, 0, 0, 13])
    np.testing.assert_array_equal(K3[:, 0, 0, 13], K[:, 0, 0, 14])


def test_paged_compaction_equals_contiguous():
    rng = np.random.default_rng(2)
    B, H, ps, D = 3, 2, 4, 3
    ctx = np.array([5, 9, 2])
    n = 5
    L = ctx + n
    cont = rng.standard_normal((1, B, H, 16, D))
    need = (L + ps - 1) // ps
    n_pages = int(need.sum()) + 3
    perm = rng.permutation(n_pages)
    pt = np.full((B, need.max()), -1)
    pages = rng.standard_normal((1, n_pages, H, ps, D))
    off = 0
    for b in range(B):
        pt[b, :need[b]] = perm[off:off + need[b]]
        off += need[b]
        for p in range(L[b]):
            pages[0, pt[b, p // ps], :, p % ps] = cont[0, b, :, p]
    path = np.array([[0, 2, 4, -1, -1], [0, 1, -1, -1, -1], [0, 3, -1, -1, -1]])
    acc = np.array([2, 1, 1])
    (c2,), nl1, _ = oracle.compact_cache([cont], ctx_lens=ctx, path=path, accept_len=acc)
    (p2,), nl2, _ = oracle.compact_cache([pages], ctx_lens=ctx, path=path, accept_len=acc,
                                         page_table=pt, page_size=ps)
    np.testing.assert_array_equal(nl1, nl2)
    for b in range(B):
        for p in range(L[b]):
            np.testing.assert_array_equal(p2[0, pt[b, p // ps], :, p % ps], c2[0, b, :, p])
