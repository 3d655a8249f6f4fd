"""Pins for the oracle's verify attention (CPU only).

Each test checks the oracle against something other than itself: a
hand-worked fixture, a one-line decode formula, torch's float64 SDPA, a
closed form (a tree row equals decode attention over the cache plus that
node's root path), an invariant (relabelling the tree), or brute force over
every small tree.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle.attention import logical_rows

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(rng, *shape):
    return rng.standard_normal(shape)


def _sdpa(q, k, v, scale, mask=None, is_causal=False, enable_gqa=False):
    """torch SDPA in float64 on CPU. q [H, Lq, D], k/v [Hkv, Lk, D]."""
    qt = torch.from_numpy(np.ascontiguousarray(q))[None]
    kt = torch.from_numpy(np.ascontiguousarray(k))[None]
    vt = torch.from_numpy(np.ascontiguousarray(v))[None]
    m = None if mask is None else torch.from_numpy(mask)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=m, is_causal=is_causal,
                                       scale=scale, enable_gqa=enable_gqa)
    return o[0].numpy()


def _random_parent(rng, n):
    p = np.empty(n, dtype=np.int32)
    p[0] = -1
    for i in range(1, n):
        p[i] = rng.integers(0, i)
    return p


def _path(parent, i):
    out = []
    while i >= 0:
        out.append(i)
        i = parent[i] if i > 0 else -1
    return out[::-1]


def test_golden_masks():
    with open(os.path.join(GOLDEN, "masks.json")) as f:
        data = json.load(f)
    for c in data["cases"]:
        got = oracle.verify_mask(c["parent"], c["ctx"]).astype(int)
        np.testing.assert_array_equal(got, np.array(c["mask"]), err_msg=c["name"])


def test_golden_tiny_attention():
    with open(os.path.join(GOLDEN, "attention_tiny.json")) as f:
        c = json.load(f)
    q = np.array(c["q"])[:, None, None]          # [N, Hq=1, D=1]
    K = np.array(c["k"])[None, :, None]          # [Hkv=1, L, 1]
    V = np.array(c["v"])[None, :, None]
    out, lse = oracle.verify_attention_seq(q, K, V, c["ctx"], c["parent"], c["scale"])
    np.testing.assert_allclose(out[:, 0, 0], c["out"], rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse[:, 0], c["lse"], rtol=0, atol=1e-14)


@pytest.mark.parametrize("ctx", [0, 1, 17, 300])
def test_single_row_is_decode_attention(ctx):
    """N = 1: a one-row chain is ordinary single-token decode attention."""
    rng = np.random.default_rng(ctx)
    Hq, Hkv, D = 6, 2, 32
    q = _rand(rng, 1, Hq, D)
    K = _rand(rng, Hkv, ctx + 1, D)
    V = _rand(rng, Hkv, ctx + 1, D)
    scale = 1 / math.sqrt(D)
    out, lse = oracle.verify_attention_seq(q, K, V, ctx, [-1], scale)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        s = scale * K[g] @ q[0, h]
        w = np.exp(s - s.max())
        np.testing.assert_allclose(out[0, h], w @ V[g] / w.sum(), rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(lse[0, h], np.log(np.exp(s).sum()), rtol=1e-12)
    # library routine: SDPA without a mask, GQA by repeat_interleave of KV heads
    ref = _sdpa(q.transpose(1, 0, 2), K, V, scale, enable_gqa=True)
    np.testing.assert_allclose(out.transpose(1, 0, 2), ref, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("ctx,n", [(0, 5), (3, 8), (100, 16), (257, 4)])
def test_chain_is_bottom_right_causal(ctx, n):
    """A chain-shaped tree equals causal attention over [cache, chain] with the
    mask aligned to the end of the key range."""
    rng = np.random.default_rng(1000 + ctx)
    Hq, Hkv, D = 4, 2, 16
    q = _rand(rng, n, Hq, D)
    K = _rand(rng, Hkv, ctx + n, D)
    V = _rand(rng, Hkv, ctx + n, D)
    scale = 0.3
    out, _ = oracle.verify_attention_seq(q, K, V, ctx, np.arange(-1, n - 1), scale)
    L = ctx + n
    bottom_right = np.tril(np.ones((n, L), dtype=bool), k=ctx)
    ref = _sdpa(q.transpose(1, 0, 2), K, V, scale, mask=bottom_right, enable_gqa=True)
    np.testing.assert_allclose(out.transpose(1, 0, 2), ref, rtol=1e-11, atol=1e-12)
    if ctx == 0:
        ref2 = _sdpa(q.transpose(1, 0, 2), K, V, scale, is_causal=True, enable_gqa=True)
        np.testing.assert_allclose(out.transpose(1, 0, 2), ref2, rtol=1e-11, atol=1e-12)


def test_top_left_causal_differs_when_ctx_positive():
    """The misaligned (top-left) causal mask is a different function once the
    draft block sits after a cache, which is why the oracle uses an explicit
    mask."""
    rng = np.random.default_rng(7)
    ctx, n, D = 5, 4, 8
    q = _rand(rng, n, 1, D)
    K = _rand(rng, 1, ctx + n, D)
    V = _rand(rng, 1, ctx + n, D)
    out, _ = oracle.verify_attention_seq(q, K, V, ctx, np.arange(-1, n - 1), 0.5)
    top_left = _sdpa(q.transpose(1, 0, 2), K, V, 0.5, is_causal=True)
    assert np.abs(out.transpose(1, 0, 2) - top_left).max() > 1e-3


@pytest.mark.parametrize("seed", range(6))
def test_tree_row_is_decode_over_root_path(seed):
    """Closed form: tree row i equals single-query attention over the cache rows
    followed by the rows of node i's root path (no mask)."""
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 24))
    ctx = int(rng.integers(0, 40))
    Hq, Hkv, D = 6, 3, 16
    parent = _random_parent(rng, n)
    q = _rand(rng, n, Hq, D)
    K = _rand(rng, Hkv, ctx + n, D)
    V = _rand(rng, Hkv, ctx + n, D)
    scale = 1 / 4
    out, lse = oracle.verify_attention_seq(q, K, V, ctx, parent, scale)
    for i in range(n):
        rows = list(range(ctx)) + [ctx + j for j in _path(parent, i)]
        ref = _sdpa(q[i][:, None, :], K[:, rows], V[:, rows], scale, enable_gqa=True)
        np.testing.assert_allclose(out[i], ref[:, 0, :], rtol=1e-11, atol=1e-12)
        for h in range(Hq):
            s = scale * K[h // 2][rows] @ q[i, h]
            np.testing.assert_allclose(lse[i, h], np.log(np.sum(np.exp(s))), rtol=1e-12)


@pytest.mark.parametrize("seed", range(4))
def test_relabelling_permutes_outputs(seed):
    """Renumbering the nodes by another topological order (and moving their KV
    rows accordingly) permutes the outputs the same way."""
    rng = np.random.default_rng(100 + seed)
    n, ctx, Hq, Hkv, D = 12, 9, 2, 1, 8
    parent = _random_parent(rng, n)
    q = _rand(rng, n, Hq, D)
    K = _rand(rng, Hkv, ctx + n, D)
    V = _rand(rng, Hkv, ctx + n, D)
    out, lse = oracle.verify_attention_seq(q, K, V, ctx, parent, 0.4)
    # random topological order: repeatedly pick a random node whose parent is placed
    order, placed = [0], {0}
    while len(order) < n:
        cand = [i for i in range(n) if i not in placed and parent[i] in placed]
        c = int(rng.choice(cand))
        order.append(c)
        placed.add(c)
    new_of_old = {old: new for new, old in enumerate(order)}
    parent2 = np.array([-1] + [new_of_old[parent[old]] for old in order[1:]])
    q2 = q[order]
    K2 = np.concatenate([K[:, :ctx], K[:, [ctx + o for o in order]]], axis=1)
    V2 = np.concatenate([V[:, :ctx], V[:, [ctx + o for o in order]]], axis=1)
    out2, lse2 = oracle.verify_attention_seq(q2, K2, V2, ctx, parent2, 0.4)
    np.testing.assert_allclose(out2, out[order], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse2, lse[order], rtol=1e-12, atol=1e-13)


def _all_parent_arrays(n):
    for choice in itertools.product(*[range(i) for i in range(1, n)]):
        yield np.array((-1,) + choice)


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6])
def test_bruteforce_all_small_trees(n):
    """Every parent array with N <= 6 ((N-1)! trees) at ctx in {0, 1, 7}."""
    rng = np.random.default_rng(n)
    D = 4
    for ctx in (0, 1, 7):
        q = _rand(rng, n, 1, D)
        K = _rand(rng, 1, ctx + n, D)
        V = _rand(rng, 1, ctx + n, D)
        for parent in _all_parent_arrays(n):
            out, _ = oracle.verify_attention_seq(q, K, V, ctx, parent, 0.7)
            for i in range(n):
                vis = list(range(ctx))
                j = i
                while j >= 0:          # collect ancestors-or-self by walking up
                    vis.append(ctx + j)
                    j = parent[j] if j > 0 else -1
                s = 0.7 * K[0][vis] @ q[i, 0]
                w = np.exp(s - s.max())
                np.testing.assert_allclose(out[i, 0], w @ V[0][vis] / w.sum(), rtol=1e-12, atol=1e-13)


def test_invalid_parents_rejected():
    with pytest.raises(ValueError):
        oracle.ancestor_matrix([-1, 1])
    with pytest.raises(ValueError):
        oracle.ancestor_matrix([0, 0])
    with pytest.raises(ValueError):
        oracle.ancestor_matrix([-1, 0, 3, 1])


def test_q4_golden_block():
    with open(os.path.join(GOLDEN, "q4_block.json")) as f:
        c = json.load(f)
    vals = oracle.q4_decode(np.array(c["codes"], dtype=np.uint8)[None],
                            np.array([c["scale_bits"]], dtype=np.uint16)[None])
    np.testing.assert_array_equal(vals[0], np.array(c["values"]))


def test_q4_all_codes_and_quantiser_error():
    """Every code decodes to d*(n-8); the write-time quantiser's round trip stays
    within half a quantisation step of the input."""
    import workloads
    d = np.float16(0.125)
    n = np.arange(32) % 16
    codes = (n[0::2] | (n[1::2] << 4)).astype(np.uint8)
    vals = oracle.q4_decode(codes[None], np.array([[d]]).astype(np.float16).view(np.uint16))
    np.testing.assert_array_equal(vals[0], 0.125 * (n - 8))
    rng = np.random.default_rng(3)
    x = rng.standard_normal((200, 256)).astype(np.float32)
    c, s = workloads.q4_encode(x)
    y = oracle.q4_decode(c, s)
    d_per = np.repeat(oracle.widen_fp16(s), 32, axis=-1)
    assert np.all(np.abs(y - x) <= d_per / 2 * (1 + 1e-3) + 1e-12)
    # a wrong nibble order or code offset breaks that bound
    swapped = ((c & 0x0F) << 4) | (c >> 4)
    assert np.abs(oracle.q4_decode(swapped, s) - x).max() > 0.5


def test_paged_rows_equal_contiguous_rows():
    """The page-table gather reads the same logical rows as contiguous storage."""
    rng = np.random.default_rng(5)
    B, H, ps, D = 3, 2, 16, 8
    L = np.array([20, 33, 47])
    cont = rng.standard_normal((B, H, 48, D)).astype(np.float32)
    need = (L + ps - 1) // ps
    n_pages = int(need.sum()) + 2
    perm = rng.permutation(n_pages)
    pt = np.full((B, need.max()), -1)
    pages = np.zeros((n_pages, H, ps, D), np.float32)
    off = 0
    for b in range(B):
        pt[b, :need[b]] = perm[off:off + need[b]]
        off += need[b]
        for p in range(L[b]):
            pages[pt[b, p // ps], :, p % ps] = cont[b, :, p]
    for b in range(B):
        for h in range(H):
            a = logical_rows(cont, None, b=b, head=h, length=int(L[b]), dtype="f32")
            g = logical_rows(pages, None, b=b, head=h, length=int(L[b]), dtype="f32",
                             page_table=pt, page_size=ps)
            np.testing.assert_array_equal(a, g)


@pytest.mark.parametrize("seed", range(5))
def test_window_equals_attention_over_the_last_rows(seed):
    """Sliding window: attention with window W equals the un-windowed
    definition run on a cache cut to its last W key rows (the rows are sliced,
    not masked), and each row equals SDPA over the window rows of its root
    path."""
    rng = np.random.default_rng(100 + seed)
    n = int(rng.integers(1, 12))
    ctx = int(rng.integers(0, 60))
    W = int(rng.integers(n, ctx + n + 5))
    Hq, Hkv, D = 4, 2, 16
    parent = _random_parent(rng, n)
    q = _rand(rng, n, Hq, D)
    K = _rand(rng, Hkv, ctx + n, D)
    V = _rand(rng, Hkv, ctx + n, D)
    out, lse = oracle.verify_attention_seq(q, K, V, ctx, parent, 0.3, window=W)
    lo = max(0, ctx + n - W)
    ref, ref_lse = oracle.verify_attention_seq(q, K[:, lo:], V[:, lo:], ctx - lo, parent, 0.3)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-13)
    for i in range(n):
        rows = list(range(lo, ctx)) + [ctx + j for j in _path(parent, i)]
        r = _sdpa(q[i][:, None, :], K[:, rows], V[:, rows], 0.3, enable_gqa=True)
        np.testing.assert_allclose(out[i], r[:, 0, :], rtol=1e-11, atol=1e-12)


def test_window_special_cases():
    rng = np.random.default_rng(9)
    n, ctx = 5, 30
    parent = _random_parent(rng, n)
    q = _rand(rng, n, 2, 8)
    K = _rand(rng, 1, ctx + n, 8)
    V = _rand(rng, 1, ctx + n, 8)
    full, _ = oracle.verify_attention_seq(q, K, V, ctx, parent, 0.5)
    for W in (ctx + n, ctx + n + 100):                  # a window over everything changes nothing
        w, _ = oracle.verify_attention_seq(q, K, V, ctx, parent, 0.5, window=W)
        np.testing.assert_array_equal(w, full)
    # W = N: the cache drops out, every row sees its root path only
    w, _ = oracle.verify_attention_seq(q, K, V, ctx, parent, 0.5, window=n)
    only, _ = oracle.verify_attention_seq(q, K[:, ctx:], V[:, ctx:], 0, parent, 0.5)
    np.testing.assert_allclose(w, only, rtol=1e-12, atol=1e-13)
    with pytest.raises(ValueError):
        oracle.verify_mask(parent, ctx, window=n - 1)
