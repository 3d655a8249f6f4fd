"""Pins for the oracle's case-level attention wrapper ``oracle.verify_attention``.

Every attention parity test and ``smoke()`` use the wrapper as their checker,
so it is pinned here on its own: for each query head the expected output is
rebuilt straight from the raw arrays of a ``workloads.Case`` with code written
in this file only — the storage read element by element (contiguous
``[seq][head][pos]``, paged ``[page][head][slot]`` through the page table,
layer 0 of a multi-layer cache), bf16 widened by torch's own conversion, the
4-bit codes and fp16 scales decoded here with bit operations, the tree mask
from a parent walk, and the attention itself by torch's float64
``scaled_dot_product_attention`` with that explicit mask.

Sources: masked GQA verify attention (the single-RTX-3090 DFlash note, "From
autoregressive to DDTree"; the draft block's mask aligned to the end of the
keys, xdnf.cn notes section 5.3); 24 query / 4 KV heads of dim 256 ("Why we
ran this test"); 16-token pages (xdnf.cn section 2); the 4-bit cache ("128K
context in 24 GB"); the sliding window (the 60K-context addendum).  Query head
h reads KV head h // (Hq / Hkv).

Each case also checks that the comparison has power: the same reference built
with query head h on KV head h % Hkv, or on layer 1 of the cache, or with the
tree mask replaced by a causal one, must disagree with the oracle.
"""
import dataclasses

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
import workloads


# ----------------------------------------------------------------------------
# independent reading of the raw storage
# ----------------------------------------------------------------------------

def _bf16_to_f64(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16)).view(torch.bfloat16)
    return t.to(torch.float64).numpy()


def _raw_to_f64(raw, dtype):
    if dtype == "f32":
        return np.asarray(raw, dtype=np.float32).astype(np.float64)
    assert dtype == "bf16"
    return _bf16_to_f64(raw)


def _decode_q4_row(codes, scales):
    """One 4-bit row: byte t holds value 2t (bits 0-3) and 2t+1 (bits 4-7);
    value i is scale[i // 32] * (code - 8), scales IEEE half."""
    d = codes.shape[-1] * 2
    out = np.empty(d, dtype=np.float64)
    sc = np.asarray(scales, dtype=np.uint16).view(np.float16).astype(np.float64)
    for t in range(codes.shape[-1]):
        byte = int(codes[t])
        out[2 * t] = sc[(2 * t) // 32] * ((byte & 15) - 8)
        out[2 * t + 1] = sc[(2 * t + 1) // 32] * ((byte >> 4) - 8)
    return out


def _storage_index(case, b, kvh, pos):
    cfg = case.cfg
    if cfg.paged:
        page = int(case.page_table[b, pos // cfg.page_size])
        return (page, kvh, pos % cfg.page_size)
    return (b, kvh, pos)


def _rows(case, b, kvh, length, which, layer=0):
    """Logical rows 0..length-1 of (sequence b, KV head kvh), float64."""
    cfg = case.cfg
    store = case.k if which == "k" else case.v
    sstore = case.k_scale if which == "k" else case.v_scale
    if case.kv_layers > 1:
        store = store[layer]
        sstore = None if sstore is None else sstore[layer]
    out = np.empty((length, cfg.head_dim))
    for pos in range(length):
        idx = _storage_index(case, b, kvh, pos)
        if cfg.kv_dtype == "q4":
            out[pos] = _decode_q4_row(store[idx], sstore[idx])
        else:
            out[pos] = _raw_to_f64(store[idx], cfg.kv_dtype)
    return out


def _tree_mask(parent, ctx, window, causal=False):
    n = len(parent)
    m = np.zeros((n, ctx + n), dtype=bool)
    m[:, :ctx] = True
    for i in range(n):
        if causal:
            m[i, ctx:ctx + i + 1] = True
            continue
        j = i
        while j >= 0:
            m[i, ctx + j] = True
            j = int(parent[j]) if j > 0 else -1
    if window:
        m[:, :max(0, ctx + n - window)] = False
    return m


def _reference(case, *, heads=None, batch=None, window=0, kv_of=None, layer=0, causal=False):
    """Per query head: fp64 SDPA with an explicit mask over the raw rows."""
    cfg = case.cfg
    B, N, Hq, Hkv, D = cfg.batch, cfg.n_nodes, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    G = Hq // Hkv
    kv_of = kv_of or (lambda h: h // G)
    out = np.full((B, N, Hq, D), np.nan)
    lse = np.full((B, N, Hq), np.nan)
    scale = 1.0 / np.sqrt(D)
    for b in (range(B) if batch is None else batch):
        ctx = int(case.ctx_lens[b])
        L = ctx + N
        mask = _tree_mask(case.parent[b], ctx, window, causal)
        qb = _raw_to_f64(case.q[b], cfg.q_dtype)                     # [N, Hq, D]
        cache = {}
        for h in (range(Hq) if heads is None else heads):
            g = kv_of(h)
            if g not in cache:
                cache[g] = (_rows(case, b, g, L, "k", layer), _rows(case, b, g, L, "v", layer))
            K, V = cache[g]
            qt = torch.from_numpy(np.ascontiguousarray(qb[:, h, :]))[None]
            kt = torch.from_numpy(K)[None]
            vt = torch.from_numpy(V)[None]
            o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(mask), scale=scale)
            out[b, :, h] = o[0].numpy()
            s = scale * (qb[:, h, :] @ K.T)
            s = np.where(mask, s, -np.inf)
            mx = s.max(axis=1)
            lse[b, :, h] = mx + np.log(np.exp(s - mx[:, None]).sum(axis=1))
    return out, lse


# ----------------------------------------------------------------------------
# cases: small shapes of every storage form
# ----------------------------------------------------------------------------

def _cfg(base, **kw):
    return dataclasses.replace(workloads.CONFIGS[base], **kw)


CASES = {
    # 24/4 heads (G = 6), bf16, contiguous, DDTree of 9 nodes
    "bf16_tree_g6": dict(cfg=_cfg("C3", head_dim=64, n_nodes=9, ctx=37, vocab=50), seed=11),
    # 32/8 heads would be slow: 4/2 heads (G = 2), 3 paged sequences of ragged length
    "bf16_paged_g2": dict(cfg=_cfg("C5", n_q_heads=4, n_kv_heads=2, head_dim=64, ctx=20, ctx_hi=70, batch=3,
                                   vocab=50), seed=12),
    # 4-bit cache, one KV head per query head (G = 1), block of 5
    "q4_g1": dict(cfg=_cfg("C4", n_q_heads=3, n_kv_heads=3, head_dim=64, n_nodes=5, ctx=41, vocab=50), seed=13),
    # 4-bit paged cache, G = 2, tree
    "q4_paged_tree": dict(cfg=_cfg("C5", n_q_heads=4, n_kv_heads=2, head_dim=64, kv_dtype="q4", tree="ddtree",
                                   draft_rule="tree", n_nodes=12, ctx=9, ctx_hi=40, batch=2, vocab=50), seed=14),
    # fp32 queries and cache, G = 2
    "f32_g2": dict(cfg=_cfg("C1", n_q_heads=4, n_kv_heads=2, ctx=30), seed=15),
    # two cache layers: attention reads layer 0
    "bf16_two_layers": dict(cfg=_cfg("C2", n_q_heads=6, n_kv_heads=2, head_dim=64, n_nodes=6, ctx=25, vocab=50),
                            seed=16, n_layers=2),
    # 4-bit, two layers (scales follow their layer)
    "q4_two_layers": dict(cfg=_cfg("C4", n_q_heads=4, n_kv_heads=2, head_dim=64, n_nodes=4, ctx=19, vocab=50),
                          seed=17, n_layers=2),
}


def _case(name, variant="peaked"):
    c = CASES[name]
    return workloads.make_case(c["cfg"], seed=c["seed"], variant=variant, n_layers=c.get("n_layers", 1),
                               capacity_pad=3)


def _close(a, b, tol=1e-12):
    both_nan = np.isnan(a) & np.isnan(b)
    assert np.array_equal(np.isnan(a), np.isnan(b)), "NaN patterns differ"
    d = np.abs(np.where(both_nan, 0.0, a - b))
    return float(d.max()) if d.size else 0.0


def _far(a, b):
    ok = ~(np.isnan(a) | np.isnan(b))
    return float(np.abs(a[ok] - b[ok]).max())


@pytest.mark.parametrize("name", sorted(CASES))
def test_wrapper_matches_per_head_sdpa(name):
    case = _case(name)
    out, lse = oracle.verify_attention(case)
    ref, rlse = _reference(case)
    assert _close(out, ref) < 1e-12
    assert _close(lse, rlse) < 1e-12
    cfg = case.cfg
    Hq, Hkv = cfg.n_q_heads, cfg.n_kv_heads
    G = Hq // Hkv
    # power: the wrong head mapping (where it differs), the other layer and a
    # causal mask in place of the tree must all be seen
    if any(h % Hkv != h // G for h in range(Hq)):
        bad, _ = _reference(case, kv_of=lambda h: h % Hkv)
        assert _far(out, bad) > 1e-3
    if case.kv_layers > 1:
        bad, _ = _reference(case, layer=1)
        assert _far(out, bad) > 1e-3
    causal = _cfg_is_tree(case)
    if causal:
        bad, _ = _reference(case, causal=True)
        assert _far(out, bad) > 1e-3


def _cfg_is_tree(case):
    p = case.parent
    return any(int(p[b, i]) != i - 1 for b in range(p.shape[0]) for i in range(1, p.shape[1]))


@pytest.mark.parametrize("name", ["bf16_tree_g6", "bf16_paged_g2", "q4_paged_tree"])
def test_wrapper_head_and_batch_subsets(name):
    """heads= / batch= compute only the asked entries; the rest stay NaN."""
    case = _case(name)
    cfg = case.cfg
    heads = [0, cfg.n_q_heads - 1] if cfg.n_q_heads > 2 else [1]
    batch = [cfg.batch - 1]
    out, lse = oracle.verify_attention(case, heads=heads, batch=batch)
    ref, rlse = _reference(case, heads=heads, batch=batch)
    assert _close(out, ref) < 1e-12 and _close(lse, rlse) < 1e-12
    assert np.isnan(out[:, :, [h for h in range(cfg.n_q_heads) if h not in heads]]).all()
    if cfg.batch > 1:
        assert np.isnan(out[:cfg.batch - 1]).all()


@pytest.mark.parametrize("name,window", [("bf16_tree_g6", 20), ("q4_paged_tree", 16), ("bf16_paged_g2", 9)])
def test_wrapper_window(name, window):
    case = _case(name)
    out, lse = oracle.verify_attention(case, window=window)
    ref, rlse = _reference(case, window=window)
    assert _close(out, ref) < 1e-12 and _close(lse, rlse) < 1e-12
    full, _ = oracle.verify_attention(case)
    assert _far(out, full) > 1e-6            # the window cut something off


def test_wrapper_plain_variant():
    """The flat (non-peaked) inputs the full-size workloads use."""
    case = _case("bf16_tree_g6", variant="")
    out, lse = oracle.verify_attention(case)
    ref, rlse = _reference(case)
    assert _close(out, ref) < 1e-12 and _close(lse, rlse) < 1e-12
