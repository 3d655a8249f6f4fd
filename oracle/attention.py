"""Masked GQA attention of the verify rows (oracle side, float64).

Definition (per sequence b, query head h, verify row i):

* rows ``j`` of the key range run over ``[0, ctx + N)``: the ``ctx`` cached
  tokens, then the N verify rows in node order;
* ``visible(i, j) = j < ctx  or  (j - ctx)`` is node i or one of its
  ancestors in the token tree (``parent[0] = -1`` is the root, the last
  committed token).  For a chain this is causal attention whose mask is
  aligned to the end of the key range: row i sees ``ctx + 0 .. ctx + i``
  (the explicit upper-triangular ``-inf`` mask of section 5.3 of the xdnf.cn
  Qwen3.8-27B speculative-decoding notes, extended by the cache);
* query head h reads KV head ``h // (Hq / Hkv)``;
* ``s_ij = scale * q_i . k_j``; ``out_i = sum_j softmax_visible(s_i)_j v_j``;
  ``lse_i = log sum_{visible j} exp(s_ij)``.

DDTree verification (the single-RTX-3090 DFlash note, sections "From
autoregressive to DDTree" and "Key breakthroughs") runs exactly this for the
budget+1 rows of the tree: each node attends to the cache and its own root
path.

Sliding window (same note, the addendum on 60K context: flash attention over
only the most recent 2,048 KV positions instead of the whole context): with a
window W >= N the key range shrinks to its last W rows, ``j >= ctx + N - W``,
for every verify row of the block alike (the draft rows always stay inside).
"""
import numpy as np

from .formats import widen, q4_decode


def ancestor_matrix(parent) -> np.ndarray:
    """``A[i, j]`` is True iff node j is node i or an ancestor of node i."""
    parent = np.asarray(parent, dtype=np.int64)
    n = len(parent)
    if n == 0:
        return np.zeros((0, 0), dtype=bool)
    if parent[0] != -1:
        raise ValueError("parent[0] must be -1 (the root)")
    for i in range(1, n):
        if not (0 <= parent[i] < i):
            raise ValueError(f"parent[{i}] = {parent[i]} is not an earlier node")
    A = np.zeros((n, n), dtype=bool)
    for i in range(n):
        j = i
        while j >= 0:
            A[i, j] = True
            j = parent[j]
    return A


def verify_mask(parent, ctx: int, window: int = 0) -> np.ndarray:
    """Explicit boolean mask ``[N, ctx + N]`` of the verify rows (``window`` > 0:
    only the last ``window`` key rows)."""
    A = ancestor_matrix(parent)
    n = A.shape[0]
    M = np.zeros((n, ctx + n), dtype=bool)
    M[:, :ctx] = True
    M[:, ctx:] = A
    if window > 0:
        if window < n:
            raise ValueError("the window must hold the N verify rows")
        M[:, :max(0, ctx + n - window)] = False
    return M


def verify_attention_seq(q, K, V, ctx: int, parent, scale: float, heads=None, window: int = 0):
    """One sequence.

    ``q``: float64 ``[N, Hq, D]``; ``K``, ``V``: float64 ``[Hkv, ctx + N, D]``
    (the logical rows); returns ``out [N, Hq, D]`` and ``lse [N, Hq]``
    (natural log).  ``heads``: optional subset of query heads to compute (the
    other entries are left NaN).
    """
    q = np.asarray(q, dtype=np.float64)
    n, hq, d = q.shape
    hkv = K.shape[0]
    group = hq // hkv
    mask = verify_mask(parent, ctx, window)
    out = np.full((n, hq, d), np.nan)
    lse = np.full((n, hq), np.nan)
    for h in (range(hq) if heads is None else heads):
        g = h // group
        s = scale * (q[:, h, :] @ K[g].T)            # [N, L]
        s = np.where(mask, s, -np.inf)
        m = s.max(axis=1, keepdims=True)
        e = np.where(mask, np.exp(s - m), 0.0)
        l = e.sum(axis=1)
        out[:, h, :] = (e @ V[g]) / l[:, None]
        lse[:, h] = m[:, 0] + np.log(l)
    return out, lse


def logical_rows(store, scale_store, *, b: int, head: int, length: int, dtype: str,
                 page_table=None, page_size: int = 0) -> np.ndarray:
    """Rows ``0 .. length-1`` of one (sequence, KV head) as float64 ``[length, D]``.

    Contiguous storage is ``[seq][head][pos][...]``; paged storage is
    ``[page][head][slot][...]`` with ``page_table[b][pos // page_size]`` naming
    the page of logical position ``pos``.
    """
    if page_table is None:
        raw = store[b, head, :length]
        sc = None if scale_store is None else scale_store[b, head, :length]
    else:
        pos = np.arange(length)
        pages = np.asarray(page_table)[b, pos // page_size]
        if np.any(pages < 0):
            raise ValueError("page table entry missing for a used position")
        raw = store[pages, head, pos % page_size]
        sc = None if scale_store is None else scale_store[pages, head, pos % page_size]
    if dtype == "q4":
        return q4_decode(raw, sc)
    return widen(raw, dtype)


def verify_attention(case, *, scale=None, heads=None, batch=None, window=0):
    """Whole-batch attention for a case object (``workloads.Case`` shape).

    Returns ``out [B, N, Hq, D]`` and ``lse [B, N, Hq]``.  ``heads`` /
    ``batch`` restrict the work to a subset (the rest stays NaN).
    """
    cfg = case.cfg
    B, N, Hq, Hkv, D = cfg.batch, cfg.n_nodes, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim
    group = Hq // Hkv
    if scale is None or scale <= 0:
        scale = 1.0 / np.sqrt(D)
    out = np.full((B, N, Hq, D), np.nan)
    lse = np.full((B, N, Hq), np.nan)
    pt = case.page_table if cfg.paged else None
    layer_k = case.k if case.kv_layers == 1 else case.k[0]
    layer_v = case.v if case.kv_layers == 1 else case.v[0]
    layer_ks = None if case.k_scale is None else (case.k_scale if case.kv_layers == 1 else case.k_scale[0])
    layer_vs = None if case.v_scale is None else (case.v_scale if case.kv_layers == 1 else case.v_scale[0])
    for b in (range(B) if batch is None else batch):
        ctx = int(case.ctx_lens[b])
        L = ctx + N
        qb = widen(case.q[b], cfg.q_dtype)
        for g in range(Hkv):
            hs = [h for h in range(g * group, (g + 1) * group) if heads is None or h in heads]
            if not hs:
                continue
            K = logical_rows(layer_k, layer_ks, b=b, head=g, length=L, dtype=cfg.kv_dtype,
                             page_table=pt, page_size=cfg.page_size)
            V = logical_rows(layer_v, layer_vs, b=b, head=g, length=L, dtype=cfg.kv_dtype,
                             page_table=pt, page_size=cfg.page_size)
            # run the single-sequence definition on this KV head only
            qg = qb[:, g * group:(g + 1) * group, :]
            o, ls = verify_attention_seq(qg, K[None], V[None], ctx, case.parent[b], scale,
                                         heads=[h - g * group for h in hs], window=window)
            for h in hs:
                out[b, :, h] = o[:, h - g * group]
                lse[b, :, h] = ls[:, h - g * group]
    return out, lse
