"""Greedy acceptance (oracle side).

Greedy verification, as the single-RTX-3090 DFlash note runs it (section
"Architecture": greedy verify only; section "Next steps": sampling is not yet
supported), accepts a draft token exactly when it equals the target model's
argmax at the draft's parent.  Over a token tree the step keeps the longest
root path whose drafts are all accepted, then appends one bonus token: the
target's argmax at the last node of that path.  The note's DDTree verifier
reads budget+1 logits rows for this (section "Key breakthroughs", the
verify-logits buffer fix).

Conventions the pages leave open, read here as:

* ties in a row's maximum go to the lowest token index;
* among equally deep accepted nodes the one with the smallest node index
  wins (the generators keep sibling tokens distinct, so with real trees the
  accepted path is unique);
* ``a`` (the accept length returned) counts accepted drafts, so ``a + 1``
  tokens are committed; node 0's draft id is the already committed token and
  is ignored.
"""
import numpy as np


def argmax_first(row) -> int:
    """Lowest index holding the maximum of a 1-D row (compared exactly)."""
    row = np.asarray(row, dtype=np.float64)
    m = row.max()
    return int(np.flatnonzero(row == m)[0])


def _depths(parent):
    n = len(parent)
    depth = [0] * n
    for i in range(1, n):
        depth[i] = depth[parent[i]] + 1
    return depth


def _result(best, am, draft, parent, n):
    path = []
    j = best
    while j >= 0:
        path.append(j)
        j = int(parent[j]) if j > 0 else -1
    path.reverse()
    a = len(path) - 1
    tokens = [int(draft[path[j]]) for j in range(1, a + 1)] + [int(am[path[a]])]
    path_out = np.full(n, -1, dtype=np.int32)
    tok_out = np.full(n, -1, dtype=np.int32)
    path_out[:a + 1] = path
    tok_out[:a + 1] = tokens
    return a, path_out, tok_out


def accept_walk(am, draft, parent):
    """Forward walk in node order: node i is accepted iff its parent is and
    ``draft[i] == am[parent[i]]``.  Returns ``(a, path, tokens)`` with ``path``
    and ``tokens`` padded to N with -1."""
    parent = [int(p) for p in parent]
    n = len(parent)
    acc = [False] * n
    acc[0] = True
    for i in range(1, n):
        p = parent[i]
        acc[i] = acc[p] and int(draft[i]) == int(am[p])
    depth = _depths(parent)
    best = 0
    for i in range(1, n):
        if acc[i] and depth[i] > depth[best]:
            best = i
    return _result(best, am, draft, parent, n)


def accept_bruteforce(am, draft, parent):
    """Independent check of ``accept_walk``: enumerate every root-to-node path,
    keep those whose every edge is accepted, take the longest (ties: the
    smallest end node)."""
    parent = [int(p) for p in parent]
    n = len(parent)
    best, best_len = 0, 0
    for end in range(n):
        chain = []
        j = end
        while j >= 0:
            chain.append(j)
            j = parent[j] if j > 0 else -1
        chain.reverse()
        ok = all(int(draft[c]) == int(am[p]) for p, c in zip(chain[:-1], chain[1:]))
        if ok and len(chain) - 1 > best_len:
            best, best_len = end, len(chain) - 1
    return _result(best, am, draft, parent, n)


def greedy_accept(logits64, draft_ids, parent):
    """Whole batch.  ``logits64``: float64 ``[B, N, V]`` (exactly widened).

    Returns ``am [B, N]``, ``accept_len [B]``, ``path [B, N]``, ``tokens [B, N]``.
    """
    B, N, _ = logits64.shape
    am = np.empty((B, N), dtype=np.int32)
    acc = np.empty(B, dtype=np.int32)
    path = np.empty((B, N), dtype=np.int32)
    tok = np.empty((B, N), dtype=np.int32)
    for b in range(B):
        for i in range(N):
            am[b, i] = argmax_first(logits64[b, i])
        acc[b], path[b], tok[b] = accept_walk(am[b], draft_ids[b], parent[b])
    return am, acc, path, tok


# ----------------------------------------------------------------------------
# stochastic verification (temperature sampling)
# ----------------------------------------------------------------------------
#
# The single-RTX-3090 DFlash note plans temperature / top-k sampling in the
# verify path (section "Next steps": only greedy decoding is wired in).  With
# a deterministic drafter the lossless form of it samples the target at every
# node and accepts a draft exactly when it equals the parent's sample:
# committed tokens are then distributed as autoregressive sampling from the
# target.  A sample of softmax(l / T) is drawn with the Gumbel-max rule,
# y = argmax_v (l_v / T + g_v) with g_v independent standard Gumbel noise; the
# noise is an input (drawn by the caller), and the key is formed in fp32 --
# the division, then the addition, each rounded to nearest -- so the argmax
# is decided identically on every implementation.  Ties go to the lowest
# index, as for the greedy argmax.


def sample_row(logits32, gumbel32, temperature) -> int:
    """Lowest index of the maximum fp32 key l / T + g of one row (numpy's
    float32 division and addition round each result to nearest)."""
    l32 = np.asarray(logits32, dtype=np.float32)
    g32 = np.asarray(gumbel32, dtype=np.float32)
    keys = (l32 / np.float32(temperature)).astype(np.float32) + g32
    assert keys.dtype == np.float32
    return int(np.argmax(keys))            # first occurrence of the maximum


def topk_threshold(logits32, top_k):
    """The k-th largest value of a row (values compared in fp32, so -0 ties
    +0); every token whose logit is >= it stays in the top-k set, ties at the
    k-th value included."""
    l32 = np.asarray(logits32, dtype=np.float32)
    return np.sort(l32.astype(np.float64))[::-1][top_k - 1]


def sample_row_topk(logits32, gumbel32, temperature, top_k) -> int:
    """Top-k sampling at temperature T: the Gumbel-max sample over the tokens
    whose logit is at least the row's k-th largest (renormalised softmax of
    l / T over that set; top_k <= 0 or >= V keeps every token)."""
    l32 = np.asarray(logits32, dtype=np.float32)
    if top_k <= 0 or top_k >= l32.size:
        return sample_row(l32, gumbel32, temperature)
    keep = l32.astype(np.float64) >= topk_threshold(l32, top_k)
    keys = (l32 / np.float32(temperature)).astype(np.float32) + np.asarray(gumbel32, dtype=np.float32)
    keys = np.where(keep, keys, np.float32(-np.inf))
    return int(np.argmax(keys))


def sample_accept(logits32, gumbel32, temperature, draft_ids, parent, top_k=0):
    """Whole batch.  ``logits32``: float32 ``[B, N, V]`` (exact widening of the
    stored logits); ``gumbel32``: float32 ``[B, N, V]``; ``top_k`` > 0
    restricts each row to its top-k tokens.  Returns ``sampled [B, N]``,
    ``accept_len [B]``, ``path [B, N]``, ``tokens [B, N]`` -- the greedy walk
    with every row's argmax replaced by its sample."""
    B, N, _ = logits32.shape
    ys = np.empty((B, N), dtype=np.int32)
    acc = np.empty(B, dtype=np.int32)
    path = np.empty((B, N), dtype=np.int32)
    tok = np.empty((B, N), dtype=np.int32)
    for b in range(B):
        for i in range(N):
            ys[b, i] = sample_row_topk(logits32[b, i], gumbel32[b, i], temperature, top_k)
        acc[b], path[b], tok[b] = accept_walk(ys[b], draft_ids[b], parent[b])
    return ys, acc, path, tok
