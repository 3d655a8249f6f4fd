"""Pins of the oracle's stochastic verification (temperature sampling by the
Gumbel-max rule, noise given): hand-worked rows, the sampling distribution
against softmax(l / T), the greedy limit and the walk it reuses."""
import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "sample_rows.json")


def test_hand_worked_rows():
    for r in json.load(open(GOLDEN))["rows"]:
        assert oracle.sample_row(r["logits"], r["gumbel"], r["temperature"]) == r["sample"]


def test_samples_follow_softmax_of_scaled_logits():
    """Gumbel-max with fresh standard Gumbel noise draws token v with
    probability softmax(l / T)_v: frequencies over 40000 draws against the
    closed form, for two temperatures (a sign or scale slip in the key shows)."""
    rng = np.random.default_rng(11)
    logits = np.array([1.5, 0.0, -0.7, 2.2, 0.9, -3.0], dtype=np.float32)
    for T in (0.7, 2.0):
        n = 40000
        u = rng.random((n, logits.size))
        g = (-np.log(-np.log(u))).astype(np.float32)
        counts = np.bincount([oracle.sample_row(logits, g[k], T) for k in range(n)], minlength=logits.size)
        p = np.exp(logits.astype(np.float64) / T)
        p /= p.sum()
        expect = n * p
        chi2 = float(np.sum((counts - expect) ** 2 / expect))
        assert chi2 < 30.0, (T, chi2, counts, expect)     # 5 dof: P(chi2 > 30) ~ 1.5e-5


def test_low_temperature_is_greedy():
    rng = np.random.default_rng(12)
    B, N, V = 2, 6, 500
    lg = rng.standard_normal((B, N, V)).astype(np.float32) * 3
    g = (-np.log(-np.log(rng.random((B, N, V))))).astype(np.float32)
    parent = np.array([[-1, 0, 1, 2, 1, 4], [-1, 0, 0, 1, 3, 3]])
    am = np.array([[oracle.argmax_first(lg[b, i]) for i in range(N)] for b in range(B)])
    drafts = am[np.arange(B)[:, None], np.maximum(parent, 0)]
    ys, acc, path, tok = oracle.sample_accept(lg, g, 1e-4, drafts, parent)
    np.testing.assert_array_equal(ys, am)
    ref = oracle.greedy_accept(lg.astype(np.float64), drafts, parent)
    np.testing.assert_array_equal(acc, ref[1])
    np.testing.assert_array_equal(path, ref[2])
    np.testing.assert_array_equal(tok, ref[3])


def test_walk_follows_the_samples():
    """The sampled walk equals the pinned greedy walk run on the samples."""
    rng = np.random.default_rng(13)
    B, N, V = 3, 9, 50
    lg = rng.standard_normal((B, N, V)).astype(np.float32)
    g = (-np.log(-np.log(rng.random((B, N, V))))).astype(np.float32)
    parent = np.array([[-1] + [int(rng.integers(0, i)) for i in range(1, N)] for _ in range(B)])
    ys0 = np.array([[oracle.sample_row(lg[b, i], g[b, i], 1.3) for i in range(N)] for b in range(B)])
    drafts = np.where(rng.random((B, N)) < 0.7, ys0[np.arange(B)[:, None], np.maximum(parent, 0)],
                      rng.integers(0, V, (B, N)))
    ys, acc, path, tok = oracle.sample_accept(lg, g, 1.3, drafts, parent)
    np.testing.assert_array_equal(ys, ys0)
    for b in range(B):
        a, pth, tk = oracle.accept_bruteforce(ys[b], drafts[b], parent[b])
        assert a == acc[b]
        np.testing.assert_array_equal(pth, path[b])
        np.testing.assert_array_equal(tk, tok[b])


def test_topk_hand_worked_rows():
    g = json.load(open(GOLDEN))
    for r in g["topk_rows"]:
        assert oracle.sample_row_topk(r["logits"], r["gumbel"], r["temperature"], r["top_k"]) == r["sample"]


def test_topk_follows_renormalised_softmax():
    """Top-k sampling draws token v of the top-k set with probability
    softmax(l / T) restricted to that set, and never a token outside it."""
    rng = np.random.default_rng(14)
    logits = np.array([1.5, 0.0, -0.7, 2.2, 0.9, -3.0, 1.1], dtype=np.float32)
    k, T, n = 3, 1.3, 40000
    u = rng.random((n, logits.size))
    g = (-np.log(-np.log(u))).astype(np.float32)
    counts = np.bincount([oracle.sample_row_topk(logits, g[i], T, k) for i in range(n)], minlength=logits.size)
    top = np.argsort(-logits.astype(np.float64))[:k]
    assert counts[np.setdiff1d(np.arange(logits.size), top)].sum() == 0
    p = np.exp(logits[top].astype(np.float64) / T)
    p /= p.sum()
    chi2 = float(np.sum((counts[top] - n * p) ** 2 / (n * p)))
    assert chi2 < 25.0, (chi2, counts, p)                   # 2 dof: P(chi2 > 25) ~ 4e-6


def test_topk_limits():
    """k >= V is plain sampling; k = 1 without ties is the argmax; the threshold
    equals numpy's partition (a library selection) and -0 ties +0."""
    rng = np.random.default_rng(15)
    V = 300
    for _ in range(20):
        l = (rng.standard_normal(V) * 2).astype(np.float32)
        g = (-np.log(-np.log(rng.random(V)))).astype(np.float32)
        assert oracle.sample_row_topk(l, g, 0.9, V) == oracle.sample_row(l, g, 0.9)
        assert oracle.sample_row_topk(l, g, 0.9, 0) == oracle.sample_row(l, g, 0.9)
        assert oracle.sample_row_topk(l, g, 0.9, 1) == oracle.argmax_first(l)
        for k in (1, 7, 50, 299):
            assert oracle.topk_threshold(l, k) == np.partition(l.astype(np.float64), V - k)[V - k]
    z = np.array([-0.0, 0.0, -1.0], dtype=np.float32)
    assert oracle.topk_threshold(z, 2) == 0.0
    assert oracle.sample_row_topk(z, np.array([0.0, 0.0, 9.0], np.float32), 1.0, 2) == 0   # both zeros stay


def test_topk_walk_uses_topk_samples():
    rng = np.random.default_rng(16)
    B, N, V = 2, 7, 80
    lg = rng.standard_normal((B, N, V)).astype(np.float32)
    g = (-np.log(-np.log(rng.random((B, N, V))))).astype(np.float32)
    parent = np.array([[-1] + [int(rng.integers(0, i)) for i in range(1, N)] for _ in range(B)])
    ys0 = np.array([[oracle.sample_row_topk(lg[b, i], g[b, i], 0.8, 5) for i in range(N)] for b in range(B)])
    drafts = ys0[np.arange(B)[:, None], np.maximum(parent, 0)]
    drafts[0, 3] = (drafts[0, 3] + 1) % V
    ys, acc, path, tok = oracle.sample_accept(lg, g, 0.8, drafts, parent, top_k=5)
    np.testing.assert_array_equal(ys, ys0)
    for b in range(B):
        ra, rp, rt = oracle.accept_walk(ys0[b], drafts[b], parent[b])
        assert acc[b] == ra and np.array_equal(path[b], rp) and np.array_equal(tok[b], rt)
