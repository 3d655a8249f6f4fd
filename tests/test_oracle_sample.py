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
