"""Pins for the oracle's argmax and greedy acceptance walk (CPU only)."""
import itertools
import json
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _scalar_argmax(row):
    best = 0
    for i in range(1, len(row)):
        if row[i] > row[best]:
            best = i
    return best


def test_argmax_matches_scalar_loop_and_numpy():
    rng = np.random.default_rng(0)
    for trial in range(50):
        n = int(rng.integers(1, 700))
        # few distinct values -> many ties
        row = rng.integers(-3, 4, size=n).astype(np.float64)
        assert oracle.argmax_first(row) == _scalar_argmax(row) == int(np.argmax(row))


def test_argmax_ties_lowest_index_bf16():
    """Planted ties across positions that a GPU reduction splits (lanes, waves,
    workgroups) resolve to the lowest index; bf16 rows tie often."""
    rng = np.random.default_rng(1)
    V = 151936
    row = workloads.bf16_bits(rng.standard_normal(V).astype(np.float32) * np.float32(np.sqrt(2)))
    w = oracle.widen_bf16(row)
    top = w.max()
    for pos in ([5, 6], [63, 64], [255, 256, 4096], [100000, 2047], [V - 1, 0]):
        r = w.copy()
        r[pos] = top + 1.0
        assert oracle.argmax_first(r) == min(pos)
    # natural ties of bf16 draws
    ties = 0
    for _ in range(20):
        r = oracle.widen_bf16(workloads.bf16_bits(
            rng.standard_normal(V).astype(np.float32) * np.float32(np.sqrt(2))))
        idx = np.flatnonzero(r == r.max())
        ties += len(idx) > 1
        assert oracle.argmax_first(r) == idx[0] == int(np.argmax(r))


def test_golden_acceptance():
    with open(os.path.join(GOLDEN, "accept_examples.json")) as f:
        data = json.load(f)
    for c in data["cases"]:
        for fn in (oracle.accept_walk, oracle.accept_bruteforce):
            a, path, tok = fn(c["am"], c["draft"], c["parent"])
            assert a == c["accept_len"], c["name"]
            assert list(path[:a + 1]) == c["path"], c["name"]
            assert list(tok[:a + 1]) == c["tokens"], c["name"]
            assert np.all(path[a + 1:] == -1) and np.all(tok[a + 1:] == -1)


@pytest.mark.parametrize("n", [1, 2, 4, 8, 16, 64])
def test_chain_all_correct_and_first_mismatch(n):
    rng = np.random.default_rng(n)
    am = rng.integers(0, 1000, size=n)
    parent = np.arange(-1, n - 1)
    draft = np.concatenate([[7], am[:-1]])
    a, path, tok = oracle.accept_walk(am, draft, parent)
    assert a == n - 1
    assert list(path) == list(range(n))
    assert list(tok) == list(draft[1:]) + [am[n - 1]]
    if n > 1:
        bad = draft.copy()
        bad[1] = am[0] + 1
        a, path, tok = oracle.accept_walk(am, bad, parent)
        assert a == 0 and path[0] == 0 and tok[0] == am[0]
        assert np.all(tok[1:] == -1)


def test_tree_all_correct_reaches_deepest_node():
    rng = np.random.default_rng(3)
    for _ in range(30):
        n = int(rng.integers(2, 40))
        parent = workloads.ddtree_parent(rng, n, chain_len=int(rng.integers(0, n)))
        am = rng.integers(0, 50, size=n)
        draft = np.array([0] + [am[parent[i]] for i in range(1, n)])
        depth = np.zeros(n, int)
        for i in range(1, n):
            depth[i] = depth[parent[i]] + 1
        a, path, _ = oracle.accept_walk(am, draft, parent)
        assert a == depth.max()
        assert path[a] == int(np.flatnonzero(depth == depth.max())[0])


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6, 7])
def test_walk_equals_bruteforce_all_trees_all_patterns(n):
    """Every tree with N <= 7 nodes and every accept/reject pattern of its edges."""
    for choice in itertools.product(*[range(i) for i in range(1, n)]):
        parent = (-1,) + choice
        am = list(range(100, 100 + n))
        for bits in range(1 << (n - 1)):
            draft = [0] * n
            for i in range(1, n):
                ok = (bits >> (i - 1)) & 1
                draft[i] = am[parent[i]] if ok else 1
            w = oracle.accept_walk(am, draft, parent)
            b = oracle.accept_bruteforce(am, draft, parent)
            assert w[0] == b[0]
            np.testing.assert_array_equal(w[1], b[1])
            np.testing.assert_array_equal(w[2], b[2])


def test_duplicate_siblings_deepest_then_smallest_index():
    # nodes 1 and 2 both match the root; node 3 (child of 2) also matches
    parent = [-1, 0, 0, 2]
    am = [5, 6, 7, 8]
    a, path, tok = oracle.accept_walk(am, [0, 5, 5, 7], parent)
    assert a == 2 and list(path[:3]) == [0, 2, 3] and list(tok[:3]) == [5, 7, 8]
    # equal depth: smaller node index wins
    a, path, tok = oracle.accept_walk(am, [0, 5, 5, 0], parent)
    assert a == 1 and list(path[:2]) == [0, 1] and list(tok[:2]) == [5, 6]


def test_logits_rows_are_budget_plus_one():
    """A DDTree of budget B verifies B + 1 rows (the root plus B drafts): the
    batch-level call reads exactly N = budget + 1 logits rows."""
    rng = np.random.default_rng(9)
    for budget in (15, 22, 40):
        n = budget + 1
        logits = rng.standard_normal((1, n, 33))
        parent = workloads.ddtree_parent(rng, n)[None]
        am, a, path, tok = oracle.greedy_accept(logits, np.zeros((1, n), np.int32), parent)
        assert am.shape == (1, n) and path.shape == (1, n)
