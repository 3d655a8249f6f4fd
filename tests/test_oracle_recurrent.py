"""Pins of the oracle's tree-aware recurrent state (conv windows along parent
chains, the gated delta rule over a token tree, the commit of the accepted
node) against hand-worked examples, torch's depthwise conv1d in float64, the
textbook matrix form of the delta rule, brute force over root paths, closed
forms and the replay of accepted tokens one at a time."""
import json
import os

import numpy as np
import pytest
import torch

import workloads
from oracle import widen_bf16, widen_fp16
from oracle.recurrent import (conv_tree, delta_net_tree, delta_rule_step, recurrent_commit,
                              root_path, tree_parent)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "recurrent_tiny.json")


def _f64(a, dtype):
    return widen_bf16(a) if dtype == "bf16" else np.asarray(a, dtype=np.float64)


# ----------------------------------------------------------------------------
# conv windows along parent chains
# ----------------------------------------------------------------------------

def test_conv_hand_worked():
    g = json.load(open(GOLDEN))["conv"]
    x = np.array(g["x"], float)[None]
    cs = np.array(g["conv_state"], float)[None]
    y = conv_tree(x, cs, np.array(g["weight"], float), np.array(g["bias"], float),
                  np.array([g["parent"]]), activation="none")
    np.testing.assert_array_equal(y[0], np.array(g["y_none"], float))


def _torch_causal_conv(seq, w, bias):
    """Depthwise causal conv by torch (cross-correlation, float64): seq [T][C],
    w [C][K] -> outputs for tokens K-1 .. T-1."""
    t = torch.from_numpy(np.ascontiguousarray(seq.T))[None]          # [1][C][T]
    wt = torch.from_numpy(np.ascontiguousarray(w))[:, None, :]         # [C][1][K]
    bt = None if bias is None else torch.from_numpy(np.asarray(bias, np.float64))
    return torch.nn.functional.conv1d(t, wt, bt, groups=w.shape[0])[0].numpy().T


def test_conv_chain_equals_torch_conv1d():
    rng = np.random.default_rng(11)
    B, N, C, K = 2, 7, 5, 4
    x = rng.standard_normal((B, N, C))
    cs = rng.standard_normal((B, K - 1, C))
    w = rng.standard_normal((C, K))
    bias = rng.standard_normal(C)
    y = conv_tree(x, cs, w, bias, None, activation="none")
    ys = conv_tree(x, cs, w, bias, None, activation="silu")
    for b in range(B):
        ref = _torch_causal_conv(np.concatenate([cs[b], x[b]]), w, bias)
        np.testing.assert_allclose(y[b], ref, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(ys[b], torch.nn.functional.silu(torch.from_numpy(ref)).numpy(),
                                   rtol=1e-13, atol=1e-13)
    # the explicit chain parent array is the same as None
    par = np.stack([workloads.chain_parent(N)] * B)
    np.testing.assert_array_equal(conv_tree(x, cs, w, bias, par, "none"), y)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_conv_tree_equals_conv_over_each_root_path(seed):
    rng = np.random.default_rng(100 + seed)
    N, C, K = 22, 6, 4
    par = workloads.ddtree_parent(rng, N)[None]
    x = rng.standard_normal((1, N, C))
    cs = rng.standard_normal((1, K - 1, C))
    w = rng.standard_normal((C, K))
    y = conv_tree(x, cs, w, None, par, "none")
    for i in range(N):
        path = root_path(par[0], i)
        ref = _torch_causal_conv(np.concatenate([cs[0], x[0, path]]), w, None)
        np.testing.assert_allclose(y[0, i], ref[-1], rtol=1e-13, atol=1e-13)
    # and siblings do differ from the row-order (DFS) conv in this tree
    rows = conv_tree(x, cs, w, None, None, "none")
    assert not np.allclose(rows, y)


def test_conv_invalid_parent_ends_the_window():
    rng = np.random.default_rng(12)
    N, C, K = 5, 3, 4
    x = rng.standard_normal((1, N, C))
    cs = rng.standard_normal((1, K - 1, C))
    w = rng.standard_normal((C, K))
    par = np.array([[-1, 0, 7, 2, -5]])               # node 2 and node 4 start new paths
    y = conv_tree(x, cs, w, None, par, "none")
    ref2 = _torch_causal_conv(np.concatenate([cs[0], x[0, [2]]]), w, None)[-1]
    ref3 = _torch_causal_conv(np.concatenate([cs[0], x[0, [2, 3]]]), w, None)[-1]
    ref4 = _torch_causal_conv(np.concatenate([cs[0], x[0, [4]]]), w, None)[-1]
    np.testing.assert_allclose(y[0, 2], ref2, atol=1e-13)
    np.testing.assert_allclose(y[0, 3], ref3, atol=1e-13)
    np.testing.assert_allclose(y[0, 4], ref4, atol=1e-13)
    assert tree_parent(par[0], 0) == -1 and tree_parent(par[0], 2) == -1


# ----------------------------------------------------------------------------
# gated delta rule over the tree
# ----------------------------------------------------------------------------

def test_delta_hand_worked():
    g = json.load(open(GOLDEN))["delta"]
    n = len(g["parent"])
    q = np.array(g["q"], float).reshape(1, n, 1, 2)
    k = np.array(g["k"], float).reshape(1, n, 1, 2)
    v = np.array(g["v"], float).reshape(1, n, 1, 2)
    gg = np.log(np.array(g["alpha"], float)).reshape(1, n, 1)
    beta = np.array(g["beta"], float).reshape(1, n, 1)
    S0 = np.array(g["state"], float).reshape(1, 1, 2, 2)
    o, st = delta_net_tree(q, k, v, gg, beta, S0, np.array([g["parent"]]), scale=1.0)
    np.testing.assert_allclose(o[0, :, 0], np.array(g["o"], float), rtol=0, atol=1e-14)
    np.testing.assert_allclose(st[0, :, 0], np.array(g["states"], float), rtol=0, atol=1e-14)


def _matrix_form_chain(q, k, v, g, beta, S0, scale):
    """The rule as printed: S_t = S_{t-1} (a_t (I - b_t k_t k_t^T)) + b_t v_t k_t^T."""
    S = S0.copy()
    outs = []
    I = np.eye(S.shape[1])
    for t in range(q.shape[0]):
        a = np.exp(g[t])
        S = S @ (a * (I - beta[t] * np.outer(k[t], k[t]))) + beta[t] * np.outer(v[t], k[t])
        outs.append(scale * S @ q[t])
    return S, np.array(outs)


def test_delta_chain_equals_matrix_form_and_head_mapping():
    rng = np.random.default_rng(21)
    B, N, Hk, Hv, Dk, Dv = 2, 6, 2, 4, 8, 5
    q = rng.standard_normal((B, N, Hk, Dk))
    k = rng.standard_normal((B, N, Hk, Dk))
    v = rng.standard_normal((B, N, Hv, Dv))
    g = -rng.uniform(0.0, 1.5, (B, N, Hv))
    beta = rng.uniform(0, 1, (B, N, Hv))
    S0 = rng.standard_normal((B, Hv, Dv, Dk))
    o, st = delta_net_tree(q, k, v, g, beta, S0, None, scale=0.3)
    # key heads repeated for consecutive value heads (torch's repeat_interleave)
    qr = torch.from_numpy(q).repeat_interleave(Hv // Hk, dim=2).numpy()
    kr = torch.from_numpy(k).repeat_interleave(Hv // Hk, dim=2).numpy()
    for b in range(B):
        for h in range(Hv):
            S, oo = _matrix_form_chain(qr[b, :, h], kr[b, :, h], v[b, :, h], g[b, :, h], beta[b, :, h],
                                       S0[b, h], 0.3)
            np.testing.assert_allclose(st[b, -1, h], S, rtol=1e-12, atol=1e-12)
            np.testing.assert_allclose(o[b, :, h], oo, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("seed", [0, 1])
def test_delta_tree_equals_chain_over_each_root_path(seed):
    rng = np.random.default_rng(200 + seed)
    N, Hk, Hv, Dk, Dv = 22, 1, 2, 6, 4
    par = workloads.ddtree_parent(rng, N)[None]
    par[0, 15] = 40                                  # an invalid entry: node 15 starts at S0
    q = rng.standard_normal((1, N, Hk, Dk))
    k = rng.standard_normal((1, N, Hk, Dk))
    v = rng.standard_normal((1, N, Hv, Dv))
    g = -rng.uniform(0.0, 1.0, (1, N, Hv))
    beta = rng.uniform(0, 1, (1, N, Hv))
    S0 = rng.standard_normal((1, Hv, Dv, Dk))
    o, st = delta_net_tree(q, k, v, g, beta, S0, par)
    for i in range(N):
        path = root_path(par[0], i)
        oc, sc = delta_net_tree(q[:, path], k[:, path], v[:, path], g[:, path], beta[:, path], S0, None)
        np.testing.assert_allclose(o[0, i], oc[0, -1], rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(st[0, i], sc[0, -1], rtol=1e-12, atol=1e-12)
    assert root_path(par[0], 15) == [15]


def test_delta_decay_only_closed_form():
    """beta = 0: nothing is written, the state only decays along the path."""
    rng = np.random.default_rng(22)
    N, Dk, Dv = 9, 4, 3
    par = workloads.ddtree_parent(rng, N, chain_len=3)[None]
    q = rng.standard_normal((1, N, 1, Dk))
    k = rng.standard_normal((1, N, 1, Dk))
    v = rng.standard_normal((1, N, 1, Dv))
    g = -rng.uniform(0, 1, (1, N, 1))
    S0 = rng.standard_normal((1, 1, Dv, Dk))
    o, st = delta_net_tree(q, k, v, g, np.zeros((1, N, 1)), S0, par, scale=1.0)
    for i in range(N):
        decay = np.exp(sum(g[0, j, 0] for j in root_path(par[0], i)))
        np.testing.assert_allclose(st[0, i, 0], decay * S0[0, 0], rtol=1e-12)
        np.testing.assert_allclose(o[0, i, 0], decay * S0[0, 0] @ q[0, i, 0], rtol=1e-12, atol=1e-14)


def test_delta_write_then_read_back():
    """a = 1, b = 1 and unit keys: reading with the key just written returns its
    value exactly (the delta rule's replacement property); with orthonormal keys
    from S0 = 0 the state is the sum of outer products v k^T."""
    rng = np.random.default_rng(23)
    N, D = 5, 8
    basis, _ = np.linalg.qr(rng.standard_normal((D, D)))
    k = basis[:N][None, :, None, :]
    v = rng.standard_normal((1, N, 1, D))
    S0 = np.zeros((1, 1, D, D))
    o, st = delta_net_tree(k, k, v, np.zeros((1, N, 1)), np.ones((1, N, 1)), S0, None, scale=1.0)
    np.testing.assert_allclose(o[0, :, 0], v[0, :, 0], atol=1e-12)
    np.testing.assert_allclose(st[0, -1, 0], sum(np.outer(v[0, t, 0], k[0, t, 0]) for t in range(N)), atol=1e-12)
    # overwriting a key replaces its value (from any prior state)
    S = rng.standard_normal((D, D))
    kk = basis[0]
    S1, o1 = delta_rule_step(S, kk, kk, v[0, 0, 0], 0.0, 1.0, 1.0)
    np.testing.assert_allclose(o1, v[0, 0, 0], atol=1e-12)


# ----------------------------------------------------------------------------
# commit of the accepted node
# ----------------------------------------------------------------------------

def test_commit_hand_worked_conv_state():
    g = json.load(open(GOLDEN))["conv"]
    x = np.array(g["x"], float)[None]
    cs = np.array(g["conv_state"], float)[None]
    for c in g["commit"]:
        S = np.zeros((1, 1, 1, 1))
        nodes = np.arange(4, dtype=float).reshape(1, 4, 1, 1, 1)
        new_s, new_c = recurrent_commit(nodes, S, x, cs, np.array([c["path"]]), np.array([c["accept_len"]]))
        np.testing.assert_array_equal(new_c[0], np.array(c["conv_state"], float))
        assert new_s[0, 0, 0, 0] == c["path"][c["accept_len"]]


def test_commit_then_next_step_equals_replay_one_token_at_a_time():
    """Verifying a tree, committing the accepted path and then verifying the next
    root gives what processing the accepted tokens one at a time gives (the
    lossless property of greedy speculative decoding, for the recurrent layers)."""
    cfg = workloads.DeltaConfig("t", 1, 12, 1, 2, 8, 4, 4, "f32", "f32", tree="ddtree")
    for seed in range(4):
        c = workloads.make_delta_case(cfg, seed)
        rng = np.random.default_rng(seed)
        N, C = cfg.n_nodes, cfg.channels
        y = conv_tree(c.x, c.conv_state, c.conv_weight, c.conv_bias, c.parent)
        o, st = delta_net_tree(c.q, c.k, c.v, c.g, c.beta, c.state, c.parent)
        new_s, new_c = recurrent_commit(st, c.state, c.x, c.conv_state, c.path, c.accept_len)
        a = int(c.accept_len[0])
        acc = [int(j) for j in c.path[0, :a + 1]]
        # one token at a time through the accepted tokens
        S, cs = c.state.astype(np.float64), c.conv_state.astype(np.float64)
        for j in acc:
            yj = conv_tree(c.x[:, [j]], cs, c.conv_weight, c.conv_bias, None)
            np.testing.assert_allclose(yj[0, 0], y[0, j], rtol=1e-12, atol=1e-12)
            oj, sj = delta_net_tree(c.q[:, [j]], c.k[:, [j]], c.v[:, [j]], c.g[:, [j]], c.beta[:, [j]], S, None)
            np.testing.assert_allclose(oj[0, 0], o[0, j], rtol=1e-12, atol=1e-12)
            S = sj[:, 0]
            cs = np.concatenate([cs[:, 1:], c.x[:, [j]].astype(np.float64)], axis=1)
        np.testing.assert_allclose(new_s, S, rtol=1e-12, atol=1e-12)
        np.testing.assert_array_equal(new_c, cs)
        # a fresh token after the commit sees the accepted history
        xn = rng.standard_normal((1, 1, C))
        np.testing.assert_allclose(conv_tree(xn, new_c, c.conv_weight, c.conv_bias, None),
                                   conv_tree(xn, cs, c.conv_weight, c.conv_bias, None), rtol=0, atol=0)


def test_commit_skips_out_of_range_entries_and_widens_f16():
    rng = np.random.default_rng(31)
    B, N, Hv, Dv, Dk, C, K = 3, 4, 2, 2, 3, 5, 3
    nodes = workloads.fp16_bits(rng.standard_normal((B, N, Hv, Dv, Dk)).astype(np.float32))
    S = rng.standard_normal((B, Hv, Dv, Dk)).astype(np.float32)
    x = workloads.bf16_bits(rng.standard_normal((B, N, C)).astype(np.float32))
    cs = workloads.bf16_bits(rng.standard_normal((B, K - 1, C)).astype(np.float32))
    path = np.array([[0, 2, 3, -1], [0, 1, -1, -1], [0, 0, 1, -1]])
    alen = np.array([2, 4, 2])                        # b=1: accept_len > N-1; b=2: path[1] < 1
    new_s, new_c = recurrent_commit(widen_fp16(nodes), S, x, cs, path, alen)
    np.testing.assert_array_equal(new_s[0], widen_fp16(nodes[0, 3]))
    np.testing.assert_array_equal(new_c[0], x[0, [2, 3]])
    assert new_c.dtype == np.uint16
    np.testing.assert_array_equal(new_s[1:], S[1:])
    np.testing.assert_array_equal(new_c[1:], cs[1:])
