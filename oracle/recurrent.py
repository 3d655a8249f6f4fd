"""Tree-aware recurrent state of the hybrid target's Gated DeltaNet layers
(oracle side).

TEST INFRASTRUCTURE ONLY: used by the tests, never by the product path.

The single-RTX-3090 DFlash note's target model is a hybrid: 48 of its 64
layers are Gated DeltaNet layers, which keep a recurrent state alongside the
KV cache ("Why we ran this test").  Verifying a token tree needs, for every
node, that layer's state after the node's root path.  The note names the two
pieces that make this work ("Key breakthroughs"): the short causal
convolution in front of the recurrence takes each node's window along its
parent chain instead of the DFS order of the rows (ggml_ssm_conv_tree), and
the tree form of the gated delta rule writes every node's state straight into
a persistent per-node buffer (ggml_gated_delta_net_tree_persist), which may be
held in f16 (the "f16 intermediate cache"); after acceptance the accepted
node's state is taken from that buffer.

The pages give neither the recurrence nor its sizes.  The readings used here:

* the recurrence is the gated delta rule of Yang, Kautz and Hatamizadeh
  ("Gated Delta Networks: Improving Mamba2 with Delta Rule", ICLR 2025), with
  the state S a dv x dk matrix per value head::

      S_t = a_t S_{t-1} + b_t (v_t - a_t S_{t-1} k_t) k_t^T,
      o_t = scale * S_t q_t,        a_t = exp(g_t),

  g the log decay and b (beta) the write strength; value head h reads key
  head h // (Hv / Hk);
* tree form: node i continues from its parent's state; a node without a valid
  parent (node 0, or an entry outside [0, i)) starts from the committed state
  S0.  Per node this is the sequential recurrence over its root path;
* the short convolution is causal and depthwise, width K: channel c of token
  t is ``bias[c] + sum_j w[c][j] * x[t - (K-1) + j][c]`` (tap K-1 on the
  token itself), optionally followed by SiLU.  In the tree, token t - m of
  node i's window is its m-th ancestor; past the root the window continues
  into the committed conv state (the K-1 inputs before the block, oldest
  first);
* commit: with the accepted root path 0 = a_0, ..., a_m, the committed state
  becomes S_{a_m} as stored in the per-node buffer, and the conv state the
  last K-1 entries of (old conv state, x_{a_0}, ..., x_{a_m}).

Everything is float64 from the exact widening of the stored inputs.

Parity status: pinned in ``tests/test_oracle_recurrent.py`` (hand-worked
examples in ``tests/golden/recurrent_tiny.json``, torch's depthwise conv1d
in float64, the textbook matrix form of the delta rule, brute force over each
node's root path, closed forms of the decay-only and write-only cases, and the
replay of the accepted tokens one at a time).
"""
import numpy as np


def tree_parent(parent_row, i: int) -> int:
    """Node i's parent, or -1 when it has none (node 0, or an entry outside [0, i))."""
    if parent_row is None:
        return i - 1
    p = int(parent_row[i])
    return p if 0 <= p < i else -1


def root_path(parent_row, i: int) -> list:
    """Node indices from the top of node i's path down to i."""
    path = [i]
    p = tree_parent(parent_row, i)
    while p >= 0:
        path.append(p)
        p = tree_parent(parent_row, p)
    return path[::-1]


def silu(y):
    return y / (1.0 + np.exp(-y))


def conv_tree(x, conv_state, weight, bias=None, parent=None, activation="silu"):
    """Causal depthwise convolution with each node's window along its parent chain.

    x           [B][N][C]   the verify block's conv inputs (float values);
    conv_state  [B][K-1][C] the committed inputs before the block, oldest first;
    weight      [C][K]      tap K-1 multiplies the token itself;
    bias        [C] or None;
    parent      [B][N] int or None (chains);
    activation  "silu" or "none".
    Returns y [B][N][C] in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    cs = np.asarray(conv_state, dtype=np.float64)
    w = np.asarray(weight, dtype=np.float64)
    B, N, C = x.shape
    K = w.shape[1]
    assert cs.shape == (B, K - 1, C)
    y = np.zeros((B, N, C))
    for b in range(B):
        prow = None if parent is None else parent[b]
        for i in range(N):
            window = []                       # newest first
            node = i
            while len(window) < K and node >= 0:
                window.append(x[b, node])
                node = tree_parent(prow, node)
            back = 1
            while len(window) < K:
                window.append(cs[b, K - 1 - back])
                back += 1
            acc = np.zeros(C) if bias is None else np.asarray(bias, dtype=np.float64).copy()
            for m, val in enumerate(window):  # m-th ancestor meets tap K-1-m
                acc += w[:, K - 1 - m] * val
            y[b, i] = silu(acc) if activation == "silu" else acc
    return y


def delta_rule_step(S, q, k, v, g, beta, scale):
    """One gated delta rule step on the dv x dk state S; returns (S_new, o)."""
    a = np.exp(g)
    decayed = a * S
    u = v - decayed @ k
    S_new = decayed + beta * np.outer(u, k)
    return S_new, scale * (S_new @ q)


def delta_net_tree(q, k, v, g, beta, state, parent=None, scale=None):
    """The gated delta rule over a token tree, every node's state kept.

    q, k   [B][N][Hk][Dk];  v [B][N][Hv][Dv];  g, beta [B][N][Hv];
    state  [B][Hv][Dv][Dk]  the committed state S0;
    parent [B][N] or None (chains);  scale None -> 1/sqrt(Dk).
    Returns (o [B][N][Hv][Dv], states [B][N][Hv][Dv][Dk]) in float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    g = np.asarray(g, dtype=np.float64)
    beta = np.asarray(beta, dtype=np.float64)
    S0 = np.asarray(state, dtype=np.float64)
    B, N, Hk, Dk = q.shape
    Hv, Dv = v.shape[2], v.shape[3]
    assert Hv % Hk == 0
    rep = Hv // Hk
    if scale is None:
        scale = 1.0 / np.sqrt(Dk)
    o = np.zeros((B, N, Hv, Dv))
    states = np.zeros((B, N, Hv, Dv, Dk))
    for b in range(B):
        prow = None if parent is None else parent[b]
        for i in range(N):                     # parents come before children
            p = tree_parent(prow, i)
            for h in range(Hv):
                S_prev = S0[b, h] if p < 0 else states[b, p, h]
                hk = h // rep
                states[b, i, h], o[b, i, h] = delta_rule_step(
                    S_prev, q[b, i, hk], k[b, i, hk], v[b, i, h], g[b, i, h], beta[b, i, h], scale)
    return o, states


def commit_ok(path_row, a: int, N: int) -> bool:
    """A sequence commits only when accept_len is in [0, N-1] and path[j] in [j, N-1] for j <= a."""
    if not 0 <= a <= N - 1:
        return False
    return all(j <= int(path_row[j]) <= N - 1 for j in range(a + 1))


def recurrent_commit(state_nodes, state, x, conv_state, path, accept_len):
    """The committed recurrent and conv state after acceptance.

    state_nodes [B][N][Hv][Dv][Dk] the per-node states as stored (float values
    or widened f16); state [B][Hv][Dv][Dk]; x [B][N][C] and conv_state
    [B][K-1][C] as stored (any dtype: entries are moved, not converted);
    path [B][N], accept_len [B] as the acceptance walk returns them.  A
    sequence whose entries are out of range keeps its old state.
    Returns (new_state float64, new_conv_state in conv_state's dtype).
    """
    new_state = np.array(state, dtype=np.float64, copy=True)
    new_conv = np.array(conv_state, copy=True)
    B, N = np.asarray(path).shape
    K1 = new_conv.shape[1]
    for b in range(B):
        a = int(accept_len[b])
        if not commit_ok(path[b], a, N):
            continue
        new_state[b] = np.asarray(state_nodes[b][int(path[b][a])], dtype=np.float64)
        seq = [conv_state[b][t] for t in range(K1)] + [x[b][int(path[b][j])] for j in range(a + 1)]
        for t in range(K1):
            new_conv[b][t] = seq[len(seq) - K1 + t]
    return new_state, new_conv
