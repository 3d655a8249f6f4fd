"""Checks of the seeded input generators (CPU only)."""
import numpy as np
import pytest

import oracle
import workloads


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -9, -2.5, 0.0], dtype=np.float32)
    b = workloads.bf16_bits(x)
    y = oracle.widen_bf16(b)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-9 rounds up
    np.testing.assert_array_equal(y, [1.0, 1.0, 1.0 + 2 ** -7, -2.5, 0.0])


@pytest.mark.parametrize("name", ["C1", "C2", "C3", "C4", "C5"])
def test_small_cases_are_well_formed(name):
    cfg = workloads.small_variant(workloads.CONFIGS[name], ctx=40, ctx_hi=90 if name == "C5" else 0,
                                  vocab=700)
    case = workloads.make_case(cfg, seed=11, capacity_pad=3)
    B, N = cfg.batch, cfg.n_nodes
    assert case.parent.shape == (B, N) and np.all(case.parent[:, 0] == -1)
    for b in range(B):
        for i in range(1, N):
            assert 0 <= case.parent[b, i] < i
    # planted target is the lowest index of the row maximum
    lg = case.logits if cfg.logits_dtype == "f32" else oracle.widen_bf16(case.logits)
    for b in range(B):
        for i in range(N):
            assert oracle.argmax_first(lg[b, i]) == case.target[b, i]
    # siblings carry distinct drafts
    for b in range(B):
        for p in range(N):
            kids = [case.draft_ids[b, i] for i in range(1, N) if case.parent[b, i] == p]
            assert len(kids) == len(set(kids))
    if cfg.paged:
        used = case.page_table[case.page_table >= 0]
        assert len(used) == len(set(used.tolist()))


def test_geometric_prefix_mean_accept_length():
    """Mean committed tokens per step for the 8-row chain is about 3.2 (the
    reading of 'geometric(0.3)-length prefix', truncated at 7 drafts)."""
    cfg = workloads.small_variant(workloads.CONFIGS["C2"], ctx=8, vocab=64)
    acc = []
    for s in range(300):
        c = workloads.make_case(cfg, seed=s)
        lg = oracle.widen_bf16(c.logits).astype(np.float64)
        _, a, _, _ = oracle.greedy_accept(lg, c.draft_ids, c.parent)
        acc.append(a[0] + 1)
    assert 2.8 < np.mean(acc) < 3.6


def test_forced_mismatch_rule():
    cfg = workloads.CONFIGS["C1"]
    seen = set()
    for s in range(60):
        c = workloads.make_case(workloads.small_variant(cfg, ctx=4, vocab=50), seed=s)
        _, a, _, _ = oracle.greedy_accept(c.logits.astype(np.float64), c.draft_ids, c.parent)
        seen.add(int(a[0]))
    assert seen == {0, 1, 2, 3}


def test_peaked_variant_makes_mask_matter():
    cfg = workloads.small_variant(workloads.CONFIGS["C3"], ctx=16, vocab=100)
    c = workloads.make_case(cfg, seed=3, variant="peaked")
    out, _ = oracle.verify_attention(c)
    assert np.abs(out).max() > 0.2


@pytest.mark.parametrize("name", sorted(workloads.DELTA_CONFIGS))
def test_delta_cases_are_well_formed(name):
    cfg = workloads.DELTA_CONFIGS[name]
    c = workloads.make_delta_case(cfg, 5)
    B, N = cfg.batch, cfg.n_nodes
    assert c.x.shape == (B, N, cfg.channels) and c.conv_state.shape == (B, cfg.conv_width - 1, cfg.channels)
    assert c.q.shape == (B, N, cfg.n_k_heads, cfg.k_dim) and c.v.shape == (B, N, cfg.n_v_heads, cfg.v_dim)
    assert c.state.shape == (B, cfg.n_v_heads, cfg.v_dim, cfg.k_dim)
    assert np.all(c.g < 0) and np.all((c.beta > 0) & (c.beta <= 1))
    for b in range(B):
        a = int(c.accept_len[b])
        path = c.path[b]
        assert path[0] == 0 and np.all(path[a + 1:] == -1)
        for j in range(1, a + 1):
            assert c.parent[b, path[j]] == path[j - 1]
