"""GPU parity of the tree-aware recurrent state (conv windows along parent
chains, the gated delta rule over the tree with every node's state persisted,
the commit of the accepted node) through the C ABI, against the CPU oracle.

Tolerances, from the arithmetic: the kernels compute in fp32 and the oracle in
fp64.  Replaying the fp32 operations on the CPU puts the fp32 error of these
workloads near 1e-8 on outputs of size 0.1 and 1e-7 on states of size 1, so
fp32 results are held to 1e-5 (absolute) + 1e-5 (relative).  A bf16 result is
the fp32 one rounded to nearest even: off by at most 2^-8 of its value (half a
bf16 step) plus the fp32 error; an f16 state at most 2^-11 of its value plus
the fp32 error.  The commit moves stored values: bit-exact.
"""
import dataclasses

import numpy as np
import pytest
import torch

import oracle
import workloads
from sv_harness import dev_tensor, say

pytestmark = pytest.mark.gpu

D = workloads.DELTA_CONFIGS


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import draft_token_verification_sv_amd as m
    return m


def _f64(a, dtype):
    return oracle.widen_bf16(a) if dtype == "bf16" else np.asarray(a, dtype=np.float64)


def _host(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def _check(got, ref, kind, what):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), what
    rel = {"f32": 1e-5, "bf16": 2.0 ** -8, "f16": 2.0 ** -11}[kind]
    err = np.abs(got - ref)
    bound = 1e-5 + rel * np.abs(ref)
    worst = float((err / bound).max())
    say(f"    {what}: max_abs={err.max():.3g} worst/bound={worst:.3g} (|ref| max {np.abs(ref).max():.3g})")
    assert worst <= 1.0, what


def _parents(kind, case):
    """Parent arrays for the tree shapes the tests cover (None = chain)."""
    B, N = case.cfg.batch, case.cfg.n_nodes
    if kind == "none":
        return None
    if kind == "case":
        return case.parent
    if kind == "chain":
        return np.stack([workloads.chain_parent(N)] * B)
    if kind == "binary":            # complete binary tree: the most parked states
        return np.stack([np.array([-1] + [(i - 1) // 2 for i in range(1, N)], np.int32)] * B)
    if kind == "star":
        return np.stack([np.array([-1] + [0] * (N - 1), np.int32)] * B)
    if kind == "forest":            # entries outside [0, i) start new paths from the committed state
        rng = np.random.default_rng(5)
        p = np.stack([workloads.ddtree_parent(rng, N, chain_len=min(3, N - 1)) for _ in range(B)])
        for b in range(B):
            for i in range(1, N, 5):
                p[b, i] = [i, -7, N + 3, 2 * i + 1][(i // 5) % 4]
        return p
    raise ValueError(kind)


# ----------------------------------------------------------------------------
# conv windows along parent chains
# ----------------------------------------------------------------------------

CONV_CASES = [
    # (label, config, kernel width, activation, bias, parents)
    ("tiny fp32 chain K4", D["D1"], 4, "silu", True, "none"),
    ("tiny fp32 tree K3", dataclasses.replace(D["D1"], n_nodes=9, tree="ddtree"), 3, "none", False, "case"),
    ("ddtree22 bf16 K4", D["D2"], 4, "silu", False, "case"),
    ("block16 bf16 K2", D["D3"], 2, "silu", True, "none"),
    ("batch8 bf16 K4", D["D4"], 4, "none", True, "chain"),
    ("forest N=23 bf16", dataclasses.replace(D["D2"], n_nodes=23), 4, "silu", True, "forest"),
    ("N=1", dataclasses.replace(D["D3"], n_nodes=1), 4, "silu", False, "none"),
    ("N=64 binary fp32 C=100", dataclasses.replace(D["D1"], n_nodes=64, n_k_heads=1, n_v_heads=1, k_dim=36,
                                                   v_dim=28, tree="ddtree"), 4, "silu", True, "binary"),
]


@pytest.mark.parametrize("case_", CONV_CASES, ids=[c[0] for c in CONV_CASES])
def test_conv_tree(sv, case_):
    label, cfg, K, act, use_bias, kind = case_
    cfg = dataclasses.replace(cfg, conv_width=K)
    say(f"[conv] {label}")
    c = workloads.make_delta_case(cfg, 41)
    par = _parents(kind, c)
    x = dev_tensor(c.x, cfg.dtype)
    cs = dev_tensor(c.conv_state, cfg.dtype)
    w = dev_tensor(c.conv_weight, "f32")
    bias = dev_tensor(c.conv_bias, "f32") if use_bias else None
    pd = None if par is None else dev_tensor(par, "i32")
    out = sv.ssm_conv_tree(x, cs, w, bias, pd, activation=act)
    torch.cuda.synchronize()
    ref = oracle.conv_tree(_f64(c.x, cfg.dtype), _f64(c.conv_state, cfg.dtype), c.conv_weight,
                           c.conv_bias if use_bias else None, par, activation=act)
    _check(_host(out), ref, cfg.dtype, "conv out")


# ----------------------------------------------------------------------------
# gated delta rule over the tree
# ----------------------------------------------------------------------------

DELTA_CASES = [
    # (label, config, parents, state dtype)
    ("tiny fp32 chain f32 states", D["D1"], "none", "f32"),
    ("tiny fp32 chain as array", D["D1"], "chain", "f32"),
    ("ddtree22 bf16 f16 states", D["D2"], "case", "f16"),
    ("ddtree22 bf16 f32 states", D["D2"], "case", "f32"),
    ("block16 bf16 f16 states", D["D3"], "none", "f16"),
    ("batch8 chains bf16", D["D4"], "chain", "f16"),
    ("N=1", dataclasses.replace(D["D3"], n_nodes=1, n_v_heads=16), "none", "f16"),
    ("N=64 binary Dk128", dataclasses.replace(D["D2"], n_nodes=64, n_k_heads=2, n_v_heads=4), "binary", "f32"),
    ("N=64 ddtree Dk128 f16", dataclasses.replace(D["D2"], n_nodes=64, n_k_heads=2, n_v_heads=6), "case", "f16"),
    ("N=31 binary fp32 Dk64", dataclasses.replace(D["D1"], n_nodes=31, n_k_heads=2, n_v_heads=4, v_dim=96,
                                                  tree="ddtree"), "binary", "f32"),
    ("N=16 star Dk64 f16", dataclasses.replace(D["D1"], n_nodes=16, k_dim=64, v_dim=32, dtype="bf16"), "star", "f16"),
    ("N=23 forest", dataclasses.replace(D["D2"], n_nodes=23, n_v_heads=16), "forest", "f16"),
    ("batch3 trees N=40", dataclasses.replace(D["D2"], batch=3, n_nodes=40, n_k_heads=4, n_v_heads=8), "case", "f32"),
]


def _delta_run(sv, c, par, sdt, **kw):
    cfg = c.cfg
    q, k, v = (dev_tensor(a, cfg.dtype) for a in (c.q, c.k, c.v))
    g, beta, state = (dev_tensor(a, "f32") for a in (c.g, c.beta, c.state))
    pd = None if par is None else dev_tensor(par, "i32")
    return sv.gated_delta_net_tree(q, k, v, g, beta, state, pd,
                                   state_dtype=torch.float16 if sdt == "f16" else torch.float32, **kw)


def _delta_ref(c, par):
    cfg = c.cfg
    return oracle.delta_net_tree(_f64(c.q, cfg.dtype), _f64(c.k, cfg.dtype), _f64(c.v, cfg.dtype), c.g, c.beta,
                                 c.state, par)


@pytest.mark.parametrize("case_", DELTA_CASES, ids=[c[0] for c in DELTA_CASES])
def test_gated_delta_net_tree(sv, case_):
    label, cfg, kind, sdt = case_
    say(f"[delta] {label}")
    c = workloads.make_delta_case(cfg, 43)
    par = _parents(kind, c)
    out, nodes = _delta_run(sv, c, par, sdt)
    torch.cuda.synchronize()
    ref_o, ref_s = _delta_ref(c, par)
    _check(_host(out), ref_o, cfg.dtype, "out")
    _check(_host(nodes), ref_s, sdt, "node states")


def test_delta_chain_as_array_matches_chain_path_bitwise(sv):
    """The tree walk (parent array) and the chain walk (no parents) take the same
    fp32 steps on a chain: identical bits."""
    c = workloads.make_delta_case(D["D3"], 44)
    o1, s1 = _delta_run(sv, c, None, "f16")
    o2, s2 = _delta_run(sv, c, _parents("chain", c), "f16")
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(s1.view(torch.int16), s2.view(torch.int16))


def test_delta_packed_views_and_bounds(sv):
    """q, k, v as views into one packed [B, N, C] conv output (the layer's
    layout); nothing written past the outputs."""
    cfg = dataclasses.replace(D["D2"], n_nodes=13, n_v_heads=16, batch=2)
    c = workloads.make_delta_case(cfg, 45)
    B, N, Hk, Hv, Dk, Dv = cfg.batch, cfg.n_nodes, cfg.n_k_heads, cfg.n_v_heads, cfg.k_dim, cfg.v_dim
    packed = np.concatenate([c.q.reshape(B, N, -1), c.k.reshape(B, N, -1), c.v.reshape(B, N, -1)], axis=2)
    pk = dev_tensor(packed, cfg.dtype)
    q = pk[:, :, :Hk * Dk].unflatten(2, (Hk, Dk))
    k = pk[:, :, Hk * Dk:2 * Hk * Dk].unflatten(2, (Hk, Dk))
    v = pk[:, :, 2 * Hk * Dk:].unflatten(2, (Hv, Dv))
    g, beta, state = (dev_tensor(a, "f32") for a in (c.g, c.beta, c.state))
    pd = dev_tensor(c.parent, "i32")
    n_out, n_st = B * N * Hv * Dv, B * N * Hv * Dv * Dk
    out_buf = torch.full((n_out + 4096,), 7.0, dtype=torch.bfloat16, device="cuda")
    st_buf = torch.full((n_st + 4096,), 3.0, dtype=torch.float16, device="cuda")
    out = out_buf[:n_out].view(B, N, Hv, Dv)
    nodes = st_buf[:n_st].view(B, N, Hv, Dv, Dk)
    sv.gated_delta_net_tree(q, k, v, g, beta, state, pd, out=out, state_nodes=nodes)
    torch.cuda.synchronize()
    assert torch.all(out_buf[n_out:] == 7.0) and torch.all(st_buf[n_st:] == 3.0)
    ref_o, ref_s = _delta_ref(c, c.parent)
    _check(_host(out), ref_o, cfg.dtype, "out")
    _check(_host(nodes), ref_s, "f16", "node states")


# ----------------------------------------------------------------------------
# commit of the accepted node
# ----------------------------------------------------------------------------

COMMIT_CASES = [
    ("ddtree22 f16 bf16", D["D2"], "f16"),
    ("batch8 f32 states bf16", D["D4"], "f32"),
    ("tiny fp32", D["D1"], "f32"),
    ("K=2 tree", dataclasses.replace(D["D2"], conv_width=2, n_v_heads=8), "f16"),
]


@pytest.mark.parametrize("case_", COMMIT_CASES, ids=[c[0] for c in COMMIT_CASES])
def test_recurrent_commit(sv, case_):
    label, cfg, sdt = case_
    say(f"[commit] {label}")
    c = workloads.make_delta_case(cfg, 47)
    B, N = cfg.batch, cfg.n_nodes
    rng = np.random.default_rng(48)
    shape = (B, N, cfg.n_v_heads, cfg.v_dim, cfg.k_dim)
    raw = rng.standard_normal(shape).astype(np.float32)
    nodes_np = workloads.fp16_bits(raw) if sdt == "f16" else raw
    path, alen = c.path.copy(), c.accept_len.copy()
    if B > 2:
        alen[1] = N                      # out of range: keeps its state
        path[2, :] = -1                  # path entry below j: keeps its state
        alen[2] = 1
    nodes = dev_tensor(nodes_np, "u16").view(torch.float16) if sdt == "f16" else dev_tensor(nodes_np, "f32")
    state = dev_tensor(c.state, "f32")
    x = dev_tensor(c.x, cfg.dtype)
    cs = dev_tensor(c.conv_state, cfg.dtype)
    sv.recurrent_commit(nodes, state, x, cs, dev_tensor(path, "i32"), dev_tensor(alen, "i32"))
    torch.cuda.synchronize()
    nodes_f = oracle.widen_fp16(nodes_np) if sdt == "f16" else nodes_np
    ref_s, ref_c = oracle.recurrent_commit(nodes_f, c.state, c.x, c.conv_state, path, alen)
    assert np.array_equal(state.cpu().numpy(), ref_s.astype(np.float32))
    got_c = cs.cpu().view(torch.int16).numpy().view(np.uint16) if cfg.dtype == "bf16" else cs.cpu().numpy()
    assert np.array_equal(got_c, ref_c)
    say(f"    accept_len={alen.tolist()} bit-exact")


SCHED_KINDS = [("D2 ddtree22", D["D2"], "case"), ("N=64 binary", dataclasses.replace(D["D2"], n_nodes=64), "binary"),
               ("N=16 star", dataclasses.replace(D["D3"], n_nodes=16), "star"),
               ("N=23 forest", dataclasses.replace(D["D2"], n_nodes=23), "forest"),
               ("chain as array", D["D3"], "chain"), ("N=1", dataclasses.replace(D["D3"], n_nodes=1), "chain"),
               ("batch3 trees N=40", dataclasses.replace(D["D2"], batch=3, n_nodes=40), "case")]


def _check_schedule_words(words, parent_row):
    """The words visit every node once, each from its parent's state: replay
    them with symbolic states (node ids) and bounded slots."""
    N = len(parent_row)
    par = [int(p) if 0 <= int(p) < i else -1 for i, p in enumerate(parent_row)]
    nodes = [int(w) & 63 for w in words[:N]]
    assert sorted(nodes) == list(range(N))
    reg, slots = -1, {}
    for t, w in enumerate(words[:N]):
        x, rc, sc = int(w) & 63, (int(w) >> 8) & 255, int(w) >> 16
        if rc == 1:
            reg = -1
        elif rc >= 2:
            reg = slots[rc - 2]
        assert reg == par[x], (t, x, reg, par[x])
        reg = x
        if sc:
            assert sc - 1 < 5
            slots[sc - 1] = x


@pytest.mark.parametrize("case_", SCHED_KINDS, ids=[c[0] for c in SCHED_KINDS])
def test_tree_schedule_shared_by_layers(sv, case_):
    """sv_tree_schedule's words are a valid walk of each tree, and the recurrence
    driven by them gives the same bits as the order computed in the kernel."""
    label, cfg, kind = case_
    say(f"[schedule] {label}")
    c = workloads.make_delta_case(cfg, 49)
    par = _parents(kind, c)
    pd = dev_tensor(par, "i32")
    sched = sv.tree_schedule(pd)
    torch.cuda.synchronize()
    words = sched.cpu().numpy()
    for b in range(cfg.batch):
        _check_schedule_words(words[b], par[b])
    o1, s1 = _delta_run(sv, c, par, "f16")
    o2, s2 = _delta_run(sv, c, par, "f16", schedule=sched)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(s1.view(torch.int16), s2.view(torch.int16))


def test_recurrent_calls_replay_in_a_graph(sv):
    """The schedule, conv, tree recurrence and commit captured in one HIP graph
    and replayed three times, with eager work between the replays, give the
    eager results every time (the calls launch kernels only: no memsets)."""
    cfg = D["D2"]
    c = workloads.make_delta_case(cfg, 51)
    x, cs0 = dev_tensor(c.x, cfg.dtype), dev_tensor(c.conv_state, cfg.dtype)
    w, bias = dev_tensor(c.conv_weight, "f32"), dev_tensor(c.conv_bias, "f32")
    q, k, v = (dev_tensor(a, cfg.dtype) for a in (c.q, c.k, c.v))
    g, beta, st0 = (dev_tensor(a, "f32") for a in (c.g, c.beta, c.state))
    pd, path, alen = dev_tensor(c.parent, "i32"), dev_tensor(c.path, "i32"), dev_tensor(c.accept_len, "i32")
    B, N, Hv, Dv, Dk = cfg.batch, cfg.n_nodes, cfg.n_v_heads, cfg.v_dim, cfg.k_dim
    sched = torch.empty((B, 64), dtype=torch.int32, device="cuda")
    conv_out = torch.empty_like(x)
    d_out = torch.empty((B, N, Hv, Dv), dtype=q.dtype, device="cuda")
    nodes = torch.empty((B, N, Hv, Dv, Dk), dtype=torch.float16, device="cuda")
    st, cs = st0.clone(), cs0.clone()

    def calls():
        sv.tree_schedule(pd, out=sched)
        sv.ssm_conv_tree(x, cs, w, bias, pd, out=conv_out)
        sv.gated_delta_net_tree(q, k, v, g, beta, st, pd, out=d_out, state_nodes=nodes, schedule=sched)
        sv.recurrent_commit(nodes, st, x, cs, path, alen)

    calls()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (sched, conv_out, d_out, nodes, st, cs)]
    st.copy_(st0)
    cs.copy_(cs0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()
    for rep in range(3):
        st.copy_(st0)                                   # eager work between the replays
        cs.copy_(cs0)
        conv_out.zero_()
        d_out.zero_()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for got, want in zip((sched, conv_out, d_out, nodes, st, cs), ref):
            assert torch.equal(got.view(torch.uint8), want.view(torch.uint8)), rep
