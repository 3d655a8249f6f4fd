"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Attention within the gates (max-abs 2e-2 for bf16 / 4-bit inputs, 1e-4 for
fp32) plus the supplementary checks (relative Frobenius error, lse error);
argmax, accept length, path, tokens and compacted caches bit-exact.
"""
import numpy as np
import pytest
import torch

import oracle
import workloads
from sv_harness import DeviceCase, check_attention, oracle_accept, q4_key_rounding, sample_accept_guarded, say

pytestmark = pytest.mark.gpu

C = workloads.CONFIGS


@pytest.fixture(scope="module")
def sv():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import draft_token_verification_sv_amd as m
    return m


def _small(name, **kw):
    return workloads.small_variant(C[name], **kw)


ATTN_CASES = [
    # (label, config, make_case kwargs)
    ("C1 tiny fp32 chain", C["C1"], {}),
    ("C2 ctx333", _small("C2", ctx=333), {}),
    ("C2 ctx1000 peaked", _small("C2", ctx=1000), {"variant": "peaked"}),
    ("C3 tree22 ctx500", _small("C3", ctx=500), {}),
    ("C3 tree23 ctx700 peaked", _small("C3", ctx=700, n_nodes=23), {"variant": "peaked"}),
    ("C3 tree22 ctx16 peaked", _small("C3", ctx=16), {"variant": "peaked"}),
    ("C3 tree22 ctx0", _small("C3", ctx=0), {"variant": "peaked"}),
    ("C4 q4 ctx700", _small("C4", ctx=700), {}),
    ("C4 q4 ctx130 peaked", _small("C4", ctx=130), {"variant": "peaked"}),
    ("C5 paged b8", _small("C5", ctx=40, ctx_hi=900), {}),
    ("C5 paged b8 peaked", _small("C5", ctx=3, ctx_hi=200), {"variant": "peaked"}),
]


@pytest.mark.parametrize("label,cfg,kw", ATTN_CASES, ids=[c[0] for c in ATTN_CASES])
@pytest.mark.parametrize("seed", [0, 1])
def test_attention_small(sv, label, cfg, kw, seed):
    say(f"[attn] {label} seed={seed}")
    case = workloads.make_case(cfg, seed=1000 * seed + 17, capacity_pad=5, **kw)
    dc = DeviceCase(case)
    out, lse = dc.attn()
    torch.cuda.synchronize()
    ma, rel, le = check_attention(case, out, lse)
    say(f"    max_abs={ma:.3g} rel={rel:.3g} lse={le:.3g}")


VARIANT_SHAPES = [
    # (label, Hq, Hkv, D, N, q, kv, paged, ctx, tree)
    ("decode N=1 G=6 bf16 (VALU)", 24, 4, 256, 1, "bf16", "bf16", False, 777, "chain"),
    ("decode N=1 G=4 paged (VALU)", 32, 8, 128, 1, "bf16", "bf16", True, 300, "chain"),
    ("N=64 max rows tree D128", 4, 2, 128, 64, "bf16", "bf16", False, 200, "ddtree"),
    ("N=3 G=8 -> 24 rows D64", 8, 1, 64, 3, "bf16", "bf16", False, 513, "chain"),
    ("R=16 exactly D256", 8, 2, 256, 4, "bf16", "bf16", False, 129, "chain"),
    ("R=16 D256 q4", 8, 2, 256, 4, "bf16", "q4", False, 129, "chain"),
    ("fp32 q bf16 kv", 4, 2, 128, 5, "f32", "bf16", False, 150, "ddtree"),
    ("fp32 q q4 kv paged", 4, 2, 256, 6, "f32", "q4", True, 90, "ddtree"),
    ("fp32 tree D256 rows>16", 12, 2, 256, 8, "f32", "f32", False, 64, "ddtree"),
    ("bf16 q4 paged tree", 12, 2, 64, 9, "bf16", "q4", True, 100, "ddtree"),
    ("many row blocks", 32, 1, 128, 12, "bf16", "bf16", False, 40, "ddtree"),
    ("q4 D256 paged tree", 12, 2, 256, 4, "bf16", "q4", True, 300, "ddtree"),
    ("q4 D256 rows 96", 24, 4, 256, 16, "bf16", "q4", False, 333, "chain"),
]


@pytest.mark.parametrize("shape", VARIANT_SHAPES, ids=[s[0] for s in VARIANT_SHAPES])
def test_attention_shapes(sv, shape):
    label, Hq, Hkv, D, N, qd, kvd, paged, ctx, tree = shape
    say(f"[attn-shape] {label}")
    cfg = workloads.Config(label, 2, Hq, Hkv, D, N, qd, kvd, "f32", 50, ctx, ctx_hi=ctx + 37,
                           tree=tree, paged=paged, q_std=0.5, kv_std=0.5,
                           draft_rule="tree" if tree == "ddtree" else "geometric")
    case = workloads.make_case(cfg, seed=5, capacity_pad=3, variant="peaked")
    dc = DeviceCase(case)
    out, lse = dc.attn()
    torch.cuda.synchronize()
    ma, rel, le = check_attention(case, out, lse)
    say(f"    max_abs={ma:.3g} rel={rel:.3g} lse={le:.3g}")


@pytest.mark.parametrize("target", [1, 5, 64, 300, 5000])
def test_attention_split_count_independent(sv, target):
    """Any number of splits gives the same answer (to fp tolerance)."""
    say(f"[attn-splits] target_wgs={target}")
    cfg = _small("C3", ctx=900)
    case = workloads.make_case(cfg, seed=3, variant="peaked")
    dc = DeviceCase(case)
    out, lse = dc.attn(tuning={"attn_target_wgs": target})
    torch.cuda.synchronize()
    check_attention(case, out, lse)


BATCH_PATHS = [
    # (label, Hq, Hkv, D, N, q, kv, paged)
    ("pipelined D128 R16 paged", 16, 4, 128, 4, "bf16", "bf16", True),
    ("pipelined D256 R48", 24, 4, 256, 8, "bf16", "bf16", False),
    ("staged q4 D128", 16, 4, 128, 4, "bf16", "q4", False),
    ("valu f32 D64", 4, 2, 64, 3, "f32", "f32", False),
]
SKEW = [0, 3100, 5, 1500, 0, 64, 777]


def _skewed_case(path, seed=11):
    label, Hq, Hkv, D, N, qd, kvd, paged = path
    cfg = workloads.Config(label, len(SKEW), Hq, Hkv, D, N, qd, kvd, "f32", 50, max(SKEW),
                           tree="ddtree", paged=paged, q_std=0.5, kv_std=0.5, draft_rule="tree")
    case = workloads.make_case(cfg, seed=seed, capacity_pad=3)
    # lengths far apart: the cache holds max(SKEW) + N positions for every
    # sequence, the call sees these lengths (both sides read the same arrays)
    case.ctx_lens = np.array(SKEW, dtype=np.int32)
    return case


@pytest.mark.parametrize("path", BATCH_PATHS, ids=[b[0] for b in BATCH_PATHS])
@pytest.mark.parametrize("target", [1, 37, 256, 4096])
def test_attention_batch_schedule(sv, path, target):
    """A batch with very different lengths (some empty) under the dynamic split
    schedule, for grids far below and far above the unit count."""
    say(f"[attn-batch] {path[0]} target_wgs={target}")
    case = _skewed_case(path)
    dc = DeviceCase(case)
    out, lse = dc.attn(tuning={"attn_target_wgs": target})
    torch.cuda.synchronize()
    ma, rel, le = check_attention(case, out, lse)
    say(f"    max_abs={ma:.3g} rel={rel:.3g} lse={le:.3g}")


@pytest.mark.parametrize("pg", [1, 2, 4])
def test_attention_position_groups(sv, pg):
    say(f"[attn-pg] posgroups={pg}")
    case = _skewed_case(BATCH_PATHS[0], seed=12)
    dc = DeviceCase(case)
    out, lse = dc.attn(tuning={"attn_posgroups": pg})
    torch.cuda.synchronize()
    check_attention(case, out, lse)


WINDOW_CASES = [("C1 tiny fp32 chain", [4, 100, 1000]), ("C2 ctx1000 peaked", [8, 100, 517, 5000]),
                ("C3 tree22 ctx500", [22, 64, 300]), ("C4 q4 ctx700", [16, 200]),
                ("C5 paged b8", [4, 50, 600]), ("C5 paged b8 peaked", [4, 137])]


@pytest.mark.parametrize("label,windows", WINDOW_CASES, ids=[w[0] for w in WINDOW_CASES])
def test_attention_window(sv, label, windows):
    """Sliding window over the key range against the oracle's windowed mask
    (windows from N, where the cache drops out, to past the whole range)."""
    cfg, kw = [(c, k) for (l, c, k) in ATTN_CASES if l == label][0]
    case = workloads.make_case(cfg, seed=6, **kw)
    dc = DeviceCase(case)
    for w in windows:
        say(f"[attn window] {label} W={w}")
        out, lse = dc.attn(window=w)
        torch.cuda.synchronize()
        check_attention(case, out, lse, ref=oracle.verify_attention(case, window=w))


OCC_CASES = ["C2 ctx333", "C2 ctx1000 peaked", "C3 tree22 ctx16 peaked", "C5 paged b8", "C5 paged b8 peaked"]


@pytest.mark.parametrize("label", OCC_CASES)
@pytest.mark.parametrize("target", [0, 37, 700])
def test_attention_two_per_cu(sv, label, target):
    """Two workgroups per CU (half-size rings, twice the units) against the oracle."""
    cfg, kw = [(c, k) for (l, c, k) in ATTN_CASES if l == label][0]
    say(f"[attn occ2] {label} target={target}")
    case = workloads.make_case(cfg, seed=5, **kw)
    out, lse = DeviceCase(case).attn(tuning={"attn_occupancy": 2, "attn_target_wgs": target})
    torch.cuda.synchronize()
    check_attention(case, out, lse)


PLAN_EDGES = [
    # (label, Hq, Hkv, D, N, tree, ctx, paged): one sequence, bf16, at the
    # planner's thresholds -- <= 6144 keys with <= 4 row tiles (half-size
    # rings at one workgroup per CU) and <= 65536 keys with > 4 row tiles
    # (blocks of <= 4 tiles, two workgroups per CU); L = ctx + N keys; and
    # the same plans over a paged cache (static schedule, page ids in LDS)
    ("short ring, L = 6144", 24, 4, 256, 8, "chain", 6136, False),
    ("full ring, L = 6145", 24, 4, 256, 8, "chain", 6137, False),
    ("5 tiles in 2 blocks", 6, 1, 256, 12, "ddtree", 5000, False),
    ("tree 22 one block, L = 4096", 6, 1, 256, 22, "ddtree", 4074, False),
    ("tree 22 blocks, L = 4097", 6, 1, 256, 22, "ddtree", 4075, False),
    ("tree 22 blocks, L = 65536", 6, 1, 256, 22, "ddtree", 65514, False),
    ("tree 22 one block, L = 65537", 6, 1, 256, 22, "ddtree", 65515, False),
    ("paged one tile", 32, 8, 128, 4, "chain", 2000, True),
    ("paged short ring", 24, 4, 256, 8, "chain", 3000, True),
    ("paged tree 22 blocks", 12, 2, 128, 22, "ddtree", 5000, True),
    ("paged full ring", 24, 4, 256, 8, "chain", 7000, True),
]

Q4_SINGLE = [
    # (label, Hq, Hkv, N, tree, ctx, paged, window): one sequence, 4-bit cache
    # of head dim 256 (pipelined kernel, static schedule)
    ("q4 paged 6 tiles", 24, 4, 16, "chain", 1500, True, 0),
    ("q4 paged tree 9 tiles", 24, 4, 22, "ddtree", 900, True, 0),
    ("q4 paged one tile windowed", 8, 2, 4, "chain", 3000, True, 700),
    ("q4 contiguous 6 tiles windowed", 24, 4, 16, "chain", 2500, False, 1000),
    # L a little over a multiple of the split: 64 splits of 256 keys, the last
    # one also takes the remaining 16 (and, windowed, of the window's keys)
    ("q4 last split takes the remainder", 24, 4, 16, "chain", 16384, False, 0),
    ("q4 paged last split takes the remainder", 24, 4, 16, "chain", 16384, True, 0),
    ("q4 tree last split takes the remainder", 24, 4, 22, "ddtree", 8192, False, 0),
    ("q4 windowed last split takes the remainder", 24, 4, 16, "chain", 20000, False, 16400),
    ("q4 two row blocks, last split takes the remainder", 2, 1, 64, "ddtree", 65536, False, 0),
]


@pytest.mark.parametrize("case_", Q4_SINGLE, ids=[c[0] for c in Q4_SINGLE])
def test_attention_q4_single_sequence(sv, case_):
    """One sequence over a 4-bit cache, paged or windowed, against the oracle."""
    label, Hq, Hkv, N, tree, ctx, paged, window = case_
    say(f"[attn q4 single] {label}")
    cfg = workloads.Config(label, 1, Hq, Hkv, 256, N, "bf16", "q4", "f32", 50, ctx, tree=tree, paged=paged,
                           q_std=0.5, kv_std=0.5, draft_rule="tree" if tree == "ddtree" else "geometric")
    case = workloads.make_case(cfg, seed=43)
    out, lse = DeviceCase(case).attn(window=window)
    torch.cuda.synchronize()
    check_attention(case, out, lse, ref=oracle.verify_attention(case, window=window))


Q4_KERNEL_CASES = [
    # (label, config, make_case kwargs, window): 4-bit caches of head dim 256
    ("C4 q4 ctx700", _small("C4", ctx=700), {}, 0),
    ("C4 q4 ctx130 peaked", _small("C4", ctx=130), {"variant": "peaked"}, 0),
    ("C4 q4 ctx2100 peaked windowed", _small("C4", ctx=2100), {"variant": "peaked"}, 900),
    ("R=16 q4 chain", workloads.Config("r16", 2, 8, 2, 256, 4, "bf16", "q4", "f32", 50, 129, ctx_hi=166,
                                       q_std=0.5, kv_std=0.5), {"variant": "peaked"}, 0),
    ("q4 paged tree 9 tiles", workloads.Config("pt9", 1, 24, 4, 256, 22, "bf16", "q4", "f32", 50, 900,
                                               tree="ddtree", paged=True, q_std=0.5, kv_std=0.5,
                                               draft_rule="tree"), {}, 0),
    ("q4 paged chain 3 tiles", workloads.Config("pc3", 2, 24, 4, 256, 8, "bf16", "q4", "f32", 50, 1100,
                                                ctx_hi=1500, paged=True, q_std=0.5, kv_std=0.5),
     {"variant": "peaked"}, 0),
    ("q4 contiguous 5 tiles ragged", workloads.Config("c5t", 1, 20, 4, 256, 15, "bf16", "q4", "f32", 50, 1333,
                                                      tree="ddtree", q_std=0.5, kv_std=0.5,
                                                      draft_rule="tree"), {}, 0),
    ("q4 batch 70", workloads.Config("b70", 70, 8, 2, 256, 4, "bf16", "q4", "f32", 50, 60, ctx_hi=400,
                                     q_std=0.5, kv_std=0.5), {"variant": "peaked"}, 0),
]


@pytest.mark.parametrize("kernel", ["cooperative", "pipelined", "wide"])
@pytest.mark.parametrize("label,cfg,kw,window", Q4_KERNEL_CASES, ids=[c[0] for c in Q4_KERNEL_CASES])
def test_attention_q4_kernels(sv, label, cfg, kw, window, kernel):
    """The kernels for 4-bit caches of head dim 256, chosen per call: the
    four-wave cooperative fp16 one, the pipelined bf16-staging one and the
    eight-wave cooperative one (the default; it hands paged blocks of three row
    tiles per wave pair to the four-wave one)."""
    say(f"[attn q4 kernel] {label} {kernel}")
    case = workloads.make_case(cfg, seed=77, capacity_pad=2, **kw)
    out, lse = DeviceCase(case).attn(window=window, tuning={"attn_q4_kernel": kernel})
    torch.cuda.synchronize()
    ref = oracle.verify_attention(case, window=window)
    check_attention(case, out, lse, ref=ref, key_rounding=q4_key_rounding(case, kernel))


def _random_q4_cases(n, seed):
    """Seeded random shapes for the 4-bit head-dim-256 kernels: 16-160 packed
    rows (GQA groups 2-8, chains and trees), 1-5 sequences of 1-3000 cached
    tokens, contiguous or paged (pages of 16 or 24), with or without a
    window."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([2, 3, 4, 6, 8]))
        n_nodes = int(rng.integers(max(1, -(-16 // g)), max(2, 160 // g) + 1))
        n_nodes = min(n_nodes, 64)
        tree = "ddtree" if rng.random() < 0.5 else "chain"
        b = int(rng.integers(1, 6))
        lo = int(rng.integers(1, 3000))
        hi = int(min(3000, lo + rng.integers(0, 1500)))
        paged = bool(rng.random() < 0.5)
        window = int(rng.integers(64, 2500)) if rng.random() < 0.3 else 0
        cfg = workloads.Config(f"rq{i}", b, hkv * g, hkv, 256, n_nodes, "bf16", "q4", "f32", 50, lo, ctx_hi=hi,
                               tree=tree, paged=paged, page_size=int(rng.choice([16, 24])), q_std=0.5,
                               kv_std=0.5, draft_rule="tree" if tree == "ddtree" else "geometric")
        variant = "peaked" if rng.random() < 0.5 else ""
        out.append((f"rq{i} B{b} {hkv * g}/{hkv} N{n_nodes} {tree} {lo}-{hi} {'paged' if paged else 'contig'}"
                    f" W{window} {variant or 'plain'}", cfg, variant, window))
    return out


RANDOM_Q4 = _random_q4_cases(32, 2024)


@pytest.mark.parametrize("label,cfg,variant,window", RANDOM_Q4, ids=[c[0] for c in RANDOM_Q4])
def test_attention_q4_random_shapes(sv, label, cfg, variant, window):
    """The default 4-bit plan (eight-wave kernel, or the four-wave one for
    paged three-tile blocks) on seeded random shapes against the oracle."""
    say(f"[attn q4 random] {label}")
    case = workloads.make_case(cfg, seed=5, capacity_pad=2, variant=variant)
    out, lse = DeviceCase(case).attn(window=window)
    torch.cuda.synchronize()
    check_attention(case, out, lse, ref=oracle.verify_attention(case, window=window))


@pytest.mark.parametrize("edge", PLAN_EDGES, ids=[e[0] for e in PLAN_EDGES])
def test_attention_plan_edges(sv, edge):
    """Launch plans on both sides of each planner threshold against the oracle."""
    label, Hq, Hkv, D, N, tree, ctx, paged = edge
    say(f"[attn plan edge] {label}")
    cfg = workloads.Config(label, 1, Hq, Hkv, D, N, "bf16", "bf16", "f32", 50, ctx, tree=tree, paged=paged,
                           q_std=0.5, kv_std=0.5, draft_rule="tree" if tree == "ddtree" else "geometric")
    case = workloads.make_case(cfg, seed=41, variant="peaked")
    out, lse = DeviceCase(case).attn()
    torch.cuda.synchronize()
    check_attention(case, out, lse)


@pytest.mark.parametrize("B", [64, 65, 1024])
def test_attention_large_batch(sv, B):
    """Batch sizes at the schedule's paths: one wavefront (<= 64 sequences),
    the whole workgroup, and 1024 sequences (the limit, four per thread)."""
    say(f"[attn-batch] B={B}")
    cfg = workloads.Config("large batch", B, 16, 4, 128, 4, "bf16", "bf16", "f32", 50, 0, ctx_hi=60 if B > 100 else 700,
                           tree="ddtree", q_std=0.5, kv_std=0.5, draft_rule="tree")
    case = workloads.make_case(cfg, seed=21 + B)
    dc = DeviceCase(case)
    out, lse = dc.attn()
    torch.cuda.synchronize()
    check_attention(case, out, lse, batch=sorted({0, 1, B // 4, B // 2, B - 2, B - 1}))


FULL = [
    # (config, query heads checked (None: all), sequences checked (None: all), variant)
    ("C2", None, None, ""),
    ("C3", None, None, ""),
    ("C3", None, None, "peaked"),
    ("C4", [0, 6, 12, 18, 23], None, ""),          # one query head of every KV head, and the last
    ("C4", [0, 6, 12, 18], None, "peaked"),
    ("C4", [1, 7, 13, 23], None, "wide"),            # the eight-wave 4-bit kernel
    ("C5", None, None, ""),
]


@pytest.mark.parametrize("name,heads,batch,variant", FULL,
                         ids=[f[0] + ("-" + f[3] if f[3] else "") for f in FULL])
def test_attention_full_size_sampled(sv, name, heads, batch, variant):
    """The configurations at their full sizes, in the launch configuration the
    benchmark times (library defaults), against the oracle on all rows (C2,
    C3, C5) or one query head of every KV head (C4: 131072 cached tokens).
    The peaked variants give each draft row's own key a score far above the
    cache's, so the tree mask decides an O(1) part of every output."""
    cfg = C[name]
    say(f"[attn-full] {cfg.name} heads={heads} batch={batch} variant={variant or 'plain'}")
    tuning = {"attn_q4_kernel": "wide"} if variant == "wide" else None
    case = workloads.make_case(cfg, seed=1, variant="" if variant == "wide" else variant)
    dc = DeviceCase(case)
    out, lse = dc.attn(tuning=tuning)
    torch.cuda.synchronize()
    ma, rel, le = check_attention(case, out, lse, heads=heads, batch=batch)
    say(f"    max_abs={ma:.3g} rel={rel:.3g} lse={le:.3g}")
    out2, lse2 = dc.attn(tuning=tuning)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)


def test_attention_repeatable(sv):
    case = workloads.make_case(_small("C2", ctx=600), seed=9)
    dc = DeviceCase(case)
    o1, l1 = dc.attn()
    o2, l2 = dc.attn()
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ---------------------------------------------------------------------------
# greedy acceptance
# ---------------------------------------------------------------------------

ACCEPT_CASES = [
    ("C1", C["C1"], {}),
    ("C2 full vocab", _small("C2", ctx=8, vocab=151936), {}),
    ("C2 perfect", _small("C2", ctx=8, vocab=151936), {"variant": "perfect"}),
    ("C3 tree22", _small("C3", ctx=8, vocab=151936), {}),
    ("C3 tree23 rescue", _small("C3", ctx=8, vocab=151936, n_nodes=23), {"force_first_mismatch": True}),
    ("C4 block16", _small("C4", ctx=8, vocab=151936), {}),
    ("C5 batch8", _small("C5", ctx=8, ctx_hi=20, vocab=151936), {}),
    ("odd vocab f32", workloads.Config("oddv", 3, 2, 1, 64, 7, "f32", "f32", "f32", 4099, 8,
                                       tree="ddtree", draft_rule="tree"), {}),
    ("odd vocab bf16", workloads.Config("oddb", 2, 2, 1, 64, 64, "bf16", "bf16", "bf16", 12345, 8,
                                        tree="ddtree", draft_rule="tree"), {}),
]


@pytest.mark.parametrize("label,cfg,kw", ACCEPT_CASES, ids=[c[0] for c in ACCEPT_CASES])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_greedy_accept(sv, label, cfg, kw, seed):
    say(f"[accept] {label} seed={seed}")
    case = workloads.make_case(cfg, seed=77 + seed, **kw)
    dc = DeviceCase(case)
    acc, path, tok, am = dc.accept()
    torch.cuda.synchronize()
    r_am, r_acc, r_path, r_tok = oracle_accept(case)
    np.testing.assert_array_equal(am.cpu().numpy(), r_am)
    np.testing.assert_array_equal(acc.cpu().numpy(), r_acc)
    np.testing.assert_array_equal(path.cpu().numpy(), r_path)
    np.testing.assert_array_equal(tok.cpu().numpy(), r_tok)
    # the planted maxima are what both found
    np.testing.assert_array_equal(r_am, case.target)


def test_argmax_natural_and_planted_ties(sv):
    """Unplanted bf16 N(0,2) rows (frequent natural ties) plus planted ties that
    straddle lanes, waves and workgroup chunks: lowest index wins."""
    rng = np.random.default_rng(4)
    B, N, V = 2, 40, 151936
    x = rng.standard_normal((B, N, V)).astype(np.float32) * np.float32(np.sqrt(2))
    bits = workloads.bf16_bits(x)
    w = oracle.widen_bf16(bits)
    plants = [(0, 0, [7, 8]), (0, 1, [4095, 4096]), (0, 2, [63, 64, 65]), (0, 3, [V - 1, 1]),
              (1, 5, [2047, 2048, 6000]), (1, 6, [0, V - 1]), (1, 7, [8191, 8192])]
    for b, i, idx in plants:
        top = np.float32(w[b, i].max() + 1.0)
        bits[b, i, idx] = workloads.bf16_bits(np.array([top], np.float32))[0]
    parent = np.stack([workloads.ddtree_parent(rng, N) for _ in range(B)])
    lg = oracle.widen_bf16(bits)
    r_am = np.array([[oracle.argmax_first(lg[b, i]) for i in range(N)] for b in range(B)])
    drafts = np.stack([workloads.drafts_from_targets(rng, parent[b], r_am[b], V, rng.random(N) < 0.7)
                       for b in range(B)])
    import draft_token_verification_sv_amd as m
    from sv_harness import dev_tensor
    acc, path, tok, am = m.greedy_accept(dev_tensor(bits, "bf16"), dev_tensor(drafts, "i32"),
                                         dev_tensor(parent, "i32"))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(am.cpu().numpy(), r_am)
    _, r_acc, r_path, r_tok = oracle.greedy_accept(lg, drafts, parent)
    np.testing.assert_array_equal(acc.cpu().numpy(), r_acc)
    np.testing.assert_array_equal(path.cpu().numpy(), r_path)
    np.testing.assert_array_equal(tok.cpu().numpy(), r_tok)


def test_argmax_signed_zero_and_negative_rows(sv):
    """Rows whose maximum is a zero (-0 and +0 are equal: the lower index
    wins), a negative value or the smallest negative subnormal, with the
    deciding entries in full 16384-logit chunks and in the ragged last one."""
    rng = np.random.default_rng(9)
    B, N, V = 1, 12, 151936
    bits = workloads.bf16_bits(-np.abs(rng.standard_normal((B, N, V)).astype(np.float32)) - np.float32(0.5))
    P0, M0, MT = 0x0000, 0x8000, 0x8001            # +0, -0, -2^-133
    plants = {0: [(5000, M0), (100, P0)],           # +0 first -> 100
              1: [(3000, P0), (200, M0)],           # -0 first -> 200
              2: [(70000, M0)],                     # a lone -0
              3: [(V - 1, M0), (V - 7, P0)],        # zeros in the ragged chunk -> V - 7
              4: [(40000, MT)],                     # the largest negative
              5: [(10, MT), (20, M0)],              # -0 above -2^-133 -> 20
              6: [(16383, P0), (16384, M0)],        # across a chunk boundary -> 16383
              7: [(147455, MT), (147456, MT)]}      # last full chunk / ragged chunk tie -> 147455
    for i, pl in plants.items():
        for idx, b16 in pl:
            bits[0, i, idx] = b16
    bits[0, 8] = bits[0, 8, 0]                       # a flat row -> 0
    bits[0, 9, [9000, 9001, 150000]] = workloads.bf16_bits(np.array([-0.25], np.float32))[0]
    parent = workloads.ddtree_parent(rng, N)[None]
    lg = oracle.widen_bf16(bits)
    r_am = np.array([[oracle.argmax_first(lg[0, i]) for i in range(N)]])
    assert list(r_am[0, :10]) == [100, 200, 70000, V - 7, 40000, 20, 16383, 147455, 0, 9000], r_am
    drafts = workloads.drafts_from_targets(rng, parent[0], r_am[0], V, rng.random(N) < 0.8)[None]
    import draft_token_verification_sv_amd as m
    from sv_harness import dev_tensor
    _, r_acc, r_path, r_tok = oracle.greedy_accept(lg, drafts, parent)
    for chunk in (0, 8192, 2048 * 8 * 3):
        acc, path, tok, am = m.greedy_accept(dev_tensor(bits, "bf16"), dev_tensor(drafts, "i32"),
                                             dev_tensor(parent, "i32"),
                                             tuning={"argmax_chunk": chunk} if chunk else None)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(am.cpu().numpy(), r_am)
        np.testing.assert_array_equal(acc.cpu().numpy(), r_acc)
        np.testing.assert_array_equal(path.cpu().numpy(), r_path)
        np.testing.assert_array_equal(tok.cpu().numpy(), r_tok)


def test_accept_repeated_calls_and_chunk_sizes(sv):
    """The workspace counters return to zero: many calls in a row, different
    shapes and chunk sizes, stay exact."""
    for k, (chunk, cfg) in enumerate([(4096, _small("C3", ctx=8, vocab=151936)),
                                      (8, _small("C2", ctx=8, vocab=1000)),
                                      (1024, _small("C5", ctx=8, ctx_hi=9, vocab=151936)),
                                      (65536, _small("C3", ctx=8, vocab=70000))]):
        for rep in range(3):
            case = workloads.make_case(cfg, seed=300 + 10 * k + rep)
            dc = DeviceCase(case)
            acc, path, tok, am = dc.accept(workspace=None, tuning={"argmax_chunk": chunk})
            torch.cuda.synchronize()
            r_am, r_acc, r_path, r_tok = oracle_accept(case)
            np.testing.assert_array_equal(am.cpu().numpy(), r_am)
            np.testing.assert_array_equal(path.cpu().numpy(), r_path)
            np.testing.assert_array_equal(tok.cpu().numpy(), r_tok)


SAMPLE_CASES = [
    ("C2 full vocab T1", _small("C2", ctx=8, vocab=151936), 1.0),
    ("C3 tree22 T0.7", _small("C3", ctx=8, vocab=151936), 0.7),
    ("C5 batch8 T1.3", _small("C5", ctx=8, ctx_hi=20, vocab=151936), 1.3),
    ("odd vocab f32 T2", workloads.Config("oddv", 3, 2, 1, 64, 7, "f32", "f32", "f32", 4099, 8,
                                          tree="ddtree", draft_rule="tree"), 2.0),
    ("odd vocab bf16 T0.3", workloads.Config("oddb", 2, 2, 1, 64, 64, "bf16", "bf16", "bf16", 12345, 8,
                                             tree="ddtree", draft_rule="tree"), 0.3),
]


@pytest.mark.parametrize("label,cfg,T", SAMPLE_CASES, ids=[c[0] for c in SAMPLE_CASES])
def test_sample_accept(sv, label, cfg, T):
    """Stochastic verification: samples, accept length, path and tokens equal
    the oracle's, bit for bit (fp32 keys l / T + g on both sides); drafts are
    built from the oracle's samples so that long paths get accepted."""
    say(f"[sample] {label}")
    rng = np.random.default_rng(41)
    case = workloads.make_case(cfg, seed=5)
    lg32 = (oracle.widen_bf16(case.logits) if cfg.logits_dtype == "bf16" else case.logits.astype(np.float64))
    lg32 = lg32.astype(np.float32)
    g = (-np.log(-np.log(rng.random(case.logits.shape)))).astype(np.float32)
    B, N = case.draft_ids.shape
    ys = np.array([[oracle.sample_row(lg32[b, i], g[b, i], T) for i in range(N)] for b in range(B)])
    par = np.maximum(case.parent, 0)
    drafts = np.where(rng.random((B, N)) < 0.8, ys[np.arange(B)[:, None], par], case.draft_ids).astype(np.int32)
    from sv_harness import dev_tensor
    acc, path, tok, y = sample_accept_guarded(dev_tensor(case.logits, cfg.logits_dtype), dev_tensor(g, "f32"), T,
                                              dev_tensor(drafts, "i32"), dev_tensor(case.parent, "i32"))
    torch.cuda.synchronize()
    r_y, r_acc, r_path, r_tok = oracle.sample_accept(lg32, g, T, drafts, case.parent)
    np.testing.assert_array_equal(y.cpu().numpy(), r_y)
    np.testing.assert_array_equal(acc.cpu().numpy(), r_acc)
    np.testing.assert_array_equal(path.cpu().numpy(), r_path)
    np.testing.assert_array_equal(tok.cpu().numpy(), r_tok)


TOPK_CASES = [
    # (label, config, temperature, top_k, special rows)
    ("C2 k=50 T1", _small("C2", ctx=8, vocab=151936), 1.0, 50, False),
    ("C3 tree22 k=1 ties", _small("C3", ctx=8, vocab=151936), 0.7, 1, False),
    ("C5 batch8 k=20 T1.3", _small("C5", ctx=8, ctx_hi=20, vocab=151936), 1.3, 20, False),
    ("C2 k=1024", _small("C2", ctx=8, vocab=151936), 0.9, 1024, False),
    ("flat and tied rows (whole-row path)", _small("C2", ctx=8, vocab=151936), 1.0, 40, True),
    ("odd vocab f32 k=7", workloads.Config("oddv", 3, 2, 1, 64, 7, "f32", "f32", "f32", 4099, 8,
                                           tree="ddtree", draft_rule="tree"), 2.0, 7, True),
    ("odd vocab bf16 k=300", workloads.Config("oddb", 2, 2, 1, 64, 64, "bf16", "bf16", "bf16", 12345, 8,
                                              tree="ddtree", draft_rule="tree"), 0.3, 300, False),
    # 625 16-byte groups for 1024 threads: k above the threads that see a logit
    ("vocab 5000 k=700", workloads.Config("v5k", 1, 2, 1, 64, 3, "bf16", "bf16", "bf16", 5000, 8), 1.0, 700, False),
]


@pytest.mark.parametrize("label,cfg,T,k,special", TOPK_CASES, ids=[c[0] for c in TOPK_CASES])
def test_sample_accept_topk(sv, label, cfg, T, k, special):
    """Top-k stochastic verification: samples, accept length, path and tokens
    equal the oracle's bit for bit.  Special rows: one all-equal row (every
    logit ties at the k-th value: the candidate list overflows and the
    whole-row passes decide) and one row whose largest value is shared by a
    quarter of the vocabulary."""
    say(f"[sample-topk] {label}")
    rng = np.random.default_rng(43)
    case = workloads.make_case(cfg, seed=6)
    logits = case.logits.copy()
    if special:
        V = logits.shape[-1]
        logits[0, 0, :] = logits[0, 0, 0]
        ties = rng.choice(V, V // 4, replace=False)
        logits[0, 1, ties] = logits[0, 1].max()
    lg32 = (oracle.widen_bf16(logits) if cfg.logits_dtype == "bf16" else logits.astype(np.float64)).astype(np.float32)
    g = (-np.log(-np.log(rng.random(logits.shape)))).astype(np.float32)
    B, N = case.draft_ids.shape
    ys = np.array([[oracle.sample_row_topk(lg32[b, i], g[b, i], T, k) for i in range(N)] for b in range(B)])
    par = np.maximum(case.parent, 0)
    drafts = np.where(rng.random((B, N)) < 0.8, ys[np.arange(B)[:, None], par], case.draft_ids).astype(np.int32)
    from sv_harness import dev_tensor
    acc, path, tok, y = sample_accept_guarded(dev_tensor(logits, cfg.logits_dtype), dev_tensor(g, "f32"), T,
                                              dev_tensor(drafts, "i32"), dev_tensor(case.parent, "i32"), top_k=k)
    torch.cuda.synchronize()
    r_y, r_acc, r_path, r_tok = oracle.sample_accept(lg32, g, T, drafts, case.parent, top_k=k)
    np.testing.assert_array_equal(y.cpu().numpy(), r_y)
    np.testing.assert_array_equal(acc.cpu().numpy(), r_acc)
    np.testing.assert_array_equal(path.cpu().numpy(), r_path)
    np.testing.assert_array_equal(tok.cpu().numpy(), r_tok)
    say(f"    accept_len={r_acc.tolist()}")


# ---------------------------------------------------------------------------
# compaction
# ---------------------------------------------------------------------------

COMPACT_CASES = [
    ("C2 chain bf16 3 layers", _small("C2", ctx=50), 3, {}),
    ("C3 tree bf16", _small("C3", ctx=60), 2, {}),
    ("C3 tree rescue", _small("C3", ctx=61, n_nodes=23), 1, {"force_first_mismatch": True}),
    ("C4 q4 chain", _small("C4", ctx=70), 2, {}),
    ("C5 paged", _small("C5", ctx=30, ctx_hi=100), 2, {}),
    ("C1 f32", C["C1"], 1, {}),
    ("tree q4 paged", workloads.Config("tqp", 3, 8, 2, 128, 20, "bf16", "q4", "bf16", 300, 20, ctx_hi=70,
                                       tree="ddtree", paged=True, draft_rule="tree"), 2, {}),
    ("tree perfect f32", workloads.Config("tpf", 2, 4, 2, 64, 30, "f32", "f32", "f32", 200, 9,
                                          tree="ddtree", draft_rule="tree"), 1, {"variant": "perfect"}),
]


@pytest.mark.parametrize("label,cfg,layers,kw", COMPACT_CASES, ids=[c[0] for c in COMPACT_CASES])
def test_kv_compact(sv, label, cfg, layers, kw):
    say(f"[compact] {label}")
    case = workloads.make_case(cfg, seed=21, capacity_pad=4, n_layers=layers, **kw)
    dc = DeviceCase(case)
    before = dc.cache_arrays_host()
    acc, path, tok, am = dc.accept()
    new_lens = sv.kv_compact(dc.kv, dc.ctx, dc.max_ctx, path, acc)
    torch.cuda.synchronize()
    after = dc.cache_arrays_host()
    _, r_acc, r_path, _ = oracle_accept(case)
    np.testing.assert_array_equal(acc.cpu().numpy(), r_acc)
    lay = (lambda a: a[None]) if layers == 1 else (lambda a: a)
    exp, r_new, _ = oracle.compact_cache([lay(a) for a in before], ctx_lens=case.ctx_lens, path=r_path,
                                         accept_len=r_acc,
                                         page_table=case.page_table if cfg.paged else None,
                                         page_size=cfg.page_size)
    for e, g in zip(exp, after):
        np.testing.assert_array_equal(lay(g), e)
    np.testing.assert_array_equal(new_lens.cpu().numpy(), r_new)


FUSED_CASES = COMPACT_CASES + [
    # many moving rows over several layers: the staging rounds of the fused
    # call (32 KB each) cut through rows and layers
    # (seed 13: 4 moving rows in sequence 0, 101 KB of rows to move)
    ("tree bf16 64 nodes 6 layers", workloads.Config("tbm", 2, 8, 4, 256, 40, "bf16", "bf16", "bf16", 500, 64,
                                                     tree="ddtree", draft_rule="tree"), 6,
     {"variant": "perfect", "seed": 13}),
    ("tree q4 64 nodes 6 layers", workloads.Config("tqm", 2, 8, 4, 256, 40, "bf16", "q4", "bf16", 500, 64,
                                                   tree="ddtree", draft_rule="tree"), 6,
     {"variant": "perfect", "seed": 13}),
]


@pytest.mark.parametrize("label,cfg,layers,kw", FUSED_CASES, ids=[c[0] for c in FUSED_CASES])
def test_accept_compact_fused(sv, label, cfg, layers, kw):
    """The one-launch acceptance + compaction against the oracle's acceptance
    and compaction (outputs, every cache array, new lengths)."""
    say(f"[fused] {label}")
    kw = dict(kw)
    case = workloads.make_case(cfg, seed=kw.pop("seed", 23), capacity_pad=4, n_layers=layers, **kw)
    for rep in range(2):              # the shared workspace comes back zeroed: a second call is exact too
        dc = DeviceCase(case)
        before = dc.cache_arrays_host()
        acc, path, tok, am, new_lens = sv.greedy_accept_compact(dc.logits, dc.drafts, dc.parent, dc.kv, dc.ctx,
                                                                dc.max_ctx)
        torch.cuda.synchronize()
        after = dc.cache_arrays_host()
        r_am, r_acc, r_path, r_tok = oracle_accept(case)
        np.testing.assert_array_equal(am.cpu().numpy(), r_am)
        np.testing.assert_array_equal(acc.cpu().numpy(), r_acc)
        np.testing.assert_array_equal(path.cpu().numpy(), r_path)
        np.testing.assert_array_equal(tok.cpu().numpy(), r_tok)
        lay = (lambda a: a[None]) if layers == 1 else (lambda a: a)
        exp, r_new, _ = oracle.compact_cache([lay(a) for a in before], ctx_lens=case.ctx_lens, path=r_path,
                                             accept_len=r_acc,
                                             page_table=case.page_table if cfg.paged else None,
                                             page_size=cfg.page_size)
        for e, g in zip(exp, after):
            np.testing.assert_array_equal(lay(g), e)
        np.testing.assert_array_equal(new_lens.cpu().numpy(), r_new)


# ---------------------------------------------------------------------------
# writing the verify block into the cache
# ---------------------------------------------------------------------------

# (label, cache dtype, D, B, n, Hkv, page_size (0: contiguous), source dtype)
APPEND_CASES = [
    ("bf16 chain block D256", "bf16", 256, 1, 8, 4, 0, "bf16"),
    ("bf16 from f32 D128 B3", "bf16", 128, 3, 5, 2, 0, "f32"),
    ("f32 from f32 D64", "f32", 64, 2, 4, 1, 0, "f32"),
    ("f32 from bf16 D64", "f32", 64, 2, 4, 1, 0, "bf16"),
    ("q4 block16 D256", "q4", 256, 1, 16, 4, 0, "bf16"),
    ("q4 from f32 D256", "q4", 256, 2, 22, 4, 0, "f32"),
    ("q4 paged D128 B3", "q4", 128, 3, 5, 2, 16, "f32"),
    ("q4 paged D64 bad page", "q4", 64, 2, 9, 2, 8, "bf16"),
    ("bf16 paged batch8 D128", "bf16", 128, 8, 4, 8, 16, "bf16"),
]


@pytest.mark.parametrize("case", APPEND_CASES, ids=[c[0] for c in APPEND_CASES])
def test_kv_append(sv, case):
    """Cache bytes after the write equal the oracle's, bit for bit (rounding
    to bf16, the 4-bit quantiser's half-precision scale and ties to even)."""
    label, dt, D, B, n, H, ps, src = case
    say(f"[append] {label}")
    from sv_harness import dev_tensor
    rng = np.random.default_rng(31)
    ctx = rng.integers(0, 40, B).astype(np.int32)
    ctx[-1] = 60                                          # clamped to max_ctx
    max_ctx = 45
    # new rows: mixed magnitudes, zero blocks and exact ties of x / d
    x = (rng.standard_normal((2, B, n, H, D)) * rng.uniform(0.01, 30, (2, B, n, H, 1))).astype(np.float32)
    x[0, 0, 0, 0, :32] = 0.0
    x[1, 0, 0, 0, :32] = np.float32(0.5) * np.arange(-16, 16, dtype=np.float32)
    if src == "bf16":
        new = [workloads.bf16_bits(x[0]), workloads.bf16_bits(x[1])]
    else:
        new = [x[0], x[1]]
    if ps == 0:
        lead = (B, H, max_ctx + n)
        pt = None
    else:
        per = (max_ctx + n + ps - 1) // ps
        pool = B * per + 3
        lead = (pool, H, ps)
        pt = rng.permutation(pool)[:B * per].reshape(B, per).astype(np.int32)
        if "bad page" in label:
            pt[0, -1] = pool + 5                          # outside the pool: skipped
    if dt == "q4":
        arrs = [rng.integers(0, 256, lead + (D // 2,), dtype=np.uint8) for _ in range(2)]
        arrs += [rng.integers(0, 2**15, lead + (D // 32,), dtype=np.uint16) for _ in range(2)]
        kinds = ["u8", "u8", "u16", "u16"]
    elif dt == "bf16":
        arrs = [rng.integers(0, 2**15, lead + (D,), dtype=np.uint16) for _ in range(2)]
        kinds = ["bf16", "bf16"]
    else:
        arrs = [rng.standard_normal(lead + (D,)).astype(np.float32) for _ in range(2)]
        kinds = ["f32", "f32"]
    dev = [dev_tensor(a, k_) for a, k_ in zip(arrs, kinds)]
    kv = sv.KVCache(k=dev[0], v=dev[1], k_scale=dev[2] if dt == "q4" else None,
                    v_scale=dev[3] if dt == "q4" else None,
                    page_table=dev_tensor(pt, "i32") if pt is not None else None)
    sv.kv_append(kv, dev_tensor(new[0], src), dev_tensor(new[1], src), dev_tensor(ctx, "i32"), max_ctx)
    torch.cuda.synchronize()
    exp = oracle.kv_append(arrs, new[0], new[1], ctx_lens=ctx, dtype=dt, src_dtype=src, max_ctx=max_ctx,
                           page_table=pt, page_size=ps)
    for e, g, k_ in zip(exp, dev, kinds):
        got = g.view(torch.int16).cpu().numpy().view(np.uint16) if k_ == "bf16" else g.cpu().numpy()
        if k_ == "u16":
            got = got.view(np.uint16)
        np.testing.assert_array_equal(got, e)


def test_verify_step_end_to_end(sv):
    """attention -> acceptance -> compaction, twice, on a paged batch."""
    cfg = _small("C5", ctx=40, ctx_hi=300, vocab=3001)
    case = workloads.make_case(cfg, seed=8, capacity_pad=8)
    dc = DeviceCase(case)
    for step in range(2):
        say(f"[step] {step}")
        arrs = dc.cache_arrays_host()
        case.k, case.v = arrs[0], arrs[1]       # the oracle reads the cache as it is now
        out, lse = dc.attn()
        acc, path, tok, am = dc.accept()
        before = dc.cache_arrays_host()
        new_lens = sv.kv_compact(dc.kv, dc.ctx, dc.max_ctx, path, acc)
        torch.cuda.synchronize()
        check_attention(case, out, lse)
        r_am, r_acc, r_path, r_tok = oracle_accept(case)
        np.testing.assert_array_equal(tok.cpu().numpy(), r_tok)
        exp, r_new, _ = oracle.compact_cache([a[None] for a in before], ctx_lens=case.ctx_lens, path=r_path,
                                             accept_len=r_acc, page_table=case.page_table,
                                             page_size=cfg.page_size)
        for e, g in zip(exp, dc.cache_arrays_host()):
            np.testing.assert_array_equal(g[None], e)
        np.testing.assert_array_equal(new_lens.cpu().numpy(), r_new)


def test_default_workspaces_are_per_stream(sv):
    """The binding's default workspaces are keyed by (kind, device, stream):
    calls on two streams never share one (a workspace serves one stream at a
    time), and each stream's results match the oracle."""
    case = workloads.make_case(_small("C3", ctx=300, vocab=3001), seed=31)
    dc = DeviceCase(case)
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for s in (s1, s2):
        with torch.cuda.stream(s):
            o, l = sv.verify_attn(dc.kv, dc.q, dc.ctx, dc.parent, dc.max_ctx)
            acc, path, tok, am = sv.greedy_accept(dc.logits, dc.drafts, dc.parent)
            outs.append((o, l, acc, path))
    torch.cuda.synchronize()
    keys = [k for k in sv._ws_cache if k[2] in (s1.cuda_stream, s2.cuda_stream)]
    assert {k[0] for k in keys} == {"attn", "accept"} and len(keys) == 4
    by = {(k[0], k[2]): sv._ws_cache[k] for k in keys}
    for kind in ("attn", "accept"):
        assert by[(kind, s1.cuda_stream)].data_ptr() != by[(kind, s2.cuda_stream)].data_ptr()
    r_am, r_acc, r_path, r_tok = oracle_accept(case)
    for o, l, acc, path in outs:
        check_attention(case, o, l)
        np.testing.assert_array_equal(acc.cpu().numpy(), r_acc)
        np.testing.assert_array_equal(path.cpu().numpy(), r_path)
