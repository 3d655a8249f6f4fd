"""Seeded synthetic inputs for the speculative-decoding verify step.

This module is shared by the tests, the benchmark and the oracle checks.  It
builds input tensors only: it holds none of the verify step's arithmetic (no
attention, no argmax, no acceptance walk, no compaction).  Every array it
returns is a plain numpy array; floating-point tensors in bf16 are returned as
their uint16 bit patterns, fp16 scales as uint16 bit patterns.

The workload shapes follow the pages on speculative decoding:

* the full-attention layers of the Qwen3.5-27B target on the single-RTX-3090
  DFlash/DDTree note ("Why we ran this test": 24 query heads, 4 KV heads,
  head dim 256);
* a DFlash block of 16 verify rows ("Architecture": greedy verify, block 16);
* a DDTree budget of 22 ("From autoregressive to DDTree"), with a chain
  pre-seeded into the tree;
* a 4-bit KV cache at 131,072 tokens of context ("128K context in 24 GB");
* 16-token KV pages (xdnf.cn speculative-decoding notes, section 2).

Reading of the draft-token rules (the pages print no input data):

* the target token of every verify row is *planted*: the generator picks it
  and writes a value above every other draw at that index, so the row's
  maximum is known by construction.  A fraction of rows gets a second, tied
  maximum at a larger index (the lower index is then the target token);
* a chain's drafts match the target token of their parent for a seeded
  prefix and differ right after it;
* tree drafts match with a per-node probability and siblings carry distinct
  tokens.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Optional

import numpy as np

__all__ = [
    "Config", "CONFIGS", "Case", "make_case", "bf16_bits", "fp16_bits",
    "q4_encode", "chain_parent", "ddtree_parent", "drafts_from_targets",
    "small_variant", "DeltaConfig", "DELTA_CONFIGS", "DeltaCase", "make_delta_case",
]


# ----------------------------------------------------------------------------
# number formats used to *store* inputs
# ----------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (inputs only)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def fp16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> IEEE half bit patterns (numpy's round to nearest even)."""
    return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def q4_encode(x: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Write-time 4-bit quantiser for KV rows (the caller's side of the cache).

    ``x``: float32 ``[..., D]`` with D a multiple of 32.  Blocks of 32
    consecutive values share one fp16 scale ``d = fp16(max|x| / 7)``; the code
    of a value is ``clamp(rint(x / d), -8, 7) + 8`` (``8`` when d is 0).
    Returns ``codes uint8 [..., D/2]`` (value 2t in the low nibble, 2t+1 in the
    high nibble) and ``scales uint16 [..., D/32]`` (fp16 bit patterns).
    """
    x = np.asarray(x, dtype=np.float32)
    D = x.shape[-1]
    assert D % 32 == 0
    blocks = x.reshape(*x.shape[:-1], D // 32, 32)
    amax = np.abs(blocks).max(axis=-1)
    d16 = (amax / np.float32(7.0)).astype(np.float16)
    d32 = d16.astype(np.float32)
    safe = np.where(d32 == 0, np.float32(1.0), d32)
    n = np.rint(blocks / safe[..., None])
    n = np.clip(n, -8, 7) + 8
    n = np.where(d32[..., None] == 0, 8, n).astype(np.uint8)
    n = n.reshape(*x.shape[:-1], D)
    codes = (n[..., 0::2] | (n[..., 1::2] << 4)).astype(np.uint8)
    return codes, d16.view(np.uint16)


# ----------------------------------------------------------------------------
# token trees
# ----------------------------------------------------------------------------

def chain_parent(n: int) -> np.ndarray:
    p = np.arange(-1, n - 1, dtype=np.int32)
    return p


def ddtree_parent(rng: np.random.Generator, n: int, chain_len: int = 9) -> np.ndarray:
    """Nodes 1..chain_len form a chain (the pre-seeded chain); later nodes hang
    off a uniformly drawn earlier node."""
    p = np.empty(n, dtype=np.int32)
    p[0] = -1
    for i in range(1, n):
        if i <= chain_len:
            p[i] = i - 1
        else:
            p[i] = rng.integers(0, i)
    return p


def _other_token(rng, vocab, avoid):
    while True:
        t = int(rng.integers(0, vocab))
        if t not in avoid:
            return t


def drafts_from_targets(rng: np.random.Generator, parent: np.ndarray,
                        target: np.ndarray, vocab: int, match: np.ndarray,
                        distinct_siblings: bool = True) -> np.ndarray:
    """Draft ids for one sequence.

    ``target[i]`` is the token the target model picks at node i (its row
    maximum).  ``match[i]`` (i >= 1) asks node i's draft to equal its parent's
    target token; otherwise the draft is a different token.  With
    ``distinct_siblings`` no two children of one node share a token (a node
    asked to match whose parent's target token is already taken by an earlier
    sibling becomes a mismatch).  Node 0's id is the committed token and is set
    to a random token.
    """
    n = len(parent)
    d = np.empty(n, dtype=np.int32)
    d[0] = rng.integers(0, vocab)
    used: dict[int, set] = {}
    for i in range(1, n):
        p = int(parent[i])
        taken = used.setdefault(p, set()) if distinct_siblings else set()
        want = int(target[p])
        if match[i] and want not in taken:
            tok = want
        else:
            tok = _other_token(rng, vocab, taken | {want})
        d[i] = tok
        taken.add(tok)
    return d


# ----------------------------------------------------------------------------
# configurations
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class Config:
    name: str
    batch: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    n_nodes: int
    q_dtype: str            # "f32" | "bf16"
    kv_dtype: str           # "f32" | "bf16" | "q4"
    logits_dtype: str       # "f32" | "bf16"
    vocab: int
    ctx: int                # fixed context (ctx_hi == 0) or lower bound
    ctx_hi: int = 0         # > 0: ctx ~ U[ctx, ctx_hi] per sequence
    tree: str = "chain"     # "chain" | "ddtree"
    paged: bool = False
    page_size: int = 16
    q_std: float = 1.0
    kv_std: float = 1.0
    logit_std: float = 1.0
    draft_rule: str = "geometric"   # "forced" | "geometric" | "tree"
    tie_rate: float = 0.07  # fraction of rows given a second tied maximum

    @property
    def group(self) -> int:
        return self.n_q_heads // self.n_kv_heads


CONFIGS = {
    # batch 1, 2 Q / 1 KV heads, head dim 64, fp32, context 256, 4-row chain
    "C1": Config("tiny_chain_f32", 1, 2, 1, 64, 4, "f32", "f32", "f32", 1000, 256,
                 q_std=1.0, kv_std=1.0, logit_std=1.0, draft_rule="forced"),
    # 24/4 heads, head dim 256, bf16, 4096 cached tokens, 8-row chain
    "C2": Config("chain_gqa_4k", 1, 24, 4, 256, 8, "bf16", "bf16", "bf16", 151936, 4096,
                 q_std=0.5, kv_std=0.5, logit_std=float(np.sqrt(2.0))),
    # DDTree of 22 nodes (root included) over 32768 cached tokens
    "C3": Config("ddtree_32k", 1, 24, 4, 256, 22, "bf16", "bf16", "bf16", 151936, 32768,
                 tree="ddtree", q_std=0.5, kv_std=0.5, logit_std=float(np.sqrt(2.0)),
                 draft_rule="tree"),
    # 16-row block over a 4-bit cache of 131072 tokens
    "C4": Config("block16_q4_128k", 1, 24, 4, 256, 16, "bf16", "q4", "bf16", 151936, 131072,
                 q_std=1.0, kv_std=1.0, logit_std=float(np.sqrt(2.0))),
    # 8 sequences, ctx ~ U[1024, 16384], 16-token pages, 32/8 heads, dim 128, 4-row chains
    "C5": Config("paged_batch8", 8, 32, 8, 128, 4, "bf16", "bf16", "bf16", 151936, 1024,
                 ctx_hi=16384, paged=True, q_std=0.5, kv_std=0.5,
                 logit_std=float(np.sqrt(2.0))),
}


def small_variant(cfg: Config, *, ctx: int = 333, ctx_hi: int = 0, vocab: int = 5003,
                  n_nodes: Optional[int] = None, batch: Optional[int] = None) -> Config:
    """The same heads / dtypes / layout at a context and vocabulary the oracle
    finishes in well under a second (still several KV tiles plus a ragged
    tail)."""
    kw = dict(ctx=ctx, ctx_hi=ctx_hi, vocab=vocab)
    if n_nodes is not None:
        kw["n_nodes"] = n_nodes
    if batch is not None:
        kw["batch"] = batch
    return dataclasses.replace(cfg, **kw)


# ----------------------------------------------------------------------------
# cases
# ----------------------------------------------------------------------------

@dataclass
class Case:
    cfg: Config
    seed: int
    ctx_lens: np.ndarray          # int32 [B]
    capacity: int                 # contiguous: positions per (seq, head); paged: pool pages
    q: np.ndarray                 # [B][N][Hq][D]  float32 or uint16 (bf16 bits)
    k: np.ndarray                 # contiguous [B][Hkv][cap][D(/2)], paged [P][Hkv][ps][D(/2)]
    v: np.ndarray
    k_scale: Optional[np.ndarray]  # q4: uint16 fp16 bits [...][D/32]
    v_scale: Optional[np.ndarray]
    page_table: Optional[np.ndarray]  # int32 [B][max_pages] (-1 = unused)
    parent: np.ndarray            # int32 [B][N]
    logits: np.ndarray            # [B][N][V] float32 or uint16 (bf16 bits)
    draft_ids: np.ndarray         # int32 [B][N]
    target: np.ndarray            # int32 [B][N]: planted row maxima (lowest index)
    kv_layers: int = 1

    @property
    def max_ctx(self) -> int:
        return int(self.ctx_lens.max())


def _normal(rng, shape, std):
    return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std))


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "bf16":
        return bf16_bits(x32)
    raise ValueError(dtype)


def _plant_logits(rng, B, N, V, std, dtype, tie_rate):
    """Row values ~ N(0, std^2), clipped to +-7.5 std, then the target token gets
    value 8 std (rounded to the storage type) so it is the row maximum."""
    top = float(8.0 * std)
    x = _normal(rng, (B, N, V), std)
    np.clip(x, -7.5 * std, 7.5 * std, out=x)
    target = np.empty((B, N), dtype=np.int32)
    for b in range(B):
        for i in range(N):
            t = int(rng.integers(0, V))
            if V > 1 and rng.random() < tie_rate:
                t2 = int(rng.integers(0, V - 1))
                t2 = t2 + 1 if t2 >= t else t2
                x[b, i, t2] = top
                t = min(t, t2)
            x[b, i, t] = top
            target[b, i] = t
    return _store(x, dtype), target


def make_case(cfg: Config, seed: int, *, variant: str = "", capacity_pad: int = 0,
              n_layers: int = 1, force_first_mismatch: bool = False) -> Case:
    """Build one seeded input set for ``cfg``.

    ``variant``: "" (plain), "peaked" (each draft row's key is set to 2x the
    query of that node's first group head, so the tree mask decides an O(1)
    part of each output), "perfect" (every draft matches).
    ``capacity_pad``: extra cache positions past ctx+N (contiguous layout) or
    spare pages (paged layout) that the verify step must leave untouched.
    ``n_layers``: cache layers (the compaction walks all of them; attention
    reads layer 0).
    """
    rng = np.random.default_rng(seed)
    B, N, Hq, Hkv, D, V = cfg.batch, cfg.n_nodes, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.vocab
    G = Hq // Hkv
    if cfg.ctx_hi > 0:
        ctx = rng.integers(cfg.ctx, cfg.ctx_hi + 1, size=B).astype(np.int32)
    else:
        ctx = np.full(B, cfg.ctx, dtype=np.int32)

    q32 = _normal(rng, (B, N, Hq, D), cfg.q_std)
    q = _store(q32, cfg.q_dtype)

    if cfg.tree == "ddtree":
        parent = np.stack([ddtree_parent(rng, N) for _ in range(B)])
    else:
        parent = np.stack([chain_parent(N) for _ in range(B)])

    # --- KV storage --------------------------------------------------------
    L = ctx + N
    page_table = None
    if cfg.paged:
        ps = cfg.page_size
        need = (L + ps - 1) // ps
        spare = max(int(np.ceil(0.1 * need.sum())), capacity_pad)
        n_pages = int(need.sum()) + spare
        perm = rng.permutation(n_pages).astype(np.int32)
        max_pages = int(need.max())
        page_table = np.full((B, max_pages), -1, dtype=np.int32)
        off = 0
        for b in range(B):
            page_table[b, :need[b]] = perm[off:off + need[b]]
            off += need[b]
        shape = (n_pages, Hkv, ps, D)
        capacity = n_pages
    else:
        capacity = int(L.max()) + capacity_pad
        shape = (B, Hkv, capacity, D)

    def draw_kv():
        # one layer of K or V in storage form; drawn per leading index to bound
        # host memory for the 128K configuration
        if cfg.kv_dtype == "q4":
            codes = np.empty(shape[:-1] + (D // 2,), np.uint8)
            scales = np.empty(shape[:-1] + (D // 32,), np.uint16)
            for i in range(shape[0]):
                for h in range(shape[1]):
                    c, s = q4_encode(_normal(rng, shape[2:], cfg.kv_std))
                    codes[i, h], scales[i, h] = c, s
            return codes, scales
        out = np.empty(shape, np.float32 if cfg.kv_dtype == "f32" else np.uint16)
        for i in range(shape[0]):
            out[i] = _store(_normal(rng, shape[1:], cfg.kv_std), cfg.kv_dtype)
        return out, None

    ks, vs, kss, vss = [], [], [], []
    for _ in range(n_layers):
        k, k_s = draw_kv()
        v, v_s = draw_kv()
        ks.append(k); vs.append(v); kss.append(k_s); vss.append(v_s)

    if variant == "peaked":
        # key of draft row m := 2 * q[node m, first head of the group]
        for b in range(B):
            for m in range(N):
                pos = int(ctx[b]) + m
                for h in range(Hkv):
                    qv = q32[b, m, h * G] * np.float32(2.0)
                    if cfg.paged:
                        pg = page_table[b, pos // cfg.page_size]
                        idx = (pg, h, pos % cfg.page_size)
                    else:
                        idx = (b, h, pos)
                    if cfg.kv_dtype == "q4":
                        c, s = q4_encode(qv[None])
                        ks[0][idx] = c[0]
                        kss[0][idx] = s[0]
                    else:
                        ks[0][idx] = _store(qv[None], cfg.kv_dtype)[0]

    stack = (lambda a: a[0]) if n_layers == 1 else (lambda a: np.stack(a))
    k_all, v_all = stack(ks), stack(vs)
    k_sc = stack(kss) if cfg.kv_dtype == "q4" else None
    v_sc = stack(vss) if cfg.kv_dtype == "q4" else None

    # --- logits and drafts ---------------------------------------------------
    logits, target = _plant_logits(rng, B, N, V, cfg.logit_std, cfg.logits_dtype, cfg.tie_rate)
    drafts = np.empty((B, N), dtype=np.int32)
    for b in range(B):
        match = np.zeros(N, dtype=bool)
        if variant == "perfect":
            match[1:] = True
        elif cfg.draft_rule == "forced":
            # p ~ U{0..4} leading correct drafts, clamped to N-1
            p = min(int(rng.integers(0, 5)), N - 1)
            match[1:p + 1] = True
        elif cfg.draft_rule == "geometric":
            # prefix length: failures before the first success, p = 0.3
            ln = min(N - 1, int(rng.geometric(0.3)) - 1)
            match[1:ln + 1] = True
        elif cfg.draft_rule == "tree":
            for i in range(1, N):
                on_chain = (i <= 9)
                match[i] = rng.random() < (0.9 if on_chain else 0.5)
        if force_first_mismatch and N > 1:
            match[1] = False
        drafts[b] = drafts_from_targets(rng, parent[b], target[b], V, match)

    return Case(cfg=cfg, seed=seed, ctx_lens=ctx, capacity=capacity, q=q,
                k=k_all, v=v_all, k_scale=k_sc, v_scale=v_sc, page_table=page_table,
                parent=parent.astype(np.int32), logits=logits, draft_ids=drafts,
                target=target, kv_layers=n_layers)


# ----------------------------------------------------------------------------
# recurrent (Gated DeltaNet) layers of the hybrid target
# ----------------------------------------------------------------------------
#
# The single-RTX-3090 note's target has 48 Gated DeltaNet layers of 64 ("Why
# we ran this test") but gives no sizes for them.  The sizes assumed here: 16
# key heads and 48 value heads of dimension 128, a conv of width 4 over the q,
# k and v channels (2 * 16 * 128 + 48 * 128 = 10240 channels).
# Input recipe: conv inputs and conv state ~ N(0, 1); conv weights
# ~ N(0, 0.5^2), bias ~ N(0, 0.1^2); q and k rows unit-length (normal draws
# divided by their norm, as the layer normalises them before the recurrence);
# v ~ N(0, 1); log decay g ~ -U(0.02, 2) (decay exp(g) in (0.14, 0.98));
# beta ~ U(0.05, 1); committed state entries ~ N(0, 0.1^2).

@dataclass(frozen=True)
class DeltaConfig:
    name: str
    batch: int
    n_nodes: int
    n_k_heads: int
    n_v_heads: int
    k_dim: int
    v_dim: int
    conv_width: int
    dtype: str              # "f32" | "bf16": q, k, v, conv inputs, conv state, outputs
    state_dtype: str        # "f32" | "f16": the per-node states as stored
    tree: str = "chain"     # "chain" | "ddtree"

    @property
    def channels(self) -> int:
        return 2 * self.n_k_heads * self.k_dim + self.n_v_heads * self.v_dim


DELTA_CONFIGS = {
    # tiny fp32 chain (fast on the oracle)
    "D1": DeltaConfig("deltanet_tiny_f32", 1, 4, 1, 2, 64, 64, 4, "f32", "f32"),
    # the DDTree budget-22 tree of the attention configuration, one sequence
    "D2": DeltaConfig("deltanet_ddtree22", 1, 22, 16, 48, 128, 128, 4, "bf16", "f16", tree="ddtree"),
    # a DFlash block of 16 rows
    "D3": DeltaConfig("deltanet_block16", 1, 16, 16, 48, 128, 128, 4, "bf16", "f16"),
    # 8 sequences, 4-row chains each
    "D4": DeltaConfig("deltanet_batch8", 8, 4, 16, 48, 128, 128, 4, "bf16", "f16"),
}


@dataclass
class DeltaCase:
    cfg: DeltaConfig
    seed: int
    parent: np.ndarray        # int32 [B][N]
    x: np.ndarray             # [B][N][C]       conv inputs (float32 or bf16 bits)
    conv_state: np.ndarray    # [B][K-1][C]     committed conv inputs, oldest first
    conv_weight: np.ndarray   # float32 [C][K]  (tap K-1 on the token itself)
    conv_bias: np.ndarray     # float32 [C]
    q: np.ndarray             # [B][N][Hk][Dk]
    k: np.ndarray             # [B][N][Hk][Dk]
    v: np.ndarray             # [B][N][Hv][Dv]
    g: np.ndarray             # float32 [B][N][Hv]  log decay
    beta: np.ndarray          # float32 [B][N][Hv]
    state: np.ndarray         # float32 [B][Hv][Dv][Dk]
    accept_len: np.ndarray    # int32 [B]  depth of the accepted node
    path: np.ndarray          # int32 [B][N] its root path, then -1


def _unit_rows(rng, shape):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    return (x / np.sqrt((x * x).sum(axis=-1, keepdims=True))).astype(np.float32)


def make_delta_case(cfg: DeltaConfig, seed: int) -> DeltaCase:
    rng = np.random.default_rng(seed)
    B, N, Hk, Hv, Dk, Dv, K = (cfg.batch, cfg.n_nodes, cfg.n_k_heads, cfg.n_v_heads,
                               cfg.k_dim, cfg.v_dim, cfg.conv_width)
    C = cfg.channels
    if cfg.tree == "ddtree":
        parent = np.stack([ddtree_parent(rng, N) for _ in range(B)])
    else:
        parent = np.stack([chain_parent(N) for _ in range(B)])
    x = _store(_normal(rng, (B, N, C), 1.0), cfg.dtype)
    conv_state = _store(_normal(rng, (B, K - 1, C), 1.0), cfg.dtype)
    w = _normal(rng, (C, K), 0.5)
    bias = _normal(rng, (C,), 0.1)
    q = _store(_unit_rows(rng, (B, N, Hk, Dk)), cfg.dtype)
    k = _store(_unit_rows(rng, (B, N, Hk, Dk)), cfg.dtype)
    v = _store(_normal(rng, (B, N, Hv, Dv), 1.0), cfg.dtype)
    g = (-rng.uniform(0.02, 2.0, size=(B, N, Hv))).astype(np.float32)
    beta = rng.uniform(0.05, 1.0, size=(B, N, Hv)).astype(np.float32)
    state = _normal(rng, (B, Hv, Dv, Dk), 0.1)
    # an accepted node per sequence (its parent chain is the accepted path)
    accept_len = np.empty(B, dtype=np.int32)
    path = np.full((B, N), -1, dtype=np.int32)
    for b in range(B):
        node = int(rng.integers(0, N))
        chain = [node]
        while parent[b, chain[-1]] >= 0:
            chain.append(int(parent[b, chain[-1]]))
        chain.reverse()
        accept_len[b] = len(chain) - 1
        path[b, :len(chain)] = chain
    return DeltaCase(cfg=cfg, seed=seed, parent=parent.astype(np.int32), x=x, conv_state=conv_state,
                     conv_weight=w, conv_bias=bias, q=q, k=k, v=v, g=g, beta=beta, state=state,
                     accept_len=accept_len, path=path)
