"""End-to-end pin of acceptance + compaction: greedy speculative decoding is
lossless.

The single-RTX-3090 DFlash note reports that its speculative output was
bit-identical to plain autoregressive decoding on a 40-token test (section
"Key breakthroughs", f16 intermediate cache).  Here a tiny deterministic
2-layer attention "language model" in float64 is decoded twice: plainly, one
token at a time with its own attention formula, and speculatively with trees
verified by the oracle (tree attention, argmax, acceptance walk, compaction).
The emitted tokens and the KV cache must come out the same.
"""
import numpy as np
import pytest

import oracle


class ToyLM:
    def __init__(self, seed, vocab=11, d=8, layers=2, hq=2, hkv=1, hd=8, max_pos=128):
        rng = np.random.default_rng(seed)
        self.V, self.d, self.nl, self.hq, self.hkv, self.hd = vocab, d, layers, hq, hkv, hd
        self.E = rng.standard_normal((vocab, d))
        self.P = rng.standard_normal((max_pos, d)) * 0.5
        self.Wq = rng.standard_normal((layers, d, hq * hd)) / np.sqrt(d)
        self.Wk = rng.standard_normal((layers, d, hkv * hd)) / np.sqrt(d)
        self.Wv = rng.standard_normal((layers, d, hkv * hd)) / np.sqrt(d)
        self.Wo = rng.standard_normal((layers, hq * hd, d)) / np.sqrt(hq * hd)
        self.U = rng.standard_normal((d, vocab)) * 2.0
        self.scale = 1 / np.sqrt(hd)

    def empty_cache(self, cap):
        return [np.zeros((self.nl, 1, self.hkv, cap, self.hd)) for _ in range(2)]

    # ---- plain autoregressive step (its own attention formula) ------------
    def ar_step(self, tok, pos, K, V):
        x = self.E[tok] + self.P[pos]
        g = self.hq // self.hkv
        for l in range(self.nl):
            q = (x @ self.Wq[l]).reshape(self.hq, self.hd)
            K[l, 0, :, pos] = (x @ self.Wk[l]).reshape(self.hkv, self.hd)
            V[l, 0, :, pos] = (x @ self.Wv[l]).reshape(self.hkv, self.hd)
            o = np.empty((self.hq, self.hd))
            for h in range(self.hq):
                kk = K[l, 0, h // g, :pos + 1]
                s = self.scale * kk @ q[h]
                w = np.exp(s - s.max())
                o[h] = w @ V[l, 0, h // g, :pos + 1] / w.sum()
            x = x + np.tanh(o.reshape(-1) @ self.Wo[l])
        return x @ self.U

    # ---- speculative verify of a token tree ---------------------------------
    def verify(self, toks, parent, ctx, K, V):
        n = len(toks)
        depth = np.zeros(n, int)
        for i in range(1, n):
            depth[i] = depth[parent[i]] + 1
        x = self.E[toks] + self.P[ctx + depth]
        for l in range(self.nl):
            q = (x @ self.Wq[l]).reshape(n, self.hq, self.hd)
            K[l, 0, :, ctx:ctx + n] = (x @ self.Wk[l]).reshape(n, self.hkv, self.hd).transpose(1, 0, 2)
            V[l, 0, :, ctx:ctx + n] = (x @ self.Wv[l]).reshape(n, self.hkv, self.hd).transpose(1, 0, 2)
            o, _ = oracle.verify_attention_seq(q, K[l, 0, :, :ctx + n], V[l, 0, :, :ctx + n],
                                               ctx, parent, self.scale)
            x = x + np.tanh(o.reshape(n, -1) @ self.Wo[l])
        return x @ self.U


def autoregressive(lm, prompt, n_gen, cap):
    K, V = lm.empty_cache(cap)
    out = list(prompt)
    for pos in range(len(prompt) - 1 + n_gen):
        logits = lm.ar_step(out[pos], pos, K, V)
        if pos >= len(prompt) - 1:
            out.append(oracle.argmax_first(logits))
    return out, K, V


def speculative(lm, prompt, n_gen, cap, propose):
    K, V = lm.empty_cache(cap)
    for pos in range(len(prompt) - 1):          # prefill all but the last prompt token
        lm.ar_step(prompt[pos], pos, K, V)
    out = list(prompt)
    ctx = len(prompt) - 1
    steps = 0
    while len(out) < len(prompt) + n_gen:
        parent, drafts = propose(out, steps)
        toks = np.array([out[-1]] + list(drafts[1:]))
        logits = lm.verify(toks, parent, ctx, K, V)
        am = np.array([oracle.argmax_first(r) for r in logits])
        a, path, tokens = oracle.accept_walk(am, toks, parent)
        pth = path[None]
        (K, V), new_lens, _ = oracle.compact_cache([K, V], ctx_lens=[ctx], path=pth, accept_len=[a])
        ctx = int(new_lens[0])
        out.extend(int(t) for t in tokens[:a + 1])
        steps += 1
    return out[:len(prompt) + n_gen], K, V, ctx


@pytest.mark.parametrize("mode", ["random", "perfect", "adversarial"])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_greedy_speculative_is_lossless(mode, seed):
    lm = ToyLM(seed)
    prompt = [1, 4, 2]
    n_gen = 24
    cap = 96
    ref, Kr, Vr = autoregressive(lm, prompt, n_gen, cap)
    rng = np.random.default_rng(100 + seed)

    def propose(out, step):
        if mode == "perfect":
            # a chain holding exactly the continuation the target will produce
            k = 5
            cont = ref[len(out):len(out) + k - 1]
            n = len(cont) + 1
            return np.arange(-1, n - 1), np.array([0] + cont)
        n = int(rng.integers(2, 9))
        parent = np.array([-1] + [int(rng.integers(0, i)) for i in range(1, n)])
        drafts = rng.integers(0, lm.V, size=n)
        if mode == "adversarial" and len(out) < len(ref):
            # the right next token sits on the *last* child of the root, behind
            # a wrong first child with a long subtree
            parent = np.array([-1, 0, 1, 2, 0])
            nxt = ref[len(out)]
            drafts = np.array([0, (nxt + 1) % lm.V, nxt, nxt, nxt])
        return parent, drafts

    got, Ks, Vs, ctx = speculative(lm, prompt, n_gen, cap, propose)
    assert got == ref
    # the committed cache rows equal those autoregressive decoding built (the
    # last step may have committed past the n_gen tokens the plain run made)
    rows = min(ctx, len(prompt) + n_gen - 1)
    assert rows >= len(prompt) + n_gen - 8
    np.testing.assert_allclose(Ks[..., :rows, :], Kr[..., :rows, :], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(Vs[..., :rows, :], Vr[..., :rows, :], rtol=1e-12, atol=1e-12)
