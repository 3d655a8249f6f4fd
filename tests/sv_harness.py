"""Shared helpers for the GPU tests: move a ``workloads.Case`` to the device,
run the library through its binding, compare with the oracle."""
import sys

import numpy as np
import torch

import oracle


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev_tensor(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    if dtype == "u8":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.uint8)).to(device)
    if dtype == "u16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device)
    if dtype == "i32":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(device)
    raise ValueError(dtype)


CANARY_BYTES = 4096
CANARY_BYTE = 0xA5


class Guarded:
    """A device buffer of `shape` and `dtype` followed by a band of
    CANARY_BYTES bytes set to CANARY_BYTE; `t` is the buffer (a contiguous
    view), `check` asserts the band is intact."""

    def __init__(self, shape, dtype, device, zero=False):
        n = int(np.prod(shape)) * torch.empty((), dtype=dtype).element_size()
        self.n = n
        self.raw = torch.empty(n + CANARY_BYTES, dtype=torch.uint8, device=device)
        if zero:
            self.raw[:n].zero_()
        else:
            self.raw[:n].fill_(0x7F)
        self.raw[n:].fill_(CANARY_BYTE)
        self.t = self.raw[:n].view(dtype).view(shape)

    def check(self, name, where=""):
        torch.cuda.synchronize()
        band = self.raw[self.n:]
        bad = int((band != CANARY_BYTE).sum())
        assert bad == 0, f"{where}: {bad} canary bytes after {name} were overwritten"


def sample_accept_guarded(logits, gumbel, T, drafts, parent, **kw):
    """sample_accept with every output and the zero-filled workspace followed
    by a canary band; checks the bands and that the workspace is all zeros
    again, then returns (accept_len, path, tokens, samples)."""
    import draft_token_verification_sv_amd as sv
    B, N, V = logits.shape
    dev = logits.device
    ws = Guarded((sv.greedy_accept_workspace_size(B, N, V),), torch.uint8, dev, zero=True)
    outs = [Guarded((B,), torch.int32, dev)] + [Guarded((B, N), torch.int32, dev) for _ in range(3)]
    res = sv.sample_accept(logits, gumbel, T, drafts, parent, workspace=ws.t, outputs=tuple(o.t for o in outs), **kw)
    for g, name in zip([ws] + outs, ("workspace", "accept_len", "path", "tokens", "samples")):
        g.check(name, "sample_accept")
    assert not bool(ws.t.any()), "acceptance workspace not returned to zero"
    return res


class DeviceCase:
    """Device copies of a case's arrays plus the binding's KVCache view."""

    def __init__(self, case, device="cuda"):
        import draft_token_verification_sv_amd as sv
        cfg = case.cfg
        self.case = case
        self.q = dev_tensor(case.q, cfg.q_dtype, device)
        if cfg.kv_dtype == "q4":
            self.k = dev_tensor(case.k, "u8", device)
            self.v = dev_tensor(case.v, "u8", device)
            self.ks = dev_tensor(case.k_scale, "u16", device)
            self.vs = dev_tensor(case.v_scale, "u16", device)
        else:
            self.k = dev_tensor(case.k, cfg.kv_dtype, device)
            self.v = dev_tensor(case.v, cfg.kv_dtype, device)
            self.ks = self.vs = None
        self.pt = dev_tensor(case.page_table, "i32", device) if cfg.paged else None
        self.kv = sv.KVCache(k=self.k, v=self.v, k_scale=self.ks, v_scale=self.vs, page_table=self.pt)
        self.ctx = dev_tensor(case.ctx_lens, "i32", device)
        self.parent = dev_tensor(case.parent, "i32", device)
        self.logits = dev_tensor(case.logits, cfg.logits_dtype, device)
        self.drafts = dev_tensor(case.draft_ids, "i32", device)
        self.max_ctx = int(case.ctx_lens.max())

    def attn(self, **kw):
        """verify_attn with out, lse and the workspace allocated here, each
        followed by a canary band that is checked after the call (unless the
        caller passes its own buffers)."""
        import draft_token_verification_sv_amd as sv
        if any(k in kw for k in ("out", "lse", "workspace")):
            return sv.verify_attn(self.kv, self.q, self.ctx, self.parent, self.max_ctx, **kw)
        cfg = self.case.cfg
        B, N, Hq = self.q.shape[:3]
        need = sv.verify_attn_workspace_size(self.kv, B, N, Hq, self.max_ctx, window=kw.get("window", 0),
                                             tuning=kw.get("tuning"))
        assert need > 0
        out = Guarded(tuple(self.q.shape), self.q.dtype, self.q.device)
        lse = Guarded((B, N, Hq), torch.float32, self.q.device)
        ws = Guarded((need,), torch.uint8, self.q.device)
        o, l = sv.verify_attn(self.kv, self.q, self.ctx, self.parent, self.max_ctx, out=out.t, lse=lse.t,
                              workspace=ws.t, **kw)
        for g, name in ((out, "out"), (lse, "lse"), (ws, "attention workspace")):
            g.check(name, cfg.name)
        return o, l

    def accept(self, **kw):
        """greedy_accept with a zero-filled workspace followed by a canary band
        (unless the caller passes one): the band must stay intact and the
        workspace must be all zeros again after the call."""
        import draft_token_verification_sv_amd as sv
        if "workspace" in kw:
            return sv.greedy_accept(self.logits, self.drafts, self.parent, **kw)
        B, N, V = self.logits.shape
        ws = Guarded((sv.greedy_accept_workspace_size(B, N, V),), torch.uint8, self.logits.device, zero=True)
        res = sv.greedy_accept(self.logits, self.drafts, self.parent, workspace=ws.t, **kw)
        ws.check("acceptance workspace", self.case.cfg.name)
        torch.cuda.synchronize()
        assert not bool(ws.t.any()), "acceptance workspace not returned to zero"
        return res

    def cache_arrays_host(self):
        """Host copies of the cache arrays in the storage form of the case."""
        def back(t, like):
            if t.dtype == torch.bfloat16:
                t = t.view(torch.int16)
            a = t.cpu().numpy()
            return a.view(like.dtype) if a.dtype != like.dtype else a
        arrs = [back(self.k, self.case.k), back(self.v, self.case.v)]
        if self.ks is not None:
            arrs += [back(self.ks, self.case.k_scale), back(self.vs, self.case.v_scale)]
        return arrs


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def q4_key_rounding(case, q4_kernel="cooperative"):
    """Relative rounding of a dequantised 4-bit key on the path the library
    plans for the case: fp16 (2^-11) on the cooperative kernels, four- or
    eight-wave (bf16 queries, head dim 256, >= 16 packed rows), bf16 (2^-8) on
    the other matrix-core kernels, none (fp32) on the vector-ALU kernel (< 16
    rows)."""
    cfg = case.cfg
    rows = (cfg.n_q_heads // cfg.n_kv_heads) * cfg.n_nodes
    if rows < 16:
        return 0.0
    if cfg.head_dim == 256 and q4_kernel in ("cooperative", "wide"):
        return 2.0 ** -11
    return 2.0 ** -8


def check_attention(case, out, lse, *, heads=None, batch=None, ref=None, key_rounding=None):
    """Attention gate of the case's dtype plus the supplementary diagnostics.
    Returns (max_abs, rel_fro, lse_err)."""
    cfg = case.cfg
    if ref is None:
        ref = oracle.verify_attention(case, heads=heads, batch=batch)
    ro, rl = ref
    go, gl = to_f64(out), to_f64(lse)
    sel = ~np.isnan(ro[..., 0])
    diff = np.abs(go[sel] - ro[sel])
    max_abs = float(diff.max())
    rel = float(np.linalg.norm(go[sel] - ro[sel]) / max(np.linalg.norm(ro[sel]), 1e-30))
    lse_err = float(np.abs(gl[sel] - rl[sel]).max())
    bf16 = cfg.q_dtype == "bf16" or cfg.kv_dtype != "f32"
    if cfg.q_dtype == "f32" and cfg.kv_dtype == "f32":
        assert max_abs <= 1e-4, (max_abs, cfg.name)
        assert lse_err <= 1e-5, (lse_err, cfg.name)
    else:
        assert max_abs <= 2e-2, (max_abs, cfg.name)
        lse_tol = 2e-2
        if cfg.kv_dtype == "q4" and cfg.q_dtype == "bf16":
            # the matrix-core paths round dequantised 4-bit keys (relative
            # error <= 2^-11 per value in fp16 on the cooperative head-dim-256
            # kernel, 2^-8 in bf16 on the others), so a score can move by up to
            # that times scale * sum_d |q_d k_d|; peaked rows reach scores ~30
            if key_rounding is None:
                key_rounding = q4_key_rounding(case)
            lse_tol += key_rounding * score_abs_bound(case, heads=heads, batch=batch)
        assert lse_err <= lse_tol, (lse_err, lse_tol, cfg.name)
        if bf16:
            assert rel <= 1e-2, (rel, cfg.name)
    assert np.all(np.isfinite(go[sel]))
    return max_abs, rel, lse_err


def score_abs_bound(case, heads=None, batch=None):
    """max over rows and keys of scale * sum_d |q_d| |k_d| (exact inputs)."""
    from oracle.attention import logical_rows
    from oracle.formats import widen
    cfg = case.cfg
    G = cfg.n_q_heads // cfg.n_kv_heads
    scale = 1.0 / np.sqrt(cfg.head_dim)
    lay = (lambda a: a) if case.kv_layers == 1 else (lambda a: a[0])
    best = 0.0
    for b in (range(cfg.batch) if batch is None else batch):
        L = int(case.ctx_lens[b]) + cfg.n_nodes
        qa = np.abs(widen(case.q[b], cfg.q_dtype))
        for g in range(cfg.n_kv_heads):
            hs = [h for h in range(g * G, (g + 1) * G) if heads is None or h in heads]
            if not hs:
                continue
            K = np.abs(logical_rows(lay(case.k), None if case.k_scale is None else lay(case.k_scale),
                                    b=b, head=g, length=L, dtype=cfg.kv_dtype,
                                    page_table=case.page_table if cfg.paged else None,
                                    page_size=cfg.page_size))
            for h in hs:
                best = max(best, float((qa[:, h, :] @ K.T).max()) * scale)
    return best


def oracle_accept(case):
    lg = case.logits.astype(np.float64) if case.cfg.logits_dtype == "f32" else oracle.widen_bf16(case.logits)
    return oracle.greedy_accept(lg, case.draft_ids, case.parent)
