"""Benchmark of one verify step on one MI355X.

A step is the whole verify path for one layer over one batch of seeded
synthetic inputs already resident in HBM: ``sv_verify_attn`` (tree/chain
masked GQA attention over the KV cache), then ``sv_greedy_accept_compact``
(vocab argmax + acceptance walk, then in-place KV compaction of the accepted
rows, in one launch; the separate ``sv_greedy_accept`` / ``sv_kv_compact``
calls are timed too, in ``breakdown_us``).  Inputs rotate over enough device
copies (>= 1 GiB) that the 256 MB Infinity Cache cannot serve the KV cache
from one step to the next.

Prints one JSON line for the headline workload (default: the 16-row block
over the 131072-token 4-bit cache, the largest single-GPU workload) with the
other workloads' results nested under ``per_config``.  ``value`` is verified
draft tokens per second (sum over sequences of N - 1 draft rows, per step
time).  ``ms_per_step`` is the mean over a HIP-graph replay of ``steps``
steps; ``step_us`` and the roofline's ``call_us`` give the median / p10 / p90
of per-call HIP-event durations over the same number of eager calls queued
behind a spin kernel (so the host never starves the queue).  ``roofline``
reports the verify-attention call (split kernel + merge kernel) against the
roof that binds it: HBM (8 TB/s) for the algorithmic bytes (every KV row of
the key range read once, plus q, out and lse), or the dense fp16/bf16 matrix
peak (2.5 PFLOP/s) for the algorithmic flops (4 * rows * keys * head_dim per
(sequence, KV head)) when those take longer at peak; both fractions are
given.  ``cpu_baseline`` times the fp64 CPU oracle on a bounded sample of
the same workload, once with every host core and once with one.
"""
import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MFMA_PEAK_TFLOPS = 2500.0       # dense bf16 / fp16 matrix peak of MI355X
METRIC = "verified draft tokens/s per verify step + achieved HBM GB/s (% of MI355X peak)"
WORKLOADS = {"C1": "C1", "C2": "C2", "C3": "C3", "C4": "C4", "C5": "C5"}
DEFAULT_CONFIG = "C4"        # 16-row block, GQA 24/4, head dim 256, 131072 cached tokens in 4 bits


def kv_bytes_per_position(cfg):
    D = cfg.head_dim
    if cfg.kv_dtype == "f32":
        return 2 * D * 4
    if cfg.kv_dtype == "bf16":
        return 2 * D * 2
    return 2 * (D // 2 + (D // 32) * 2)          # 4-bit codes + fp16 scales, K and V


def attn_algorithmic_bytes(cfg, ctx_lens, window=0):
    qb = 4 if cfg.q_dtype == "f32" else 2
    lens = ctx_lens + cfg.n_nodes
    if window:
        lens = np.minimum(lens, window)
    rows = int(np.sum(lens))
    kv = rows * cfg.n_kv_heads * kv_bytes_per_position(cfg)
    q_out = 2 * cfg.batch * cfg.n_nodes * cfg.n_q_heads * cfg.head_dim * qb
    lse = cfg.batch * cfg.n_nodes * cfg.n_q_heads * 4
    return kv + q_out + lse


def attn_algorithmic_flops(cfg, ctx_lens, window=0):
    """Q K^T and P V over every (row, key) pair of the key range: 4 * D flops
    per pair, rows = G * N per (sequence, KV head)."""
    lens = ctx_lens + cfg.n_nodes
    if window:
        lens = np.minimum(lens, window)
    return 4.0 * cfg.n_q_heads * cfg.n_nodes * cfg.head_dim * float(np.sum(lens))


def uses_matrix_cores(cfg):
    return cfg.q_dtype == "bf16" and cfg.kv_dtype in ("bf16", "q4") and cfg.group * cfg.n_nodes >= 16


def source_hash():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "draft_token_verification_sv_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def committed_counters(workload):
    """The committed rocprofv3 counter summary of the workload's dominant call
    (attention, or the tree recurrence), if it was taken on the current kernel
    sources: HBM bytes per call and matrix-core busy fraction."""
    path = os.path.join(ROOT, "profiles", "attn_traffic.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        data = json.load(f)
    ent = data.get(workload)
    if not ent or ent.get("source_hash") != source_hash():
        return {}
    return ent


def measured_traffic(workload, per_launch_bytes=None):
    return committed_counters(workload).get("bytes_per_call")


def _blas_threads():
    """Threads numpy's BLAS may use (the oracle's only parallel part)."""
    try:
        from threadpoolctl import threadpool_info
        return int(max([i.get("num_threads", 1) for i in threadpool_info()] or [1]))
    except Exception:
        return int(os.environ.get("OMP_NUM_THREADS", "1"))


def cpu_baseline(cfg_key, seconds, one_core=False):
    """The oracle (unchanged) on a sample of the same workload: whole verify
    steps (at least one) on the host cores, repeated for about `seconds`;
    `one_core` limits numpy's BLAS (the oracle's only parallel part) to one
    thread."""
    import contextlib
    import oracle
    import workloads
    cfg = workloads.CONFIGS[cfg_key]
    case = workloads.make_case(cfg, seed=1)
    lg = case.logits.astype(np.float64) if cfg.logits_dtype == "f32" else oracle.widen_bf16(case.logits)
    try:
        from threadpoolctl import threadpool_limits
        limit = threadpool_limits(1) if one_core else contextlib.nullcontext()
    except Exception:
        limit = contextlib.nullcontext()
    steps = 0
    with limit:
        threads = 1 if one_core else _blas_threads()
        t0 = time.perf_counter()
        while True:
            oracle.verify_attention(case)
            am, acc, path, tok = oracle.greedy_accept(lg, case.draft_ids, case.parent)
            arrs = [case.k[None], case.v[None]]
            if case.k_scale is not None:
                arrs += [case.k_scale[None], case.v_scale[None]]
            oracle.compact_cache(arrs, ctx_lens=case.ctx_lens, path=path, accept_len=acc,
                                 page_table=case.page_table if cfg.paged else None, page_size=cfg.page_size)
            steps += 1
            if time.perf_counter() - t0 >= seconds:
                break
        dt = time.perf_counter() - t0
    drafts = cfg.batch * (cfg.n_nodes - 1)
    return {"value": drafts * steps / dt, "unit": "verified draft tokens/s", "cores": threads,
            "host_cpus": len(os.sched_getaffinity(0)), "kind": "oracle",
            "sample": f"{steps} whole verify steps of the {cfg.name} workload (attention, argmax + walk, "
                      f"compaction) in {dt:.1f} s, fp64 numpy, {threads} BLAS thread(s)"}


def recurrent_cpu_baseline(key, seconds):
    """The oracle (unchanged) on a sample of the recurrent workload: the tree
    conv, the tree recurrence and the commit of one layer over the first value
    heads (a key head's worth at a time), repeated for about `seconds`; the
    time is scaled to all heads."""
    import oracle
    import workloads
    cfg = workloads.DELTA_CONFIGS[key]
    c = workloads.make_delta_case(cfg, seed=2)
    f64 = (lambda a: oracle.widen_bf16(a)) if cfg.dtype == "bf16" else (lambda a: np.asarray(a, np.float64))
    rep = cfg.n_v_heads // cfg.n_k_heads
    q, k, v = f64(c.q)[:, :, :1], f64(c.k)[:, :, :1], f64(c.v)[:, :, :rep]
    par = c.parent if cfg.tree != "chain" else None
    x, cs = f64(c.x), f64(c.conv_state)
    t0 = time.perf_counter()
    oracle.conv_tree(x, cs, c.conv_weight, c.conv_bias, par)           # every channel, once
    t_conv = time.perf_counter() - t0
    calls = 0
    t0 = time.perf_counter()
    while True:
        o, st = oracle.delta_net_tree(q, k, v, c.g[:, :, :rep], c.beta[:, :, :rep], c.state[:, :rep], par)
        oracle.recurrent_commit(st, c.state[:, :rep], c.x, c.conv_state, c.path, c.accept_len)
        calls += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    per_call = t_conv + dt / calls * (cfg.n_v_heads / rep)
    return {"value": round(per_call * 1e6, 1), "unit": "us per layer call (conv + tree recurrence + commit)",
            "cores": _blas_threads(), "kind": "oracle",
            "sample": f"the conv over all channels once ({t_conv * 1e3:.1f} ms), then {calls} tree recurrences + "
                      f"commits on {rep} of {cfg.n_v_heads} value heads in {dt:.1f} s, scaled x{cfg.n_v_heads // rep} "
                      f"to all heads; fp64 numpy"}


def delta_algorithmic_bytes(cfg):
    """Bytes one sv_gated_delta_net_tree call must move: the committed state read,
    q, k, v, decay and beta read once, every node's state and output written."""
    B, N, Hk, Hv, Dk, Dv = cfg.batch, cfg.n_nodes, cfg.n_k_heads, cfg.n_v_heads, cfg.k_dim, cfg.v_dim
    e = 2 if cfg.dtype == "bf16" else 4
    se = 2 if cfg.state_dtype == "f16" else 4
    return (B * Hv * Dv * Dk * 4 + B * N * (2 * Hk * Dk + Hv * Dv) * e + B * N * Hv * 8
            + B * N * Hv * Dv * e + B * N * Hv * Dv * Dk * se)


def recurrent_bench(sv, dev, key, steps, rotate_bytes, capture, timed):
    """Times the tree-aware recurrent state calls of one Gated DeltaNet layer
    (conv, tree recurrence with every node's state persisted, commit) with the
    committed and per-node states rotated over >= rotate_bytes of HBM."""
    import torch
    import workloads
    cfg = workloads.DELTA_CONFIGS[key]
    c = workloads.make_delta_case(cfg, seed=2)
    B, N, Hv, Dk, Dv = cfg.batch, cfg.n_nodes, cfg.n_v_heads, cfg.k_dim, cfg.v_dim

    def up(x, kind):
        x = np.ascontiguousarray(x)
        if kind == "bf16":
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(x).to(dev)

    kind = cfg.dtype
    x, cs = up(c.x, kind), up(c.conv_state, kind)
    w, bias = up(c.conv_weight, "f32"), up(c.conv_bias, "f32")
    q, k, v = up(c.q, kind), up(c.k, kind), up(c.v, kind)
    g, beta = up(c.g, "f32"), up(c.beta, "f32")
    parent = up(c.parent, "i32") if cfg.tree != "chain" else None
    path, alen = up(c.path, "i32"), up(c.accept_len, "i32")
    sdt = torch.float16 if cfg.state_dtype == "f16" else torch.float32
    state0 = up(c.state, "f32")
    per = state0.numel() * 4 + B * N * Hv * Dv * Dk * (2 if sdt == torch.float16 else 4)
    n_rot = max(1, int(np.ceil(rotate_bytes / per)))
    states = [state0] + [state0.clone() for _ in range(n_rot - 1)]
    nodes = [torch.empty((B, N, Hv, Dv, Dk), dtype=sdt, device=dev) for _ in range(n_rot)]
    conv_out = torch.empty_like(x)
    d_out = torch.empty((B, N, Hv, Dv), dtype=q.dtype, device=dev)
    cs_c = cs.clone()

    def conv(i):
        sv.ssm_conv_tree(x, cs, w, bias, parent, activation="silu", out=conv_out)

    # the visiting order is computed once per verify step and shared by every
    # recurrent layer (timed separately)
    sched = sv.tree_schedule(parent) if parent is not None else None

    def schedule(i):
        sv.tree_schedule(parent, out=sched)

    def delta(i):
        sv.gated_delta_net_tree(q, k, v, g, beta, states[i % n_rot], parent, out=d_out, state_nodes=nodes[i % n_rot],
                                schedule=sched)

    def commit(i):
        sv.recurrent_commit(nodes[i % n_rot], states[(i + 1) % n_rot], x, cs_c, path, alen)

    for i in range(3):
        conv(i), delta(i), commit(i)
    torch.cuda.synchronize()
    conv_us = timed(capture(conv)) / steps * 1e3
    delta_us = timed(capture(delta)) / steps * 1e3
    commit_us = timed(capture(commit)) / steps * 1e3
    sched_us = timed(capture(schedule)) / steps * 1e3 if parent is not None else 0.0
    nbytes = delta_algorithmic_bytes(cfg)
    achieved = nbytes / (delta_us * 1e-6) / 1e9
    return {
        "workload": f"{cfg.name}: batch {B}, {N} rows ({cfg.tree}), {cfg.n_k_heads} key / {Hv} value heads, "
                    f"dims {Dk}/{Dv}, conv width {cfg.conv_width}, {cfg.dtype} inputs, {cfg.state_dtype} node states",
        "breakdown_us": {"ssm_conv_tree": round(conv_us, 2), "gated_delta_net_tree": round(delta_us, 2),
                         "recurrent_commit": round(commit_us, 2),
                         "tree_schedule (once per verify step, shared by the layers)": round(sched_us, 2)},
        "rotation_copies": n_rot,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": measured_traffic(cfg.name, nbytes),
                     "kernel": "sv_gated_delta_net_tree", "algorithmic_bytes": int(nbytes)},
    }


def _pcts(us):
    a = np.asarray(us, dtype=np.float64)
    return {"median": round(float(np.median(a)), 2), "p10": round(float(np.percentile(a, 10)), 2),
            "p90": round(float(np.percentile(a, 90)), 2), "n": int(a.size)}


def run_workload(sv, dev, key, args, steps, full):
    """Times one workload: the step (attention + fused acceptance/compaction)
    and the attention call from HIP-graph replays of `steps` calls, their
    per-call distributions from HIP events, and (full) every other call of the
    verify path for the breakdown.  Returns the workload's record."""
    import torch
    import workloads
    cfg = workloads.CONFIGS[key]
    case = workloads.make_case(cfg, seed=1)
    tuning = {}
    if args.target_wgs:
        tuning["attn_target_wgs"] = args.target_wgs
    if args.attn_q4_kernel != "default":
        tuning["attn_q4_kernel"] = args.attn_q4_kernel
    tuning = tuning or None
    window = args.window

    def up(x, kind):
        x = np.ascontiguousarray(x)
        if kind == "bf16":
            return torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
        if kind == "u16":
            return torch.from_numpy(x.view(np.int16)).to(dev)
        return torch.from_numpy(x).to(dev)

    qk = "bf16" if cfg.q_dtype == "bf16" else "f32"
    base = {"q": up(case.q, qk), "logits": up(case.logits, "bf16" if cfg.logits_dtype == "bf16" else "f32")}
    if cfg.kv_dtype == "q4":
        base.update(k=up(case.k, "u8"), v=up(case.v, "u8"), ks=up(case.k_scale, "u16"), vs=up(case.v_scale, "u16"))
    else:
        kk = "bf16" if cfg.kv_dtype == "bf16" else "f32"
        base.update(k=up(case.k, kk), v=up(case.v, kk))
    ctx = up(case.ctx_lens.astype(np.int32), "i32")
    parent = up(case.parent.astype(np.int32), "i32")
    drafts = up(case.draft_ids.astype(np.int32), "i32")
    pt = up(case.page_table.astype(np.int32), "i32") if cfg.paged else None
    max_ctx = int(case.ctx_lens.max())
    per_copy = sum(t.numel() * t.element_size() for t in base.values())
    n_copies = max(1, int(np.ceil(args.rotate_bytes / per_copy)))
    copies = [base] + [{k: t.clone() for k, t in base.items()} for _ in range(n_copies - 1)]

    B, N, Hq, D = cfg.batch, cfg.n_nodes, cfg.n_q_heads, cfg.head_dim
    kvs = [sv.KVCache(k=c["k"], v=c["v"], k_scale=c.get("ks"), v_scale=c.get("vs"), page_table=pt)
           for c in copies]
    outs = [torch.empty_like(base["q"]) for _ in range(2)]
    lse = torch.empty((B, N, Hq), dtype=torch.float32, device=dev)
    acc = torch.empty(B, dtype=torch.int32, device=dev)
    path = torch.empty((B, N), dtype=torch.int32, device=dev)
    tok = torch.empty((B, N), dtype=torch.int32, device=dev)
    new_lens = torch.empty(B, dtype=torch.int32, device=dev)
    ws_a = torch.empty(sv.verify_attn_workspace_size(kvs[0], B, N, Hq, max_ctx, window=window, tuning=tuning),
                       dtype=torch.uint8, device=dev)
    ws_g = torch.zeros(sv.greedy_accept_workspace_size(B, N, cfg.vocab), dtype=torch.uint8, device=dev)

    def attn(i):
        c, kv = copies[i % n_copies], kvs[i % n_copies]
        sv.verify_attn(kv, c["q"], ctx, parent, max_ctx, out=outs[i & 1], lse=lse, workspace=ws_a,
                       window=window, tuning=tuning)

    def accept(i):
        sv.greedy_accept(copies[i % n_copies]["logits"], drafts, parent, workspace=ws_g,
                         outputs=(acc, path, tok, None))

    def compact(i):
        sv.kv_compact(kvs[i % n_copies], ctx, max_ctx, path, acc, new_lens=new_lens)

    def accept_compact(i):
        sv.greedy_accept_compact(copies[i % n_copies]["logits"], drafts, parent, kvs[i % n_copies], ctx, max_ctx,
                                 workspace=ws_g, outputs=(acc, path, tok, None), new_lens=new_lens)

    # one verify step: attention, then acceptance and compaction in one launch
    def step(i):
        attn(i)
        accept_compact(i)

    # warm-up: eager steps (first launches, code objects, caches)
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # The timed work is replayed from HIP graphs (the launch path a serving
    # loop uses); each graph holds exactly `steps` consecutive calls over the
    # rotation.  Events are recorded on the stream the calls go to.
    def capture(fn):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                fn(args.warmup + i)
        torch.cuda.synchronize()
        return g

    def timed(g):
        s = torch.cuda.current_stream(dev)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        g.replay()                       # untimed replay (graph upload)
        torch.cuda.synchronize()
        e0.record(s)
        g.replay()
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1)

    def per_call(fns):
        """HIP-event durations of each call of `fns` over `steps` eager
        rounds.  A spin kernel goes first so that every call is queued before
        the first one starts (the host never starves the queue; `queued`
        says whether that held)."""
        s = torch.cuda.current_stream(dev)
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(fns) + 1)] for _ in range(steps)]
        torch.cuda.synchronize()
        torch.cuda._sleep(int(args.spin_cycles))
        for i in range(steps):
            for j, fn in enumerate(fns):
                ev[i][j].record(s)
                fn(args.warmup + steps + i)
            ev[i][-1].record(s)
        queued = not ev[0][0].query()
        torch.cuda.synchronize()
        return [[ev[i][j].elapsed_time(ev[i][j + 1]) * 1e3 for i in range(steps)] for j in range(len(fns))], queued

    total_ms = timed(capture(step))
    attn_total_ms = timed(capture(attn))
    (attn_calls, ac_calls), queued = per_call([attn, accept_compact])
    step_calls = [a + b for a, b in zip(attn_calls, ac_calls)]

    ms_per_step = total_ms / steps
    value = B * (N - 1) / (ms_per_step / 1e3)
    attn_us = attn_total_ms / steps * 1e3
    nbytes = attn_algorithmic_bytes(cfg, case.ctx_lens, window)
    flops = attn_algorithmic_flops(cfg, case.ctx_lens, window)
    gbps = nbytes / (attn_us * 1e-6) / 1e9
    tflops = flops / (attn_us * 1e-6) / 1e12
    hbm = {"achieved": round(gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s", "frac": round(gbps / HBM_PEAK_GBPS, 4),
           "algorithmic_bytes": int(nbytes)}
    mfma = {"achieved": round(tflops, 1), "peak": MFMA_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / MFMA_PEAK_TFLOPS, 4), "algorithmic_flops": flops}
    # the binding roof: the one whose peak takes longer for this call's work
    mfma_bound = uses_matrix_cores(cfg) and flops / (MFMA_PEAK_TFLOPS * 1e12) > nbytes / (HBM_PEAK_GBPS * 1e9)
    roof = dict(mfma if mfma_bound else hbm)
    roof = {"bound": "mfma" if mfma_bound else "hbm", **roof}
    counters = {} if window else committed_counters(cfg.name)
    roof["traffic"] = counters.get("bytes_per_call")
    roof["kernel"] = "sv_verify_attn (split + merge kernels)"
    roof["call_us"] = {"mean": round(attn_us, 2), **_pcts(attn_calls)}
    roof["hbm"] = hbm
    if uses_matrix_cores(cfg):
        roof["mfma"] = dict(mfma, busy_frac_counters=counters.get("mfma_busy_frac"))
    rec = {
        "value": round(value, 1),
        "ms_per_step": round(ms_per_step, 5),
        "step_us": _pcts(step_calls),
        "events_queued_ahead": bool(queued),
        "config": {"workload": cfg.name, "batch": B, "n_q_heads": Hq, "n_kv_heads": cfg.n_kv_heads,
                   "head_dim": D, "n_nodes": N, "tree": cfg.tree, "kv": cfg.kv_dtype,
                   "kv_layout": "paged16" if cfg.paged else "contiguous",
                   "ctx": int(cfg.ctx) if not cfg.ctx_hi else [int(cfg.ctx), int(cfg.ctx_hi)],
                   "vocab": cfg.vocab, "rotation_copies": n_copies, "window": window, "seed": 1},
        "dtype": "bf16" if cfg.q_dtype == "bf16" else "f32",
        "roofline": roof,
    }
    if full:
        def app_rows():
            rng_new = np.random.default_rng(977)
            x = (rng_new.standard_normal((B, N, cfg.n_kv_heads, D)) * 0.5).astype(np.float32)
            return up(x, "f32") if cfg.q_dtype == "f32" else up(workloads.bf16_bits(x), "bf16")
        new_rows = [app_rows(), app_rows()]
        # stochastic verification at T = 0.8 with standard Gumbel noise drawn once on the device
        gen = torch.Generator(device=dev)
        gen.manual_seed(991)
        gumbel = -torch.log(-torch.log(torch.rand(base["logits"].shape, generator=gen, device=dev,
                                                  dtype=torch.float32).clamp_(1e-12, 1.0)))

        def sample(i):
            sv.sample_accept(copies[i % n_copies]["logits"], gumbel, 0.8, drafts, parent, workspace=ws_g,
                             outputs=(acc, path, tok, None))

        def sample_topk(i):
            sv.sample_accept(copies[i % n_copies]["logits"], gumbel, 0.8, drafts, parent, workspace=ws_g,
                             outputs=(acc, path, tok, None), top_k=50)

        def append(i):
            sv.kv_append(kvs[i % n_copies], new_rows[0], new_rows[1], ctx, max_ctx)

        us = lambda fn: round(timed(capture(fn)) / steps * 1e3, 2)
        rec["breakdown_us"] = {
            "verify_attn": round(attn_us, 2), "greedy_accept": us(accept), "kv_compact": us(compact),
            "greedy_accept_compact": us(accept_compact),
            "sample_accept T=0.8 (not in the step)": us(sample),
            "sample_accept_topk k=50 T=0.8 (not in the step)": us(sample_topk),
            # last: it rewrites the draft rows of the rotated caches
            "kv_append (not in the step)": us(append),
        }
        a_host = acc.cpu().numpy()
        rec["accepted_tokens_per_step"] = int(np.sum(a_host + 1))
    del copies, kvs, base, outs, ws_a, ws_g
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default=DEFAULT_CONFIG, choices=sorted(WORKLOADS))
    ap.add_argument("--per-config", default="all",
                    help="other workloads timed beside the headline ('all', 'none' or e.g. 'C2,C3')")
    ap.add_argument("--per-config-steps", type=int, default=100)
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--rotate-bytes", type=float, default=1.1 * 2 ** 30)
    ap.add_argument("--target-wgs", type=int, default=0, help="attention grid target (0: library default)")
    ap.add_argument("--attn-q4-kernel", default="default", choices=["default", "cooperative", "pipelined", "wide"],
                    help="kernel for 4-bit caches of head dim 256 (default: the library's choice)")
    ap.add_argument("--spin-cycles", type=float, default=1e8,
                    help="spin kernel ahead of the per-call event timing (clock cycles)")
    ap.add_argument("--window", type=int, default=0,
                    help="sliding-window attention over the last W key rows (0: the whole key range)")
    ap.add_argument("--recurrent", default="D2", choices=["none", "D1", "D2", "D3", "D4"],
                    help="Gated DeltaNet tree-state workload timed beside the step (none: skip)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="BYTES",
                    help="only run 5 device-to-device copies of BYTES bytes (reference kernel for "
                         "scaling the FETCH_SIZE / WRITE_SIZE counters) and exit")
    args = ap.parse_args()

    if args.copy_calibration:
        import torch
        src = torch.ones(args.copy_calibration, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": args.copy_calibration, "copies": 5}), flush=True)
        return

    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}); "
              "the verify path would shard by sequence or by KV head with no exchange between GPUs",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import draft_token_verification_sv_amd as sv

    dev = torch.device("cuda:0")
    head = run_workload(sv, dev, args.config, args, args.steps, full=True)
    print(f"bench: {args.config} done ({head['ms_per_step'] * 1e3:.1f} us per step)", file=sys.stderr, flush=True)
    others = [] if args.per_config == "none" else (
        [k for k in sorted(WORKLOADS) if k != args.config] if args.per_config == "all"
        else [k for k in args.per_config.split(",") if k and k != args.config])
    per_config = {}
    for key in others:
        r = run_workload(sv, dev, key, args, args.per_config_steps, full=False)
        per_config[key] = {"workload": r["config"]["workload"], "value": r["value"],
                           "ms_per_step": r["ms_per_step"], "step_us": r["step_us"],
                           "attn_us": r["roofline"]["call_us"], "bound": r["roofline"]["bound"],
                           "frac": r["roofline"]["frac"], "hbm_frac": r["roofline"]["hbm"]["frac"],
                           "traffic": r["roofline"]["traffic"],
                           "algorithmic_bytes": r["roofline"]["hbm"]["algorithmic_bytes"]}
        print(f"bench: {key} done ({r['ms_per_step'] * 1e3:.1f} us per step)", file=sys.stderr, flush=True)

    rec = {
        "metric": METRIC,
        "value": head["value"],
        "unit": "verified draft tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "step_us": head["step_us"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic",
        "config": head["config"],
        "roofline": head["roofline"],
        "breakdown_us": head["breakdown_us"],
        "accepted_tokens_per_step": head["accepted_tokens_per_step"],
        "events_queued_ahead": head["events_queued_ahead"],
        "per_config": per_config,
    }
    if args.target_wgs or args.attn_q4_kernel != "default":
        rec["tuning"] = {"attn_target_wgs": args.target_wgs, "attn_q4_kernel": args.attn_q4_kernel}
    if args.recurrent != "none":
        def capture_timed(steps):
            def capture(fn):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for i in range(steps):
                        fn(i)
                torch.cuda.synchronize()
                return g

            def timed(g):
                s = torch.cuda.current_stream(dev)
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                g.replay()
                torch.cuda.synchronize()
                e0.record(s)
                g.replay()
                e1.record(s)
                torch.cuda.synchronize()
                return e0.elapsed_time(e1)
            return capture, timed
        capture, timed = capture_timed(args.steps)
        rec["recurrent"] = recurrent_bench(sv, dev, args.recurrent, args.steps, args.rotate_bytes, capture, timed)
        if not args.no_cpu_baseline:
            rec["recurrent"]["cpu_baseline"] = recurrent_cpu_baseline(args.recurrent, min(5.0, args.cpu_seconds))
    if not args.no_cpu_baseline:
        allc = cpu_baseline(args.config, args.cpu_seconds)
        one = cpu_baseline(args.config, args.cpu_seconds, one_core=True)
        rec["cpu_baseline"] = dict(allc, one_core={k: one[k] for k in ("value", "unit", "cores", "sample")})
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
